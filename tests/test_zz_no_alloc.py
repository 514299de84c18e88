"""mm3_index_decode_static, the fused decode that allocates nothing (its
score workspace is the library's own per-GPU device array): on the same
inputs its ids -- and its scores when scores_out is given -- equal those of
mm3_index_decode with a caller workspace, on consecutive calls that reuse the
one array with smaller batches after larger ones."""
import numpy as np
import pytest
import torch

import sparse_attention_block_paged_amd as mm3
from workloads import KFMT_NVFP4, config, make

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _rg(w):
    return dict(cu_seqlens_q=w.cu_seqlens_q, prefix_lens=w.prefix_lens)


def _call(fn, w, scores=False, **kw):
    out = torch.full((w.heads, w.rows, w.topk), -7, dtype=torch.int32, device=DEV)
    s = torch.full((w.heads, w.rows, w.score_width), float("nan"), device=DEV) if scores else None
    fn(w.q, w.kdata, w.block_table, w.seq_lens, w.query_len, w.max_seq_len, w.sm_scale, w.topk,
       w.init_blocks, w.local_blocks, kscales=w.kscales, out=out, scores_out=s, **_rg(w), **kw)
    torch.cuda.synchronize()
    return out, s


def _same(w, label):
    print(f"no-alloc {label}: R={w.num_reqs} rows={w.rows} H={w.heads}", flush=True)
    want, _ = _call(mm3.mm3_index_decode, w)
    got, _ = _call(mm3.mm3_index_decode_static, w)
    assert torch.equal(got, want), f"{label}: static workspace ids differ"
    want_s, s_ref = _call(mm3.mm3_index_decode, w, scores=True)
    got_s, s_got = _call(mm3.mm3_index_decode_static, w, scores=True)
    assert torch.equal(got_s, want_s) and torch.equal(got_s, want)
    assert torch.equal(torch.nan_to_num(s_got, nan=7.0), torch.nan_to_num(s_ref, nan=7.0))


def test_static_workspace_matches_caller_workspace():
    """Larger batches first, then smaller ones on the same array: the chunked
    prefill (its scores fill the whole 64 MiB), the long decode, the NVFP4
    decode, a ragged mixed batch, then a small decode batch."""
    _same(config(4, device=DEV), "chunked prefill")
    _same(config(3, device=DEV), "long decode")
    _same(config(5, device=DEV, R=32), "nvfp4 decode")
    _same(make(name="mixed", R=10, lens=(1300, 5000), Q=1200, H=4, max_seq_len=8192, topk=8, I=1,
               L=2, kfmt=0, seed=9, device=DEV, qlens=[1, 2, 3, 4, 500, 0, 4, 1200, 2, 64],
               prefix="tail"), "mixed ragged")
    _same(config(2, device=DEV, R=8, lens=(900, 6000), max_seq_len=8192), "small decode batch")


def test_static_sparse_table_matches():
    w = config(3, device=DEV, R=6, lens=(1000, 9000), max_seq_len=9216)
    abt = torch.randint(0, 10**6, (w.num_reqs, w.nb_max * 2), dtype=torch.int32, device=DEV)
    res = []
    for fn in (mm3.mm3_index_decode, mm3.mm3_index_decode_static):
        st = torch.full((w.rows, w.topk * 2), -7, dtype=torch.int32, device=DEV)
        ctx = torch.full((w.rows,), -7, dtype=torch.int32, device=DEV)
        out, _ = _call(fn, w, attention_block_table=abt, sparse_block_table_out=st,
                       sparse_context_lens_out=ctx, pages_per_block=2, block_page_stride=2)
        res.append((out, st, ctx))
    for a, b in zip(*res):
        assert torch.equal(a, b)


def test_static_rejects_a_batch_past_its_workspace():
    """Scores of 4 heads x 32800 rows x 128 blocks exceed 64 MiB: the call is
    refused before anything runs, out untouched; with scores_out it runs."""
    w = config(4, device=DEV, Q=8200)
    out = torch.full((w.heads, w.rows, w.topk), -7, dtype=torch.int32, device=DEV)
    with pytest.raises(mm3.Mm3Error) as e:
        mm3.mm3_index_decode_static(w.q, w.kdata, w.block_table, w.seq_lens, w.query_len,
                                    w.max_seq_len, w.sm_scale, w.topk, w.init_blocks,
                                    w.local_blocks, out=out)
    assert e.value.code == -3 and "67174400" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out == -7)
    got, _ = _call(mm3.mm3_index_decode_static, w, scores=True)
    want, _ = _call(mm3.mm3_index_decode, w)
    assert torch.equal(got, want)
