"""Seeded random batches through every call path, every row against the
oracle: key format, heads, rows per request, lengths, top-k, forced blocks
and the ragged layouts are drawn per case, so share and tile boundaries,
write-out groups, the one-launch small-batch path and both selectors meet
combinations the hand-picked cases do not.  Each case is small enough for
the oracle to check every row in a few seconds."""
import numpy as np
import pytest
import torch

import sparse_attention_block_paged_amd as mm3
from tests import _parity as P
from tests.test_gpu_parity import (DEV, _np, _ragged_kw, full_check, run_fused, run_prefill_select,
                                   run_split)
from workloads import KFMT_BF16, KFMT_NVFP4, make

pytestmark = pytest.mark.gpu

SEEDS = list(range(64))


def draw(seed):
    """One batch: (label, make() arguments, rng for the case's other draws)."""
    rng = np.random.default_rng(1000 + seed)
    kfmt = int(rng.choice([KFMT_BF16, KFMT_NVFP4]))
    H = int(rng.choice([1, 2, 4, 8]))
    mode = str(rng.choice(["decode", "prefill", "ragged"]))
    R = int(rng.integers(1, 5))
    msl = int(rng.choice([128, 300, 1000, 2048, 2500, 4096]))
    lo = int(rng.integers(1, msl + 1))
    lens = (min(lo, msl), msl)
    topk = int(rng.choice([4, 8, 16, 20, 33]))
    I = int(rng.integers(0, 3))
    L = int(rng.integers(0, 4))
    if I + L > topk:
        I, L = 1, 1
    kw = dict(name=f"random{seed}", R=R, lens=lens, H=H, max_seq_len=msl, topk=topk, I=I, L=L,
              kfmt=kfmt, seed=seed, device=DEV)
    if mode == "decode":
        kw["Q"] = int(rng.integers(1, 16 // H + 1))
    elif mode == "prefill":
        kw["Q"] = int(rng.integers(16 // H + 1, max(16 // H + 2, 300 // H)))
    else:
        Q = int(rng.integers(1, max(2, 400 // H)))
        kw["Q"] = Q
        kw["qlens"] = [(0, Q)] * R
        kw["prefix"] = str(rng.choice(["none", "tail", "gap"]))
        if kw["prefix"] == "none":
            kw["prefix"] = None
    label = (f"random{seed} {mode} {'nvfp4' if kfmt else 'bf16'} R={R} H={H} Q={kw['Q']} "
             f"msl={msl} topk={topk} I={I} L={L} prefix={kw.get('prefix')}")
    return label, kw, rng


def sparse_check(w, ids, rng, seed):
    """One index head: mm3_index_decode with the sparse-table arguments gives
    the same ids, and the table and context lengths the oracle builds."""
    import oracle
    P_ = int(rng.choice([1, 2, 4]))
    stride = P_ * int(rng.choice([1, 2]))
    abt = torch.randint(0, 10**6, (w.num_reqs, max(1, w.nb_max) * stride), dtype=torch.int32,
                        device=DEV)
    st = torch.full((w.rows, w.topk * P_), -7, dtype=torch.int32, device=DEV)
    ctx = torch.full((w.rows,), -7, dtype=torch.int32, device=DEV)
    out = torch.full((1, w.rows, w.topk), -7, dtype=torch.int32, device=DEV)
    mm3.mm3_index_decode(w.q, w.kdata, w.block_table, w.seq_lens, w.query_len, w.max_seq_len,
                         w.sm_scale, w.topk, w.init_blocks, w.local_blocks, kscales=w.kscales, out=out,
                         attention_block_table=abt, sparse_block_table_out=st,
                         sparse_context_lens_out=ctx, pages_per_block=P_, block_page_stride=stride,
                         **_ragged_kw(w))
    torch.cuda.synchronize()
    assert torch.equal(out, ids), f"random{seed}: ids with the sparse table differ"
    st_ref, ctx_ref = oracle.sparse_block_table(ids[0].cpu().numpy(), w.seq_lens.cpu().numpy(),
                                                w.query_len, abt.cpu().numpy(), P_, stride,
                                                cu_seqlens_q=_np(w.cu_seqlens_q),
                                                prefix_lens=_np(w.prefix_lens))
    assert np.array_equal(st.cpu().numpy(), st_ref), f"random{seed}: sparse table (P={P_}, stride={stride})"
    assert np.array_equal(ctx.cpu().numpy(), ctx_ref), f"random{seed}: sparse context lengths"
    print(f"random{seed}: sparse table P={P_} stride={stride}", flush=True)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_batch(seed):
    label, kw, rng = draw(seed)
    w = make(**kw)
    print(f"case {label}: rows={w.rows}", flush=True)
    s1, o1 = run_split(w)
    full_check(w, s1, o1, f"random{seed} split")
    s2, o2 = run_fused(w, with_scores=True)
    full_check(w, s2, o2, f"random{seed} fused")
    assert torch.equal(o1, o2), "the two call paths chose different ids"
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32)), "the two call paths' scores differ"
    _, o3 = run_fused(w, with_scores=False)
    assert torch.equal(o1, o3), "the workspace-only call chose different ids"
    n = mm3.mm3_index_decode_launches(w.q, w.kdata, w.block_table, w.seq_lens, w.query_len,
                                      w.max_seq_len, w.sm_scale, kscales=w.kscales, **_ragged_kw(w))
    assert n in (1, 2)
    print(f"random{seed}: {n} launch(es) in mm3_index_decode", flush=True)
    # the call that allocates nothing (the library's own score workspace)
    o4 = torch.full_like(o1, -7)
    mm3.mm3_index_decode_static(w.q, w.kdata, w.block_table, w.seq_lens, w.query_len, w.max_seq_len,
                                w.sm_scale, w.topk, w.init_blocks, w.local_blocks, o4,
                                kscales=w.kscales, **_ragged_kw(w))
    torch.cuda.synchronize()
    assert torch.equal(o1, o4), "mm3_index_decode_static chose different ids"
    # the selection again with each row's block count given instead of positions
    pos = P.row_positions(w.seq_lens.cpu().numpy(), w.query_len, _np(w.cu_seqlens_q),
                          _np(w.prefix_lens))
    nv = torch.from_numpy(np.where(pos >= 0, pos // 128 + 1, 0).astype(np.int32)).to(DEV)
    o5 = torch.full_like(o1, -7)
    mm3.mm3_index_topk_blocks(s1, nv, w.max_seq_len, w.topk, w.init_blocks, w.local_blocks, out=o5)
    torch.cuda.synchronize()
    assert torch.equal(o1, o5), "mm3_index_topk_blocks chose different ids"
    if w.heads == 1:
        sparse_check(w, o1, rng, seed)
    if w.cu_seqlens_q is None:
        p = mm3.make_problem(w.q, w.kdata, w.block_table, w.seq_lens, w.query_len, w.max_seq_len,
                             w.sm_scale, w.kscales)
        try:
            mm3.prefill_select_workspace_bytes(p, w.topk, True)
        except mm3.Mm3Error:
            return  # not a batch the fused prefill selection takes
        print(f"random{seed}: fused prefill selection too", flush=True)
        s6, o6 = run_prefill_select(w, with_scores=True)
        assert torch.equal(o1, o6), "the fused prefill selection chose different ids"
        assert torch.equal(torch.nan_to_num(s1, nan=7.0), torch.nan_to_num(s6, nan=7.0))
