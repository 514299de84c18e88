"""Seeded random batches through both call paths (mm3_index_score then
mm3_index_topk, and mm3_index_decode), every row against the oracle: key
format, heads, rows per request, lengths, top-k, forced blocks and the ragged
layouts are drawn per case, so share and tile boundaries, write-out groups,
the one-launch small-batch path and both selectors meet combinations the
hand-picked cases do not.  Each case is small enough for the oracle to check
every row in a few seconds."""
import numpy as np
import pytest
import torch

import sparse_attention_block_paged_amd as mm3
from tests.test_gpu_parity import (DEV, _ragged_kw, full_check, run_fused, run_prefill_select,
                                   run_split)
from workloads import KFMT_BF16, KFMT_NVFP4, make

pytestmark = pytest.mark.gpu

SEEDS = list(range(64))


def draw(seed):
    """One batch: (label, make() arguments)."""
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
    return label, kw


@pytest.mark.parametrize("seed", SEEDS)
def test_random_batch(seed):
    label, kw = draw(seed)
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
    if w.cu_seqlens_q is None:
        p = mm3.make_problem(w.q, w.kdata, w.block_table, w.seq_lens, w.query_len, w.max_seq_len,
                             w.sm_scale, w.kscales)
        try:
            mm3.prefill_select_workspace_bytes(p, w.topk, True)
        except mm3.Mm3Error:
            return  # not a batch the fused prefill selection takes
        print(f"random{seed}: fused prefill selection too", flush=True)
        s4, o4 = run_prefill_select(w, with_scores=True)
        assert torch.equal(o1, o4), "the fused prefill selection chose different ids"
        assert torch.equal(torch.nan_to_num(s1, nan=7.0), torch.nan_to_num(s4, nan=7.0))
