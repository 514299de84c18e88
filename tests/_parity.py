"""Comparison helpers for the GPU parity tests (HIP path vs the CPU oracle).

Bar: scores within 1e-3 relative or 1e-4 absolute of the oracle on every
visible (head, row, block); block ids bit-exact, except where a row's
selected set differs only by non-forced blocks whose oracle score is within
that same tolerance of the oracle's k-th (smallest selected non-forced)
score -- a near-tie at the k-th boundary, counted and reported.
"""
from __future__ import annotations

import numpy as np

import oracle

RTOL = 1e-3
ATOL = 1e-4


def tol(x):
    return np.maximum(ATOL, RTOL * np.abs(x))


def check_scores(s_gpu, s_ref, rows=None):
    """s_* [H, T, W]; s_ref NaN where not visible.  With rows, only those rows
    are compared.  GPU entries outside the visible set must still hold the NaN
    the test pre-filled (nothing else is written)."""
    if rows is not None:
        s_gpu, s_ref = s_gpu[:, rows], s_ref[:, rows]
    vis = ~np.isnan(s_ref)
    untouched = np.isnan(s_gpu[:, :, : s_ref.shape[2]])
    assert np.array_equal(vis, ~untouched), (
        f"written set differs: {int((vis & untouched).sum())} visible entries unwritten, "
        f"{int((~vis & ~untouched).sum())} invisible entries written")
    err = np.abs(s_gpu[vis] - s_ref[vis])
    bad = err > tol(s_ref[vis])
    assert not bad.any(), (
        f"{int(bad.sum())} scores out of tolerance; worst err {err.max():.3g}")
    return float(err.max()) if err.size else 0.0


def _forced(nv, I, L):
    return set(range(min(I, nv))) | set(range(max(0, nv - L), nv))


def row_positions(seq_lens, Q, cu=None, prefix=None):
    """Position of every row [T] (int64).  Uniform batches: request r's row j
    at seq_lens[r] - Q + j.  Ragged: rows cu[r]..cu[r+1]-1, row j at
    prefix[r] + j, or seq_lens[r] - rows + j without prefix."""
    seq = np.asarray(seq_lens, dtype=np.int64)
    if cu is None:
        t = np.arange(seq.size * Q)
        return seq[t // Q] - Q + t % Q
    cu = np.asarray(cu, dtype=np.int64)
    n = np.diff(cu)
    first = np.asarray(prefix, dtype=np.int64) if prefix is not None else seq - n
    req = np.repeat(np.arange(seq.size), n)
    j = np.arange(int(cu[-1])) - cu[req]
    return first[req] + j


def check_ids(ids_gpu, ids_ref, s_ref, seq_lens, Q, topk, I, L, rows=None, cu=None, prefix=None):
    """ids_* [H, T, topk] int32.  Returns the number of near-tie rows."""
    H = ids_ref.shape[0]
    pos_all = row_positions(seq_lens, Q, cu, prefix)
    rows = range(ids_ref.shape[1]) if rows is None else rows
    near = 0
    for h in range(H):
        for t in rows:
            g, o = ids_gpu[h, t], ids_ref[h, t]
            if np.array_equal(g, o):
                continue
            pos = int(pos_all[t])
            nv = pos // 128 + 1 if pos >= 0 else 0
            F = _forced(nv, I, L)
            gs = set(int(x) for x in g if x >= 0)
            os_ = set(int(x) for x in o if x >= 0)
            sel = [int(x) for x in g if x >= 0]
            assert sel == sorted(gs) and len(sel) == len(gs), f"row (h={h},t={t}) not ascending/distinct: {g}"
            assert list(g[len(sel):]) == [-1] * (topk - len(sel)), f"row (h={h},t={t}) bad padding: {g}"
            diff = gs ^ os_
            assert len(gs) == len(os_), f"row (h={h},t={t}) selects {len(gs)} vs oracle {len(os_)}: {g} vs {o}"
            assert not (diff & F), f"row (h={h},t={t}) differs on forced blocks: {g} vs {o}"
            kth = min(s_ref[h, t, b] for b in os_ - F)
            for b in diff:
                assert abs(s_ref[h, t, b] - kth) <= tol(kth), (
                    f"row (h={h},t={t}) differs beyond a near-tie: {g} vs oracle {o}; "
                    f"block {b} score {s_ref[h, t, b]} vs k-th {kth}")
            near += 1
    return near


def check_invariants(ids, seq_lens, Q, topk, I, L, cu=None, prefix=None):
    """Every row: ascending distinct ids < nv, trailing -1 only, count =
    min(topk, nv), forced blocks present.  Vectorised over [H, T, topk]."""
    H, T, K = ids.shape
    pos = row_positions(seq_lens, Q, cu, prefix)
    assert pos.size == T
    nv = np.where(pos >= 0, pos // 128 + 1, 0)
    cnt = np.minimum(nv, topk)
    valid = ids >= 0
    n_valid = valid.sum(-1)
    assert np.array_equal(n_valid, np.broadcast_to(cnt, (H, T))), "wrong id count"
    slot = np.arange(K)
    want_valid = np.broadcast_to(slot[None, None, :] < cnt[None, :, None], valid.shape)
    assert np.array_equal(valid, want_valid), "-1 not trailing"
    diffs = np.diff(ids, axis=-1)
    inner = np.broadcast_to(slot[None, None, 1:] < cnt[None, :, None], diffs.shape)
    assert np.all(diffs[inner] > 0), "ids not strictly ascending"
    assert np.all(ids[valid] < np.broadcast_to(nv[None, :, None], ids.shape)[valid]), "id >= nv"
    # forced blocks: first min(I, nv) ids are 0..; last L selected are nv-L..nv-1
    for i in range(I):
        m = nv > i
        assert np.all(ids[:, m, i] == i), "init block missing"
    for l in range(1, L + 1):
        m = nv >= l
        last = np.take_along_axis(ids, (cnt - l).clip(0)[None, :, None].repeat(H, 0), -1)[..., 0]
        assert np.all(last[:, m] == (nv - l)[m][None, :]), "local block missing"


def oracle_forward(a, width, topk, I, L, rows=None):
    return oracle.forward(a["q_bits"], a["kfmt"], a["kdata"], a["kscales"], a["block_table"],
                          a["seq_lens"], a["query_len"], a["sm_scale"], topk, I, L, width,
                          rows=rows, cu_seqlens_q=a.get("cu_seqlens_q"),
                          prefix_lens=a.get("prefix_lens"))
