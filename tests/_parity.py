"""Comparison helpers for the GPU parity tests (HIP path vs the CPU oracle).

Bar: scores within 1e-3 relative or 1e-4 absolute of the oracle on every
visible (head, row, block); block ids bit-exact, except where a row's
selected set differs only by non-forced blocks whose oracle score is within
that same tolerance of the oracle's k-th (smallest selected non-forced)
score -- a near-tie at the k-th boundary, counted, reported and bounded.

A near-tie is only a difference the rounding of distinct values can explain:
the oracle also returns every score before its one rounding to fp32 (sm_scale
times the fp64 block maximum), and two blocks whose unrounded scores are equal
hold keys with the same largest dot product -- a true tie, which must go to
the lower id on both sides.  A GPU row that swaps such a pair fails.

This module imports numpy and the oracle only (no torch), so the oracle
worker processes of the GPU tests can import it.
"""
from __future__ import annotations

import numpy as np

import oracle

RTOL = 1e-3
ATOL = 1e-4

# (label, (head, row) pairs compared, near-tie rows, exact boundary ties),
# appended by record() and printed at the end of the session
LOG: list = []


def tol(x):
    return np.maximum(ATOL, RTOL * np.abs(x))


def near_tie_bound(pairs: int) -> int:
    """Most near-tie rows a comparison of `pairs` (head, row) pairs may hold.
    A row flips only when its k-th gap is within the GPU's fp32 accumulation
    error (~1e-6 relative), which the workloads' score spacing (~0.03 at the
    k-th boundary) makes rarer than 1 in 10^4; the bound leaves a tenfold
    margin."""
    return max(2, pairs // 1000)


def record(label: str, pairs: int, near: int, ties: int):
    assert near <= near_tie_bound(pairs), (
        f"{label}: {near} near-tie rows in {pairs} compared, above the bound "
        f"{near_tie_bound(pairs)}")
    LOG.append((label, int(pairs), int(near), int(ties)))


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


def check_scores(s_gpu, s_ref):
    """s_* [H, n, W] over the same rows; s_ref NaN where not visible.  GPU
    entries outside the visible set must still hold the NaN the test
    pre-filled (nothing else is written).  Returns the largest error."""
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


def _masks(ids, s64, pos, topk, I, L):
    """Per (head, row): visible, forced and oracle-selected block masks
    [H, n, W] of the rows at positions pos."""
    H, n, W = s64.shape
    nv = np.where(pos >= 0, pos // 128 + 1, 0)
    b = np.arange(W)
    vis = b[None, :] < nv[:, None]
    forced = vis & ((b[None, :] < I) | (b[None, :] >= nv[:, None] - L))
    sel = np.zeros((H, n, W + 1), dtype=bool)
    np.put_along_axis(sel, np.where(ids >= 0, ids, W).astype(np.int64), True, axis=-1)
    return nv, vis, forced, sel[..., :W]


def boundary_ties(ids_ref, s64, pos, topk, I, L):
    """(head, row) pairs whose k-th boundary is an exact tie: the oracle's
    smallest selected non-forced block and its best unselected one have
    equal unrounded scores."""
    nv, vis, forced, sel = _masks(ids_ref, s64, pos, topk, I, L)
    cand = (vis & ~forced)[None]
    kth = np.where(sel & cand, s64, np.inf).min(-1)
    best_out = np.where(~sel & cand, s64, -np.inf).max(-1)
    return int(((kth == best_out) & (nv > topk)[None, :]).sum())


def check_ids(ids_gpu, ids_ref, s_ref, s64, pos, topk, I, L):
    """ids_* [H, n, topk], s_ref / s64 [H, n, W] and pos [n] over the same
    rows.  Returns the number of near-tie rows (selected sets that differ
    within the rule above)."""
    pos = np.asarray(pos, dtype=np.int64)
    rows_h, rows_t = np.nonzero((ids_gpu != ids_ref).any(-1))
    for h, t in zip(rows_h.tolist(), rows_t.tolist()):
        g, o = ids_gpu[h, t], ids_ref[h, t]
        p = int(pos[t])
        nv = p // 128 + 1 if p >= 0 else 0
        F = set(range(min(I, nv))) | set(range(max(0, nv - L), nv))
        gs = set(int(x) for x in g if x >= 0)
        os_ = set(int(x) for x in o if x >= 0)
        sel = [int(x) for x in g if x >= 0]
        where = f"row (h={h}, local t={t}, pos={p})"
        assert sel == sorted(gs) and len(sel) == len(gs), f"{where} not ascending/distinct: {g}"
        assert list(g[len(sel):]) == [-1] * (topk - len(sel)), f"{where} bad padding: {g}"
        assert len(gs) == len(os_), f"{where} selects {len(gs)} vs oracle {len(os_)}: {g} vs {o}"
        diff = gs ^ os_
        assert not (diff & F), f"{where} differs on forced blocks: {g} vs {o}"
        assert all(b < nv for b in gs), f"{where} selects an invisible block: {g}"
        assert os_ - F, f"{where} differs where every selected block is forced: {g} vs {o}"
        kth = min(s_ref[h, t, b] for b in os_ - F)
        for b in diff:
            assert abs(s_ref[h, t, b] - kth) <= tol(kth), (
                f"{where} differs beyond a near-tie: {g} vs oracle {o}; "
                f"block {b} score {s_ref[h, t, b]} vs k-th {kth}")
        for b_gpu in gs - os_:
            for b_orc in os_ - gs:
                assert s64[h, t, b_gpu] != s64[h, t, b_orc], (
                    f"{where} breaks an exact tie toward the higher id: GPU {g} vs oracle {o}; "
                    f"blocks {b_orc} and {b_gpu} have the same unrounded score {s64[h, t, b_orc]!r}")
    return len(rows_h)


def compare(s_gpu, ids_gpu, s_ref, s64, ids_ref, pos, topk, I, L):
    """Scores (when s_gpu is given) and ids of the same rows.  Returns
    (max score error, near-tie rows, exact boundary ties)."""
    err = check_scores(s_gpu, s_ref) if s_gpu is not None else 0.0
    near = check_ids(ids_gpu, ids_ref, s_ref, s64, pos, topk, I, L)
    ties = boundary_ties(ids_ref, s64, pos, topk, I, L)
    return err, near, ties


def oracle_forward(a, width, topk, I, L, rows=None):
    """(scores, unrounded scores, ids) of the oracle for host arrays a."""
    return oracle.forward(a["q_bits"], a["kfmt"], a["kdata"], a["kscales"], a["block_table"],
                          a["seq_lens"], a["query_len"], a["sm_scale"], topk, I, L, width,
                          rows=rows, cu_seqlens_q=a.get("cu_seqlens_q"),
                          prefix_lens=a.get("prefix_lens"), with64=True)


def positions_of(a):
    return row_positions(a["seq_lens"], a["query_len"], a.get("cu_seqlens_q"),
                         a.get("prefix_lens"))


def check_task(task):
    """One comparison job, run in an oracle worker process: host arrays a of
    some requests, the local rows to compare (None: all), and the GPU's
    scores (or None) and ids of exactly those rows.  Returns (rows compared,
    max score error, near-tie rows, exact boundary ties); a mismatch raises."""
    a, rows, width, topk, I, L, s_gpu, ids_gpu = task
    s_ref, s64, ids_ref = oracle_forward(a, width, topk, I, L, rows=rows)
    pos = positions_of(a)
    if rows is not None:
        rows = np.asarray(rows)
        s_ref, s64, ids_ref, pos = s_ref[:, rows], s64[:, rows], ids_ref[:, rows], pos[rows]
    err, near, ties = compare(s_gpu, ids_gpu, s_ref, s64, ids_ref, pos, topk, I, L)
    return ids_ref.shape[0] * ids_ref.shape[1], err, near, ties


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
