"""Pins for the oracle's top-k selection and sparse block table (CPU only).

Selection (page "vllm.models.minimax_m3.amd.ops.index_topk", module docstring;
minimax_m3_index_decode docstring; page "indexer_cp_exchange", module
docstring on pinned forced blocks): per (head, row), the best topk visible
blocks with the init and local blocks always kept, 0-indexed ids, -1 padding.

Pins: hand-worked rows (tests/golden/topk_cases.txt), torch's stable sort in
the unforced case, closed forms (nv <= topk, all-equal scores), and the
exchange property every correct selection has on random rows with ties.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "topk_cases.txt")


def _one_row(scores, k, I, L):
    """Select for a single row with nv = len(scores): R=1, Q=1 and a length
    that puts the row in the last visible block."""
    nv = len(scores)
    s = np.asarray(scores, dtype=np.float32).reshape(1, 1, nv)
    seq = np.array([(nv - 1) * 128 + 1], dtype=np.int32)
    return oracle.topk(s, seq, 1, k, I, L)[0, 0]


def test_golden_rows():
    n = 0
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            head, sc, want = [p.split() for p in line.split("|")]
            k, I, L = map(int, head)
            got = _one_row([float(x) for x in sc], k, I, L)
            assert got.tolist() == [int(x) for x in want], line
            n += 1
    assert n >= 10


def _forced(nv, I, L):
    return set(range(min(I, nv))) | set(range(max(0, nv - L), nv))


def _check_row(ids, scores, nv, k, I, L):
    ids = list(ids)
    sel = [i for i in ids if i >= 0]
    assert ids == sel + [-1] * (k - len(sel))  # -1 only as trailing padding
    assert sel == sorted(set(sel))  # ascending, distinct
    assert all(0 <= i < nv for i in sel)
    assert len(sel) == min(k, nv)
    F = _forced(nv, I, L)
    assert F <= set(sel)
    chosen = set(sel) - F
    rest = set(range(nv)) - set(sel)
    for x in chosen:
        for y in rest:
            assert scores[x] > scores[y] or (scores[x] == scores[y] and x < y)


@pytest.mark.parametrize("seed", range(6))
def test_exchange_property_random_rows(seed):
    rng = np.random.default_rng(seed)
    for _ in range(200):
        nv = int(rng.integers(1, 80))
        k = int(rng.integers(1, 20))
        I = int(rng.integers(0, 3))
        L = int(rng.integers(0, 3))
        if I + L > k:
            continue
        # few distinct values -> many ties
        sc = rng.integers(-4, 5, size=nv).astype(np.float32) * np.float32(0.5)
        sc[rng.random(nv) < 0.1] = -0.0
        got = _one_row(sc, k, I, L)
        _check_row(got, sc, nv, k, I, L)


def test_unforced_equals_stable_sort():
    rng = np.random.default_rng(3)
    for _ in range(100):
        nv = int(rng.integers(17, 200))
        sc = rng.integers(0, 30, size=nv).astype(np.float32)
        k = 16
        got = _one_row(sc, k, 0, 0)
        order = torch.sort(torch.from_numpy(-sc), stable=True).indices[:k]
        assert got.tolist() == sorted(order.tolist())


def test_small_rows_take_everything():
    rng = np.random.default_rng(4)
    for nv in range(1, 17):
        got = _one_row(rng.standard_normal(nv), 16, 1, 2)
        assert got.tolist() == list(range(nv)) + [-1] * (16 - nv)


def test_all_equal_scores():
    for nv in [20, 100, 1000]:
        got = _one_row(np.full(nv, 3.0), 16, 1, 2)
        assert got.tolist() == list(range(0, 14)) + [nv - 2, nv - 1]


def test_rows_before_position_zero_are_empty():
    s = np.zeros((1, 8, 16), dtype=np.float32)
    seq = np.array([2, 0], dtype=np.int32)  # Q=4: rows 0,1 and 4..7 have pos < 0
    got = oracle.topk(s, seq, 4, 3, 1, 1)
    for t in [0, 1, 4, 5, 6, 7]:
        assert got[0, t].tolist() == [-1, -1, -1]
    assert got[0, 2].tolist() == [0, -1, -1]


def test_multi_head_rows_are_independent():
    rng = np.random.default_rng(5)
    H, T, W = 3, 8, 32
    s = rng.standard_normal((H, T, W)).astype(np.float32)
    seq = np.array([2000, 3000], dtype=np.int32)
    got = oracle.topk(s, seq, 4, 5, 1, 1)
    for h in range(H):
        alone = oracle.topk(s[h:h + 1], seq, 4, 5, 1, 1)
        assert np.array_equal(got[h], alone[0])


def test_rejects_bad_arguments():
    s = np.zeros((1, 4, 16), dtype=np.float32)
    seq = np.array([500], dtype=np.int32)
    with pytest.raises(ValueError):
        oracle.topk(s, seq, 4, 2, 2, 1)  # I + L > topk


def test_sparse_block_table_hand_worked():
    # P = 2 attention pages per 128-token block, stride 2P = 4 entries
    abt = np.array([[10, 11, 12, 13, 20, 21, 22, 23, 30, 31, 32, 33, 40, 41, 42, 43]],
                   dtype=np.int32)
    pos = 3 * 128 + 9  # nv = 4, last block holds 10 visible tokens
    seq = np.array([pos + 1], dtype=np.int32)
    ids = np.array([[0, 2, 3, -1]], dtype=np.int32)
    sp, ctx = oracle.sparse_block_table(ids, seq, 1, abt, 2, 4)
    assert sp.tolist() == [[10, 11, 30, 31, 40, 41, -1, -1]]
    assert ctx.tolist() == [128 + 128 + 10]
    # stride P: block b's pages are entries [2b, 2b+2)
    sp, ctx = oracle.sparse_block_table(ids, seq, 1, abt, 2, 2)
    assert sp.tolist() == [[10, 11, 20, 21, 22, 23, -1, -1]]
    assert ctx.tolist() == [266]


# ------------------------------------------------------------ ragged rows

def test_ragged_rows_select_by_their_own_position():
    """Ragged batch (cu_seqlens_q, prefix_lens): each row selects as a
    single-row problem whose position is prefix + j."""
    rng = np.random.default_rng(7)
    seq = np.array([3000, 700, 5000], dtype=np.int32)
    cu = np.array([0, 2, 2, 7], dtype=np.int32)  # request 1 has no rows
    pre = np.array([1500, 0, 4000], dtype=np.int32)
    T, W = 7, 48
    s = rng.integers(-8, 8, size=(1, T, W)).astype(np.float32)
    got = oracle.topk(s, seq, 5, 6, 1, 2, cu_seqlens_q=cu, prefix_lens=pre)
    for r in range(3):
        for j in range(cu[r + 1] - cu[r]):
            t = cu[r] + j
            nv = (int(pre[r]) + j) // 128 + 1
            _check_row(got[0, t], s[0, t], nv, 6, 1, 2)
            assert got[0, t].tolist() == _one_row(s[0, t, :nv], 6, 1, 2).tolist()


def test_ragged_without_prefix_uses_the_last_tokens():
    s = np.zeros((1, 3, 16), dtype=np.float32)
    seq = np.array([129, 1], dtype=np.int32)
    cu = np.array([0, 2, 3], dtype=np.int32)
    # request 0: rows at positions 127, 128 (nv 1, 2); request 1: position 0
    got = oracle.topk(s, seq, 2, 4, 0, 0, cu_seqlens_q=cu)
    assert got[0].tolist() == [[0, -1, -1, -1], [0, 1, -1, -1], [0, -1, -1, -1]]


def test_ragged_sparse_table_context_lengths():
    abt = np.arange(100, 140, dtype=np.int32).reshape(2, 20)
    seq = np.array([1000, 300], dtype=np.int32)
    cu = np.array([0, 1, 3], dtype=np.int32)
    pre = np.array([260, 129], dtype=np.int32)
    ids = np.array([[0, 2, -1], [0, 1, -1], [1, -1, -1]], dtype=np.int32)
    sp, ctx = oracle.sparse_block_table(ids, seq, 2, abt, 1, 1, cu_seqlens_q=cu, prefix_lens=pre)
    assert sp.tolist() == [[100, 102, -1], [120, 121, -1], [121, -1, -1]]
    # row 0 at 260: block 0 full, block 2 holds 260-256+1 = 5; row 1 at 129:
    # 128 + 2; row 2 at 130: block 1 holds 3
    assert ctx.tolist() == [133, 130, 3]
