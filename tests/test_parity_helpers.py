"""The GPU parity checkers, exercised on the CPU with oracle outputs and
planted mistakes (so a broken checker cannot pass a broken kernel)."""
import numpy as np
import pytest

from tests import _parity as P
from workloads import config, host_arrays


@pytest.fixture(scope="module")
def case():
    w = config(2, device="cpu", R=4, lens=(300, 3000), max_seq_len=4096)
    a = host_arrays(w)
    s, s64, ids = P.oracle_forward(a, w.score_width, w.topk, w.init_blocks, w.local_blocks)
    return w, a, s, s64, ids


def _ids(w, a, g, ids, s, s64):
    return P.check_ids(g, ids, s, s64, P.positions_of(a), w.topk, w.init_blocks, w.local_blocks)


def _inv(w, a, ids):
    P.check_invariants(ids, a["seq_lens"], w.query_len, w.topk, w.init_blocks, w.local_blocks)


def test_accepts_oracle_output(case):
    w, a, s, s64, ids = case
    _inv(w, a, ids)
    assert _ids(w, a, ids, ids, s, s64) == 0
    assert P.check_scores(s.copy(), s) == 0.0


def _row_with_choice(w, a, ids):
    """A (head, row) that has more visible blocks than topk."""
    for t in range(ids.shape[1]):
        pos = int(a["seq_lens"][t // w.query_len]) - w.query_len + t % w.query_len
        if pos // 128 + 1 > w.topk:
            return 1 % ids.shape[0], t, pos // 128 + 1
    raise AssertionError("no row with a choice")


@pytest.mark.parametrize("mistake", ["hole", "unsorted", "dup", "out_of_range", "drop_init",
                                     "drop_local", "swap_worse"])
def test_planted_id_mistakes_are_caught(case, mistake):
    w, a, s, s64, ids = case
    h, t, nv = _row_with_choice(w, a, ids)
    bad = ids.copy()
    row = bad[h, t]
    if mistake == "hole":
        row[3] = -1
    elif mistake == "unsorted":
        row[[2, 3]] = row[[3, 2]]
    elif mistake == "dup":
        row[3] = row[2]
    elif mistake == "out_of_range":
        row[-1] = nv
    elif mistake == "drop_init":
        row[0] = [b for b in range(nv) if b not in row][0]
        row.sort()
    elif mistake == "drop_local":
        row[-1] = [b for b in range(nv) if b not in row][0]
        row.sort()
    elif mistake == "swap_worse":
        chosen = [b for b in row if b not in (0, nv - 1, nv - 2)]
        rest = [b for b in range(nv) if b not in row]
        worst_rest = min(rest, key=lambda b: s[h, t, b])
        row[list(row).index(chosen[0])] = worst_rest
        row.sort()
    with pytest.raises(AssertionError):
        _inv(w, a, bad)
        _ids(w, a, bad, ids, s, s64)


def _boundary(w, ids, s, h, t, nv):
    """The oracle's k-th (smallest selected non-forced) block and its best
    unselected one, for row (h, t)."""
    row = ids[h, t]
    forced = {0, nv - 1, nv - 2}
    kth_b = min((b for b in row if b not in forced), key=lambda b: s[h, t, b])
    out_b = max((b for b in range(nv) if b not in row), key=lambda b: s[h, t, b])
    return kth_b, out_b


def _swap(ids, h, t, a_b, b_b):
    g = ids.copy()
    g[h, t, list(g[h, t]).index(a_b)] = b_b
    g[h, t].sort()
    return g


def test_near_tie_is_accepted(case):
    """A block just inside the tolerance of the k-th, with a different
    unrounded score, may be swapped for it."""
    w, a, s, s64, ids = case
    h, t, nv = _row_with_choice(w, a, ids)
    kth_b, out_b = _boundary(w, ids, s, h, t, nv)
    s2, s64b = s.copy(), s64.copy()
    s2[h, t, out_b] = s2[h, t, kth_b] - 1e-5  # within tolerance below the k-th
    s64b[h, t, out_b] = s64b[h, t, kth_b] - 1e-5
    g = _swap(ids, h, t, kth_b, out_b)
    assert P.check_ids(g, ids, s2, s64b, P.positions_of(a), w.topk, w.init_blocks,
                       w.local_blocks) == 1


def test_exact_tie_toward_higher_id_is_caught(case):
    """Blocks with equal unrounded scores are a true tie: the oracle keeps the
    lower id, and a GPU row that keeps the higher one fails, even though the
    score gap (0) is inside the tolerance."""
    w, a, s, s64, ids = case
    h, t, nv = _row_with_choice(w, a, ids)
    kth_b, out_b = _boundary(w, ids, s, h, t, nv)
    s2, s64b = s.copy(), s64.copy()
    s2[h, t, out_b] = s2[h, t, kth_b]
    s64b[h, t, out_b] = s64b[h, t, kth_b]
    g = _swap(ids, h, t, kth_b, out_b)
    with pytest.raises(AssertionError, match="exact tie"):
        P.check_ids(g, ids, s2, s64b, P.positions_of(a), w.topk, w.init_blocks, w.local_blocks)
    # equal fp32 scores from distinct unrounded values: a near-tie
    s64b[h, t, out_b] = np.nextafter(s64b[h, t, kth_b], -np.inf)
    assert P.check_ids(g, ids, s2, s64b, P.positions_of(a), w.topk, w.init_blocks,
                       w.local_blocks) == 1


def test_boundary_ties_counted():
    """One row, hand-made: 8 visible blocks, topk 4, 1 init + 1 local block;
    the oracle selects {0, 3, 5, 7}.  With block 2's unrounded score equal to
    block 3's (the k-th), the boundary is an exact tie; lowered by one ulp,
    it is not."""
    s64 = np.array([[[9.0, 1.0, 4.0, 4.0, 2.0, 6.0, 3.0, 0.5]]])
    ids = np.array([[[0, 3, 5, 7]]], dtype=np.int32)
    pos = np.array([8 * 128 - 1])
    # blocks 2 and 3 tie at 4.0; the oracle keeps 2 (the lower id)
    assert P.boundary_ties(np.array([[[0, 2, 5, 7]]], dtype=np.int32), s64, pos, 4, 1, 1) == 1
    s64[0, 0, 2] = np.nextafter(4.0, 0.0)
    assert P.boundary_ties(ids, s64, pos, 4, 1, 1) == 0
    # fewer visible blocks than topk: no boundary at all
    assert P.boundary_ties(ids, s64, np.array([3 * 128 - 1]), 4, 1, 1) == 0


def test_near_tie_bound_enforced():
    P.record("bound-ok", 5000, 5, 0)
    with pytest.raises(AssertionError, match="above the bound"):
        P.record("bound-exceeded", 5000, 6, 0)
    del P.LOG[-1:]


def test_planted_score_mistakes_are_caught(case):
    w, a, s, s64, ids = case
    g = s.copy()
    vis = np.argwhere(~np.isnan(s))
    h, t, b = vis[len(vis) // 2]
    g[h, t, b] *= 1.01
    with pytest.raises(AssertionError):
        P.check_scores(g, s)
    g = s.copy()
    g[h, t, b] = np.nan  # unwritten visible entry
    with pytest.raises(AssertionError):
        P.check_scores(g, s)
    g = s.copy()
    inv = np.argwhere(np.isnan(s))[0]
    g[tuple(inv)] = 0.0  # write outside the visible set
    with pytest.raises(AssertionError):
        P.check_scores(g, s)


def test_row_positions_hand_worked():
    """Positions of a uniform and of a ragged batch, written out by hand."""
    seq = np.array([10, 3], dtype=np.int32)
    assert P.row_positions(seq, 4).tolist() == [6, 7, 8, 9, -1, 0, 1, 2]
    cu = np.array([0, 2, 2, 5], dtype=np.int32)
    seq3 = np.array([10, 7, 300], dtype=np.int32)
    # no prefix: each request's rows are its last tokens
    assert P.row_positions(seq3, 8, cu).tolist() == [8, 9, 297, 298, 299]
    pre = np.array([4, 0, 128], dtype=np.int32)
    assert P.row_positions(seq3, 8, cu, pre).tolist() == [4, 5, 128, 129, 130]


def test_ragged_checkers_catch_a_shifted_position():
    """On a ragged batch the invariant checker uses the ragged positions: ids
    computed for positions one block later must fail it."""
    from workloads import make
    w = make(name="rg", R=3, lens=(700, 3000), Q=300, H=1, max_seq_len=4096, topk=4, I=1, L=1,
             kfmt=0, seed=3, device="cpu", qlens=[2, 300, 5], prefix="tail")
    a = host_arrays(w)
    s, s64, ids = P.oracle_forward(a, w.score_width, w.topk, w.init_blocks, w.local_blocks)
    P.check_invariants(ids, a["seq_lens"], w.query_len, w.topk, w.init_blocks, w.local_blocks,
                       cu=a["cu_seqlens_q"], prefix=a["prefix_lens"])
    with pytest.raises(AssertionError):
        P.check_invariants(ids, a["seq_lens"], w.query_len, w.topk, w.init_blocks,
                           w.local_blocks, cu=a["cu_seqlens_q"], prefix=a["prefix_lens"] + 128)
