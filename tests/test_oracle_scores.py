"""Pins for the oracle's block scores (CPU only).

What the oracle computes (page "vllm.models.minimax_m3.amd.ops.index_topk",
module docstring and minimax_m3_index_score docstring): for every query row
and visible 128-token block, the maximum over the block's causally visible
tokens of sm_scale * (q . k), with one shared key per token.

Pins, none of which re-types the oracle:
  * a numpy float64 matmul over the flattened, de-paged context with a causal
    mask and a reshape-amax per 128 keys (a different algorithm);
  * torch CPU float32 matmul + amax, within float32 error;
  * a closed form for the partial last block (monotone keys);
  * invariances: poisoned unread slots, page permutation, power-of-two
    sm_scale, head permutation.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import KFMT_BF16, KFMT_NVFP4, cdiv, host_arrays, make

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _keys_f64(a, page_ids):
    """[n_pages, 128, 128] float64 keys of the given pages."""
    if a["kfmt"] == KFMT_BF16:
        return _bf16_to_f64(a["kdata"][page_ids])
    nb = a["kdata"][page_ids].astype(np.int64)
    nib = np.stack([nb & 15, nb >> 4], axis=-1).reshape(nb.shape[0], 128, 128)
    sc = np.repeat(a["kscales"][page_ids], 16, axis=-1)
    # dequant through the oracle's scalar codec would not be independent; use
    # torch's e4m3 decode, the E2M1 table and torch's fp8 cast for rounding
    sv = torch.from_numpy(sc.astype(np.uint8).copy()).view(torch.float8_e4m3fn).double()
    mag = torch.tensor(E2M1, dtype=torch.float64)[torch.from_numpy(nib & 7)]
    sgn = torch.where(torch.from_numpy(nib & 8) > 0, -1.0, 1.0).double()
    # satfinite: clamp to +-448 first (only poison slots reach it here)
    prod = (mag * sgn * sv).float().clamp(-448.0, 448.0)
    return prod.to(torch.float8_e4m3fn).double().numpy()


def brute_scores(a, width, with64=False):
    q = _bf16_to_f64(a["q_bits"])
    T, H, _ = q.shape
    Q = a["query_len"]
    out = np.full((H, T, width), np.nan, dtype=np.float32)
    out64 = np.full((H, T, width), np.nan, dtype=np.float64)
    for r, L in enumerate(a["seq_lens"]):
        nb = cdiv(int(L), 128)
        if nb == 0:
            continue
        K = _keys_f64(a, a["block_table"][r, :nb]).reshape(nb * 128, 128)
        for j in range(Q):
            t = r * Q + j
            pos = int(L) - Q + j
            if pos < 0:
                continue
            nv = pos // 128 + 1
            dots = q[t] @ K[: nv * 128].T  # [H, nv*128]
            dots[:, pos + 1:] = -np.inf
            m = dots.reshape(H, nv, 128).max(-1)
            # sm_scale crosses the boundary as an fp32 value
            out64[:, t, :nv] = float(np.float32(a["sm_scale"])) * m
            out[:, t, :nv] = (a["sm_scale"] * m).astype(np.float32)
    return (out, out64) if with64 else out


def _small(seed, kfmt=KFMT_BF16, R=3, lens=(1, 700), Q=4, H=2, msl=1024, **kw):
    return make(name="t", R=R, lens=lens, Q=Q, H=H, max_seq_len=msl, topk=4,
                I=1, L=1, kfmt=kfmt, seed=seed, device="cpu", **kw)


def _oracle_scores(a, width, rows=None):
    return oracle.block_scores(a["q_bits"], a["kfmt"], a["kdata"], a["kscales"],
                               a["block_table"], a["seq_lens"], a["query_len"],
                               a["sm_scale"], width, rows=rows)


def _same(x, y, rtol=0.0, atol=0.0):
    vis = ~np.isnan(y)
    assert np.array_equal(np.isnan(x), np.isnan(y))
    np.testing.assert_allclose(x[vis], y[vis], rtol=rtol, atol=atol)


@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("kfmt", [KFMT_BF16, KFMT_NVFP4])
def test_vs_numpy_float64(seed, kfmt):
    w = _small(seed, kfmt=kfmt)
    a = host_arrays(w)
    _same(_oracle_scores(a, w.score_width), brute_scores(a, w.score_width), rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("kfmt", [KFMT_BF16, KFMT_NVFP4])
def test_scores64_vs_numpy_float64(kfmt):
    """The oracle's unrounded scores (sm_scale * the fp64 block maximum) equal
    a numpy float64 matmul's to fp64 summation-order error, and round to the
    fp32 scores exactly."""
    w = _small(4, kfmt=kfmt, R=3, lens=(200, 1000))
    a = host_arrays(w)
    s64 = np.full((w.heads, w.rows, w.score_width), np.nan)
    s32 = oracle.block_scores(a["q_bits"], a["kfmt"], a["kdata"], a["kscales"],
                              a["block_table"], a["seq_lens"], a["query_len"],
                              a["sm_scale"], w.score_width, out64=s64)
    _, b64 = brute_scores(a, w.score_width, with64=True)
    vis = ~np.isnan(b64)
    assert np.array_equal(vis, ~np.isnan(s64))
    np.testing.assert_allclose(s64[vis], b64[vis], rtol=1e-12, atol=1e-12)
    assert np.array_equal(s64[vis].astype(np.float32), s32[vis])


def test_scores64_equal_for_copied_keys():
    """Two blocks holding the same keys, in any slot order, get bit-equal
    unrounded scores (the tie a checker must treat as exact), while blocks
    whose fp64 maxima differ get different unrounded scores."""
    w = _small(8, R=1, lens=(900, 900), Q=4, H=2)
    bt = w.block_table[0]
    src = w.kdata[bt[1]].clone()
    w.kdata[bt[3]] = src.roll(37, dims=0)  # block 3: block 1's keys, rotated
    a = host_arrays(w)
    s64 = np.full((w.heads, w.rows, w.score_width), np.nan)
    oracle.block_scores(a["q_bits"], a["kfmt"], a["kdata"], a["kscales"], a["block_table"],
                        a["seq_lens"], a["query_len"], a["sm_scale"], w.score_width, out64=s64)
    assert np.array_equal(s64[:, :, 1], s64[:, :, 3])
    assert not np.array_equal(s64[:, :, 1], s64[:, :, 2])


def test_vs_torch_fp32_special_case():
    """One request, one head: scores equal torch fp32 q@K^T, masked, amax
    over 128 keys, times sm_scale (fp32 rounding error only)."""
    w = _small(11, R=1, lens=(900, 900), Q=8, H=1)
    a = host_arrays(w)
    got = _oracle_scores(a, w.score_width)
    q = w.q.float()[:, 0]  # [8, 128]
    nb = cdiv(900, 128)
    K = w.kdata[w.block_table[0, :nb].long()].float().reshape(-1, 128)
    s = q @ K.T
    pos = torch.arange(900 - 8, 900)
    s[torch.arange(s.shape[1])[None, :] > pos[:, None]] = -float("inf")
    m = s.reshape(8, nb, 128).amax(-1) * w.sm_scale
    for j in range(8):
        nv = int(pos[j]) // 128 + 1
        np.testing.assert_allclose(got[0, j, :nv], m[j, :nv].numpy(), rtol=2e-5, atol=2e-5)


def test_partial_block_closed_form():
    """q = c e0 and key[0] strictly increasing with the slot in the block
    (1 + s/128, exact in bf16): the block score is sm_scale * c * key[0] of
    the last visible token."""
    L, Q = 1000, 4
    w = _small(5, R=1, lens=(L, L), Q=Q, H=1)
    c = 2.0
    w.q.zero_()
    w.q[:, 0, 0] = c
    bt = w.block_table[0]
    for p in range(L):
        w.kdata[bt[p // 128], p % 128, 0] = 1.0 + (p % 128) / 128.0
    a = host_arrays(w)
    got = _oracle_scores(a, w.score_width)
    for j in range(Q):
        pos = L - Q + j
        for b in range(pos // 128 + 1):
            last = min(pos, 128 * b + 127)
            # sm_scale crosses the boundary as an fp32 value
            want = float(np.float32(w.sm_scale)) * c * (1.0 + (last - 128 * b) / 128.0)
            assert got[0, j, b] == np.float32(want)


def test_poisoned_unread_slots_change_nothing():
    w = _small(6)
    a = host_arrays(w)
    base = _oracle_scores(a, w.score_width)
    # overwrite every slot that no visible block covers with a huge value
    kd = a["kdata"].copy()
    used = np.zeros(kd.shape[:2], dtype=bool)
    for r, L in enumerate(a["seq_lens"]):
        for p in range(int(L)):
            used[a["block_table"][r, p // 128], p % 128] = True
    kd[~used] = np.uint16(0x7F00)  # bf16 1.7e38
    a2 = dict(a, kdata=kd)
    _same(_oracle_scores(a2, w.score_width), base)


def test_page_permutation_invariance():
    w = _small(7)
    a = host_arrays(w)
    base = _oracle_scores(a, w.score_width)
    rng = np.random.default_rng(0)
    perm = rng.permutation(a["kdata"].shape[0])  # new page p' holds old page perm[p']
    inv = np.argsort(perm)
    a2 = dict(a, kdata=a["kdata"][perm], block_table=inv[a["block_table"]].astype(np.int32))
    _same(_oracle_scores(a2, w.score_width), base)


def test_power_of_two_scale_is_exact():
    w = _small(8)
    a = host_arrays(w)
    base = _oracle_scores(a, w.score_width)
    a2 = dict(a, sm_scale=a["sm_scale"] * 4.0)
    _same(_oracle_scores(a2, w.score_width), base * np.float32(4.0))


def test_head_permutation_equivariance():
    w = _small(9, H=3)
    a = host_arrays(w)
    base = _oracle_scores(a, w.score_width)
    a2 = dict(a, q_bits=np.ascontiguousarray(a["q_bits"][:, ::-1]))
    _same(_oracle_scores(a2, w.score_width), base[::-1])


def test_rows_subset_matches_full():
    w = _small(10)
    a = host_arrays(w)
    full = _oracle_scores(a, w.score_width)
    rows = [0, 5, 7, 11]
    sub = _oracle_scores(a, w.score_width, rows=rows)
    _same(sub[:, rows], full[:, rows])
    other = [t for t in range(w.rows) if t not in rows]
    assert np.isnan(sub[:, other]).all()


def test_short_requests_have_no_rows():
    """seq_len < query_len: early rows sit before position 0 and see nothing."""
    w = _small(12, R=2, lens=(2, 2), Q=4, H=1, fixed_lens=[2, 0])
    a = host_arrays(w)
    got = _oracle_scores(a, w.score_width)
    assert np.isnan(got[0, [0, 1, 4, 5, 6, 7]]).all()
    assert not np.isnan(got[0, [2, 3], 0]).any()


# ---------------------------------------------------------------- ragged
#
# Ragged batches (page "ops.index_topk", minimax_m3_index_score signature:
# cu_seqlens_q row offsets and prefix_lens).  Request r owns rows
# cu[r]..cu[r+1]-1; its row j sits at prefix_lens[r] + j, or at
# seq_lens[r] - rows + j when no prefix_lens are given.

def _ragged_positions(a):
    seq = a["seq_lens"].astype(np.int64)
    cu = a["cu_seqlens_q"].astype(np.int64)
    out = []
    for r in range(seq.size):
        n = int(cu[r + 1] - cu[r])
        p0 = int(a["prefix_lens"][r]) if a["prefix_lens"] is not None else int(seq[r]) - n
        out += [(r, int(cu[r]) + j, p0 + j) for j in range(n)]
    return out


def brute_scores_ragged(a, width):
    """The numpy float64 pin above, with rows and positions from the ragged
    batch description."""
    q = _bf16_to_f64(a["q_bits"])
    T, H, _ = q.shape
    out = np.full((H, T, width), np.nan, dtype=np.float32)
    for r, t, pos in _ragged_positions(a):
        if pos < 0:
            continue
        nv = pos // 128 + 1
        K = _keys_f64(a, a["block_table"][r, :nv]).reshape(nv * 128, 128)
        dots = q[t] @ K.T
        dots[:, pos + 1:] = -np.inf
        out[:, t, :nv] = (a["sm_scale"] * dots.reshape(H, nv, 128).max(-1)).astype(np.float32)
    return out


def _ragged_small(seed, kfmt=KFMT_BF16, prefix=None, qlens=(3, 0, 1, 7, 2), H=2, msl=1024,
                  lens=(1, 900)):
    return make(name="t", R=len(qlens), lens=lens, Q=8, H=H, max_seq_len=msl, topk=4, I=1, L=1,
                kfmt=kfmt, seed=seed, device="cpu", qlens=list(qlens), prefix=prefix)


def _oracle_ragged(a, width, rows=None):
    return oracle.block_scores(a["q_bits"], a["kfmt"], a["kdata"], a["kscales"],
                               a["block_table"], a["seq_lens"], a["query_len"],
                               a["sm_scale"], width, rows=rows,
                               cu_seqlens_q=a["cu_seqlens_q"], prefix_lens=a["prefix_lens"])


@pytest.mark.parametrize("prefix", [None, "tail", "gap"])
@pytest.mark.parametrize("kfmt", [KFMT_BF16, KFMT_NVFP4])
def test_ragged_vs_numpy_float64(kfmt, prefix):
    w = _ragged_small(21, kfmt=kfmt, prefix=prefix)
    a = host_arrays(w)
    assert a["cu_seqlens_q"].tolist()[-1] == w.rows
    _same(_oracle_ragged(a, w.score_width), brute_scores_ragged(a, w.score_width),
          rtol=1e-6, atol=1e-6)


def test_ragged_gap_keys_are_invisible():
    """With prefix_lens below seq_len - rows, the keys after the last row's
    position hold poison (a huge value); no score may see it."""
    w = _ragged_small(22, prefix="gap", qlens=(5, 8, 2), lens=(300, 900))
    a = host_arrays(w)
    assert (a["prefix_lens"] + np.diff(a["cu_seqlens_q"]) < a["seq_lens"]).any()
    got = _oracle_ragged(a, w.score_width)
    assert np.nanmax(np.abs(got)) < 100.0


def test_ragged_equals_requests_alone():
    """A ragged batch scores each request as a uniform one-request batch with
    query_len = its rows and seq_len = its last row's position + 1."""
    w = _ragged_small(23, prefix="gap", qlens=(4, 1, 6, 0, 3))
    a = host_arrays(w)
    full = _oracle_ragged(a, w.score_width)
    cu = a["cu_seqlens_q"]
    for r in range(a["seq_lens"].size):
        n = int(cu[r + 1] - cu[r])
        if n == 0:
            continue
        end = int(a["prefix_lens"][r]) + n
        alone = oracle.block_scores(a["q_bits"][cu[r]:cu[r + 1]], a["kfmt"], a["kdata"],
                                    a["kscales"], a["block_table"][r:r + 1],
                                    np.array([end], dtype=np.int32), n, a["sm_scale"],
                                    w.score_width)
        _same(full[:, cu[r]:cu[r + 1]], alone)


def test_ragged_rows_subset_matches_full():
    w = _ragged_small(24, prefix="tail")
    a = host_arrays(w)
    full = _oracle_ragged(a, w.score_width)
    rows = [0, 3, 4, 10]
    sub = _oracle_ragged(a, w.score_width, rows=rows)
    _same(sub[:, rows], full[:, rows])


def test_ragged_rejects_rows_outside_the_batch():
    w = _ragged_small(25)
    a = host_arrays(w)
    with pytest.raises(ValueError):
        _oracle_ragged(a, w.score_width, rows=[w.rows])
