"""CPU oracle for the block-scored paged index top-k (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it, and it
shares no code with the HIP library: ``mm3_oracle.c`` is a plain, fp64,
brute-force restatement of what the pages define (page "ops.index_topk",
module docstring and the minimax_m3_index_decode / minimax_m3_index_topk
docstrings; page "indexer_nvfp4", module docstring for the NVFP4 key value).

Every function here takes and returns host numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mm3_oracle.c")
_LIB = os.path.join(_HERE, "libmm3oracle.so")

BLOCK = 128
DIM = 128


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, so every double op
    rounds as written)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
             "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build(force=False)  # only when missing or older than its source
        lib = ctypes.CDLL(_LIB)
        P, I64, I32, F32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        lib.oracle_e2m1_value.argtypes = [I32]
        lib.oracle_e2m1_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [I32]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_rn_satfinite.argtypes = [ctypes.c_double]
        lib.oracle_e4m3_rn_satfinite.restype = ctypes.c_double
        lib.oracle_nvfp4_element.argtypes = [I32, I32]
        lib.oracle_nvfp4_element.restype = ctypes.c_double
        lib.oracle_block_scores.argtypes = [
            P, I64, I64, I32, I32, P, P, I64, P, I64, P, I32, I32, P, P, F32,
            P, P, I64, I64, P, I64]
        lib.oracle_block_scores.restype = I32
        lib.oracle_topk.argtypes = [
            P, I64, I64, I32, P, I32, I32, P, P, I32, I32, I32, P, I64, I64, P, I64]
        lib.oracle_topk.restype = I32
        lib.oracle_sparse_block_table.argtypes = [
            P, I64, I32, P, I32, I32, P, P, P, I64, I32, I32, P, I64, P]
        lib.oracle_sparse_block_table.restype = I32
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def e2m1_value(nib: int) -> float:
    return _load().oracle_e2m1_value(int(nib))


def e4m3_value(byte: int) -> float:
    return _load().oracle_e4m3_value(int(byte))


def e4m3_rn_satfinite(x: float) -> float:
    return _load().oracle_e4m3_rn_satfinite(float(x))


def nvfp4_element(nib: int, scale_byte: int) -> float:
    return _load().oracle_nvfp4_element(int(nib), int(scale_byte))


def _rows_arg(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r, r.size


def _ragged(cu_seqlens_q, prefix_lens, R):
    """int32 host copies of the optional ragged-batch arrays (or None)."""
    cu = pre = None
    if cu_seqlens_q is not None:
        cu = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
        assert cu.shape == (R + 1,) and cu[0] == 0 and (np.diff(cu) >= 0).all()
    if prefix_lens is not None:
        assert cu is not None, "prefix_lens needs cu_seqlens_q"
        pre = np.ascontiguousarray(prefix_lens, dtype=np.int32)
        assert pre.shape == (R,)
    return cu, pre


def total_rows(seq_lens, query_len, cu_seqlens_q=None):
    if cu_seqlens_q is not None:
        return int(np.asarray(cu_seqlens_q)[-1])
    return int(np.asarray(seq_lens).size) * int(query_len)


def block_scores(q_bits, kfmt, kdata, kscales, block_table, seq_lens,
                 query_len, sm_scale, width, rows=None, out=None,
                 cu_seqlens_q=None, prefix_lens=None, out64=None):
    """Scores [H, T, width] fp32 (unwritten entries stay NaN).
    out64: optional float64 array of the same shape that receives each score
    before its rounding to fp32 (sm_scale * the fp64 block maximum).

    q_bits: uint16 [T, H, 128] (bf16 bit patterns); kfmt 0: kdata uint16
    [pages,128,128]; kfmt 1: kdata uint8 [pages,128,64] nibbles and kscales
    uint8 [pages,128,8]; block_table int32 [R, W]; seq_lens int32 [R].
    Ragged batches: cu_seqlens_q int32 [R+1] (request r owns rows
    cu[r]..cu[r+1]-1) and optionally prefix_lens int32 [R] (position of the
    request's first row; default seq_lens - rows).
    """
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    T, H, D = q_bits.shape
    assert D == DIM
    kdata = np.ascontiguousarray(kdata)
    if kfmt == 0:
        assert kdata.dtype == np.uint16 and kdata.shape[1:] == (BLOCK, DIM)
    else:
        assert kdata.dtype == np.uint8 and kdata.shape[1:] == (BLOCK, DIM // 2)
        kscales = np.ascontiguousarray(kscales, dtype=np.uint8)
        assert kscales.shape == (kdata.shape[0], BLOCK, DIM // 16)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    R = sl.size
    cu, pre = _ragged(cu_seqlens_q, prefix_lens, R)
    assert T == total_rows(sl, query_len, cu)
    if out is None:
        out = np.full((H, T, width), np.nan, dtype=np.float32)
    assert out.dtype == np.float32 and out.flags.c_contiguous
    if out64 is not None:
        assert out64.dtype == np.float64 and out64.flags.c_contiguous and out64.shape == out.shape
    rr, nr = _rows_arg(rows)
    rc = _load().oracle_block_scores(
        _ptr(q_bits), H * D, D, H, kfmt, _ptr(kdata),
        _ptr(kscales) if kfmt == 1 else None, kdata.shape[0], _ptr(bt),
        bt.shape[1], _ptr(sl), R, query_len, _ptr(cu), _ptr(pre),
        float(sm_scale), _ptr(out), _ptr(out64), out.shape[1] * out.shape[2], out.shape[2],
        _ptr(rr), nr)
    if rc != 0:
        raise ValueError("oracle_block_scores rejected its arguments")
    return out


def topk(scores, seq_lens, query_len, topk_, init_blocks, local_blocks,
         rows=None, out=None, cu_seqlens_q=None, prefix_lens=None):
    """Block ids [H, T, topk] int32 from scores [H, T, W] fp32."""
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    H, T, W = scores.shape
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    cu, pre = _ragged(cu_seqlens_q, prefix_lens, sl.size)
    assert T >= total_rows(sl, query_len, cu)
    if out is None:
        out = np.full((H, T, topk_), -7, dtype=np.int32)
    rr, nr = _rows_arg(rows)
    rc = _load().oracle_topk(
        _ptr(scores), T * W, W, H, _ptr(sl), sl.size, query_len, _ptr(cu),
        _ptr(pre), topk_, init_blocks, local_blocks, _ptr(out),
        out.shape[1] * out.shape[2], out.shape[2], _ptr(rr), nr)
    if rc != 0:
        raise ValueError("oracle_topk rejected its arguments")
    return out


def sparse_block_table(topk_idx, seq_lens, query_len, abt, pages_per_block,
                       block_page_stride, cu_seqlens_q=None, prefix_lens=None):
    """(sparse [T, topk*P] int32, ctx_lens [T] int32) for one index head."""
    ti = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, K = ti.shape
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    cu, pre = _ragged(cu_seqlens_q, prefix_lens, sl.size)
    assert T == total_rows(sl, query_len, cu)
    abt = np.ascontiguousarray(abt, dtype=np.int32)
    sparse = np.full((T, K * pages_per_block), -7, dtype=np.int32)
    ctx = np.full((T,), -7, dtype=np.int32)
    rc = _load().oracle_sparse_block_table(
        _ptr(ti), K, K, _ptr(sl), sl.size, query_len, _ptr(cu), _ptr(pre),
        _ptr(abt), abt.shape[1], pages_per_block, block_page_stride,
        _ptr(sparse), sparse.shape[1], _ptr(ctx))
    if rc != 0:
        raise ValueError("oracle_sparse_block_table rejected its arguments")
    return sparse, ctx


def forward(q_bits, kfmt, kdata, kscales, block_table, seq_lens, query_len,
            sm_scale, topk_, init_blocks, local_blocks, width, rows=None,
            cu_seqlens_q=None, prefix_lens=None, with64=False):
    """Scores then ids, the whole path on the CPU (rows: optional subset).
    Returns (scores, ids), or (scores, scores64, ids) with with64."""
    s64 = None
    if with64:
        T, H = np.asarray(q_bits).shape[:2]
        s64 = np.full((H, T, width), np.nan, dtype=np.float64)
    s = block_scores(q_bits, kfmt, kdata, kscales, block_table, seq_lens,
                     query_len, sm_scale, width, rows=rows,
                     cu_seqlens_q=cu_seqlens_q, prefix_lens=prefix_lens, out64=s64)
    # unwritten (invisible) entries are never read by the selection
    ids = topk(s, seq_lens, query_len, topk_, init_blocks, local_blocks, rows=rows,
               cu_seqlens_q=cu_seqlens_q, prefix_lens=prefix_lens)
    return (s, s64, ids) if with64 else (s, ids)
