"""ctypes binding of libmm3idx.so (include/mm3_index.h).

Argument marshalling only: torch tensors are turned into device pointers,
strides and the current HIP stream, and the C library does the rest.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback, so a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmm3idx.so")

MM3_OK = 0
MM3_EINVAL = -1
MM3_EUNSUPPORTED = -2
MM3_EWORKSPACE = -3
MM3_EHIP = -4
KFMT_BF16 = 0
KFMT_NVFP4 = 1
BLOCK = 128
HEAD_DIM = 128

EXPORTED = (
    "mm3_index_score", "mm3_index_topk", "mm3_index_topk_blocks", "mm3_index_decode_workspace_bytes",
    "mm3_index_decode", "mm3_index_decode_static", "mm3_index_prefill_select",
    "mm3_index_prefill_select_workspace_bytes", "mm3_build_sparse_block_table",
    "mm3_index_topk_selector", "mm3_index_decode_launches", "mm3_last_error", "mm3_version",
)
STATIC_SCRATCH_BYTES = 64 << 20


class Mm3Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"mm3 error {code}: {msg}")
        self.code = code


class Rows(ctypes.Structure):
    _fields_ = [
        ("seq_lens", ctypes.c_void_p),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("prefix_lens", ctypes.c_void_p),
        ("num_reqs", ctypes.c_int32),
        ("query_len", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
    ]


class Problem(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("q_tok_stride", ctypes.c_int64),
        ("q_head_stride", ctypes.c_int64),
        ("heads", ctypes.c_int32),
        ("kfmt", ctypes.c_int32),
        ("kdata", ctypes.c_void_p),
        ("kscales", ctypes.c_void_p),
        ("num_pages", ctypes.c_int64),
        ("block_table", ctypes.c_void_p),
        ("bt_row_stride", ctypes.c_int64),
        ("bt_width", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("rows", Rows),
    ]


class SparseOut(ctypes.Structure):
    _fields_ = [
        ("attention_block_table", ctypes.c_void_p),
        ("abt_row_stride", ctypes.c_int64),
        ("abt_width", ctypes.c_int32),
        ("pages_per_block", ctypes.c_int32),
        ("block_page_stride", ctypes.c_int32),
        ("sparse_table", ctypes.c_void_p),
        ("st_row_stride", ctypes.c_int64),
        ("sparse_ctx_lens", ctypes.c_void_p),
    ]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                "(the HIP library is required; there is no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        PP = ctypes.POINTER(Problem)
        PR = ctypes.POINTER(Rows)
        PS = ctypes.POINTER(SparseOut)
        L.mm3_index_score.argtypes = [PP, P, I64, I64, I32, P]
        L.mm3_index_score.restype = ctypes.c_int
        L.mm3_index_topk.argtypes = [P, I64, I64, I32, I32, PR, I32, I32, I32, P, I64, I64, P]
        L.mm3_index_topk.restype = ctypes.c_int
        L.mm3_index_topk_blocks.argtypes = [P, I64, I64, I32, I32, P, I32, I32, I32, I32, I32, P,
                                            I64, I64, P]
        L.mm3_index_topk_blocks.restype = ctypes.c_int
        L.mm3_index_decode_workspace_bytes.argtypes = [PP, I32, I32]
        L.mm3_index_decode_workspace_bytes.restype = SZ
        L.mm3_index_decode.argtypes = [PP, I32, I32, I32, P, I64, I64, P, I64, I64, I32, P, SZ, PS, P]
        L.mm3_index_decode.restype = ctypes.c_int
        L.mm3_index_prefill_select_workspace_bytes.argtypes = [PP, I32, I32]
        L.mm3_index_prefill_select_workspace_bytes.restype = SZ
        L.mm3_index_prefill_select.argtypes = [PP, I32, I32, I32, P, I64, I64, P, I64, I64, I32, P, SZ, P]
        L.mm3_index_prefill_select.restype = ctypes.c_int
        L.mm3_index_decode_static.argtypes = [PP, I32, I32, I32, P, I64, I64, P, I64, I64, I32, PS, P]
        L.mm3_index_decode_static.restype = ctypes.c_int
        L.mm3_build_sparse_block_table.argtypes = [P, I64, I32, PR, PS, P]
        L.mm3_build_sparse_block_table.restype = ctypes.c_int
        L.mm3_index_topk_selector.argtypes = [P, I64, I64, I32, I32, I32, I32, I32, I32, I32]
        L.mm3_index_topk_selector.restype = ctypes.c_char_p
        L.mm3_index_decode_launches.argtypes = [PP, P, I64, I64, PS]
        L.mm3_index_decode_launches.restype = ctypes.c_int
        L.mm3_last_error.argtypes = []
        L.mm3_last_error.restype = ctypes.c_char_p
        L.mm3_version.argtypes = []
        L.mm3_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(rc: int):
    if rc != MM3_OK:
        raise Mm3Error(rc, lib().mm3_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor, stream=None):
    if stream is not None:
        return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)
    if t.is_cuda:
        return int(torch.cuda.current_stream(t.device).cuda_stream)
    return None


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def score_width(max_seq_len: int) -> int:
    """Default score row width: cdiv(max_seq_len, 128) rounded up to 16."""
    return cdiv(cdiv(max_seq_len, BLOCK), 16) * 16


def _int32_vec(t, n, what):
    if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous() or t.shape[0] != n:
        raise ValueError(f"{what} must be contiguous int32 [{n}]")


def make_rows(seq_lens, query_len, max_seq_len, total_q, cu_seqlens_q=None,
              prefix_lens=None) -> Rows:
    """Marshal the row map (uniform, or ragged with cu_seqlens_q and optional
    prefix_lens; query_len is then the bound on every request's rows)."""
    if seq_lens.dtype != torch.int32 or seq_lens.dim() != 1 or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be contiguous int32 [reqs]")
    R = seq_lens.shape[0]
    if cu_seqlens_q is not None:
        _int32_vec(cu_seqlens_q, R + 1, "cu_seqlens_q")
    if prefix_lens is not None:
        if cu_seqlens_q is None:
            raise ValueError("prefix_lens needs cu_seqlens_q")
        _int32_vec(prefix_lens, R, "prefix_lens")
    for t in (cu_seqlens_q, prefix_lens):
        if t is not None and t.device != seq_lens.device:
            raise ValueError("row-map tensors must be on the same device")
    m = Rows()
    m.seq_lens = seq_lens.data_ptr()
    m.cu_seqlens_q = _ptr(cu_seqlens_q)
    m.prefix_lens = _ptr(prefix_lens)
    m.num_reqs = R
    m.query_len = int(query_len)
    m.total_q = int(total_q)
    m.max_seq_len = int(max_seq_len)
    return m


def make_problem(q, kdata, block_table, seq_lens, query_len, max_seq_len, sm_scale,
                 kscales=None, cu_seqlens_q=None, prefix_lens=None) -> Problem:
    """Marshal tensors into the C problem struct (no copies)."""
    if q.dtype != torch.bfloat16 or q.dim() != 3 or q.shape[2] != HEAD_DIM or q.stride(2) != 1:
        raise ValueError("q: expected bf16 of shape [tokens, heads, 128] with unit stride along the last dim")
    if kscales is None:
        if kdata.dtype != torch.bfloat16 or tuple(kdata.shape[1:]) != (BLOCK, HEAD_DIM) \
                or not kdata.is_contiguous():
            raise ValueError("bf16 index cache must be contiguous [pages, 128, 128]")
        kfmt = KFMT_BF16
    else:
        if kdata.dtype != torch.uint8 or tuple(kdata.shape[1:]) != (BLOCK, HEAD_DIM // 2) \
                or not kdata.is_contiguous():
            raise ValueError("NVFP4 nibbles must be contiguous uint8 [pages, 128, 64]")
        if kscales.dtype != torch.uint8 or tuple(kscales.shape) != (kdata.shape[0], BLOCK, HEAD_DIM // 16) \
                or not kscales.is_contiguous():
            raise ValueError("NVFP4 scales must be contiguous uint8 [pages, 128, 8]")
        kfmt = KFMT_NVFP4
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be int32 [reqs, width] with unit column stride")
    rows = make_rows(seq_lens, query_len, max_seq_len, q.shape[0], cu_seqlens_q, prefix_lens)
    devs = {t.device for t in (q, kdata, block_table, seq_lens) + ((kscales,) if kscales is not None else ())}
    if len(devs) != 1:
        raise ValueError("q, the index cache, the block table and the lengths have to share one device")
    p = Problem()
    p.q = q.data_ptr()
    p.q_tok_stride = q.stride(0)
    p.q_head_stride = q.stride(1)
    p.heads = q.shape[1]
    p.kfmt = kfmt
    p.kdata = kdata.data_ptr()
    p.kscales = _ptr(kscales)
    p.num_pages = kdata.shape[0]
    p.block_table = block_table.data_ptr()
    p.bt_row_stride = block_table.stride(0)
    p.bt_width = block_table.shape[1]
    p.sm_scale = float(sm_scale)
    p.rows = rows
    return p


def mm3_index_score(q, kdata, block_table, seq_lens, query_len, max_seq_len, sm_scale,
                    kscales=None, scores=None, stream=None, cu_seqlens_q=None, prefix_lens=None):
    """Block scores [heads, tokens, width] fp32 (only visible entries written).
    Ragged batches: cu_seqlens_q int32 [reqs+1] and optional prefix_lens
    int32 [reqs] on the device; query_len is then max_query_len."""
    p = make_problem(q, kdata, block_table, seq_lens, query_len, max_seq_len, sm_scale, kscales,
                     cu_seqlens_q, prefix_lens)
    if scores is None:
        scores = torch.empty((q.shape[1], q.shape[0], score_width(max_seq_len)),
                             dtype=torch.float32, device=q.device)
    if scores.dtype != torch.float32 or scores.dim() != 3 or scores.stride(2) != 1:
        raise ValueError("scores must be fp32 [heads, >=tokens, width] with unit column stride")
    _check(lib().mm3_index_score(ctypes.byref(p), scores.data_ptr(), scores.stride(0),
                                 scores.stride(1), scores.shape[2], _stream(q, stream)))
    return scores


def mm3_index_topk(scores, seq_lens, query_len, max_seq_len, topk, init_blocks, local_blocks,
                   out=None, stream=None, cu_seqlens_q=None, prefix_lens=None, total_q=None):
    """Block ids [heads, tokens, topk] int32, written into out[:, :tokens] in place.
    Ragged batches take tokens from total_q, else from the score tensor's rows."""
    H = scores.shape[0]
    if cu_seqlens_q is None:
        T = seq_lens.shape[0] * int(query_len)
    else:
        T = int(scores.shape[1] if total_q is None else total_q)
    rows = make_rows(seq_lens, query_len, max_seq_len, T, cu_seqlens_q, prefix_lens)
    if out is None:
        out = torch.empty((H, T, topk), dtype=torch.int32, device=scores.device)
    if scores.dtype != torch.float32 or scores.stride(2) != 1:
        raise ValueError("scores must be fp32 with unit column stride")
    if out.dtype != torch.int32 or out.dim() != 3 or out.stride(2) != 1 or out.shape[2] != topk \
            or out.shape[0] != H or out.shape[1] < T:
        raise ValueError("out must be int32 [heads, >=tokens, topk] with unit column stride")
    _check(lib().mm3_index_topk(scores.data_ptr(), scores.stride(0), scores.stride(1),
                                scores.shape[2], H, ctypes.byref(rows), int(topk), int(init_blocks),
                                int(local_blocks), out.data_ptr(), out.stride(0), out.stride(1),
                                _stream(scores, stream)))
    return out


def mm3_index_topk_blocks(scores, row_blocks, max_seq_len, topk, init_blocks, local_blocks,
                          out=None, stream=None):
    """Block ids [heads, tokens, topk] int32 with each row's visible-block
    count taken from row_blocks (int32 [tokens] on the device)."""
    H = scores.shape[0]
    if row_blocks.dtype != torch.int32 or row_blocks.dim() != 1 or not row_blocks.is_contiguous():
        raise ValueError("row_blocks must be contiguous int32 [tokens]")
    T = row_blocks.shape[0]
    if out is None:
        out = torch.empty((H, T, topk), dtype=torch.int32, device=scores.device)
    if scores.dtype != torch.float32 or scores.stride(2) != 1:
        raise ValueError("scores must be fp32 with unit column stride")
    if out.dtype != torch.int32 or out.dim() != 3 or out.stride(2) != 1 or out.shape[2] != topk \
            or out.shape[0] != H or out.shape[1] < T:
        raise ValueError("out must be int32 [heads, >=tokens, topk] with unit column stride")
    _check(lib().mm3_index_topk_blocks(scores.data_ptr(), scores.stride(0), scores.stride(1),
                                       scores.shape[2], H, row_blocks.data_ptr(), T,
                                       int(max_seq_len), int(topk), int(init_blocks),
                                       int(local_blocks), out.data_ptr(), out.stride(0),
                                       out.stride(1), _stream(scores, stream)))
    return out


def decode_workspace_bytes(p: Problem, topk: int, with_scores_out: bool) -> int:
    n = lib().mm3_index_decode_workspace_bytes(ctypes.byref(p), int(topk), int(with_scores_out))
    err = lib().mm3_last_error().decode()
    if n == 0 and err:
        raise Mm3Error(MM3_EINVAL, err)
    return n


def make_sparse_out(attention_block_table, pages_per_block, block_page_stride, sparse_table,
                    sparse_ctx_lens) -> SparseOut:
    """Marshal the sparse block-table outputs (all int32, contiguous rows)."""
    for t in (attention_block_table, sparse_table, sparse_ctx_lens):
        if t.dtype != torch.int32 or t.stride(-1) != 1:
            raise ValueError("sparse-table tensors must be int32 with contiguous rows")
    if attention_block_table.dim() != 2 or sparse_table.dim() != 2 or sparse_ctx_lens.dim() != 1:
        raise ValueError("attention_block_table and sparse_table are 2-D, sparse_ctx_lens 1-D")
    o = SparseOut()
    o.attention_block_table = attention_block_table.data_ptr()
    o.abt_row_stride = attention_block_table.stride(0)
    o.abt_width = attention_block_table.shape[1]
    o.pages_per_block = int(pages_per_block)
    o.block_page_stride = int(block_page_stride)
    o.sparse_table = sparse_table.data_ptr()
    o.st_row_stride = sparse_table.stride(0)
    o.sparse_ctx_lens = sparse_ctx_lens.data_ptr()
    return o


def mm3_index_decode(q, kdata, block_table, seq_lens, query_len, max_seq_len, sm_scale, topk,
                     init_blocks, local_blocks, kscales=None, out=None, scores_out=None,
                     workspace=None, stream=None, cu_seqlens_q=None, prefix_lens=None,
                     attention_block_table=None, sparse_block_table_out=None,
                     sparse_context_lens_out=None, pages_per_block=None, block_page_stride=None):
    """Scores then top-k in one call; returns out [heads, tokens, topk] int32.
    With the sparse-table arguments (all together, one index head) the
    selector also writes sparse_block_table_out [tokens, >= topk * P] and
    sparse_context_lens_out [tokens]."""
    sp_args = (attention_block_table, sparse_block_table_out, sparse_context_lens_out,
               pages_per_block, block_page_stride)
    if any(x is not None for x in sp_args) and any(x is None for x in sp_args):
        raise ValueError("the sparse-table arguments go together: pass all of them or none")
    sparse = None
    if attention_block_table is not None:
        sparse = make_sparse_out(attention_block_table, pages_per_block, block_page_stride,
                                 sparse_block_table_out, sparse_context_lens_out)
    p = make_problem(q, kdata, block_table, seq_lens, query_len, max_seq_len, sm_scale, kscales,
                     cu_seqlens_q, prefix_lens)
    H, T = q.shape[1], q.shape[0]
    if out is None:
        out = torch.empty((H, T, topk), dtype=torch.int32, device=q.device)
    if out.dtype != torch.int32 or out.dim() != 3 or out.stride(2) != 1:
        raise ValueError("out must be int32 [heads, >=tokens, topk] with unit column stride")
    need = decode_workspace_bytes(p, topk, scores_out is not None)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if scores_out is not None:
        if scores_out.dtype != torch.float32 or scores_out.stride(2) != 1:
            raise ValueError("scores_out must be fp32 with unit column stride")
        sh, sr, sw = scores_out.stride(0), scores_out.stride(1), scores_out.shape[2]
    else:
        sh = sr = sw = 0
    _check(lib().mm3_index_decode(ctypes.byref(p), int(topk), int(init_blocks), int(local_blocks),
                                  out.data_ptr(), out.stride(0), out.stride(1), _ptr(scores_out),
                                  sh, sr, sw, ws_ptr, ws_bytes,
                                  None if sparse is None else ctypes.byref(sparse),
                                  _stream(q, stream)))
    return out


def prefill_select_workspace_bytes(p: Problem, topk: int, with_scores_out: bool) -> int:
    n = lib().mm3_index_prefill_select_workspace_bytes(ctypes.byref(p), int(topk),
                                                       int(with_scores_out))
    err = lib().mm3_last_error().decode()
    if n == 0 and err:
        raise Mm3Error(MM3_EUNSUPPORTED, err)
    return n


def mm3_index_prefill_select(q, kdata, block_table, seq_lens, query_len, max_seq_len, sm_scale,
                             topk, init_blocks, local_blocks, kscales=None, out=None,
                             scores_out=None, workspace=None, stream=None):
    """The prefill scorer with the selection fused in (uniform prefill-shaped
    batches); returns out [heads, tokens, topk] int32."""
    p = make_problem(q, kdata, block_table, seq_lens, query_len, max_seq_len, sm_scale, kscales)
    H, T = q.shape[1], q.shape[0]
    if out is None:
        out = torch.empty((H, T, topk), dtype=torch.int32, device=q.device)
    if out.dtype != torch.int32 or out.dim() != 3 or out.stride(2) != 1:
        raise ValueError("out must be int32 [heads, >=tokens, topk] with unit column stride")
    if workspace is None:
        n = prefill_select_workspace_bytes(p, topk, scores_out is not None)
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)
    if scores_out is not None:
        if scores_out.dtype != torch.float32 or scores_out.stride(2) != 1:
            raise ValueError("scores_out must be fp32 with unit column stride")
        sh, sr, sw = scores_out.stride(0), scores_out.stride(1), scores_out.shape[2]
    else:
        sh = sr = sw = 0
    _check(lib().mm3_index_prefill_select(ctypes.byref(p), int(topk), int(init_blocks),
                                          int(local_blocks), out.data_ptr(), out.stride(0),
                                          out.stride(1), _ptr(scores_out), sh, sr, sw,
                                          workspace.data_ptr(),
                                          workspace.numel() * workspace.element_size(),
                                          _stream(q, stream)))
    return out


def mm3_index_decode_static(q, kdata, block_table, seq_lens, query_len, max_seq_len, sm_scale,
                            topk, init_blocks, local_blocks, out, kscales=None, scores_out=None,
                            stream=None, cu_seqlens_q=None, prefix_lens=None,
                            attention_block_table=None, sparse_block_table_out=None,
                            sparse_context_lens_out=None, pages_per_block=None,
                            block_page_stride=None):
    """mm3_index_decode without a workspace argument: the library's own
    per-GPU score workspace (64 MiB) serves when scores_out is None.  out
    must be given: nothing here allocates device memory."""
    sp_args = (attention_block_table, sparse_block_table_out, sparse_context_lens_out,
               pages_per_block, block_page_stride)
    if any(x is not None for x in sp_args) and any(x is None for x in sp_args):
        raise ValueError("the sparse-table arguments go together: pass all of them or none")
    sparse = None
    if attention_block_table is not None:
        sparse = make_sparse_out(attention_block_table, pages_per_block, block_page_stride,
                                 sparse_block_table_out, sparse_context_lens_out)
    p = make_problem(q, kdata, block_table, seq_lens, query_len, max_seq_len, sm_scale, kscales,
                     cu_seqlens_q, prefix_lens)
    if out is None or out.dtype != torch.int32 or out.dim() != 3 or out.stride(2) != 1:
        raise ValueError("out must be given: int32 [heads, >=tokens, topk] with unit column stride")
    if scores_out is not None:
        if scores_out.dtype != torch.float32 or scores_out.stride(2) != 1:
            raise ValueError("scores_out must be fp32 with unit column stride")
        sh, sr, sw = scores_out.stride(0), scores_out.stride(1), scores_out.shape[2]
    else:
        sh = sr = sw = 0
    _check(lib().mm3_index_decode_static(ctypes.byref(p), int(topk), int(init_blocks),
                                         int(local_blocks), out.data_ptr(), out.stride(0),
                                         out.stride(1), _ptr(scores_out), sh, sr, sw,
                                         None if sparse is None else ctypes.byref(sparse),
                                         _stream(q, stream)))
    return out


def mm3_build_sparse_block_table(topk_idx, seq_lens, query_len, max_seq_len,
                                 attention_block_table, pages_per_block, block_page_stride,
                                 sparse_table=None, sparse_ctx_lens=None, stream=None,
                                 cu_seqlens_q=None, prefix_lens=None):
    """(sparse_table [tokens, topk*P], sparse_ctx_lens [tokens]) for one head."""
    if topk_idx.dim() == 3:
        if topk_idx.shape[0] != 1:
            raise ValueError("the sparse table is built for one index head")
        topk_idx = topk_idx[0]
    T, K = topk_idx.shape[0], topk_idx.shape[1]
    P = int(pages_per_block)
    if sparse_table is None:
        sparse_table = torch.empty((T, K * P), dtype=torch.int32, device=topk_idx.device)
    if sparse_ctx_lens is None:
        sparse_ctx_lens = torch.empty((T,), dtype=torch.int32, device=topk_idx.device)
    if topk_idx.dtype != torch.int32 or topk_idx.stride(-1) != 1:
        raise ValueError("topk_idx must be int32 with contiguous rows")
    rows = make_rows(seq_lens, query_len, max_seq_len, T, cu_seqlens_q, prefix_lens)
    sp = make_sparse_out(attention_block_table, P, block_page_stride, sparse_table, sparse_ctx_lens)
    _check(lib().mm3_build_sparse_block_table(
        topk_idx.data_ptr(), topk_idx.stride(0), K, ctypes.byref(rows), ctypes.byref(sp),
        _stream(topk_idx, stream)))
    return sparse_table, sparse_ctx_lens


def mm3_index_decode_launches(q, kdata, block_table, seq_lens, query_len, max_seq_len, sm_scale,
                              kscales=None, scores_out=None, cu_seqlens_q=None, prefix_lens=None,
                              sparse=None):
    """How mm3_index_decode runs this problem: 1 (scores and selection in one
    launch) or 2 (scorer, then selector).  sparse: a SparseOut or None."""
    p = make_problem(q, kdata, block_table, seq_lens, query_len, max_seq_len, sm_scale, kscales,
                     cu_seqlens_q, prefix_lens)
    sh = sr = 0
    if scores_out is not None:
        sh, sr = scores_out.stride(0), scores_out.stride(1)
    n = lib().mm3_index_decode_launches(ctypes.byref(p), _ptr(scores_out), sh, sr,
                                        None if sparse is None else ctypes.byref(sparse))
    _check(min(n, 0))
    return n


def mm3_index_topk_selector(scores, total_q, max_seq_len, topk, by_row_blocks=False,
                            sparse=False) -> str:
    """Name of the selector kernel a selection over this score tensor launches
    (mm3_index_topk, mm3_index_topk_blocks with by_row_blocks, or the fused
    decode's selection with its sparse table).  scores may be any tensor with
    the layout (fp32 [heads, >=total_q, width], unit column stride); it is
    not read."""
    if scores.stride(-1) != 1 or scores.dim() != 3:
        raise ValueError("scores must be [heads, tokens, width] with unit column stride")
    name = lib().mm3_index_topk_selector(scores.data_ptr(), scores.stride(0), scores.stride(1),
                                         scores.shape[2], scores.shape[0], int(total_q),
                                         int(max_seq_len), int(topk), int(bool(by_row_blocks)),
                                         int(bool(sparse)))
    if name is None:
        raise Mm3Error(MM3_EINVAL, lib().mm3_last_error().decode())
    return name.decode()


def version() -> str:
    return lib().mm3_version().decode()
