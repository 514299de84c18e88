"""MI355X (gfx950) block-scored paged index top-k: the MiniMax-M3 lightning
indexer hot path as a C-ABI HIP library (libmm3idx.so) with a thin ctypes
binding.  PyTorch supplies device memory and streams only."""
from ._binding import (BLOCK, HEAD_DIM, KFMT_BF16, KFMT_NVFP4, LIB_PATH, Mm3Error,
                       Problem, Rows, SparseOut, decode_workspace_bytes, lib, make_problem,
                       make_rows, make_sparse_out,
                       mm3_build_sparse_block_table, mm3_index_decode, mm3_index_decode_launches,
                       mm3_index_decode_static,
                       mm3_index_prefill_select, mm3_index_score,
                       mm3_index_topk, mm3_index_topk_blocks, mm3_index_topk_selector,
                       prefill_select_workspace_bytes, score_width, version)
