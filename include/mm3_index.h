/*
 * mm3_index.h -- C ABI of libmm3idx.so: block-scored, paged index top-k
 * (the MiniMax-M3 lightning indexer) on AMD Instinct MI355X (gfx950).
 *
 * What it computes.  Index queries q [tokens, heads, 128] (bf16) score every
 * 128-token block of a paged index-K cache shared by all heads, one page per
 * block, reached through an int32 block table and int32 sequence lengths.  A
 * block's score is the maximum over its causally visible tokens of
 * sm_scale * (q . k); each (head, token) row then selects its top-k block
 * ids, with the leading "init" and trailing "local" blocks always kept and
 * -1 padding.  Sources: page "vllm.models.minimax_m3.amd.ops.index_topk"
 * (module docstring; minimax_m3_index_decode, minimax_m3_index_score and
 * minimax_m3_index_topk docstrings and signatures), page
 * "vllm.models.minimax_m3.amd.ops.indexer_context_parallel"
 * (check_context_score_inputs: layout rules; indexer_context_scores:
 * capture-stable max_seq_len and in-place out), page
 * "vllm.models.minimax_m3.amd.indexer_nvfp4" (module docstring: NVFP4 keys
 * score as e4m3_rn_satfinite(e2m1 * scale)).
 *
 * Conventions shared by every entry point
 *  - Rows (struct mm3_rows).  Uniform batches: request r owns rows
 *    t = r*query_len + j, j < query_len, and row j sits at position
 *    pos = seq_lens[r] - query_len + j.  Ragged batches (cu_seqlens_q given;
 *    page "ops.index_topk", minimax_m3_index_score and minimax_m3_index_topk
 *    signatures): request r owns rows cu_seqlens_q[r] <= t <
 *    cu_seqlens_q[r+1], and its row j sits at prefix_lens[r] + j, or, without
 *    prefix_lens, at seq_lens[r] - n_r + j (n_r = its row count: the chunk is
 *    the request's last n_r tokens).  A row at pos sees the nv = pos/128 + 1
 *    blocks b <= pos/128 and in block b the tokens 128*b + s <= pos.  Rows
 *    with pos < 0 see nothing.
 *  - Pointers are DEVICE pointers unless a parameter says "host".  The
 *    mm3_problem struct itself is read on the host during the call only.
 *  - Strides are in ELEMENTS of the pointed-to type.
 *  - stream is a hipStream_t (NULL = the legacy default stream).  All work is
 *    enqueued asynchronously on it; nothing is read back to the host, no
 *    device memory is allocated, and the grid depends only on host-side
 *    arguments (never on device seq_lens), so every call can be captured in
 *    a HIP graph and replayed with new device values.
 *  - Ownership: the caller owns every buffer; the library keeps no pointer
 *    after a call returns.
 *  - Errors: every host-checkable rule is checked before anything is
 *    enqueued; a non-zero return leaves every output untouched.
 *    mm3_last_error() then describes it (thread-local).  Device VALUES
 *    (lengths, row offsets, prefixes, page ids) are preconditions, listed
 *    with mm3_rows and mm3_problem, and not checked.
 */
#ifndef MM3_INDEX_H
#define MM3_INDEX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define MM3_OK 0
#define MM3_EINVAL (-1)       /* an argument breaks a rule listed below */
#define MM3_EUNSUPPORTED (-2) /* valid, but outside what the call supports */
#define MM3_EWORKSPACE (-3)   /* workspace NULL, misaligned or too small */
#define MM3_EHIP (-4)         /* a HIP launch failed; message has the HIP error */

/* index-K page formats */
#define MM3_KFMT_BF16 0  /* kdata: bf16 [num_pages][128][128] */
#define MM3_KFMT_NVFP4 1 /* kdata: u8 nibbles [num_pages][128][64], element 2i
                            in the low nibble of byte i, 2i+1 in the high one;
                            kscales: u8 e4m3 [num_pages][128][8], scale g
                            covers d in [16g, 16g+16); key element =
                            e4m3_rn_satfinite(e2m1(nibble) * e4m3(scale)) */

#define MM3_BLOCK 128     /* tokens per sparse block == tokens per page */
#define MM3_HEAD_DIM 128  /* index head dimension */
#define MM3_MAX_BLOCKS 65534 /* cdiv(max_seq_len, 128) must stay below 65535 */
#define MM3_MAX_TOPK 1024
#define MM3_MAX_ROWS 2147482624 /* total_q bound: 2^31 - 1024 (grids round rows up to whole workgroups) */

/*
 * How rows map to requests and positions (see "Rows" above).
 *   seq_lens     int32 [num_reqs], contiguous; each in [0, max_seq_len].
 *   cu_seqlens_q NULL (uniform batch), or int32 [num_reqs + 1], contiguous:
 *                cu[0] == 0, non-decreasing, every n_r = cu[r+1] - cu[r] <=
 *                query_len, cu[num_reqs] == total_q.
 *   prefix_lens  NULL, or (ragged batches only) int32 [num_reqs], contiguous:
 *                prefix_lens[r] >= 0 and prefix_lens[r] + n_r <= seq_lens[r].
 *   num_reqs     >= 0.
 *   query_len    >= 1: rows per request; with cu_seqlens_q, a bound on every
 *                n_r (the pages' max_query_len), which sizes grids.
 *   total_q      rows in all (tokens); == num_reqs * query_len without
 *                cu_seqlens_q.  At most MM3_MAX_ROWS (2^31 - 1024);
 *                heads * query_len below 2^31.
 *   max_seq_len  capture-stable bound on every seq_lens[r] (e.g. the model's
 *                maximum length, not the batch maximum); sizes the grids.
 * The arrays live on the device and their VALUES are preconditions, not
 * checked: values outside these ranges make the kernels read out of bounds.
 */
typedef struct mm3_rows {
    const int32_t* seq_lens;
    const int32_t* cu_seqlens_q;
    const int32_t* prefix_lens;
    int32_t num_reqs;
    int32_t query_len;
    int32_t total_q;
    int32_t max_seq_len;
} mm3_rows;

/*
 * The scoring problem (page "ops.index_topk", minimax_m3_index_decode and
 * minimax_m3_index_score signatures; page "indexer_context_parallel",
 * check_context_score_inputs).
 *   q            bf16, element (t, h, d) at q[t*q_tok_stride + h*q_head_stride + d];
 *                D contiguous; 16-byte aligned; both strides multiples of 8.
 *   heads        index heads H >= 1 (each head selects its own blocks).
 *   kfmt/kdata/kscales/num_pages  the page pool (formats above), 16-byte
 *                aligned, num_pages >= 1; kscales NULL for bf16.
 *   block_table  int32, entry (r, b) at block_table[r*bt_row_stride + b];
 *                bt_width >= cdiv(rows.max_seq_len, 128); bt_row_stride >=
 *                bt_width.  Entries of every visible block must lie in
 *                [0, num_pages) (a device precondition, not checked).
 *   rows         the batch's rows (struct above); q holds rows.total_q tokens.
 *   sm_scale     finite, > 0.
 */
typedef struct mm3_problem {
    const void* q;
    int64_t q_tok_stride;
    int64_t q_head_stride;
    int32_t heads;
    int32_t kfmt;
    const void* kdata;
    const uint8_t* kscales;
    int64_t num_pages;
    const int32_t* block_table;
    int64_t bt_row_stride;
    int32_t bt_width;
    float sm_scale;
    mm3_rows rows;
} mm3_problem;

/*
 * mm3_index_score -- block scores (page "ops.index_topk",
 * minimax_m3_index_score): for every token row and head, one score per
 * causally visible 128-token block, the block's largest scaled dot product.
 *   scores  fp32, element (h, t, b) at scores[h*s_head_stride + t*s_row_stride + b],
 *           s_width >= cdiv(max_seq_len,128) columns per row,
 *           s_row_stride >= s_width, s_head_stride >= total_q*s_row_stride.
 *           Written: every visible (h, t, b); nothing else is touched.
 *   score = fl32(sm_scale * max over visible tokens of the fp32-accumulated
 *           dot product of q[t, h, :] and the key).
 * A request with heads * n_r <= 16 rows is scored by the bandwidth-bound
 * decode scorer, a larger one by the MFMA prefill scorer; a ragged batch may
 * mix both kinds in one call.  Both take either key format (both decode
 * NVFP4 keys to bf16 in registers, just before the multiplies).  q and keys are
 * expected finite: a score whose block holds a NaN or infinite product is
 * unspecified.
 */
/* (scores, and the problem's block_table, may be NULL when
 * cdiv(max_seq_len, 128) == 0: no row sees a block, so nothing is read or
 * written there; the same holds for the selection calls below.) */
int mm3_index_score(const mm3_problem* p, float* scores, int64_t s_head_stride,
                    int64_t s_row_stride, int32_t s_width, void* stream);

/*
 * mm3_index_topk -- per (head, row) selection from a score tensor (page
 * "ops.index_topk", minimax_m3_index_topk; forced blocks pinned as in page
 * "indexer_cp_exchange", module docstring).
 *   scores laid out as in mm3_index_score; only visible entries are read.
 *   With F = [0, min(I,nv)) U [max(0,nv-L), nv):
 *     nv <= topk -> ids 0..nv-1;  else F plus the topk-|F| best other blocks
 *     by (score descending, id ascending; -0 == +0).
 *   rows as in mm3_problem (the same batch the scores were computed for).
 *   out int32, row (h, t) at out[h*o_head_stride + t*o_row_stride], written in
 *   place: the selected ids ascending, then -1 up to topk.  Rows t >= total_q
 *   are not touched (stable address for graph capture).
 *   1 <= topk <= 1024, 0 <= I, 0 <= L, I + L <= topk,
 *   o_row_stride >= topk, o_head_stride >= total_q*o_row_stride.
 */
int mm3_index_topk(const float* scores, int64_t s_head_stride,
                   int64_t s_row_stride, int32_t s_width, int32_t heads,
                   const mm3_rows* rows, int32_t topk, int32_t init_blocks,
                   int32_t local_blocks, int32_t* out, int64_t o_head_stride,
                   int64_t o_row_stride, void* stream);

/*
 * mm3_index_topk_blocks -- the selection of mm3_index_topk with each row's
 * visible-block count given directly instead of derived from its position
 * (page "indexer_nvfp4", MiniMaxM3IndexerRocmNvfp4Impl: the prefill selector
 * takes the row block counts the metadata builder materialises,
 * num_valid_pages).
 *   row_blocks int32 [total_q], contiguous: nv of row t, in
 *              [0, cdiv(max_seq_len,128)] (a device precondition, not
 *              checked); the row's scores are read for blocks b < nv.
 *   Forced blocks, ordering, padding, out and the stride rules as in
 *   mm3_index_topk.
 */
int mm3_index_topk_blocks(const float* scores, int64_t s_head_stride,
                          int64_t s_row_stride, int32_t s_width, int32_t heads,
                          const int32_t* row_blocks, int32_t total_q,
                          int32_t max_seq_len, int32_t topk,
                          int32_t init_blocks, int32_t local_blocks,
                          int32_t* out, int64_t o_head_stride,
                          int64_t o_row_stride, void* stream);

/*
 * Sparse block-table output: the attention pages of the selected blocks and
 * each row's sparse context length, for ONE index head (page
 * "ops.index_topk", minimax_m3_index_decode: attention_block_table,
 * sparse_block_table_out, sparse_context_lens_out and block_page_stride,
 * which come together).
 *   attention_block_table  int32, request r's row at abt[r*abt_row_stride];
 *              sparse block b owns entries [b*block_page_stride,
 *              b*block_page_stride + pages_per_block);
 *              abt_width >= cdiv(max_seq_len,128) * block_page_stride;
 *              abt_row_stride >= abt_width.
 *   pages_per_block P >= 1; block_page_stride in {P, 2P}.
 *   sparse_table int32, row t at sparse_table[t*st_row_stride], st_row_stride
 *              >= topk*P: slot j*P+i = abt[r][b_j*stride + i] for the row's
 *              j-th id b_j, -1 for the slots of -1 ids.
 *   sparse_ctx_lens int32 [total_q]: sum over the row's ids b of the tokens
 *              of b it sees, min(128, pos - 128*b + 1); 0 when pos < 0.
 * Every pointer 4-byte aligned.  Attention-table entries are read only for
 * selected blocks.
 */
typedef struct mm3_sparse_out {
    const int32_t* attention_block_table;
    int64_t abt_row_stride;
    int32_t abt_width;
    int32_t pages_per_block;
    int32_t block_page_stride;
    int32_t* sparse_table;
    int64_t st_row_stride;
    int32_t* sparse_ctx_lens;
} mm3_sparse_out;

/*
 * Workspace bytes mm3_index_decode needs for this problem when it is given
 * no scores_out buffer (0 when scores_out is given).  Host-only, no HIP call.
 * Returns 0 and sets mm3_last_error() if p is invalid.
 */
size_t mm3_index_decode_workspace_bytes(const mm3_problem* p, int32_t topk,
                                        int32_t with_scores_out);

/*
 * mm3_index_decode -- scores then top-k in one call (page "ops.index_topk",
 * minimax_m3_index_decode: the decode block scores and the top-k selection
 * of them in the same call, out written in place at a stable address).
 *   out / topk / init_blocks / local_blocks as in mm3_index_topk.
 *   scores_out  optional (NULL = keep scores in the workspace); when given it
 *               receives the scores exactly as mm3_index_score writes them.
 *   workspace   device memory of >= mm3_index_decode_workspace_bytes(),
 *               256-byte aligned (NULL allowed when that is 0).  Its contents
 *               need no initialisation; overlapping calls must not share it.
 *   sparse      optional (NULL = none): the sparse block table of the
 *               selected ids, built by the selector as it writes them (no
 *               extra launch); needs heads == 1.
 */
int mm3_index_decode(const mm3_problem* p, int32_t topk, int32_t init_blocks,
                     int32_t local_blocks, int32_t* out, int64_t o_head_stride,
                     int64_t o_row_stride, float* scores_out,
                     int64_t s_head_stride, int64_t s_row_stride,
                     int32_t s_width, void* workspace, size_t workspace_bytes,
                     const mm3_sparse_out* sparse, void* stream);

/*
 * mm3_index_prefill_select -- the prefill scorer with the selection fused in
 * (page "ops.index_topk": minimax_m3_index_score followed by
 * minimax_m3_index_topk, in one scorer pass): the workgroup that completes a
 * 512-row tile's blocks selects the tile's rows itself, with no separate
 * selector launch.  Arguments, outputs and rules as in mm3_index_decode
 * (without the sparse table).  Measured slower than mm3_index_decode on the
 * chunked-prefill shapes -- the tiles complete at the end of the scorer's
 * shares, where one workgroup per tile selects with far less parallelism
 * than the selector launch -- so it is a separate call, not a default.
 *   Batches: uniform (no cu_seqlens_q) with heads * query_len > 16, topk <=
 *   16, cdiv(max_seq_len, 128) <= 512, at most 65536 (request, 512-row tile)
 *   units, and scores 16-byte aligned with row and head strides multiples
 *   of 4 (the workspace's scores are); others get MM3_EUNSUPPORTED.
 *   workspace   device memory of >= mm3_index_prefill_select_workspace_bytes(),
 *               256-byte aligned, required (it holds per-tile counters even
 *               with scores_out); its contents need no initialisation (the
 *               call resets the counters); overlapping calls must not share it.
 */
size_t mm3_index_prefill_select_workspace_bytes(const mm3_problem* p, int32_t topk,
                                                int32_t with_scores_out);
int mm3_index_prefill_select(const mm3_problem* p, int32_t topk, int32_t init_blocks,
                             int32_t local_blocks, int32_t* out, int64_t o_head_stride,
                             int64_t o_row_stride, float* scores_out,
                             int64_t s_head_stride, int64_t s_row_stride,
                             int32_t s_width, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * mm3_index_decode_static -- mm3_index_decode for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same computation, arguments and rules
 * as mm3_index_decode, without the workspace arguments: when scores_out is
 * NULL the scores go to a workspace the library holds in device memory of
 * its own, MM3_STATIC_SCRATCH_BYTES (64 MiB) per GPU, allocated when the
 * library's code is loaded onto the GPU and kept until the process ends.
 * Nothing is allocated or freed by the call.
 *   Limit: mm3_index_decode_workspace_bytes(p, topk, 0) at most
 *   MM3_STATIC_SCRATCH_BYTES (enough for heads * total_q *
 *   round_up(cdiv(max_seq_len, 128), 16) <= 16 Mi scores, e.g. 4 heads x
 *   32768 rows x 128 blocks), else MM3_EWORKSPACE and nothing enqueued.
 *   Sharing: every call on one GPU uses that GPU's one workspace, which
 *   holds the last call's scores afterwards (nothing in it needs to start
 *   at zero).  Calls that overlap on one GPU -- on different streams, or
 *   from different host threads without ordering -- race on it; order them
 *   on one stream, or give one of them scores_out or mm3_index_decode.
 */
#define MM3_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int mm3_index_decode_static(const mm3_problem* p, int32_t topk,
                            int32_t init_blocks, int32_t local_blocks,
                            int32_t* out, int64_t o_head_stride,
                            int64_t o_row_stride, float* scores_out,
                            int64_t s_head_stride, int64_t s_row_stride,
                            int32_t s_width, const mm3_sparse_out* sparse,
                            void* stream);

/*
 * mm3_build_sparse_block_table -- the sparse block table (mm3_sparse_out)
 * of ids already selected, for ONE index head (page "ops.index_topk",
 * minimax_m3_index_decode, the optional table arguments).
 *   topk_idx   int32 row t at topk_idx[t*o_row_stride], ids as mm3_index_topk
 *              writes them (ascending, -1 padded).
 *   rows       the batch's rows, as in mm3_problem.
 */
int mm3_build_sparse_block_table(const int32_t* topk_idx, int64_t o_row_stride,
                                 int32_t topk, const mm3_rows* rows,
                                 const mm3_sparse_out* sparse, void* stream);

/*
 * mm3_index_topk_selector -- which selector kernel a selection call launches
 * for a score tensor of this layout and these sizes: mm3_index_topk
 * (by_row_blocks = 0, sparse = 0), mm3_index_topk_blocks (by_row_blocks = 1),
 * or the selection inside mm3_index_decode (sparse = 1 when it builds the
 * sparse block table; scores = the scores_out or workspace pointer it is
 * given).  The kernels (one wave per row with a ballot search, or lanes that
 * select rows by themselves) give identical ids; this names the one that
 * runs, for tests and benchmarks.  Arguments as in those calls (scores is
 * only inspected for its alignment).  Host only, no HIP call.
 * Returns the kernel's name with its template arguments (host string, valid
 * until the next call on this thread), or NULL with mm3_last_error() set for
 * arguments those calls reject.
 */
const char* mm3_index_topk_selector(const float* scores, int64_t s_head_stride,
                                    int64_t s_row_stride, int32_t s_width,
                                    int32_t heads, int32_t total_q,
                                    int32_t max_seq_len, int32_t topk,
                                    int32_t by_row_blocks, int32_t sparse);

/*
 * mm3_index_decode_launches -- how mm3_index_decode runs this problem: 1 when
 * it scores and selects in one launch (every request holds at most 16 rows,
 * heads * query_len <= 16, and sees at most 16 blocks, cdiv(max_seq_len, 128)
 * <= 16; at most 256 requests; no sparse table; scores_out, if given,
 * addressable through one buffer descriptor), 2 when it launches the scorer
 * then the selector.  Both give identical scores and ids (page
 * "ops.index_topk", minimax_m3_index_decode: score then select, one
 * call); this names the path that runs, for tests and benchmarks.
 * Arguments as in mm3_index_decode (scores_out is only inspected, with its
 * strides).  Host only, no HIP call.  Returns 1 or 2, or a negative MM3_E*
 * code with mm3_last_error() set when p is invalid.
 */
int mm3_index_decode_launches(const mm3_problem* p, const float* scores_out,
                              int64_t s_head_stride, int64_t s_row_stride,
                              const mm3_sparse_out* sparse);

/* Message for the last non-OK return on this thread ("" if none).  Host
 * pointer, valid until the next call on this thread. */
const char* mm3_last_error(void);

/* Library version string (host pointer, static). */
const char* mm3_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MM3_INDEX_H */
