// mm3_abi.hip -- the C ABI declared in include/mm3_index.h: host-side
// validation, launch policy and kernel launches.  No device memory is
// allocated or read here, and grids depend only on host arguments, so every
// entry point can be captured in a HIP graph.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "mm3_index.h"
#include "mm3_launch.h"

using namespace mm3;

// Score workspace of mm3_index_decode_static: device memory the library owns,
// one copy per GPU (zero at load; held until the process ends).  Host code
// never uses this name as an address: scratch_ptr() looks the copy of the
// current device up once and passes that address on.
static __device__ __align__(256) uint8_t scratch[MM3_STATIC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return MM3_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MM3_EHIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
}

bool aligned(const void* p, size_t n) { return ((uintptr_t)p % n) == 0; }

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The row map every entry point takes (page "ops.index_topk":
// minimax_m3_index_decode for uniform batches, minimax_m3_index_score and
// minimax_m3_index_topk for cu_seqlens_q / prefix_lens; page
// "indexer_context_parallel", check_context_score_inputs: tokens ==
// requests * query_len).  heads is 0 when the caller has no heads.
int check_rows(const mm3_rows* m, int32_t heads) {
  if (!m) return fail(MM3_EINVAL, "rows is NULL");
  if (m->query_len < 1) return fail(MM3_EINVAL, "query_len must be >= 1, got %d", m->query_len);
  if (m->num_reqs < 0) return fail(MM3_EINVAL, "num_reqs must be >= 0, got %d", m->num_reqs);
  if (m->total_q < 0) return fail(MM3_EINVAL, "total_q must be >= 0, got %d", m->total_q);
  if (m->total_q > MM3_MAX_ROWS)
    return fail(MM3_EINVAL, "total_q must be at most 2^31 - 1024, got %d", m->total_q);
  if (m->max_seq_len < 0) return fail(MM3_EINVAL, "max_seq_len must be >= 0");
  if (!m->seq_lens) return fail(MM3_EINVAL, "seq_lens must be non-NULL");
  if (!aligned(m->seq_lens, 4) || !aligned(m->cu_seqlens_q, 4) || !aligned(m->prefix_lens, 4))
    return fail(MM3_EINVAL, "seq_lens, cu_seqlens_q and prefix_lens must be 4-byte aligned");
  if ((int64_t)heads * m->query_len > INT32_MAX)
    return fail(MM3_EINVAL, "heads * query_len must be below 2^31");
  if (m->num_reqs == 0 && m->total_q != 0)
    return fail(MM3_EINVAL, "total_q must be 0 without requests, got %d", m->total_q);
  if (!m->cu_seqlens_q) {
    if (m->prefix_lens) return fail(MM3_EINVAL, "prefix_lens needs cu_seqlens_q");
    if ((int64_t)m->num_reqs * m->query_len != m->total_q)
      return fail(MM3_EINVAL, "total_q (%d) must equal num_reqs * query_len (%lld) without cu_seqlens_q",
                  m->total_q, (long long)m->num_reqs * m->query_len);
  }
  const int64_t nb = cdiv64(m->max_seq_len, MM3_BLOCK);
  if (nb > MM3_MAX_BLOCKS)
    return fail(MM3_EINVAL, "cdiv(max_seq_len,128) = %lld must be below 65535", (long long)nb);
  return MM3_OK;
}

// Rules every scorer entry point shares (page "indexer_context_parallel",
// check_context_score_inputs and indexer_context_scores; page
// "ops.index_topk", minimax_m3_index_decode).
int check_problem(const mm3_problem* p) {
  if (!p) return fail(MM3_EINVAL, "problem is NULL");
  if (p->heads < 1) return fail(MM3_EINVAL, "heads must be >= 1, got %d", p->heads);
  int rc = check_rows(&p->rows, p->heads);
  if (rc) return rc;
  const int64_t nb = cdiv64(p->rows.max_seq_len, MM3_BLOCK);
  if (!(isfinite(p->sm_scale) && p->sm_scale > 0.0f))
    return fail(MM3_EINVAL, "sm_scale must be finite and > 0");
  if (p->kfmt != MM3_KFMT_BF16 && p->kfmt != MM3_KFMT_NVFP4)
    return fail(MM3_EINVAL, "unknown index-K format %d", p->kfmt);
  if (p->num_pages < 1) return fail(MM3_EINVAL, "index cache must hold >= 1 page");
  if (!p->q || !p->kdata || (!p->block_table && nb > 0))
    return fail(MM3_EINVAL, "q, kdata and block_table must be non-NULL");
  if (p->kfmt == MM3_KFMT_NVFP4 && !p->kscales)
    return fail(MM3_EINVAL, "NVFP4 index cache needs kscales");
  if (!aligned(p->q, 16) || !aligned(p->kdata, 16) || (p->kscales && !aligned(p->kscales, 2)))
    return fail(MM3_EINVAL, "q and kdata must be 16-byte aligned, kscales 2-byte aligned");
  if (p->q_tok_stride % 8 || p->q_head_stride % 8 || p->q_tok_stride < 0 || p->q_head_stride < 0)
    return fail(MM3_EINVAL, "q strides must be non-negative multiples of 8 elements");
  if (p->heads > 1 && p->q_head_stride < MM3_HEAD_DIM)
    return fail(MM3_EINVAL, "q head stride must be >= 128 (D contiguous, heads disjoint)");
  if (p->bt_width < nb)
    return fail(MM3_EINVAL, "block table width %d narrower than cdiv(max_seq_len,128) = %lld",
                p->bt_width, (long long)nb);
  if (p->rows.num_reqs > 1 && p->bt_row_stride < p->bt_width)
    return fail(MM3_EINVAL, "block table row stride must be >= its width");
  return MM3_OK;
}

int check_scores(const mm3_problem* p, const float* s, int64_t sh, int64_t sr, int32_t sw) {
  const int64_t T = p->rows.total_q;
  const int64_t nb = cdiv64(p->rows.max_seq_len, MM3_BLOCK);
  if (!s && nb > 0) return fail(MM3_EINVAL, "scores must be non-NULL");
  if (!aligned(s, 4)) return fail(MM3_EINVAL, "scores must be 4-byte aligned");
  if (sw < nb) return fail(MM3_EINVAL, "score width %d < cdiv(max_seq_len,128) = %lld", sw, (long long)nb);
  if (T > 1 && sr < sw) return fail(MM3_EINVAL, "score row stride must be >= score width");
  if (p->heads > 1 && sh < T * sr) return fail(MM3_EINVAL, "score head stride must be >= tokens * row stride");
  if (sh < 0 || sr < 0) return fail(MM3_EINVAL, "score strides must be non-negative");
  return MM3_OK;
}

int check_select(int32_t topk, int32_t I, int32_t L) {
  if (topk < 1 || topk > MM3_MAX_TOPK) return fail(MM3_EINVAL, "topk must be in [1, 1024], got %d", topk);
  if (I < 0 || L < 0) return fail(MM3_EINVAL, "init_blocks and local_blocks must be >= 0");
  if ((int64_t)I + L > topk)
    return fail(MM3_EINVAL, "init_blocks + local_blocks (%d) exceeds topk (%d)", I + L, topk);
  return MM3_OK;
}

int check_out(int32_t* out, int64_t oh, int64_t orow, int32_t heads, int64_t T, int32_t topk) {
  if (!out) return fail(MM3_EINVAL, "out must be non-NULL");
  if (!aligned(out, 4)) return fail(MM3_EINVAL, "out must be 4-byte aligned");
  if (oh < 0 || orow < 0) return fail(MM3_EINVAL, "out strides must be non-negative");
  if (T > 1 && orow < topk) return fail(MM3_EINVAL, "out row stride must be >= topk");
  if (heads > 1 && oh < T * orow) return fail(MM3_EINVAL, "out head stride must be >= tokens * row stride");
  return MM3_OK;
}

// The sparse-table output (page "ops.index_topk", minimax_m3_index_decode:
// the table arguments come together, one index head, page stride P or 2P,
// the attention table wide enough for every block).
int check_sparse(const mm3_sparse_out* s, const mm3_rows* rows, int32_t topk, int32_t heads) {
  if (!s->attention_block_table || !s->sparse_table || !s->sparse_ctx_lens)
    return fail(MM3_EINVAL, "the sparse-table arguments go together: all of them non-NULL");
  if (heads != 1)
    return fail(MM3_EINVAL, "the sparse block table is built for one index head, got %d", heads);
  const int32_t P = s->pages_per_block;
  if (P < 1) return fail(MM3_EINVAL, "pages_per_block must be >= 1");
  if (s->block_page_stride != P && s->block_page_stride != 2 * P)
    return fail(MM3_EINVAL, "block_page_stride must be P or 2P (P=%d), got %d", P, s->block_page_stride);
  const int64_t nb = cdiv64(rows->max_seq_len, MM3_BLOCK);
  if ((int64_t)s->abt_width < nb * s->block_page_stride)
    return fail(MM3_EINVAL, "attention block table narrower than cdiv(max_seq_len,128)*stride");
  if (rows->num_reqs > 1 && s->abt_row_stride < s->abt_width)
    return fail(MM3_EINVAL, "attention block table row stride must be >= its width");
  if (s->abt_row_stride < 0 || s->st_row_stride < 0)
    return fail(MM3_EINVAL, "sparse-table strides must be non-negative");
  if (rows->total_q > 1 && s->st_row_stride < (int64_t)topk * P)
    return fail(MM3_EINVAL, "sparse table row stride must be >= topk * pages_per_block");
  if (!aligned(s->sparse_table, 4) || !aligned(s->sparse_ctx_lens, 4) ||
      !aligned(s->attention_block_table, 4))
    return fail(MM3_EINVAL, "int32 buffers must be 4-byte aligned");
  return MM3_OK;
}

SparseOut sparse_of(const mm3_sparse_out* s) {
  SparseOut o{};
  o.abt = s->attention_block_table;
  o.abt_row = s->abt_row_stride;
  o.table = s->sparse_table;
  o.st_row = s->st_row_stride;
  o.ctx_lens = s->sparse_ctx_lens;
  o.pages_per_block = s->pages_per_block;
  o.block_page_stride = s->block_page_stride;
  return o;
}

Rows rows_of(const mm3_rows* m) {
  Rows r{};
  r.seq_lens = m->seq_lens;
  r.cu = m->cu_seqlens_q;
  r.prefix = m->cu_seqlens_q ? m->prefix_lens : nullptr;
  r.num_reqs = m->num_reqs;
  r.qlen = m->query_len;
  r.tokens = m->total_q;
  return r;
}

ScoreArgs score_args(const mm3_problem* p, float* s, int64_t sh, int64_t sr) {
  ScoreArgs a{};
  a.q = static_cast<const uint16_t*>(p->q);
  a.q_tok = p->q_tok_stride;
  a.q_head = p->q_head_stride;
  a.kdata = static_cast<const uint8_t*>(p->kdata);
  a.kscales = p->kscales;
  a.bt = p->block_table;
  a.bt_stride = p->bt_row_stride;
  a.rows = rows_of(&p->rows);
  a.scores = s;
  a.s_head = sh;
  a.s_row = sr;
  a.heads = p->heads;
  a.route = kRouteAll;
  a.nb_max = (int32_t)cdiv64(p->rows.max_seq_len, MM3_BLOCK);
  a.sm_scale = p->sm_scale;
  // Decode fallback grid: each wave scores a few pages; aim for enough
  // workgroups to cover the chip several times at the capture-stable size.
  const int64_t total = (int64_t)p->rows.num_reqs * a.nb_max;
  int bpw = 4;  // blocks per workgroup (4 waves)
  while (bpw < 32 && total / bpw > 8192) bpw *= 2;
  a.blocks_per_wg = bpw;
  const int64_t T = p->rows.total_q;
  const int64_t extent = T == 0 ? 0 : ((int64_t)(p->heads - 1) * sh + (T - 1) * sr + a.nb_max) * 4;
  a.s_bytes = extent <= 0x7FFFFFC0 ? (int32_t)extent : 0;
  return a;
}

// Batches that mm3_index_decode scores and selects in one launch: every
// request is a decode request (heads * query_len <= kDecodeRows) that sees at
// most kSmallBlocks blocks, there are few enough of them for one workgroup
// each, no sparse table is asked for, and scores_out (if given) is addressable
// through one buffer descriptor.
bool small_decode_ok(const mm3_problem* p, const float* scores_out, int64_t sh, int64_t sr,
                     const mm3_sparse_out* sparse) {
  const int64_t nb = cdiv64(p->rows.max_seq_len, MM3_BLOCK);
  if (sparse || nb < 1 || nb > kSmallBlocks || p->rows.num_reqs > kSmallMaxReqs) return false;
  if ((int64_t)p->heads * p->rows.query_len > kDecodeRows) return false;
  return !scores_out || score_args(p, const_cast<float*>(scores_out), sh, sr).s_bytes > 0;
}

// Launch policy.  A request with heads * n_r <= 16 rows goes to the decode
// scorer (one MFMA tile of query rows, bandwidth-bound), a larger one to the
// MFMA prefill scorer.  Uniform batches take one of them for every request.
// Ragged batches may hold both kinds, so both launch, each taking only its
// own requests (decided on the device from cu_seqlens_q); the decode one
// sizes its query tile for the largest row count it can take.
int launch_scores(const mm3_problem* p, float* s, int64_t sh, int64_t sr, hipStream_t st) {
  ScoreArgs a = score_args(p, s, sh, sr);
  const bool bf16 = p->kfmt == MM3_KFMT_BF16;
  const int64_t H = p->heads, Q = p->rows.query_len;
  bool decode, prefill;
  ScoreArgs d = a, f = a;
  if (!p->rows.cu_seqlens_q) {
    decode = H * Q <= kDecodeRows;
    prefill = !decode;
  } else {
    decode = H <= kDecodeRows;
    prefill = H * Q > kDecodeRows;
    d.route = kRouteDecode;
    d.rows.qlen = (int32_t)(Q < kDecodeRows / H ? Q : kDecodeRows / H);
    f.route = kRoutePrefill;
  }
  hipError_t e = hipSuccess;
  if (decode) e = bf16 ? launch_decode_score_bf16(d, st) : launch_decode_score_nvfp4(d, st);
  if (e == hipSuccess && prefill) e = bf16 ? launch_prefill_score_bf16(f, st) : launch_prefill_score_nvfp4(f, st);
  return e == hipSuccess ? MM3_OK : hip_fail(e, "scorer launch");
}

// Bytes from a score tensor's base to one past its last element, or 0 when
// that is 2^31 - 64 or more (kernels that address it through one buffer
// descriptor then take another path).
int32_t score_bytes(int64_t sh, int64_t sr, int64_t sw, int64_t heads, int64_t T) {
  if (T == 0) return 0;
  const int64_t extent = ((heads - 1) * sh + (T - 1) * sr + sw) * 4;
  return extent > 0 && extent <= 0x7FFFFFC0 ? (int32_t)extent : 0;
}

TopkArgs topk_args(const float* s, int64_t sh, int64_t sr, int32_t sw, int32_t heads,
                   const mm3_rows* rows, int32_t topk, int32_t I, int32_t L, int32_t* out, int64_t oh,
                   int64_t orow) {
  TopkArgs a{};
  a.scores = s;
  a.s_head = sh;
  a.s_row = sr;
  a.s_width = sw;
  a.rows = rows_of(rows);
  a.out = out;
  a.o_head = oh;
  a.o_row = orow;
  a.heads = heads;
  a.topk = topk;
  a.init_blocks = I;
  a.local_blocks = L;
  a.nb_max = (int32_t)cdiv64(rows->max_seq_len, MM3_BLOCK);
  a.s_bytes = score_bytes(sh, sr, sw, heads, rows->total_q);
  return a;
}

size_t round256(size_t n) { return (n + 255) & ~size_t(255); }

// Bytes of the decode workspace's score area (0 with scores_out).
size_t workspace_score_bytes(const mm3_problem* p, int32_t with_scores_out) {
  if (with_scores_out) return 0;
  const int64_t T = p->rows.total_q;
  const int64_t width = cdiv64(cdiv64(p->rows.max_seq_len, MM3_BLOCK), 16) * 16;
  return round256((size_t)(p->heads * T * width) * sizeof(float));
}

// int32 words the fused prefill selection needs after the score area (a
// counter and an owner per row tile), or 0 when the batch cannot take it:
// uniform batches whose requests all go to the prefill scorer, no sparse
// table, a selection the lane selector takes (the score layout is checked
// at the call).
int fused_prefill_counters(const mm3_problem* p, int32_t topk, const mm3_sparse_out* sparse) {
  if (sparse || p->rows.cu_seqlens_q || p->rows.total_q == 0 || p->rows.max_seq_len == 0 ||
      (int64_t)p->heads * p->rows.query_len <= kDecodeRows)
    return 0;
  ScoreArgs sa = score_args(p, nullptr, 0, 0);
  TopkArgs sel{};
  sel.topk = topk;
  sel.heads = p->heads;
  sel.s_bytes = 1;
  return prefill_select_counters(sa, sel);
}

// The device address of `scratch` on the current device, looked up the
// first time a device asks (with that device current) and kept per device.
// Returns nullptr after setting the error message when the lookup fails.
void* scratch_ptr() {
  static std::mutex mu;
  static void* ptrs[64] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice"), nullptr;
  if (dev < 0 || dev >= 64) return fail(MM3_EHIP, "device index %d out of range", dev), nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e, "hipGetSymbolAddress(scratch)"), nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

}  // namespace

extern "C" {

const char* mm3_last_error(void) { return g_err.c_str(); }

const char* mm3_version(void) { return "mm3idx 0.2 gfx950"; }

int mm3_index_score(const mm3_problem* p, float* scores, int64_t s_head_stride,
                    int64_t s_row_stride, int32_t s_width, void* stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if ((rc = check_scores(p, scores, s_head_stride, s_row_stride, s_width))) return rc;
  if (p->rows.total_q == 0 || p->rows.max_seq_len == 0) return ok();
  if ((rc = launch_scores(p, scores, s_head_stride, s_row_stride, (hipStream_t)stream))) return rc;
  return ok();
}

int mm3_index_topk(const float* scores, int64_t s_head_stride, int64_t s_row_stride,
                   int32_t s_width, int32_t heads, const mm3_rows* rows, int32_t topk,
                   int32_t init_blocks, int32_t local_blocks, int32_t* out, int64_t o_head_stride,
                   int64_t o_row_stride, void* stream) {
  if (heads < 1) return fail(MM3_EINVAL, "heads must be >= 1");
  int rc = check_rows(rows, 0);
  if (rc) return rc;
  const int64_t nb = cdiv64(rows->max_seq_len, MM3_BLOCK);
  if ((rc = check_select(topk, init_blocks, local_blocks))) return rc;
  const int64_t T = rows->total_q;
  if (!scores && nb > 0) return fail(MM3_EINVAL, "scores must be non-NULL");
  if (!aligned(scores, 4)) return fail(MM3_EINVAL, "scores must be 4-byte aligned");
  if (s_width < nb) return fail(MM3_EINVAL, "score width < cdiv(max_seq_len,128)");
  if (s_head_stride < 0 || s_row_stride < 0) return fail(MM3_EINVAL, "score strides must be non-negative");
  if (T > 1 && s_row_stride < s_width) return fail(MM3_EINVAL, "score row stride must be >= score width");
  if (heads > 1 && s_head_stride < T * s_row_stride)
    return fail(MM3_EINVAL, "score head stride must be >= tokens * row stride");
  if ((rc = check_out(out, o_head_stride, o_row_stride, heads, T, topk))) return rc;
  if (T == 0) return ok();
  TopkArgs a = topk_args(scores, s_head_stride, s_row_stride, s_width, heads, rows, topk,
                         init_blocks, local_blocks, out, o_head_stride, o_row_stride);
  hipError_t e = launch_topk(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "top-k launch");
  return ok();
}

int mm3_index_topk_blocks(const float* scores, int64_t s_head_stride, int64_t s_row_stride,
                          int32_t s_width, int32_t heads, const int32_t* row_blocks,
                          int32_t total_q, int32_t max_seq_len, int32_t topk, int32_t init_blocks,
                          int32_t local_blocks, int32_t* out, int64_t o_head_stride,
                          int64_t o_row_stride, void* stream) {
  if (heads < 1) return fail(MM3_EINVAL, "heads must be >= 1");
  if (total_q < 0) return fail(MM3_EINVAL, "total_q must be >= 0, got %d", total_q);
  if (total_q > MM3_MAX_ROWS) return fail(MM3_EINVAL, "total_q must be at most 2^31 - 1024, got %d", total_q);
  if (max_seq_len < 0) return fail(MM3_EINVAL, "max_seq_len must be >= 0");
  const int64_t nb = cdiv64(max_seq_len, MM3_BLOCK);
  if (nb > MM3_MAX_BLOCKS)
    return fail(MM3_EINVAL, "cdiv(max_seq_len,128) = %lld must be below 65535", (long long)nb);
  int rc = check_select(topk, init_blocks, local_blocks);
  if (rc) return rc;
  if (!row_blocks) return fail(MM3_EINVAL, "row_blocks must be non-NULL");
  if (!aligned(row_blocks, 4)) return fail(MM3_EINVAL, "row_blocks must be 4-byte aligned");
  const int64_t T = total_q;
  if (!scores && nb > 0) return fail(MM3_EINVAL, "scores must be non-NULL");
  if (!aligned(scores, 4)) return fail(MM3_EINVAL, "scores must be 4-byte aligned");
  if (s_width < nb) return fail(MM3_EINVAL, "score width < cdiv(max_seq_len,128)");
  if (s_head_stride < 0 || s_row_stride < 0) return fail(MM3_EINVAL, "score strides must be non-negative");
  if (T > 1 && s_row_stride < s_width) return fail(MM3_EINVAL, "score row stride must be >= score width");
  if (heads > 1 && s_head_stride < T * s_row_stride)
    return fail(MM3_EINVAL, "score head stride must be >= tokens * row stride");
  if ((rc = check_out(out, o_head_stride, o_row_stride, heads, T, topk))) return rc;
  if (T == 0) return ok();
  TopkArgs a{};
  a.scores = scores;
  a.s_head = s_head_stride;
  a.s_row = s_row_stride;
  a.s_width = s_width;
  a.rows.tokens = total_q;  // rows map unused: nv comes from row_blocks
  a.out = out;
  a.o_head = o_head_stride;
  a.o_row = o_row_stride;
  a.heads = heads;
  a.topk = topk;
  a.init_blocks = init_blocks;
  a.local_blocks = local_blocks;
  a.nb_max = (int32_t)nb;
  a.row_blocks = row_blocks;
  a.s_bytes = score_bytes(s_head_stride, s_row_stride, s_width, heads, T);
  hipError_t e = launch_topk(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "top-k launch");
  return ok();
}

size_t mm3_index_decode_workspace_bytes(const mm3_problem* p, int32_t topk, int32_t with_scores_out) {
  if (check_problem(p)) return 0;
  if (check_select(topk, 0, 0)) return 0;
  g_err.clear();
  return workspace_score_bytes(p, with_scores_out);
}

size_t mm3_index_prefill_select_workspace_bytes(const mm3_problem* p, int32_t topk, int32_t with_scores_out) {
  if (check_problem(p)) return 0;
  if (check_select(topk, 0, 0)) return 0;
  if (p->rows.total_q == 0) return ok(), 0;  // nothing to score or select
  if (p->rows.max_seq_len == 0) return ok(), workspace_score_bytes(p, with_scores_out);
  const int nctr = fused_prefill_counters(p, topk, nullptr);
  if (nctr == 0) {
    fail(MM3_EUNSUPPORTED, "the batch cannot take the fused prefill selection (it needs a uniform batch "
                           "whose requests all go to the prefill scorer, topk <= 16, rows of at most 512 "
                           "blocks and at most 65536 row tiles)");
    return 0;
  }
  g_err.clear();
  return workspace_score_bytes(p, with_scores_out) + round256((size_t)nctr * sizeof(int32_t));
}

int mm3_index_decode(const mm3_problem* p, int32_t topk, int32_t init_blocks,
                     int32_t local_blocks, int32_t* out, int64_t o_head_stride,
                     int64_t o_row_stride, float* scores_out, int64_t s_head_stride,
                     int64_t s_row_stride, int32_t s_width, void* workspace,
                     size_t workspace_bytes, const mm3_sparse_out* sparse, void* stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if ((rc = check_select(topk, init_blocks, local_blocks))) return rc;
  const int64_t T = p->rows.total_q;
  if ((rc = check_out(out, o_head_stride, o_row_stride, p->heads, T, topk))) return rc;
  if (sparse && (rc = check_sparse(sparse, &p->rows, topk, p->heads))) return rc;
  float* s = scores_out;
  int64_t sh = s_head_stride, sr = s_row_stride;
  int32_t sw = s_width;
  const size_t score_area = workspace_score_bytes(p, s != nullptr);
  if (s) {
    if ((rc = check_scores(p, s, sh, sr, sw))) return rc;
  } else {
    if (score_area && (!workspace || workspace_bytes < score_area || !aligned(workspace, 256)))
      return fail(MM3_EWORKSPACE, "workspace must be 256-byte aligned and hold %zu bytes (got %zu)",
                  mm3_index_decode_workspace_bytes(p, topk, 0), workspace_bytes);
    sw = (int32_t)(cdiv64(cdiv64(p->rows.max_seq_len, MM3_BLOCK), 16) * 16);
    sr = sw;
    sh = T * sr;
    s = static_cast<float*>(workspace);
  }
  if (T == 0) return ok();
  hipStream_t st = (hipStream_t)stream;
  TopkArgs a = topk_args(s, sh, sr, sw, p->heads, &p->rows, topk, init_blocks, local_blocks, out,
                         o_head_stride, o_row_stride);
  if (small_decode_ok(p, scores_out, sh, sr, sparse)) {
    // one launch: the scores stay on chip unless the caller asked for them
    ScoreArgs sa = score_args(p, scores_out, sh, sr);
    if (!scores_out) sa.s_bytes = 0;
    const hipError_t e = launch_decode_small(sa, a, p->kfmt == MM3_KFMT_BF16 ? 0 : 1, st);
    return e == hipSuccess ? ok() : hip_fail(e, "small-batch decode launch");
  }
  if (sparse) {
    a.sp = sparse_of(sparse);
    a.sparse = 1;
  }
  if (p->rows.max_seq_len > 0 && (rc = launch_scores(p, s, sh, sr, st))) return rc;
  hipError_t e = launch_topk(a, st);
  if (e != hipSuccess) return hip_fail(e, "top-k launch");
  return ok();
}

int mm3_index_decode_launches(const mm3_problem* p, const float* scores_out, int64_t s_head_stride,
                              int64_t s_row_stride, const mm3_sparse_out* sparse) {
  const int rc = check_problem(p);
  if (rc) return rc;
  g_err.clear();
  return small_decode_ok(p, scores_out, s_head_stride, s_row_stride, sparse) ? 1 : 2;
}

const char* mm3_index_topk_selector(const float* scores, int64_t s_head_stride, int64_t s_row_stride,
                                    int32_t s_width, int32_t heads, int32_t total_q, int32_t max_seq_len,
                                    int32_t topk, int32_t by_row_blocks, int32_t sparse) {
  if (heads < 1) return fail(MM3_EINVAL, "heads must be >= 1"), nullptr;
  if (total_q < 0 || total_q > MM3_MAX_ROWS)
    return fail(MM3_EINVAL, "total_q must be in [0, 2^31 - 1024], got %d", total_q), nullptr;
  if (max_seq_len < 0) return fail(MM3_EINVAL, "max_seq_len must be >= 0"), nullptr;
  const int64_t nb = cdiv64(max_seq_len, MM3_BLOCK);
  if (nb > MM3_MAX_BLOCKS)
    return fail(MM3_EINVAL, "cdiv(max_seq_len,128) = %lld must be below 65535", (long long)nb), nullptr;
  if (topk < 1 || topk > MM3_MAX_TOPK) return fail(MM3_EINVAL, "topk must be in [1, 1024], got %d", topk), nullptr;
  if (s_width < nb) return fail(MM3_EINVAL, "score width < cdiv(max_seq_len,128)"), nullptr;
  if (s_head_stride < 0 || s_row_stride < 0) return fail(MM3_EINVAL, "score strides must be non-negative"), nullptr;
  if (sparse && (heads != 1 || by_row_blocks))
    return fail(MM3_EINVAL, "the sparse block table is built for one index head, from positions"), nullptr;
  TopkArgs a{};
  a.scores = scores;
  a.s_head = s_head_stride;
  a.s_row = s_row_stride;
  a.s_width = s_width;
  a.rows.tokens = total_q;
  a.heads = heads;
  a.topk = topk;
  a.nb_max = (int32_t)nb;
  a.sparse = sparse ? 1 : 0;
  a.row_blocks = by_row_blocks ? reinterpret_cast<const int32_t*>(16) : nullptr;  // only tested for NULL
  a.s_bytes = score_bytes(s_head_stride, s_row_stride, s_width, heads, total_q);
  g_err.clear();
  return topk_kernel_name(a);
}

int mm3_index_prefill_select(const mm3_problem* p, int32_t topk, int32_t init_blocks,
                             int32_t local_blocks, int32_t* out, int64_t o_head_stride,
                             int64_t o_row_stride, float* scores_out, int64_t s_head_stride,
                             int64_t s_row_stride, int32_t s_width, void* workspace,
                             size_t workspace_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if ((rc = check_select(topk, init_blocks, local_blocks))) return rc;
  const int64_t T = p->rows.total_q;
  if ((rc = check_out(out, o_head_stride, o_row_stride, p->heads, T, topk))) return rc;
  if (T == 0) return ok();
  if (p->rows.max_seq_len == 0)  // no row sees a block: the selector writes the -1 rows
    return mm3_index_decode(p, topk, init_blocks, local_blocks, out, o_head_stride, o_row_stride,
                            scores_out, s_head_stride, s_row_stride, s_width, workspace,
                            workspace_bytes, nullptr, stream);
  const int nctr = fused_prefill_counters(p, topk, nullptr);
  if (nctr == 0)
    return fail(MM3_EUNSUPPORTED, "the batch cannot take the fused prefill selection (it needs a uniform "
                                  "batch whose requests all go to the prefill scorer, topk <= 16, rows of at "
                                  "most 512 blocks and at most 65536 row tiles)");
  float* s = scores_out;
  int64_t sh = s_head_stride, sr = s_row_stride;
  int32_t sw = s_width;
  const size_t score_area = workspace_score_bytes(p, s != nullptr);
  const size_t need = score_area + round256((size_t)nctr * sizeof(int32_t));
  if (s && (rc = check_scores(p, s, sh, sr, sw))) return rc;
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
    return fail(MM3_EWORKSPACE, "workspace must be 256-byte aligned and hold %zu bytes (got %zu)", need,
                workspace_bytes);
  if (!s) {
    sw = (int32_t)(cdiv64(cdiv64(p->rows.max_seq_len, MM3_BLOCK), 16) * 16);
    sr = sw;
    sh = T * sr;
    s = static_cast<float*>(workspace);
  }
  TopkArgs a = topk_args(s, sh, sr, sw, p->heads, &p->rows, topk, init_blocks, local_blocks, out,
                         o_head_stride, o_row_stride);
  if (!lanes_layout_ok(a))
    return fail(MM3_EUNSUPPORTED, "the fused prefill selection reads score rows 16 bytes at a time: scores "
                                  "16-byte aligned, row and head strides multiples of 4, under 2 GiB");
  int32_t* ctr = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) + score_area);
  hipError_t e = launch_prefill_score_select(score_args(p, s, sh, sr), p->kfmt, a, ctr, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fused scorer launch");
  return ok();
}

int mm3_index_decode_static(const mm3_problem* p, int32_t topk, int32_t init_blocks,
                            int32_t local_blocks, int32_t* out, int64_t o_head_stride,
                            int64_t o_row_stride, float* scores_out, int64_t s_head_stride,
                            int64_t s_row_stride, int32_t s_width, const mm3_sparse_out* sparse,
                            void* stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if ((rc = check_select(topk, init_blocks, local_blocks))) return rc;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (!scores_out) {
    const size_t need = workspace_score_bytes(p, 0);
    if (need > MM3_STATIC_SCRATCH_BYTES)
      return fail(MM3_EWORKSPACE,
                  "the scores of this batch need %zu bytes of workspace, more than the %zu the "
                  "library holds for mm3_index_decode_static; pass scores_out or call "
                  "mm3_index_decode with a workspace",
                  need, (size_t)MM3_STATIC_SCRATCH_BYTES);
    if (!(ws = scratch_ptr())) return MM3_EHIP;
    ws_bytes = MM3_STATIC_SCRATCH_BYTES;
  }
  return mm3_index_decode(p, topk, init_blocks, local_blocks, out, o_head_stride, o_row_stride,
                          scores_out, s_head_stride, s_row_stride, s_width, ws, ws_bytes, sparse,
                          stream);
}

int mm3_build_sparse_block_table(const int32_t* topk_idx, int64_t o_row_stride, int32_t topk,
                                 const mm3_rows* rows, const mm3_sparse_out* sparse, void* stream) {
  if (!topk_idx || !sparse)
    return fail(MM3_EINVAL, "the sparse-table arguments go together: all of them non-NULL");
  if (topk < 1 || topk > MM3_MAX_TOPK) return fail(MM3_EINVAL, "topk must be in [1, 1024]");
  int rc = check_rows(rows, 0);
  if (rc) return rc;
  if ((rc = check_sparse(sparse, rows, topk, 1))) return rc;
  const int64_t T = rows->total_q;
  if (T > 1 && o_row_stride < topk) return fail(MM3_EINVAL, "topk row stride must be >= topk");
  if (o_row_stride < 0) return fail(MM3_EINVAL, "topk row stride must be non-negative");
  if (!aligned(topk_idx, 4)) return fail(MM3_EINVAL, "int32 buffers must be 4-byte aligned");
  if (T == 0) return ok();
  SparseTableArgs a{};
  a.topk_idx = topk_idx;
  a.o_row = o_row_stride;
  a.rows = rows_of(rows);
  a.sp = sparse_of(sparse);
  a.topk = topk;
  hipError_t e = launch_sparse_table(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sparse-table launch");
  return ok();
}

}  // extern "C"
