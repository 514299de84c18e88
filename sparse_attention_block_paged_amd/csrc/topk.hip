// topk.hip -- per (head, row) block selection and the sparse block table.
//
// What it computes (page "vllm.models.minimax_m3.amd.ops.index_topk", module
// docstring and minimax_m3_index_topk / minimax_m3_index_decode docstrings;
// page "indexer_cp_exchange", module docstring, for the pinned forced
// blocks): each (head, row) keeps the init and local blocks and fills the
// rest of its topk slots with the best-scoring other visible blocks,
// 0-indexed, -1 padded.  Ties go to the lower block id; ids are written in
// ascending order.
//
// Design.  Two selectors with identical results: one wave per row with a
// ballot search over the row's keys (mm3_select.h), and lanes that select
// rows by themselves with sorting networks (mm3_lanes.h), for batches with
// many rows.  Both replace the pages' packed 64-bit (score, id) keys and
// partial-top-k merges with a single pass that needs no workspace.
#include <stdio.h>

#include "mm3_device.h"
#include "mm3_lanes.h"
#include "mm3_select.h"
#include "mm3_launch.h"
#include "mm3_rows.h"

namespace mm3 {

// SPARSE: also the row's sparse block table (one index head, page
// "ops.index_topk", minimax_m3_index_decode: table construction fused into
// the selector).
// rows (waves) per workgroup; 8 and 16 measured equal or slower
constexpr int kTopkWaves = 4;

// One wave per run of RPW consecutive (head, row)s.  A row's scores go out
// first: their address needs only the row, so their latency overlaps that of
// the loads nv depends on (the request's length, or the row's block count).
// With RPW > 1 the next row's scores (and block count, when given) are loaded
// before the current row is selected, so a wave keeps them in flight while it
// searches; the next row's position follows from the current one while both
// rows are in one request, and is looked up only past its end.
template <int E, bool SPARSE, int RPW, bool ROWB>
__global__ __launch_bounds__(64 * kTopkWaves) void topk_kernel(TopkArgs a) {
  constexpr int ER = E > 0 ? E : 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.y;
  int t = (blockIdx.x * kTopkWaves + wave) * RPW;
  if (t >= a.rows.tokens) return;
  const int t_end = min(a.rows.tokens, t + RPW);
  float raw[ER];
  if constexpr (E > 0) load_row<E>(a, h, t, lane, raw);
  RowInfo ri = row_info(a, t);
  if constexpr (RPW == 1) {
    select_row<E, SPARSE>(a, h, t, ri, raw, lane);
  } else {
    while (true) {
      // the next row's loads (the last row reloads itself, unused)
      const int tn = t + 1 < t_end ? t + 1 : t;
      float raw_n[ER];
      int nv_n = 0;
      if constexpr (E > 0) load_row<E>(a, h, tn, lane, raw_n);
      if constexpr (ROWB) nv_n = a.row_blocks[tn];
      // keep these loads ahead of the selection's stores
      asm volatile("" ::: "memory");
      select_row<E, SPARSE>(a, h, t, ri, raw, lane);
      if (tn == t) break;
      for (int e = 0; e < ER; ++e) raw[e] = raw_n[e];
      t = tn;
      if constexpr (ROWB) {
        ri.nv = nv_n;
      } else if (t < ri.row_end) {
        ri.pos += 1;
        ri.nv = blocks_at(ri.pos);
      } else {
        ri = row_info(a, t);
      }
    }
  }
}

// One wave per 64/SPLIT consecutive rows of head blockIdx.y.
template <int NC, bool ROWB, int SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void topk_lanes_kernel(TopkArgs a) {
  __shared__ __attribute__((aligned(16))) float tr[4][64 * kLaneRowFloats];
  const int wave = threadIdx.x >> 6;
  const int t0 = (blockIdx.x * 4 + wave) * (64 / SPLIT);
  lane_select<NC, ROWB, SPLIT>(a, blockIdx.y, t0, a.rows.tokens, tr[wave]);
}

#ifndef MM3_TOPK_RPW
#define MM3_TOPK_RPW 4
#endif
#ifndef MM3_TOPK_LANES
#define MM3_TOPK_LANES 1
#endif

template <bool SPARSE, int RPW, bool ROWB>
static void launch_topk_t(const TopkArgs& a, hipStream_t s) {
  const int T = a.rows.tokens;
  const int waves = (T + RPW - 1) / RPW;
  dim3 grid((waves + kTopkWaves - 1) / kTopkWaves, a.heads), block(64 * kTopkWaves);
  const int nb = a.nb_max;
  if (nb <= 64)
    hipLaunchKernelGGL((topk_kernel<1, SPARSE, RPW, ROWB>), grid, block, 0, s, a);
  else if (nb <= 128)
    hipLaunchKernelGGL((topk_kernel<2, SPARSE, RPW, ROWB>), grid, block, 0, s, a);
  else if (nb <= 256)
    hipLaunchKernelGGL((topk_kernel<4, SPARSE, RPW, ROWB>), grid, block, 0, s, a);
  else if (nb <= 512)
    hipLaunchKernelGGL((topk_kernel<8, SPARSE, RPW, ROWB>), grid, block, 0, s, a);
  else if (nb <= 1024)
    hipLaunchKernelGGL((topk_kernel<16, SPARSE, RPW, ROWB>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((topk_kernel<0, SPARSE, RPW, ROWB>), grid, block, 0, s, a);
}

// Which form of the lane selector takes a batch, or none (split == 0: one
// wave per row).  It needs topk within the kept list, score rows that the
// 16-byte loads can read, and (head, row) pairs enough for about one wave per
// SIMD (below that the ballot search measured faster).  A lane takes
// 16*kLaneChunks blocks of a row (64: registers for four waves per SIMD), and
// 1, 2, 4 or 8 lanes share a row of up to 64, 128, 256 or 512 blocks.
#ifndef MM3_LANE1_MIN_ROWS
#define MM3_LANE1_MIN_ROWS 65536  // rows of up to 64 blocks
#endif
#ifndef MM3_LANE2_MIN_ROWS
#define MM3_LANE2_MIN_ROWS 24576  // up to 128
#endif
#ifndef MM3_LANE4_MIN_ROWS
#define MM3_LANE4_MIN_ROWS 16384  // up to 256
#endif
#ifndef MM3_LANE8_MIN_ROWS
#define MM3_LANE8_MIN_ROWS 8192   // up to 512
#endif
bool lanes_layout_ok(const TopkArgs& a) {
  return a.s_bytes > 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0 && a.s_row % 4 == 0 &&
         (a.heads == 1 || a.s_head % 4 == 0);
}

static int lanes_split(const TopkArgs& a, int64_t rows) {
  const bool ok = a.topk <= kLaneTop && lanes_layout_ok(a);
  const int nb = a.nb_max;
  if (!ok || nb > 512) return 0;
  const int64_t min_rows = nb <= 64    ? MM3_LANE1_MIN_ROWS
                           : nb <= 128 ? MM3_LANE2_MIN_ROWS
                           : nb <= 256 ? MM3_LANE4_MIN_ROWS
                                       : MM3_LANE8_MIN_ROWS;
  if (rows < min_rows) return 0;
  int split = 1;
  while (16 * kLaneChunks * split < nb) split *= 2;
  return split <= 8 ? split : 0;
}

template <bool ROWB>
static void launch_topk_lanes(const TopkArgs& a, int split, hipStream_t s) {
  constexpr int NC = kLaneChunks;
  const int rows_per_wg = 4 * 64 / split;
  dim3 grid((a.rows.tokens + rows_per_wg - 1) / rows_per_wg, a.heads), block(256);
  switch (split) {
    case 1: hipLaunchKernelGGL((topk_lanes_kernel<NC, ROWB, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((topk_lanes_kernel<NC, ROWB, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((topk_lanes_kernel<NC, ROWB, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((topk_lanes_kernel<NC, ROWB, 8>), grid, block, 0, s, a); break;
    default: break;  // lanes_split returns 1, 2, 4 or 8 only
  }
}

// Which selector kernel takes a batch: the lane selector (split lanes per
// row), or one wave per row (rpw rows per wave, E keys per lane, 0 for the
// form that re-reads long rows).
struct TopkPlan {
  int split;
  int rpw;
  int E;
  bool sparse;
  bool rowb;
};

static TopkPlan plan_topk(const TopkArgs& a) {
  TopkPlan p{};
  // several rows per wave only when there are rows enough to keep every
  // wave slot of the chip busy that way (prefill-sized batches)
  const int64_t rows = (int64_t)a.rows.tokens * a.heads;
  const bool multi = MM3_TOPK_RPW > 1 && rows >= 65536 && a.nb_max <= 1024;
  p.rowb = a.row_blocks != nullptr;
  p.sparse = a.sparse != 0;
  p.split = (!a.sparse && MM3_TOPK_LANES) ? lanes_split(a, rows) : 0;
  p.rpw = (!p.split && !p.sparse && multi) ? MM3_TOPK_RPW : 1;
  const int nb = a.nb_max;
  p.E = nb <= 64 ? 1 : nb <= 128 ? 2 : nb <= 256 ? 4 : nb <= 512 ? 8 : nb <= 1024 ? 16 : 0;
  return p;
}

// No row of the batch sees a block (cdiv(max_seq_len, 128) == 0): every id
// is -1, and with a sparse table every slot -1 and every context length 0.
// The selectors are not launched then: their branch-free row loads assume a
// score row of at least one column.
__global__ __launch_bounds__(256) void no_blocks_kernel(TopkArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= a.rows.tokens) return;
  for (int h = 0; h < a.heads; ++h)
    for (int k = lane; k < a.topk; k += 64) a.out[(int64_t)h * a.o_head + (int64_t)t * a.o_row + k] = -1;
  if (a.sparse) {
    int32_t* st = a.sp.table + (int64_t)t * a.sp.st_row;
    for (int x = lane; x < a.topk * a.sp.pages_per_block; x += 64) st[x] = -1;
    if (lane == 0) a.sp.ctx_lens[t] = 0;
  }
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.nb_max == 0) {
    hipLaunchKernelGGL(no_blocks_kernel, dim3((a.rows.tokens + 3) / 4), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const TopkPlan p = plan_topk(a);
  if (p.split) {
    if (p.rowb)
      launch_topk_lanes<true>(a, p.split, s);
    else
      launch_topk_lanes<false>(a, p.split, s);
  } else if (p.sparse)
    launch_topk_t<true, 1, false>(a, s);
  else if (p.rpw > 1 && p.rowb)
    launch_topk_t<false, MM3_TOPK_RPW, true>(a, s);
  else if (p.rpw > 1)
    launch_topk_t<false, MM3_TOPK_RPW, false>(a, s);
  else
    launch_topk_t<false, 1, false>(a, s);
  return hipGetLastError();
}

const char* topk_kernel_name(const TopkArgs& a) {
  if (a.nb_max == 0) return "no_blocks_kernel";
  const TopkPlan p = plan_topk(a);
  static thread_local char buf[96];
  if (p.split)
    snprintf(buf, sizeof buf, "topk_lanes_kernel<%d, %s, %d>", kLaneChunks, p.rowb ? "true" : "false",
             p.split);
  else
    snprintf(buf, sizeof buf, "topk_kernel<%d, %s, %d, %s>", p.E, p.sparse ? "true" : "false", p.rpw,
             (p.rpw > 1 && p.rowb) ? "true" : "false");
  return buf;
}

// ------------------------------------------------------ sparse block table
//
// For one index head (page "ops.index_topk", minimax_m3_index_decode, the
// optional sparse-table arguments): the P attention pages of each selected
// block, and the number of tokens the row's sparse context holds.  One wave
// per row; lanes walk the topk*P output slots.

__global__ __launch_bounds__(256) void sparse_table_kernel(SparseTableArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.rows.tokens) return;
  const int r = row_request(a.rows, t);
  const ReqRows rr = req_rows(a.rows, r);
  const int pos = rr.p0 + (t - rr.row0);
  const int32_t* ids = a.topk_idx + (int64_t)t * a.o_row;
  const int32_t* abt = a.sp.abt + (int64_t)r * a.sp.abt_row;
  int32_t* st = a.sp.table + (int64_t)t * a.sp.st_row;
  const int P = a.sp.pages_per_block, slots = a.topk * P;
  for (int x = lane; x < slots; x += 64) {
    const int k = x / P, i = x - k * P;
    const int b = ids[k];
    st[x] = b < 0 ? -1 : abt[(int64_t)b * a.sp.block_page_stride + i];
  }
  int len = 0;
  for (int k = lane; k < a.topk; k += 64) {
    const int b = ids[k];
    if (b >= 0 && pos >= 0) len += max(0, min(kBlock, pos - kBlock * b + 1));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) len += __shfl_xor(len, off, 64);
  if (lane == 0) a.sp.ctx_lens[t] = len;
}

hipError_t launch_sparse_table(const SparseTableArgs& a, hipStream_t s) {
  const int T = a.rows.tokens;
  hipLaunchKernelGGL(sparse_table_kernel, dim3((T + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mm3
