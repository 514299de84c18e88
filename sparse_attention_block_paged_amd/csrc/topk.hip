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
// Design.  One wavefront per row.  Each lane holds the scores of blocks
// lane, lane+64, ... as order-preserving u32 keys (forced blocks get the
// largest key), so the k-th largest key T is found by a bitwise search (at
// most 32 steps) whose counts are wave ballots + scalar popcounts; it stops
// as soon as exactly topk keys lie at or above the running threshold, since
// no lower bit can change that set.  Blocks with
// key > T are taken, and keys == T are taken in ascending id order until
// topk are chosen; the same ballot prefix counts (mbcnt) give each chosen id
// its output slot, so the row is written already sorted.  This replaces the
// pages' packed 64-bit (score, id) keys and partial-top-k merges with a
// single-pass threshold select that needs no workspace.
#include <stdio.h>

#include "mm3_device.h"
#include "mm3_lanes.h"
#include "mm3_launch.h"
#include "mm3_rows.h"

namespace mm3 {

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// Selection key of block b with score v (v is not read for b >= nv).
__device__ __forceinline__ uint32_t key_of(float v, int b, int nv, int I, int L) {
  if (b >= nv) return 0u;  // not a candidate (every finite score maps above 0)
  if (b < I || b >= nv - L) return kForcedKey;
  return order_key(v);
}

__device__ __forceinline__ uint32_t block_key(const float* srow, int b, int nv, int I, int L) {
  return key_of(b < nv ? srow[b] : 0.f, b, nv, I, L);
}

// Writes a selected id at its output slot and, with a sparse table, the
// block's attention pages at the same slot; each lane sums the context
// tokens of the ids it wrote.
template <bool SPARSE>
struct Emit {
  int32_t* orow;
  const int32_t* abt;  // the request's attention-table row
  int32_t* st;         // the row's sparse-table row
  int P, stride, pos;
  int len;
  __device__ __forceinline__ void operator()(int slot, int id) {
    orow[slot] = id;
    if constexpr (SPARSE) {
      for (int i = 0; i < P; ++i) st[slot * P + i] = abt[(int64_t)id * stride + i];
      len += min(kBlock, pos - kBlock * id + 1);
    }
  }
};

// E keys per lane in registers: rows with nv <= 64*E.  raw[e] holds the
// score of block 64e + lane, loaded before nv was known.
template <int E, typename EmitT>
__device__ void select_regs(const float* raw, int nv, const TopkArgs& a, EmitT& emit, int lane) {
  uint32_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = key_of(raw[e], 64 * e + lane, nv, a.init_blocks, a.local_blocks);
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) cnt += __popcll(__ballot(key[e] >= cand));
    if (cnt >= a.topk) T = cand;
    if (cnt == a.topk) break;  // exactly topk keys >= T: the rest of T cannot change the set
  }
  int gt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) gt += __popcll(__ballot(key[e] > T));
  const int need = a.topk - gt;
  int base = 0, tie_base = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t tmask = __ballot(key[e] == T);
    const bool sel = key[e] > T || (key[e] == T && tie_base + lanes_below(tmask) < need);
    const uint64_t smask = __ballot(sel);
    if (sel) emit(base + lanes_below(smask), 64 * e + lane);
    base += __popcll(smask);
    tie_base += __popcll(tmask);
  }
}

// Any nv: keys re-read from the score row on every pass.
template <typename EmitT>
__device__ void select_generic(const float* srow, int nv, const TopkArgs& a, EmitT& emit, int lane) {
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int cnt = 0;
    for (int b0 = 0; b0 < nv; b0 += 64)
      cnt += __popcll(__ballot(block_key(srow, b0 + lane, nv, a.init_blocks, a.local_blocks) >= cand));
    if (cnt >= a.topk) T = cand;
    if (cnt == a.topk) break;
  }
  int gt = 0;
  for (int b0 = 0; b0 < nv; b0 += 64)
    gt += __popcll(__ballot(block_key(srow, b0 + lane, nv, a.init_blocks, a.local_blocks) > T));
  const int need = a.topk - gt;
  int base = 0, tie_base = 0;
  for (int b0 = 0; b0 < nv; b0 += 64) {
    const uint32_t k = block_key(srow, b0 + lane, nv, a.init_blocks, a.local_blocks);
    const uint64_t tmask = __ballot(k == T);
    const bool sel = k > T || (k == T && tie_base + lanes_below(tmask) < need);
    const uint64_t smask = __ballot(sel);
    if (sel) emit(base + lanes_below(smask), b0 + lane);
    base += __popcll(smask);
    tie_base += __popcll(tmask);
  }
}

// SPARSE: also the row's sparse block table (one index head, page
// "ops.index_topk", minimax_m3_index_decode: table construction fused into
// the selector).
// rows (waves) per workgroup; 8 and 16 measured equal or slower
constexpr int kTopkWaves = 4;

// Row t's request, position and visible-block count, and the end of its
// request's rows.
struct RowInfo {
  int r, pos, nv, row_end;
};

__device__ __forceinline__ int blocks_at(int pos) { return pos < 0 ? 0 : pos / kBlock + 1; }

__device__ __forceinline__ RowInfo row_info(const TopkArgs& a, int t) {
  RowInfo ri{0, -1, 0, 0};
  if (a.row_blocks != nullptr) {
    ri.nv = a.row_blocks[t];  // given per row (never with a sparse table)
  } else {
    ri.r = row_request(a.rows, t);
    const ReqRows rr = req_rows(a.rows, ri.r);
    ri.pos = rr.p0 + (t - rr.row0);
    ri.nv = blocks_at(ri.pos);
    ri.row_end = rr.row0 + rr.n;
  }
  return ri;
}

// The scores of blocks 64e + lane of row t.  Columns past the score width
// read the row's last column instead (every such block is past nv, so the
// value is never used): no branch around the loads, which keeps the
// compiler's wait counts exact when loads of the next row are in flight.
template <int E>
__device__ __forceinline__ void load_row(const TopkArgs& a, int h, int t, int lane, float* raw) {
  const float* srow = a.scores + (int64_t)h * a.s_head + (int64_t)t * a.s_row;
#pragma unroll
  for (int e = 0; e < E; ++e) raw[e] = srow[min(64 * e + lane, a.s_width - 1)];
}

template <int E, bool SPARSE>
__device__ __forceinline__ void select_row(const TopkArgs& a, int h, int t, const RowInfo& ri,
                                           const float* raw, int lane) {
  const int nv = ri.nv, pos = ri.pos;
  int32_t* orow = a.out + (int64_t)h * a.o_head + (int64_t)t * a.o_row;
  Emit<SPARSE> emit{orow, nullptr, nullptr, 0, 0, pos, 0};
  if constexpr (SPARSE) {
    emit.abt = a.sp.abt + (int64_t)ri.r * a.sp.abt_row;
    emit.st = a.sp.table + (int64_t)t * a.sp.st_row;
    emit.P = a.sp.pages_per_block;
    emit.stride = a.sp.block_page_stride;
  }
  if (nv <= a.topk) {
    // every visible block, then -1
    for (int k = lane; k < a.topk; k += 64) orow[k] = k < nv ? k : -1;
    if constexpr (SPARSE) {
      const int P = emit.P;
      for (int x = lane; x < a.topk * P; x += 64) {
        const int k = x / P, i = x - k * P;
        emit.st[x] = k < nv ? emit.abt[(int64_t)k * emit.stride + i] : -1;
      }
      if (lane == 0) a.sp.ctx_lens[t] = pos + 1 > 0 ? pos + 1 : 0;  // all of blocks 0..pos/128
    }
    return;
  }
  if constexpr (E > 0) {
    select_regs<E>(raw, nv, a, emit, lane);
  } else {
    const float* srow = a.scores + (int64_t)h * a.s_head + (int64_t)t * a.s_row;
    select_generic(srow, nv, a, emit, lane);
  }
  if constexpr (SPARSE) {
    // nv > topk: all topk slots hold ids, no padding
    int len = emit.len;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) len += __shfl_xor(len, off, 64);
    if (lane == 0) a.sp.ctx_lens[t] = len;
  }
}

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

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
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
