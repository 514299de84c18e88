// mm3_select.h -- one wave selects one (head, row): the ballot search over
// order-preserving keys (page "vllm.models.minimax_m3.amd.ops.index_topk",
// module docstring and minimax_m3_index_topk / minimax_m3_index_decode
// docstrings; forced blocks pinned as in page "indexer_cp_exchange", module
// docstring).  Each lane holds the scores of blocks lane, lane + 64, ... as
// order-preserving u32 keys (forced blocks get the largest key), so the k-th
// largest key T is found by a bitwise search (at most 32 steps) whose counts
// are wave ballots + scalar popcounts; it stops as soon as exactly topk keys
// lie at or above the running threshold, since no lower bit can change that
// set.  Blocks with key > T are taken, and keys == T in ascending id order
// until topk are chosen; the same ballot prefix counts (mbcnt) give each
// chosen id its output slot, so the row is written already sorted.  Used by
// the selector kernels (topk.hip).
#pragma once

#include "mm3_device.h"
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

}  // namespace mm3
