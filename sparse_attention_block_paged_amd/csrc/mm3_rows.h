// mm3_rows.h -- device side of the row map: which request a row belongs to
// and at which position it sits (page "vllm.models.minimax_m3.amd.ops.
// index_topk": uniform decode batches in minimax_m3_index_decode, ragged
// cu_seqlens_q / prefix_lens batches in minimax_m3_index_score and
// minimax_m3_index_topk).
#pragma once

#include "mm3_device.h"
#include "mm3_launch.h"

namespace mm3 {

// Request r's rows: the first row, how many, and the first one's position
// (row j of the request sits at p0 + j).
struct ReqRows {
  int row0;
  int n;
  int p0;
};

// SCALAR: r is wave-uniform and the loads go through the scalar cache (the
// arrays are read-only for the whole launch).
template <bool SCALAR>
__device__ __forceinline__ int ld_i32(const int32_t* p, int i) {
  if constexpr (SCALAR)
    return ((const int32_t __attribute__((address_space(4)))*)p)[i];
  else
    return p[i];
}

template <bool SCALAR = false>
__device__ __forceinline__ ReqRows req_rows(const Rows& m, int r) {
  ReqRows q;
  if (m.cu == nullptr) {
    q.row0 = r * m.qlen;
    q.n = m.qlen;
    q.p0 = ld_i32<SCALAR>(m.seq_lens, r) - m.qlen;
  } else {
    q.row0 = ld_i32<SCALAR>(m.cu, r);
    q.n = ld_i32<SCALAR>(m.cu, r + 1) - q.row0;
    q.p0 = m.prefix != nullptr ? ld_i32<SCALAR>(m.prefix, r) : ld_i32<SCALAR>(m.seq_lens, r) - q.n;
  }
  return q;
}

// Blocks the request's last row sees: every block any of its rows sees.
__device__ __forceinline__ int req_blocks(int p0, int n) {
  const int pl = p0 + n - 1;
  return (n > 0 && pl >= 0) ? pl / kBlock + 1 : 0;
}

// Whether a scorer launch with this route takes a request of n rows.
__device__ __forceinline__ bool routed(int route, int heads, int n) {
  if (route == kRouteAll) return true;
  const bool small = heads * n <= kDecodeRows;
  return route == kRouteDecode ? small : !small;
}

// The request that owns row t.  t must be wave-uniform and the whole wave
// active.  Ragged batches: the last r with cu[r] <= t (that request owns t
// even when requests before it are empty), found 64 entries per step -- each
// lane tests one candidate and a ballot keeps the last that passes -- so
// 4096 requests take two dependent loads.
__device__ __forceinline__ int row_request(const Rows& m, int t) {
  if (m.cu == nullptr) return t / m.qlen;
  const int lane = threadIdx.x & 63;
  int lo = 0, n = m.num_reqs;  // the answer lies in [lo, lo + n); cu[lo] <= t
  while (n > 1) {
    const int step = (n + 63) >> 6;
    const int off = lane * step;
    const int idx = lo + min(off, n - 1);  // in [lo, lo + n): every lane loads in bounds
    const bool ok = off < n && m.cu[idx] <= t;
    const uint64_t bal = __ballot(ok);  // lanes 0..k (cu is sorted); lane 0 always
    const int k = 63 - __builtin_clzll(bal);
    lo += k * step;
    n = min(step, n - k * step);
  }
  return lo;
}

}  // namespace mm3
