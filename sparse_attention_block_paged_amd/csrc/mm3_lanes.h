// mm3_lanes.h -- per (head, row) selection by lanes that select rows by
// themselves (page "vllm.models.minimax_m3.amd.ops.index_topk", module
// docstring and minimax_m3_index_topk: top-k blocks per query token, forced
// init and local blocks pinned as in page "indexer_cp_exchange", module
// docstring; ties to the lower id, ids ascending, -1 padded).  Used by the
// selector kernel (topk.hip) and by the prefill scorer's fused selection
// (prefill_score.hip).
#pragma once

#include "mm3_device.h"
#include "mm3_launch.h"
#include "mm3_rows.h"

namespace mm3 {

__device__ __forceinline__ int lanes_blocks_at(int pos) { return pos < 0 ? 0 : pos / kBlock + 1; }

// ---- lanes that select rows by themselves
//
// For batches with many rows (prefill chunks), lanes select (head, row) pairs
// by themselves.  The selection then runs on the vector units, a wave's rows
// in each instruction, instead of as the per-row ballot search above, whose
// scalar popcounts, compares and branches all queue on the CU's one scalar
// unit (about 8 scalar instructions per search step, ~15 steps per row).
// SPLIT lanes share a row, each taking 16*NC of its blocks.  The wave reads
// its rows in chunks of 16 blocks with coalesced loads (64 contiguous bytes
// per row part and chunk) and hands each lane its chunk through LDS.  A lane
// keeps its part's keys in registers, and the 16 largest of them sorted:
//   * each chunk of 16 keys is sorted by a bitonic network;
//   * the elementwise max of the kept list (descending) and the reversed
//     chunk holds the 16 largest of both, as a bitonic sequence;
//   * a half-cleaner cascade sorts it again.
// The lanes of a row then merge their kept lists the same way.  The topk-th
// kept key is the threshold T.  A second pass over the registers takes the
// blocks above T, and those equal to T in ascending id order until topk are
// chosen: the same set as the ballot search, written in the same ascending
// order.
constexpr int kLaneTop = 16;  // kept keys per lane: topk <= 16
// A lane takes 16*kLaneChunks blocks of a row (64: registers for four waves
// per SIMD), and 1, 2, 4 or 8 lanes share a row of up to 64, 128, 256 or 512
// blocks.
#ifndef MM3_LANE_CHUNKS
#define MM3_LANE_CHUNKS 4
#endif
constexpr int kLaneChunks = MM3_LANE_CHUNKS;
// 16*kLaneChunks blocks per lane and at most 8 lanes per row must cover the
// 512-block rows the lane path accepts.
static_assert(kLaneChunks >= 4 && kLaneChunks % 2 == 0, "lane selector chunks");

__device__ __forceinline__ void cx_desc(uint32_t& hi, uint32_t& lo) {
  const uint32_t m = max(hi, lo);
  lo = min(hi, lo);
  hi = m;
}

// 16 keys into descending order.
__device__ __forceinline__ void sort16_desc(uint32_t (&x)[16]) {
#pragma unroll
  for (int k = 2; k <= 16; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int l = i ^ j;
        if (l > i) {
          // runs with bit k clear descend, the others ascend; the last
          // stage (k = 16) leaves one descending run
          if ((i & k) == 0)
            cx_desc(x[i], x[l]);
          else
            cx_desc(x[l], x[i]);
        }
      }
}

// top (descending) := the 16 largest of top and x (both descending).
__device__ __forceinline__ void merge16_desc(uint32_t (&top)[16], const uint32_t (&x)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) top[i] = max(top[i], x[15 - i]);
#pragma unroll
  for (int j = 8; j > 0; j >>= 1)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if ((i & j) == 0) cx_desc(top[i], top[i + j]);
}

// The last request in [lo, hi] whose first row is <= t (ragged batches;
// cu[lo] <= t).
__device__ __forceinline__ int lane_request(const Rows& m, int t, int lo, int hi) {
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (m.cu[mid] <= t)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// The selection key of key_of, without branches or per-block compares
// (compare results are 64-bit scalar masks, and a chunk's worth of them
// spills).  Per chunk of 16 blocks a lane makes two 16-bit masks, of its
// visible and of its forced blocks; block i of the chunk takes its bits by
// a sign-extending bit-field extract (0 or all ones).  Adding +0 turns -0
// into +0 and leaves every other finite value as it is.
__device__ __forceinline__ uint32_t chunk_key(float v, int i, uint32_t vism, uint32_t fm) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  const uint32_t k = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);  // order_key
  return (k | (uint32_t)__builtin_amdgcn_sbfe((int)fm, i, 1)) & (uint32_t)__builtin_amdgcn_sbfe((int)vism, i, 1);
}

// Bits [0, min(max(n, 0), 16)) of a 16-bit mask.
__device__ __forceinline__ uint32_t low_bits16(int n) { return (1u << min(max(n, 0), 16)) - 1u; }

// (k > thr, k == thr) as 0/1, each compare's mask used by the next
// instruction (the compiler would gather a run of compares first).
__device__ __forceinline__ void cmp_bits(uint32_t k, uint32_t thr, uint32_t& gt, uint32_t& eq) {
  asm("v_cmp_gt_u32 vcc, %2, %3\n\t"
      "v_cndmask_b32 %0, 0, 1, vcc\n\t"
      "v_cmp_eq_u32 vcc, %2, %3\n\t"
      "v_cndmask_b32 %1, 0, 1, vcc"
      : "=&v"(gt), "=&v"(eq)
      : "v"(k), "v"(thr)
      : "vcc");
}

// Sum of v over the parts below `part` of a row (parts sit 64/SPLIT lanes
// apart): a log-step scan over the parts.  The whole wave must be active.
template <int SPLIT>
__device__ __forceinline__ int parts_below_t(int v, int part) {
  int incl = v;
#pragma unroll
  for (int d = 1; d < SPLIT; d <<= 1) {
    const int x = __shfl_up(incl, d * (64 / SPLIT));
    incl += part >= d ? x : 0;
  }
  return incl - v;
}

// Per-wave LDS row of one chunk (16 scores), padded so that both the
// chunk's writes (16 rows x 64 bytes per instruction) and the lanes' row
// reads spread over the banks.
constexpr int kLaneRowFloats = 20;
// Chunks whose loads a wave keeps in flight ahead of the one it sorts.
#ifndef MM3_LANE_AHEAD
#define MM3_LANE_AHEAD 2
#endif
constexpr int kLaneAhead = MM3_LANE_AHEAD;

// One chunk (16 blocks) of the wave's 64 rows with coalesced loads: load q
// takes rows 16q + l/4 (l = lane), 16 bytes each at column 4*(l%4) of the
// chunk, so each instruction reads 16 runs of 64 contiguous bytes.
__device__ __forceinline__ void lane_chunk_load(f32x4 (&g)[4], const __amdgpu_buffer_rsrc_t& rs,
                                                const uint32_t (&roff)[4], int c) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    g[q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)roff[q], 64 * c, 0));
}

// Rows of 16*NC*SPLIT blocks at most; the score rows are 16-byte aligned and
// the tensor spans s_bytes < 2 GiB (checked by the launcher).  SPLIT lanes
// share a row (a power of two up to 8; lanes l, l + 64/SPLIT, ...): part p
// takes its blocks [16*NC*p, 16*NC*(p + 1)).  After the sorting pass the
// parts merge their kept lists, ties go to the lower parts first, and each
// part writes its ids after those of the parts below it.
//
// lane_select: one wave selects head h's rows t0 .. t0 + 64/SPLIT - 1; rows
// at or past t_end are not selected (their loads stay in bounds and go
// unused).  trw: the wave's LDS area of 64 * kLaneRowFloats floats, 16-byte
// aligned.  The whole wave must be active.
template <int NC, bool ROWB, int SPLIT>
__device__ __forceinline__ void lane_select(const TopkArgs& a, int h, int t0, int t_end, float* trw) {
  constexpr int RW = 64 / SPLIT;  // rows per wave
  const int lane = threadIdx.x & 63;
  if (t0 >= t_end) return;
  const int T = t_end;
  const int half = lane / RW;   // which part of the row this lane takes
  const int b0 = 16 * NC * half;  // its first block
  const int t = t0 + lane % RW;
  const bool live = t < T;
  const int tc = live ? t : T - 1;
  // The loads nv depends on go out first.  Memory loads retire in issue
  // order, so nv's wait then leaves the first chunks' score loads in
  // flight.  (A ragged batch's request search, whose loads depend on each
  // other, completes before them.)  Raw values only, no arithmetic on them
  // yet, which would wait: row t of request r sits at seq_lens[r] - c1 + t
  // (c1 = the request's end row), or at prefix[r] + t - c0 (c0 = its first
  // row) with prefix lengths.
  int nv_raw = 0, base = 0, c0 = 0, c1 = 0;
  const Rows& m = a.rows;
  if constexpr (ROWB) {
    nv_raw = a.row_blocks[tc];
  } else if (m.cu == nullptr) {
    const int r = tc / m.qlen;
    c1 = (r + 1) * m.qlen;
    base = m.seq_lens[r];
  } else {
    // the wave's rows lie in requests [r_lo, r_hi]
    const int r_lo = row_request(m, t0);
    const int r_hi = row_request(m, min(t0 + RW - 1, T - 1));
    const int r = lane_request(m, tc, r_lo, r_hi);
    c0 = m.cu[r];
    c1 = m.cu[r + 1];
    base = m.prefix != nullptr ? m.prefix[r] : m.seq_lens[r];
  }
  __builtin_amdgcn_sched_barrier(0);
  // The scores, one chunk ahead.  One buffer descriptor spans the score
  // tensor (under 2 GiB, checked by the launcher); rows past the batch read
  // its last row, and columns past a row's width read the next row (or
  // zeros past the tensor's end): all of them belong to blocks >= nv, whose
  // values are not used.
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.scores, (short)0, a.s_bytes, 0x00020000);
  // load q, lane l: LDS row p = 16q + l/4, i.e. the part p / RW of the
  // wave's row p % RW -- the row and part that lane p works on
  // Offsets are unsigned: a row near the end of a tensor of almost 2 GiB can
  // reach past 2^31 here; such bytes lie past the descriptor's range, read as
  // zeros, and belong to blocks past nv.
  uint32_t roff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int p = 16 * q + lane / 4;
    const int tq = min(t0 + p % RW, T - 1);
    roff[q] = (uint32_t)(((int64_t)h * a.s_head + (int64_t)tq * a.s_row) * 4) +
              (uint32_t)(64 * NC * (p / RW) + 16 * (lane % 4));
  }
  constexpr int PD = NC < kLaneAhead ? NC : kLaneAhead;  // chunks in flight
  f32x4 g[PD][4];
#pragma unroll
  for (int c = 0; c < PD; ++c) lane_chunk_load(g[c], rs, roff, c);
  __builtin_amdgcn_sched_barrier(0);
  int nv = 0;
  if constexpr (ROWB)
    nv = live ? nv_raw : 0;
  else
    nv = live ? lanes_blocks_at(m.prefix != nullptr ? base + tc - c0 : base - c1 + tc) : 0;
  const int I = a.init_blocks, L = a.local_blocks;
  // the row's keys, in place of its scores (both passes read them), made
  // chunk by chunk: a chunk's sort waits only for its own loads
  uint32_t kk[16 * NC];
  uint32_t top[kLaneTop];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    // chunk c through the wave's LDS rows: written as loaded, read back one
    // row per lane; chunk c + PD's loads go out in between.  (The fences
    // keep the compiler from moving LDS accesses across the exchange, as it
    // sees only each lane's own addresses; one wave's LDS accesses execute
    // in order.)
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<f32x4*>(trw + (16 * q + lane / 4) * kLaneRowFloats + 4 * (lane % 4)) = g[c % PD][q];
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    if (c + PD < NC) lane_chunk_load(g[c % PD], rs, roff, c + PD);
    f32x4 rv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) rv[j] = *reinterpret_cast<const f32x4*>(trw + lane * kLaneRowFloats + 4 * j);
    // this chunk's blocks from cb = b0 + 16c: visible ones [cb, nv) and
    // forced ones [cb, I) and [nv - L, nv), as bits of the chunk
    const int cb = b0 + 16 * c;
    const uint32_t vism = low_bits16(nv - cb);
    const uint32_t fm = low_bits16(I - cb) | (vism & ~low_bits16(nv - L - cb));
    uint32_t x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      kk[16 * c + i] = chunk_key(rv[i / 4][i % 4], i, vism, fm);
      x[i] = kk[16 * c + i];
    }
    sort16_desc(x);
    if (c == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) top[i] = x[i];
    } else {
      merge16_desc(top, x);
    }
    // the next chunk's exchange stays after this chunk's sort, so the loads
    // in flight have the sort's time to arrive
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (SPLIT >= 2) {
    // Merge with the parts at lane distance 32, 16, ..., RW in turn.  A lane
    // swap (distances 32 and 16) leaves this lane's list in one copy and its
    // partner's in the other, the same way round for every entry; below 16 a
    // lane shuffle brings the partner's.  Merging the two gives the 16
    // largest of both.
    uint32_t other[kLaneTop];
#pragma unroll
    for (int d = 32; d >= RW; d >>= 1) {
#pragma unroll
      for (int i = 0; i < kLaneTop; ++i) {
        if (d == 32) {
          const auto r = __builtin_amdgcn_permlane32_swap(top[i], top[i], false, false);
          top[i] = r[0];
          other[i] = r[1];
        } else if (d == 16) {
          const auto r = __builtin_amdgcn_permlane16_swap(top[i], top[i], false, false);
          top[i] = r[0];
          other[i] = r[1];
        } else {
          other[i] = (uint32_t)__shfl_xor((int)top[i], d);
        }
      }
      merge16_desc(top, other);
    }
  }
  const int K = a.topk;
  uint32_t thr = top[0];
#pragma unroll
  for (int j = 1; j < kLaneTop; ++j)
    if (j < K) thr = top[j];
  int gt = 0;
#pragma unroll
  for (int j = 0; j < kLaneTop; ++j) gt += (j < K && top[j] > thr) ? 1 : 0;
  const int need = K - gt;
  // The selection as a bitmask (bit b of word b/32), then the ids in
  // ascending order from it: no branch or store inside the block loop.
  // Blocks above T, and of those equal to T the first `need` by id.  Blocks
  // past nv have key 0 and every visible block a key above 0, so a
  // threshold of 0 (fewer than topk visible) takes no ties.
  constexpr int NW = NC / 2;
  uint32_t selm[NW], eqm[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) selm[w] = eqm[w] = 0u;
#pragma unroll
  for (int b = 0; b < 16 * NC; ++b) {
    uint32_t gtb, eqb;
    cmp_bits(kk[b], thr, gtb, eqb);
    selm[b / 32] |= gtb << (b % 32);
    eqm[b / 32] |= eqb << (b % 32);
  }
  int left = thr != 0u ? need : 0;
  if constexpr (SPLIT >= 2) {
    // the lower parts' ties come first
    int n_eq = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) n_eq += __popc(eqm[w]);
    left = max(0, left - parts_below_t<SPLIT>(n_eq, half));
  }
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    uint32_t x = eqm[w], keep = 0u;
    const int n = __popc(x);
    if (left >= n) {
      keep = x;
      left -= n;
    } else {
      for (int j = 0; j < left; ++j) {
        const uint32_t lb = x & (0u - x);
        keep |= lb;
        x ^= lb;
      }
      left = 0;
    }
    selm[w] |= keep;
  }
  // each part's ids follow those of the parts below it
  int slot0 = 0;
  if constexpr (SPLIT >= 2) {
    int n_sel = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) n_sel += __popc(selm[w]);
    slot0 = parts_below_t<SPLIT>(n_sel, half);
  }
  if (!live) return;
  int32_t* orow = a.out + (int64_t)h * a.o_head + (int64_t)tc * a.o_row;
  for (int j = 0; slot0 + j < K; ++j) {
    int id = -1;
    bool found = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (!found && selm[w] != 0u) {
        id = b0 + 32 * w + __builtin_ctz(selm[w]);
        selm[w] &= selm[w] - 1u;
        found = true;
      }
    }
    // the top part of the row (the whole row if unsplit) also pads the
    // rest with -1; the others write their ids only
    if (half == SPLIT - 1 || found) orow[slot0 + j] = id;
  }
}

}  // namespace mm3
