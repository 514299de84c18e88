// decode_score.hip -- split-K decode block scorer for gfx950.
//
// What it computes (page "vllm.models.minimax_m3.amd.ops.index_topk", module
// docstring and minimax_m3_index_decode): for each request, its H*n index
// query rows (H heads x n decode positions, <= 16) score every visible
// 128-token block of the paged, shared index-K cache as the maximum over the
// block's causally visible tokens of sm_scale * (q . k).  n may differ per
// request (ragged batches: spec-decode rows, or the decode part of a mixed
// batch).
//
// Design.  Decode is a bandwidth-bound GEMV: every key (256 B bf16, 72 B
// NVFP4) is read once and serves all H*n rows of its request.  One wavefront
// scores one page (= one block) at a time:
//   * the page is loaded straight into MFMA A-operand registers with 16-byte
//     loads: lane l takes token 16*tt + l%16 and 16 contiguous bytes of it,
//     so each load instruction reads 16 tokens x 64 contiguous bytes and the
//     wave's 32 loads cover the 32 KiB page exactly once;
//   * v_mfma_f32_16x16x32_bf16 multiplies 16 tokens by the 16 padded query
//     rows (B operand, kept in registers for the workgroup's lifetime);
//   * the block maximum is an in-register max over each lane's 4 tokens per
//     tile and 8 tiles, masked only on a causally partial block, then a
//     2-step cross-lane max (lanes l, l^16, l^32).
// The default grid is one workgroup per CU, each taking an equal slice of
// the batch's (request, block) pairs (decode_score_cu); above 4096 requests
// or 2 GiB of scores, a grid of (block chunks, requests) sized from
// max_seq_len (decode_score_chunked).  Both grids depend on host arguments
// only, so they are fixed under graph capture.  Unlike the pages' Triton
// split-K kernel there is no per-chunk partial result: a block's score is
// complete inside one wave, so the split needs no merge.
#include <atomic>

#include "mm3_device.h"
#include "mm3_fp4.h"
#include "mm3_launch.h"
#include "mm3_rows.h"
#include "mm3_select.h"

namespace mm3 {

// ------------------------------------------------------------------ scorer

// A wave scores one block (page) as two halves of 64 tokens.  Half h of the
// page is held as the 16 contiguous KiB it spans, one 16-byte piece per lane
// and load (bf16), or as 4 tiles of 16 nibble bytes plus their 2 scale bytes
// (NVFP4).
template <int KFMT>
struct HalfBuf;
template <>
struct HalfBuf<0> {
  u32x4 v[16];
};

// Cache policy of the key loads: non-temporal (each key is read once per
// pass; streaming it past the caches is worth ~12% of bandwidth with whole
// 1 KiB runs per load instruction).
constexpr int kKeyLoadPolicy = 2;

// bf16 half pages reach the MFMA operand layout through a per-wave 8 KiB
// LDS area, a quarter page (32 tokens x 256 B) at a time.
constexpr int kTransposeBytes = 32 * kDim * 2;
template <>
struct HalfBuf<1> {
  u32x4 nib[4];
  u32x2 scl;  // the 8 scale bytes of token l of the half (lane l)
};

// A decode request's first-row position and row count (<= 16) in one word.
__device__ __forceinline__ int pack_req(int p0, int n) { return p0 * 32 + n; }
__device__ __forceinline__ int packed_p0(int v) { return v >> 5; }  // arithmetic: floor
__device__ __forceinline__ int packed_n(int v) { return v & 31; }

// The block a wave works on: request r, logical block b, the request's rows
// (pack_req of the first one's position and their count; the first row) and
// the page the block table maps b to (all wave-uniform).
struct Cur {
  int r;
  int b;
  int pk;
  int row0;
  int64_t page;
};

struct QRows {
  bf16x8 qb[4];
  int pos;   // position of this lane's row (MFMA column n), -1 if none
  int t;     // its token row
  int h;     // its head
};

// Raw query loads for one request, before the NVFP4 element reordering.
struct QRaw {
  u32x4 v[4];
};

// Buffer descriptor over [base, base + bytes); bytes == 0 makes every load
// through it return zeros without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, 0x00020000);
}

// Issue the query loads of c's request: column n = row j*H + h of the
// request.  Lanes without a row (n >= H*rows) and calls with live == false
// get zeros.
template <int KFMT>
__device__ __forceinline__ QRaw issue_q(const ScoreArgs& a, const Cur& c, int n, int g, bool live) {
  const int H = a.heads;
  const int j = n / H, h = n - (n / H) * H;
  const uint16_t* base = a.q + (int64_t)c.row0 * a.q_tok;
  const __amdgpu_buffer_rsrc_t rs = rsrc(base, live ? 0x7FFFFFF0 : 0);
  const int row = n < H * packed_n(c.pk) ? (int)(((int64_t)j * a.q_tok + (int64_t)h * a.q_head) * 2) : 0x7FFFFFF0;
  QRaw q;
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
    // bf16: k-group g, step kc covers d = 32*kc + 8*g .. +8 (natural order);
    // NVFP4: lane group g takes the 32 dims [32g, 32g+32), step kc 8 of them
    const int d = KFMT == 0 ? 32 * kc + 8 * g : 32 * g + 8 * kc;
    q.v[kc] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, row + d * 2, 0, 0));
  }
  return q;
}

// Register copy the compiler cannot fold: the destination is written by a
// VALU move, never directly by a (possibly conditional) load, so code that
// reads it waits only for that load here, not at every later use.
__device__ __forceinline__ uint32_t opaque_mov(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
  return r;
}

// Finish the query operands of c's request (row bookkeeping; NVFP4 element
// order {0,2,4,6,1,3,5,7} within each 8-element step to match the keys).
template <int KFMT>
__device__ __forceinline__ void set_q(QRows& q, const QRaw& raw, const ScoreArgs& a, const Cur& c, int n) {
  const int H = a.heads;
  const int j = n / H;
  q.h = n - j * H;
  q.t = c.row0 + j;
  q.pos = n < H * packed_n(c.pk) ? packed_p0(c.pk) + j : -1;
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
    const u32x4 v = raw.v[kc];
    u32x4 p;
    if constexpr (KFMT == 0) {
      p.x = opaque_mov(v.x);
      p.y = opaque_mov(v.y);
      p.z = opaque_mov(v.z);
      p.w = opaque_mov(v.w);
    } else {
      p.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);  // e0, e2
      p.y = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);  // e4, e6
      p.z = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);  // e1, e3
      p.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);  // e5, e7
    }
    q.qb[kc] = as_bf16x8(p);
  }
}

// Issue the loads of half `half` of a page.  The page base is wave-uniform
// and goes into a buffer descriptor (scalar registers) sized to exactly one
// page, so no load can leave the page; each lane keeps one 32-bit offset.
// live == false issues the same instructions with an empty descriptor: they
// return zeros and move no data, which keeps the loop free of branches
// around loads (and the wait counts exact).
//   bf16: load i reads KiB i of the half: lane l takes token 4i + l/16 of the
//   half, 16-byte chunk l%16 (whole 128-byte lines per instruction).
//   NVFP4: load tt reads tokens 16tt + l%16 of the half, nibble bytes
//   16(l/16).. (again one contiguous KiB); one more load brings the half's
//   512 scale bytes, token l's 8 to lane l (the multiply fetches the pair
//   it needs from that lane).
template <int KFMT>
__device__ __forceinline__ void issue_half(HalfBuf<KFMT>& buf, const ScoreArgs& a, int64_t page,
                                           int half, int n, int g, bool live) {
  if constexpr (KFMT == 0) {
    const __amdgpu_buffer_rsrc_t rs = rsrc(a.kdata + page * (kBlock * kDim * 2), live ? kBlock * kDim * 2 : 0);
    const int voff = 16 * (16 * g + n);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      buf.v[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, half * 16384 + i * 1024, kKeyLoadPolicy));
  } else {
    const __amdgpu_buffer_rsrc_t rn = rsrc(a.kdata + page * (kBlock * kDim / 2), live ? kBlock * kDim / 2 : 0);
    const __amdgpu_buffer_rsrc_t rsc = rsrc(a.kscales + page * (kBlock * kDim / 16), live ? kBlock * kDim / 16 : 0);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      buf.nib[tt] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rn, n * (kDim / 2) + 16 * g, (4 * half + tt) * 1024,
                                                       kKeyLoadPolicy));
    buf.scl = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_raw_buffer_load_b64(rsc, 8 * (16 * g + n), half * 512,
                                                    kKeyLoadPolicy));
  }
}

// Multiply half `half` of a page by the query rows and fold its tokens into
// this lane's running maximum m (lane l: row l%16, tokens 4*(l/16) + 0..3 of
// each 16-token tile).  lim: token s of the block is visible iff s <= lim.
// bf16: each quarter (32 tokens) is written to the wave's LDS area tb as
// loaded -- token t's 16-byte chunk c at slot c ^ (t & 15) of its 256-byte
// row -- and read back as MFMA A operands (token 16tt + l%16, chunk
// 4kc + l/16); the XOR keeps both the writes (8 chunks of one token) and the
// reads (one chunk of 8 tokens) free of bank conflicts.
template <int KFMT>
__device__ __forceinline__ void compute_half(const HalfBuf<KFMT>& buf, const QRows& q, const u32x2* lut,
                                             uint8_t* tb, int half, bool full, int lim, int n, int g,
                                             float& m) {
  auto fold = [&](const f32x4& acc, int s0) {
    if (full) {
      m = fmaxf(m, fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3])));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (s0 + i <= lim) m = fmaxf(m, acc[i]);
    }
  };
  if constexpr (KFMT == 0) {
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      // the wave's lanes exchange data through tb: keep the compiler from
      // moving these writes above the previous quarter's reads, or the
      // reads below above these writes (it only sees each lane's own
      // addresses; the hardware keeps one wave's LDS accesses in order)
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = 4 * j + g;
        *reinterpret_cast<u32x4*>(tb + t * (kDim * 2) + ((n ^ (t & 15)) << 4)) = buf.v[8 * qq + j];
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int t = 16 * tt + n;
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(tb + t * (kDim * 2) + (((4 * kc + g) ^ n) << 4));
          acc = mfma16(as_bf16x8(v), q.qb[kc], acc);
        }
        fold(acc, 64 * half + 32 * qq + 16 * tt + 4 * g);
      }
    }
  } else {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      // scale bytes 2g, 2g+1 (dims [32g, 32g+32)) of token 16tt + n, held by
      // lane 16tt + n
      const int src = (16 * tt + n) * 4;
      const uint32_t wx = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)buf.scl.x);
      const uint32_t wy = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)buf.scl.y);
      const uint32_t sc = ((g < 2 ? wx : wy) >> (16 * (g & 1))) & 0xFFFFu;
      const u32x2 t0 = lut[sc & 0xFF];
      const u32x2 t1 = lut[sc >> 8];
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      acc = mfma16(as_bf16x8(fp4x8_to_bf16(buf.nib[tt].x, t0)), q.qb[0], acc);
      acc = mfma16(as_bf16x8(fp4x8_to_bf16(buf.nib[tt].y, t0)), q.qb[1], acc);
      acc = mfma16(as_bf16x8(fp4x8_to_bf16(buf.nib[tt].z, t1)), q.qb[2], acc);
      acc = mfma16(as_bf16x8(fp4x8_to_bf16(buf.nib[tt].w, t1)), q.qb[3], acc);
      fold(acc, 64 * half + 16 * tt + 4 * g);
    }
  }
}

__device__ __forceinline__ int64_t page_of(const ScoreArgs& a, int r, int b) {
  const int32_t __attribute__((address_space(4)))* bt =
      (const int32_t __attribute__((address_space(4)))*)a.bt;
  return bt[(int64_t)r * a.bt_stride + b];
}

// Block scores are staged, not stored as they are produced: on gfx9 stores
// and loads retire in order on one counter, so a store in the middle of the
// page stream makes every later wait on page data wait for that store too.
// Each wave keeps up to kStage (row, block) scores -- value and byte offset --
// in its own LDS area and writes them out when the area is full (every
// kStage / (H*n) blocks, rare) and once after its last page load, with
// consecutive blocks of a row on adjacent lanes.
constexpr int kStage = 512;

__device__ __forceinline__ void flush_scores(const __amdgpu_buffer_rsrc_t& srs, const float* stv,
                                             const int32_t* sto, int nblk, int HQ, int lane) {
  const int total = nblk * HQ;
  for (int e0 = 0; e0 < total; e0 += 64) {
    const int e = e0 + lane;
    const int row = e / nblk, i = e - (e / nblk) * nblk;  // row-major: blocks of a row adjacent
    const bool ok = e < total;
    const int idx = ok ? i * HQ + row : 0;
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, stv[idx]), srs,
                                          ok ? sto[idx] : 0x7FFFFFF0, 0, 0);
  }
}

// Blocks whose loads a wave keeps in flight besides the one it multiplies:
// one (its second half in flight while the first is multiplied, the next
// block's first half while the second is).  bf16 half pages take 64
// registers, so that is all that fits; NVFP4 half pages take 18, but a
// deeper ring costs waves per SIMD, and the NVFP4 scorer is bound by its
// decode more than by loads in flight (2 and 3 blocks measured slower).
#ifndef MM3_FP4_RING
#define MM3_FP4_RING 1
#endif
template <int KFMT>
constexpr int kRingBlocks = KFMT == 0 ? 1 : MM3_FP4_RING;

// One block of the ring: the walker's position, whether it is real, its two
// half pages, and the query loads of its request when that request differs
// from the previous block's.
template <int KFMT>
struct RingBlock {
  Cur c;
  bool live;
  bool new_req;
  QRaw qraw;
  HalfBuf<KFMT> h0, h1;
};

// Score every block the walker hands this wave, in order.  Block i's loads
// are issued when block i - kRingBlocks is multiplied (its first half after
// that block's first half, its second half after the second), so the wave
// always has about kRingBlocks blocks of keys in flight.  A block that starts
// a new request also brings that request's query rows, loaded with its pages.
// Loads are issued unconditionally (empty descriptors where there is nothing
// to fetch), so the loop has no branch around a load and the wait counts
// stay exact.  STAGED == false (score tensors past 2 GiB) stores each value
// directly.
template <int KFMT, bool STAGED, typename Walk>
__device__ __forceinline__ void score_wave(const ScoreArgs& a, const u32x2* lut, uint8_t* tb, Walk& walk,
                                           float* stv, int32_t* sto) {
  constexpr int DB = kRingBlocks<KFMT>;
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int HQ = a.heads * a.rows.qlen;  // stage columns: the most rows a request has
  const int stage_blocks = kStage / HQ;
  RingBlock<KFMT> ring[DB];
  if (!walk.first(ring[0].c)) return;
  QRows q;
  // the first block's query rows and pages load together; the query operands
  // are set up once both are on their way
  const QRaw raw0 = issue_q<KFMT>(a, ring[0].c, n, g, true);
  ring[0].live = true;
  ring[0].new_req = false;
  issue_half<KFMT>(ring[0].h0, a, ring[0].c.page, 0, n, g, true);
  issue_half<KFMT>(ring[0].h1, a, ring[0].c.page, 1, n, g, true);
  set_q<KFMT>(q, raw0, a, ring[0].c, n);
  Cur last = ring[0].c;  // the last block issued (the walker's position)
  bool more = true;      // the walker has not run out
#pragma unroll
  for (int j = 1; j < DB; ++j) {
    RingBlock<KFMT>& rb = ring[j];
    rb.c = last;
    rb.live = more && walk.next(rb.c);
    more = rb.live;
    rb.new_req = rb.live && rb.c.r != last.r;
    rb.qraw = issue_q<KFMT>(a, rb.c, n, g, rb.new_req);
    issue_half<KFMT>(rb.h0, a, rb.c.page, 0, n, g, rb.live);
    issue_half<KFMT>(rb.h1, a, rb.c.page, 1, n, g, rb.live);
    if (rb.live) last = rb.c;
  }
  const __amdgpu_buffer_rsrc_t srs = rsrc(a.scores, STAGED ? a.s_bytes : 0);
  int staged = 0;  // blocks in the stage (wave-uniform)
  while (true) {
#pragma unroll
    for (int j = 0; j < DB; ++j) {
      RingBlock<KFMT>& rb = ring[j];
      if (!rb.live) goto done;
      const Cur cur = rb.c;
      if (rb.new_req) set_q<KFMT>(q, rb.qraw, a, cur, n);
      // the block that takes this slot
      Cur nxt = last;
      const bool has_next = more && walk.next(nxt);
      more = has_next;
      const bool new_req = has_next && nxt.r != last.r;
      __builtin_amdgcn_sched_barrier(0);
      const bool full = kBlock * cur.b + (kBlock - 1) <= packed_p0(cur.pk);  // the first row sees all of it
      const int lim = q.pos - kBlock * cur.b;
      float m = -INFINITY;
      compute_half<KFMT>(rb.h0, q, lut, tb, 0, full, lim, n, g, m);
      __builtin_amdgcn_sched_barrier(0);
      rb.qraw = issue_q<KFMT>(a, nxt, n, g, new_req);
      issue_half<KFMT>(rb.h0, a, nxt.page, 0, n, g, has_next);
      __builtin_amdgcn_sched_barrier(0);
      compute_half<KFMT>(rb.h1, q, lut, tb, 1, full, lim, n, g, m);
      __builtin_amdgcn_sched_barrier(0);
      issue_half<KFMT>(rb.h1, a, nxt.page, 1, n, g, has_next);
      __builtin_amdgcn_sched_barrier(0);
      m = wave_max_xor16(m);
      m = wave_max_xor32(m);
      const bool writer = n < HQ && q.pos >= kBlock * cur.b;
      const int64_t off = (int64_t)q.h * a.s_head + (int64_t)q.t * a.s_row + cur.b;
      if constexpr (STAGED) {
        if (g == 0 && n < HQ) {
          stv[staged * HQ + n] = m * a.sm_scale;
          sto[staged * HQ + n] = writer ? (int32_t)(off * 4) : 0x7FFFFFF0;
        }
        if (++staged == stage_blocks) {
          flush_scores(srs, stv, sto, staged, HQ, lane);
          staged = 0;
        }
      } else {
        if (g == 0 && writer) a.scores[off] = m * a.sm_scale;
      }
      rb.c = nxt;
      rb.live = has_next;
      rb.new_req = new_req;
      if (has_next) last = nxt;
    }
  }
done:
  if constexpr (STAGED) flush_scores(srs, stv, sto, staged, HQ, lane);
}


// ---- per-CU scorer
//
// One workgroup per CU holds all of the CU's waves.  The batch's (request,
// block) pairs, flattened request-major, are cut into equal contiguous slices,
// one per workgroup (each builds the prefix sum of the requests' block counts
// in LDS to map a flattened index back to its request).  Inside a workgroup
// the waves take the slice's blocks one at a time from an LDS counter, so a
// wave the SIMD arbiter favours simply scores more blocks: with fixed
// per-wave shares the waves of one CU finished up to ~50% apart and the CU
// idled on its slowest wave.  The slices of all CUs finish within a few
// percent of each other.

struct SharedWalk {
  const ScoreArgs* a;
  const int32_t* pre;  // LDS: pre[r] = blocks of requests < r
  const int32_t* sl;   // LDS: pack_req(p0, rows) per request
  const int32_t* r0;   // LDS: first row per request
  uint32_t* counter;   // LDS: next block of the slice, counted from lo
  int64_t lo, hi;      // the workgroup's slice of the flattened block list
  int64_t gb;          // the block just taken
  int64_t req_lo, req_hi;  // flattened range of the current request

  __device__ __forceinline__ bool take() {
    uint32_t v = 0;
    if ((threadIdx.x & 63) == 0) v = atomicAdd(counter, 1u);
    gb = lo + (int64_t)__builtin_amdgcn_readfirstlane(v);
    return gb < hi;
  }
  __device__ __forceinline__ void fill(Cur& c) {
    req_lo = __builtin_amdgcn_readfirstlane(pre[c.r]);
    req_hi = __builtin_amdgcn_readfirstlane(pre[c.r + 1]);
    c.pk = __builtin_amdgcn_readfirstlane(sl[c.r]);
    c.row0 = __builtin_amdgcn_readfirstlane(r0[c.r]);
    c.b = (int)(gb - req_lo);
    // finish the LDS reads before the scalar page load, so that later waits
    // on LDS never also wait on that load
    __builtin_amdgcn_sched_barrier(0);
    c.page = page_of(*a, c.r, c.b);
  }
  __device__ __forceinline__ bool first(Cur& c) {
    if (!take()) return false;
    int l = 0, u = a->rows.num_reqs;  // last r with pre[r] <= gb
    while (u - l > 1) {
      const int mid = (l + u) >> 1;
      if (pre[mid] <= gb) l = mid; else u = mid;
    }
    c.r = __builtin_amdgcn_readfirstlane(l);
    fill(c);
    return true;
  }
  // blocks come out of the counter in increasing order, so the request only
  // moves forward
  __device__ __forceinline__ bool next(Cur& c) {
    if (!take()) return false;
    if (gb < req_hi) {
      c.b = (int)(gb - req_lo);
      c.page = page_of(*a, c.r, c.b);
      return true;
    }
    int r = c.r;
    while (pre[r + 1] <= gb) ++r;
    c.r = __builtin_amdgcn_readfirstlane(r);
    fill(c);
    return true;
  }
};

// waves per workgroup (= per CU): what the register budget allows
template <int KFMT>
constexpr int kCuWaves = KFMT == 0 ? 8 : 16;

template <int KFMT>
__global__ __launch_bounds__(64 * kCuWaves<KFMT>) void decode_score_cu(ScoreArgs a) {
  constexpr int W = kCuWaves<KFMT>;
  constexpr int NT = 64 * W;
  extern __shared__ int32_t smem[];
  __shared__ u32x2 lut[KFMT == 1 ? 256 : 1];
  __shared__ int32_t part[W];
  __shared__ uint32_t next_blk;
  __shared__ float stage_v[W][kStage];
  __shared__ int32_t stage_o[W][kStage];
  __shared__ __attribute__((aligned(16))) uint8_t tbuf[W][KFMT == 0 ? kTransposeBytes : 16];
  const int R = a.rows.num_reqs;
  int32_t* pre = smem;              // [R + 1]
  int32_t* sl = smem + R + 1;       // [R]
  int32_t* r0s = smem + 2 * R + 1;  // [R]
  const int per = (R + NT - 1) / NT;
  const int r0 = min(R, (int)threadIdx.x * per), r1 = min(R, r0 + per);
  // the table load goes out first, so its latency overlaps the length loads'
  u32x2 lut_v{0u, 0u};
  if constexpr (KFMT == 1) {
    if (threadIdx.x < 256) lut_v = lut_entry();
  }
  int sum = 0;
  for (int r = r0; r < r1; ++r) {
    const ReqRows q = req_rows(a.rows, r);
    // requests this launch does not take count as no rows
    const int v = routed(a.route, a.heads, q.n) ? pack_req(q.p0, q.n) : pack_req(0, 0);
    sl[r] = v;
    r0s[r] = q.row0;
    sum += req_blocks(packed_p0(v), packed_n(v));
  }
  if constexpr (KFMT == 1) {
    if (threadIdx.x < 256) lut[threadIdx.x] = lut_v;
  }
  // exclusive scan of the partial sums: within each wave by lane shifts,
  // then over the wave totals (two barriers in all)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  int incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  if (lane == 63) part[wave] = incl;
  if (threadIdx.x == 0) next_blk = 0;
  __syncthreads();
  int base = incl - sum, total_blocks = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const int pw = part[w];
    base += w < wave ? pw : 0;
    total_blocks += pw;
  }
  for (int r = r0; r < r1; ++r) {
    pre[r] = base;
    const int v = sl[r];
    base += req_blocks(packed_p0(v), packed_n(v));
  }
  if (threadIdx.x == NT - 1) pre[R] = total_blocks;
  __syncthreads();
  const int64_t total = total_blocks;
  const int64_t lo = total * blockIdx.x / gridDim.x;
  const int64_t hi = total * (blockIdx.x + 1) / gridDim.x;
  SharedWalk walk{&a, pre, sl, r0s, &next_blk, lo, hi, 0, 0, 0};
  score_wave<KFMT, true>(a, lut, tbuf[wave], walk, stage_v[wave], stage_o[wave]);
}

// ---- per-request chunk scorer (any batch size)
//
// Grid (block chunks, requests): workgroup (x, r) covers blocks
// [x*bpw, (x+1)*bpw) of request r and returns at once past its end.

template <int STEP>
struct ChunkWalkT {
  const ScoreArgs* a;
  int r;
  ReqRows rr;
  int b, b_end;
  __device__ __forceinline__ bool first(Cur& c) {
    if (b >= b_end) return false;
    c.r = r;
    c.pk = pack_req(rr.p0, rr.n);
    c.row0 = rr.row0;
    c.b = b;
    c.page = page_of(*a, r, b);
    return true;
  }
  __device__ __forceinline__ bool next(Cur& c) {
    b += STEP;
    if (b >= b_end) return false;
    c.b = b;
    c.page = page_of(*a, r, b);
    return true;
  }
};

using ChunkWalk = ChunkWalkT<4>;

template <int KFMT>
__global__ __launch_bounds__(256) void decode_score_chunked(ScoreArgs a) {
  __shared__ u32x2 lut[KFMT == 1 ? 256 : 1];
  __shared__ __attribute__((aligned(16))) uint8_t tbuf[4][KFMT == 0 ? kTransposeBytes : 16];
  const int r = blockIdx.y;
  const ReqRows rr = req_rows(a.rows, r);
  if (!routed(a.route, a.heads, rr.n)) return;
  const int nb = req_blocks(rr.p0, rr.n);
  const int b_begin = blockIdx.x * a.blocks_per_wg;
  if (b_begin >= nb) return;
  if constexpr (KFMT == 1) {
    fill_lut(lut);
    __syncthreads();
  }
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  ChunkWalk walk{&a, r, rr, b_begin + wave, min(nb, b_begin + a.blocks_per_wg)};
  score_wave<KFMT, false>(a, lut, tbuf[wave], walk, nullptr, nullptr);
}

// Blocks b, b + STEP, ... below b_end of request r, the first one's page id
// already loaded.
template <int STEP>
struct SmallWalk {
  const ScoreArgs* a;
  int r;
  ReqRows rr;
  int b, b_end;
  int64_t page0;
  __device__ __forceinline__ bool first(Cur& c) {
    if (b >= b_end) return false;
    c.r = r;
    c.pk = pack_req(rr.p0, rr.n);
    c.row0 = rr.row0;
    c.b = b;
    c.page = page0;
    return true;
  }
  __device__ __forceinline__ bool next(Cur& c) {
    b += STEP;
    if (b >= b_end) return false;
    c.b = b;
    c.page = page_of(*a, r, b);
    return true;
  }
};

// ---- small batches: scores and selection in one launch
//
// For requests that see few blocks the two-launch path is bound by latency:
// two kernel launches and a score round trip through global memory for a
// few microseconds of work.  Here one workgroup takes one request: its waves
// score blocks wave, wave + W, ... with the same wave loop as the per-CU
// scorer (so the scores are the same bits), the scores stay in the waves'
// LDS stages (and go to global memory too when the caller asks for them),
// and after a barrier each wave selects rows of the request from the LDS.
// The selection is that of the selector kernels (page "ops.index_topk",
// minimax_m3_index_topk; forced blocks pinned as in page
// "indexer_cp_exchange", module docstring): block b of a row holds the
// selection key key_of(score, b, nv, I, L), and the row takes the blocks of
// rank < topk under (key descending, id ascending); with at most kSmallBlocks
// blocks a lane per block counts its rank directly.

template <int KFMT>
__global__ __launch_bounds__(64 * kCuWaves<KFMT>) void decode_small(ScoreArgs a, TopkArgs t) {
  constexpr int W = kCuWaves<KFMT>;
  __shared__ u32x2 lut[KFMT == 1 ? 256 : 1];
  __shared__ float stage_v[W][kStage];
  __shared__ int32_t stage_o[W][kStage];
  __shared__ __attribute__((aligned(16))) uint8_t tbuf[W][KFMT == 0 ? kTransposeBytes : 16];
  const int r = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  // the table load and the page id of the wave's first block (block
  // `wave`, read only below cdiv(max_seq_len, 128), which the block table's
  // width covers) go out first, so their latency overlaps the row lookup's
  u32x2 lut_v{0u, 0u};
  if constexpr (KFMT == 1) {
    if (threadIdx.x < 256) lut_v = lut_entry();
  }
  const int64_t page0 = wave < a.nb_max ? page_of(a, r, wave) : 0;
  const ReqRows rr = req_rows<true>(a.rows, r);
  if constexpr (KFMT == 1) {
    if (threadIdx.x < 256) lut[threadIdx.x] = lut_v;
    __syncthreads();
  }
  // at most kSmallBlocks when seq_lens <= max_seq_len, as every scorer
  // assumes; clamped so that a length past it cannot index past the stage
  const int nbr = min(req_blocks(rr.p0, rr.n), kSmallBlocks);
  SmallWalk<W> walk{&a, r, rr, wave, nbr, page0};
  score_wave<KFMT, true>(a, lut, tbuf[wave], walk, stage_v[wave], stage_o[wave]);
  __syncthreads();
  const int H = a.heads;
  const int HQ = H * a.rows.qlen;  // stage stride: column n holds row n = j H + h
  for (int row = wave; row < H * rr.n; row += W) {
    const int j = row / H, h = row - j * H;
    const int nv = blocks_at(rr.p0 + j);
    uint32_t key = 0;
    if (lane < nbr) key = key_of(stage_v[lane % W][(lane / W) * HQ + row], lane, nv, t.init_blocks, t.local_blocks);
    int rank = 0;
#pragma unroll
    for (int b = 0; b < kSmallBlocks; ++b) {
      const uint32_t kb = (uint32_t)__builtin_amdgcn_readlane((int)key, b);
      rank += (kb > key || (kb == key && b < lane)) ? 1 : 0;
    }
    const bool take = key != 0 && rank < t.topk;
    const uint64_t m = __ballot(take);
    int32_t* orow = t.out + (int64_t)h * t.o_head + (int64_t)(rr.row0 + j) * t.o_row;
    if (take) orow[lanes_below(m)] = lane;
    for (int k = __popcll(m) + lane; k < t.topk; k += 64) orow[k] = -1;
  }
}

// ------------------------------------------------------------------ launch

// Largest batch whose lengths and prefix sums fit the per-CU scorer's LDS.
constexpr int kCuMaxReqs = 4096;

// Compute units of the current device, cached per device (host threads may
// race on the first call; they store the same value).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  int n = dev < 64 ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int KFMT>
static hipError_t launch_decode(const ScoreArgs& a, hipStream_t s) {
  const size_t lds = (size_t)(3 * a.rows.num_reqs + 1) * sizeof(int32_t);
  if (a.rows.num_reqs <= kCuMaxReqs && a.s_bytes > 0) {
    // one workgroup per CU: its LDS and registers leave room for no second
    hipLaunchKernelGGL(decode_score_cu<KFMT>, dim3(device_cus()), dim3(64 * kCuWaves<KFMT>), lds, s, a);
  } else {
    const int chunks = (a.nb_max + a.blocks_per_wg - 1) / a.blocks_per_wg;
    hipLaunchKernelGGL(decode_score_chunked<KFMT>, dim3(chunks, a.rows.num_reqs, 1), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_decode_score_bf16(const ScoreArgs& a, hipStream_t s) { return launch_decode<0>(a, s); }

hipError_t launch_decode_small(const ScoreArgs& a, const TopkArgs& t, int kfmt, hipStream_t s) {
  if (kfmt == 0)
    hipLaunchKernelGGL(decode_small<0>, dim3(a.rows.num_reqs), dim3(64 * kCuWaves<0>), 0, s, a, t);
  else
    hipLaunchKernelGGL(decode_small<1>, dim3(a.rows.num_reqs), dim3(64 * kCuWaves<1>), 0, s, a, t);
  return hipGetLastError();
}

hipError_t launch_decode_score_nvfp4(const ScoreArgs& a, hipStream_t s) { return launch_decode<1>(a, s); }

}  // namespace mm3
