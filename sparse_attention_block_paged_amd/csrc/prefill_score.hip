// prefill_score.hip -- MFMA block scorer for chunked prefill on gfx950.
//
// What it computes (page "vllm.models.minimax_m3.amd.ops.index_topk",
// minimax_m3_index_score: per query token and head, the largest scaled
// dot product over the causally visible keys of each 128-token index-K
// block; causal within the chunk; chunks of different lengths and prefixes
// in one ragged batch).
//
// Design.  With many query rows per request the score is a dense product
// [rows x 128] . [128 x keys] followed by a max over each 128-key block, so it
// runs on the bf16 matrix cores.
//   * Work unit: 512 flattened (position, head) rows of one request -- all
//     heads of a position share its causal bound -- against one key block.
//     A request's row tile x has one step per block it can see.  The steps of
//     all tiles of all requests form one list; each persistent workgroup takes
//     an equal contiguous share of it (a prefix scan over the tiles finds the
//     start), so the chip stays full to the end whatever the causal triangle
//     and the length mix look like.  Every (row, block) score is produced by
//     exactly one step: shares need no merge.
//   * Wave w owns rows 128w..128w+127 of the tile (with the default four
//     waves) as four 32-row MFMA B tiles held in registers (loaded again only
//     when the share crosses into the next tile); each key fragment read from
//     LDS feeds four MFMAs.
//   * Key pages (32 KiB) go global -> LDS by direct DMA (no registers), double
//     buffered one block ahead, with a 16-byte-chunk XOR swizzle (chunk c of
//     token s at c ^ (s & 15)) so the A-operand reads of 32 tokens x 16 B are
//     free of bank conflicts.
//   * v_mfma_f32_32x32x16_bf16 with keys as A (rows = tokens) and queries as
//     B (columns = rows): each lane holds one query row and 16 tokens per tile,
//     so the block max is an in-register max plus one cross-lane step (l ^ 32);
//     the causal mask is applied only on blocks that cross a row's position.
//   * Each wave stages its rows' scores in LDS and writes them every 8 blocks
//     as row-contiguous 32-byte runs (one 4-byte store per row and block would
//     scatter over 64 rows per instruction).
//   * NVFP4 keys: the raw page (8 KiB of nibbles, 1 KiB of scales) is copied
//     the same way, and each wave decodes the fragments it multiplies in
//     registers, each k-step's 8 elements in the shadow of the previous
//     k-step's multiplies (the same table decode as the decode scorer).
// Two workgroups (80 KiB of LDS each with bf16 keys, 36 KiB with NVFP4) share
// a CU, so one's barrier or copy wait is covered by the other's multiplies;
// wave priorities that fall with the progress through a share keep the two
// abreast to the end.
//
// Fused selection (SEL > 0; page "ops.index_topk": minimax_m3_index_score
// followed by minimax_m3_index_topk, here in one launch).  A row tile's
// steps are split between the shares of two or three workgroups.  When a
// wave finishes its part of a tile it publishes its score stores (release at
// device scope) and adds its step count to the tile's counter; the wave whose
// count completes the tile (every wave of every part: waves x steps) records
// its workgroup as the tile's owner.  After its share, each workgroup
// selects the rows of the tiles it owns with the lane selector (SEL lanes
// per row), in its then idle LDS.  No workgroup ever waits for another, and
// the selection stays out of the multiply loop and its registers.  Counters
// and owners are reset by a small kernel launched just before.
#include <atomic>

#include "mm3_device.h"
#include "mm3_fp4.h"
#include "mm3_lanes.h"
#include "mm3_launch.h"
#include "mm3_rows.h"

namespace mm3 {

constexpr int kPageBytes = kBlock * kDim * 2;              // 32 KiB
// Four waves of 128 rows, two workgroups per CU.  Eight waves of 64 rows (one
// workgroup per CU, its waves in step at every block) read each key fragment
// for two multiplies instead of four and measured 3-7% slower.
#ifndef MM3_PF_WAVES
#define MM3_PF_WAVES 4
#endif
constexpr int kPfWaves = MM3_PF_WAVES;                       // waves per workgroup
constexpr int kPfWaveRows = kPrefillRows / kPfWaves;         // query rows per wave
constexpr int kPfQt = kPfWaveRows / 32;                      // 32-row MFMA B tiles per wave
constexpr int kPfWgPerCu = 8 / kPfWaves;                     // two waves per SIMD
static_assert(kPfWaves == 4 || kPfWaves == 8, "row tile");
constexpr int kPfStage = 8;                                  // blocks staged per write-out
static_assert(kPfStage == 8, "the write-out's lanes take two column groups of four");
#ifndef MM3_PF_AHEAD
#define MM3_PF_AHEAD 3
#endif
constexpr int kPfAhead = MM3_PF_AHEAD;                       // k-steps a fragment read runs ahead
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfCopies = kPageBytes / (kPfThreads * 16);    // 16-byte copies per thread per page
constexpr int kPfStageFloats = kPfWaveRows * kPfStage;       // per wave
constexpr int kPfLds = 2 * kPageBytes + kPfWaves * kPfStageFloats * 4;  // 80 KiB
// NVFP4 keys: the page (8 KiB nibbles + 1 KiB scales) is copied into one of
// two slots, and each wave decodes the fragments it multiplies in registers
// (no decoded page in LDS).  Nibble row of token t (64 bytes, 4 chunks of 16):
// chunk c at 16 (c ^ ((t >> 1) & 3)), so that a wave's 16-byte reads of one
// chunk of 32 consecutive tokens hit distinct banks.
constexpr int kFp4NibBytes = kBlock * kDim / 2;    // 8 KiB
constexpr int kFp4ScaleBytes = kBlock * kDim / 16;  // 1 KiB
constexpr int kPfFp4Stage0 = 0;                                      // nibble slots
constexpr int kPfFp4Scale0 = kPfFp4Stage0 + 2 * kFp4NibBytes;       // scale slots
constexpr int kPfFp4Lut = kPfFp4Scale0 + 2 * kFp4ScaleBytes;        // E4M3 table
constexpr int kPfFp4Scores = kPfFp4Lut + 256 * 8;                   // score stage
constexpr int kPfLdsFp4 = kPfFp4Scores + kPfWaves * kPfStageFloats * 4;  // 36 KiB
template <int KFMT>
constexpr int kPfLdsOf = KFMT == 0 ? kPfLds : kPfLdsFp4;
// Above this many (request, row tile) units the start-finding scan of the
// balanced grid costs more than it saves: one workgroup per unit instead.
constexpr int kPfBalancedMaxUnits = 1 << 16;
// Relative share sizes of workgroups on even- and odd-numbered XCDs.
constexpr int kPfXcdWeightEven = 1030;
constexpr int kPfXcdWeightOdd = 970;

#define MM3_AS3 __attribute__((address_space(3)))
#define MM3_AS4 __attribute__((address_space(4)))

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Blocks that the last row of row tile x of a request (n positions from p0,
// H heads each) can see: the tile's step count, 0 for a tile past the
// request's rows.  Rows are ordered by position, so the last row bounds them.
__device__ __forceinline__ int tile_blocks(int p0, int n, int x, int H) {
  const int HQ = H * n;
  if (x * kPrefillRows >= HQ) return 0;
  const int rl = min(HQ, (x + 1) * kPrefillRows) - 1;
  const int pl = p0 + rl / H;
  return pl < 0 ? 0 : pl / kBlock + 1;
}

// One 16-byte global -> LDS copy per lane: LDS bytes [lds, lds + 1 KiB) get
// the 64 lanes' 16-byte pieces at gbase + voff, in lane order.  Written as
// assembly so the compiler does not track it (it cannot tell the two page
// buffers apart and would wait for every copy in flight before each LDS
// read); the ring's explicit waits and barriers order it.  The compiler
// treats M0 as reserved (a clobber of it is ignored); no compiler-generated
// code in this kernel reads M0, so the asm may set it freely.
__device__ __forceinline__ void copy16_to_lds(uint32_t lds, const uint8_t* gbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(gbase)
               : "memory");
}

// Wait for this thread's copies (and any other vector memory access), then a
// workgroup barrier.  The empty asm keeps LDS accesses from moving across it.
__device__ __forceinline__ void ring_sync() {
  asm volatile("" ::: "memory");
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Position in the list of (unit, block) steps: unit u = row tile x of
// request r (rows row0.., n of them, positions p0..), its step count nv and
// the current block b.
struct PfCursor {
  int u, r, x, p0, n, row0, nv, b;
};

template <int KFMT, bool BALANCED, int SEL>
__global__ __launch_bounds__(kPfThreads, kPfWgPerCu) void prefill_score_kernel(ScoreArgs a, int units, int tiles,
                                                                              TopkArgs sel, int32_t* ctr) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kPfLdsOf<KFMT>];
  // bf16: two page buffers (kbuf0, kbuf1).  NVFP4: two slots of raw nibbles
  // and scales, and the E4M3 table.
  uint8_t* const kbuf0 = smem;
  uint8_t* const kbuf1 = smem + kPageBytes;
  float* const stage_all = reinterpret_cast<float*>(smem + (KFMT == 0 ? 2 * kPageBytes : kPfFp4Scores));
  u32x2* const lut = reinterpret_cast<u32x2*>(smem + kPfFp4Lut);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = a.heads;
  const int32_t MM3_AS4* bt_s = (const int32_t MM3_AS4*)a.bt;

  auto unit_at = [&](PfCursor& c, int u) {
    c.u = u;
    c.r = u / tiles;
    c.x = u - c.r * tiles;
    const ReqRows q = req_rows<true>(a.rows, c.r);
    c.p0 = q.p0;
    c.n = q.n;
    c.row0 = q.row0;
    c.nv = routed(a.route, H, q.n) ? tile_blocks(q.p0, q.n, c.x, H) : 0;
  };
  // steps of unit v (any lane's own v); a lane walks its units in order, so
  // it keeps the last request's rows and loads each request once
  int memo_r = -1;
  ReqRows memo_q{0, 0, 0};
  bool memo_routed = false;
  auto unit_steps = [&](int v) {
    const int r = v / tiles;
    if (r != memo_r) {
      memo_r = r;
      memo_q = req_rows(a.rows, r);
      memo_routed = routed(a.route, H, memo_q.n);
    }
    return memo_routed ? tile_blocks(memo_q.p0, memo_q.n, v - r * tiles, H) : 0;
  };
  // next step of the list (callers guarantee one exists)
  auto advance = [&](PfCursor& c) {
    if (++c.b < c.nv) return;
    do {
      unit_at(c, c.u + 1);
    } while (c.nv == 0);
    c.b = 0;
  };

  // ---- this workgroup's share: steps [s0, s0 + nsteps) of the list
  PfCursor cur;
  int nsteps;
  if constexpr (BALANCED) {
    int* const scan = reinterpret_cast<int*>(stage_all);  // scratch until the first block
    const int t = threadIdx.x;
    const int lo = (int)((int64_t)units * t / kPfThreads);
    const int hi = (int)((int64_t)units * (t + 1) / kPfThreads);
    int part = 0;
    for (int v = lo; v < hi; ++v) part += unit_steps(v);
    int incl = part;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    if (lane == 63) scan[wave] = incl;
    __syncthreads();
    int pre = incl - part, total = 0;
#pragma unroll
    for (int w = 0; w < kPfWaves; ++w) {
      const int sw = scan[w];
      pre += w < wave ? sw : 0;
      total += sw;
    }
    total = __builtin_amdgcn_readfirstlane(total);
    // Workgroups are dealt to the 8 XCDs round-robin; renumber so that each
    // XCD takes one contiguous stretch of the list (its requests' pages stay
    // in its own L2).  Under this load the odd-numbered XCDs run at a ~5%
    // lower clock than the even ones (the same cycles per step, 1.70-1.74
    // against 1.77-1.84 GHz), so their workgroups' shares are weighted
    // 0.97 against 1.03.
    const int G = gridDim.x, g = blockIdx.x;
    int64_t s0, s1;
    if (G % 8 == 0) {
      const int x = g % 8, per = G / 8;
      const int64_t w_x = x % 2 == 0 ? kPfXcdWeightEven : kPfXcdWeightOdd;
      // weight of the XCDs before x (half of them even), then of x's
      // workgroups before this one
      const int64_t w0 = (int64_t)per * ((x + 1) / 2 * kPfXcdWeightEven + x / 2 * kPfXcdWeightOdd) + w_x * (g / 8);
      const int64_t wtot = (int64_t)per * 4 * (kPfXcdWeightEven + kPfXcdWeightOdd);
      s0 = (int64_t)total * w0 / wtot;
      s1 = (int64_t)total * (w0 + w_x) / wtot;
    } else {
      s0 = (int64_t)total * g / G;
      s1 = (int64_t)total * (g + 1) / G;
    }
    nsteps = (int)(s1 - s0);
    if (part > 0 && pre <= s0 && s0 < pre + part) {
      int acc = pre;
      for (int v = lo; v < hi; ++v) {
        const int n = unit_steps(v);
        if (s0 < acc + n) {
          scan[8] = v;
          scan[9] = (int)(s0 - acc);
          break;
        }
        acc += n;
      }
    }
    __syncthreads();
    if (nsteps == 0) return;  // workgroup-uniform
    unit_at(cur, __builtin_amdgcn_readfirstlane(scan[8]));
    cur.b = __builtin_amdgcn_readfirstlane(scan[9]);
  } else {
    unit_at(cur, blockIdx.x);
    cur.b = 0;
    nsteps = cur.nv;
    if (nsteps == 0) return;
  }

  // ---- this wave's query rows of the current tile
  const int nl = lane & 31, kg = lane >> 5;
  bf16x8 qb[kPfQt][8];
  int pos_q[kPfQt];
  int wave_pos_min = 0, wave_pos_max = -1;
  bool wave_live = false;
  auto load_q = [&]() __attribute__((always_inline)) {
    const int HQ = H * cur.n;  // >= 1: the unit has steps
    const int wrow0 = cur.x * kPrefillRows + kPfWaveRows * wave;
#pragma unroll
    for (int qt = 0; qt < kPfQt; ++qt) {
      const int i = wrow0 + 32 * qt + nl;
      const bool ok = i < HQ;
      const int ic = ok ? i : HQ - 1;
      const int j = ic / H, h = ic - j * H;
      pos_q[qt] = ok ? cur.p0 + j : -1;
      const uint16_t* qp = a.q + (int64_t)(cur.row0 + j) * a.q_tok + (int64_t)h * a.q_head;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        // k-step kk: bf16 keys, dims 16kk + 8kg .. +8 (the swizzled page's
        // chunk 2kk + kg); NVFP4 keys, dims 64kg + 8kk .. +8 (each lane half
        // decodes one half of the token's nibble row)
        const u32x4 v = ld16(qp + (KFMT == 0 ? 16 * kk + 8 * kg : 64 * kg + 8 * kk));
        if constexpr (KFMT == 0) {
          qb[qt][kk] = as_bf16x8(v);
        } else {
          // decoded NVFP4 chunks hold their 8 elements in the order
          // {0,2,4,6,1,3,5,7}; the query operand follows it
          u32x4 pv;
          pv.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);
          pv.y = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);
          pv.z = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);
          pv.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);
          qb[qt][kk] = as_bf16x8(pv);
        }
      }
    }
    wave_live = wrow0 < HQ;
    wave_pos_min = cur.p0 + min(wrow0, HQ - 1) / H;
    wave_pos_max = cur.p0 + min(wrow0 + kPfWaveRows - 1, HQ - 1) / H;
    // land them now: a query load still pending at the loop would make the
    // compiler wait inside every step, and so on the copies in flight
    wait_vmcnt<0>();
  };

  // ---- page copies.  One copy instruction of a wave moves 1 KiB (4 tokens);
  // a round of all the workgroup's waves moves kCopyRound bytes.  Copy k of
  // wave w fills LDS bytes [k kCopyRound + w KiB, +1 KiB): lane l the 16-byte
  // slot of token t = 4 kPfWaves k + t0 (t0 = 4w + l/16) at slot l%16, which
  // holds chunk (l%16) ^ (t & 15) of the token (t & 15 == t0 & 15).
  constexpr int kCopyRound = 1024 * kPfWaves;
  const int t0 = 4 * wave + (lane >> 4);
  const uint32_t src0 = t0 * (kDim * 2) + (((lane & 15) ^ (t0 & 15)) << 4);
  // copy k of page pg into the buffer whose wave slot is l0 (the round steps
  // go on the scalar base: one offset register for all)
  auto copy_one = [&](uint32_t l0, const uint8_t* pg, int k) __attribute__((always_inline)) {
    copy16_to_lds(l0 + kCopyRound * k, pg + kCopyRound * k, src0);
  };
  auto wave_slot = [&](uint8_t* kl) { return (uint32_t)(uintptr_t)(MM3_AS3 uint8_t*)kl + 1024 * wave; };
  auto page_bytes = [&](int64_t page) -> const uint8_t* { return a.kdata + page * kPageBytes; };
  // The page id of a step, by a vector load: issued a step before its copy,
  // it completes behind that step's multiplies (the ring barrier waits for
  // it), where a scalar load right before the copy would hold the wave for
  // its latency at every step.  The opaque zero offset keeps it a vector
  // load.
  auto page_load = [&](const PfCursor& c) __attribute__((always_inline)) {
    int z = 0;
    asm volatile("" : "+v"(z));
    return a.bt[(int64_t)c.r * a.bt_stride + c.b + z];
  };

  // NVFP4: copy k of wave w moves nibble KiB kPfWaves k + w of the page (the
  // 8 KiB in 8 / kPfWaves rounds), and wave 0 also moves the 1 KiB of scales,
  // into slot `slot`.  Lane l fills the 16-byte slot p = l % 4 of token
  // (base + l / 4), whose (t >> 1) & 3 is (l >> 3) & 3 (the base is a
  // multiple of 16 tokens): it holds chunk p ^ ((l >> 3) & 3).
  const uint32_t nsrc0 = 16 * (lane & ~3) + 16 * ((lane & 3) ^ ((lane >> 3) & 3));
  auto copy_fp4 = [&](int slot, int64_t page) __attribute__((always_inline)) {
    const uint8_t* nib = a.kdata + page * kFp4NibBytes;
    const uint32_t l0 =
        (uint32_t)(uintptr_t)(MM3_AS3 uint8_t*)(smem + kPfFp4Stage0 + slot * kFp4NibBytes) + 1024 * wave;
#pragma unroll
    for (int k = 0; k < kFp4NibBytes / kCopyRound; ++k)
      copy16_to_lds(l0 + kCopyRound * k, nib + kCopyRound * k + 1024 * wave, nsrc0);
    if (wave == 0)
      copy16_to_lds((uint32_t)(uintptr_t)(MM3_AS3 uint8_t*)(smem + kPfFp4Scale0 + slot * kFp4ScaleBytes),
                    a.kscales + page * kFp4ScaleBytes, 16 * lane);
  };
  float* const stage = stage_all + wave * kPfStageFloats;
  // stage layout: row rho (0..127 of the wave), column c (block b & 7) at
  // 8 rho + 4 ((c >> 2) ^ (rho & 1)) + (c & 3): a row's column groups of four
  // stay contiguous for the write-out's 16-byte reads
  // Scores block b (its keys in page buffer kl, or NVFP4 slot `slot`) into
  // stage column col.
  auto compute = [&](const uint8_t* kl, int slot, int b, int col) __attribute__((always_inline)) {
    if (!(wave_live && wave_pos_max >= kBlock * b)) return;
    // every row of the wave sees the whole block
    const bool full = kBlock * b + (kBlock - 1) <= wave_pos_min;
    float m[kPfQt];
#pragma unroll
    for (int qt = 0; qt < kPfQt; ++qt) m[qt] = -INFINITY;
    f32x16 acc[kPfQt];
    // After token tile tt's last k-step: acc[qt][i] holds token
    // 32tt + 8(i/4) + 4kg + i%4 against row nl of tile qt.
    auto tile_max = [&](int tt) __attribute__((always_inline)) {
      if (full) {
#pragma unroll
        for (int qt = 0; qt < kPfQt; ++qt)
#pragma unroll
          for (int i = 0; i < 16; ++i) m[qt] = fmaxf(m[qt], acc[qt][i]);
      } else {
#pragma unroll
        for (int qt = 0; qt < kPfQt; ++qt) {
          // visible iff 8(i/4) + i%4 <= pos - 128b - 32tt - 4kg
          const int d = pos_q[qt] - kBlock * b - 32 * tt - 4 * kg;
#pragma unroll
          for (int i = 0; i < 16; ++i)
            m[qt] = fmaxf(m[qt], 8 * (i >> 2) + (i & 3) <= d ? acc[qt][i] : -INFINITY);
        }
      }
    };
    auto multiply = [&](const bf16x8& key, int kk) __attribute__((always_inline)) {
#pragma unroll
      for (int qt = 0; qt < kPfQt; ++qt) {
        if (kk == 0) acc[qt] = f32x16{};
        acc[qt] = mfma32(key, qb[qt][kk], acc[qt]);
      }
    };
    if constexpr (KFMT == 0) {
      // Key fragment of step st: tokens 32(st/8) + nl, 16-byte chunk
      // 2(st%8) + kg, stored at slot chunk ^ (tok & 15) of the token's 256-byte
      // row.  With tok & 15 == nl & 15 == 2p + e, the chunk
      // slot (2kk + kg) ^ (2p + e) is 2(kk ^ p) + (kg ^ e), so the address is
      // a0 ^ (kk << 5) plus 8 KiB per token tile, a0 holding the kk = 0 slot
      // (the buffers are 256-byte aligned, so bits 5..7 of a0 are exactly p).
      // The asm hides a0's loop invariance: hoisted out of the step loop, the
      // eight per-kk addresses would stay live next to the 192 query and
      // accumulator registers and spill.
      uint32_t a0 = (uint32_t)(uintptr_t)(const MM3_AS3 uint8_t*)kl + nl * (kDim * 2) +
                    (((kg ^ nl) & 1) << 4) + (((nl >> 1) & 7) << 5);
      asm volatile("" : "+v"(a0));
      auto frag = [&](int st) {
        const uint32_t addr = (a0 ^ ((st & 7) << 5)) + (st >> 3) * 32 * (kDim * 2);
        return as_bf16x8(*(const MM3_AS3 u32x4*)(uintptr_t)addr);
      };
      // Fragments are read kPfAhead steps before their multiplies; the
      // scheduling barrier at the end of each step pins that order (left
      // alone, the scheduler sinks each read next to its use and the wave then
      // waits out the full LDS latency at every step).
      bf16x8 fr[kPfAhead + 1];
#pragma unroll
      for (int p = 0; p < kPfAhead; ++p) fr[p] = frag(p);
#pragma unroll
      for (int st = 0; st < 32; ++st) {
        const int tt = st >> 3, kk = st & 7;
        if (st + kPfAhead < 32) fr[(st + kPfAhead) % (kPfAhead + 1)] = frag(st + kPfAhead);
        multiply(fr[st % (kPfAhead + 1)], kk);
        if (kk == 7) tile_max(tt);
        // also keeps the next tile's multiplies (fresh accumulators) below the
        // max: overlapping them needs a second set of 64 accumulator
        // registers, which the two-waves-per-SIMD budget does not have (the
        // other wave on the SIMD fills the matrix pipe meanwhile)
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // NVFP4: lane (nl, kg) multiplies token 32tt + nl, dims 64kg + 8kk ..
      // +8 at k-step (tt, kk): nibble dword kk of the lane's half row
      // (chunks 2kg and 2kg + 1, words W0 for kk < 4 and W1 after), under
      // scale byte kk / 2 of the token's scale word (bytes 4kg .. 4kg + 3 of
      // its 8).  Each pair of k-steps takes one table entry: the 8 E4M3 codes
      // of that scale.  The fragment of k-step st + 1 is decoded during k-step
      // st, its vector instructions placed between st's four multiplies, so
      // the matrix pipe is fed while the decode runs.  Reads lead their use:
      // W1 is read at kk = 0 of its tile, the next tile's W0 at kk = 4 and its
      // scale word at kk = 0, a pair's table entry three k-steps before the
      // decode of its first k-step.
      const int sw = (nl >> 1) & 3;
      const uint32_t nb0 = (uint32_t)(uintptr_t)(const MM3_AS3 uint8_t*)(smem + kPfFp4Stage0 + slot * kFp4NibBytes);
      const uint32_t sb0 = (uint32_t)(uintptr_t)(const MM3_AS3 uint8_t*)(smem + kPfFp4Scale0 + slot * kFp4ScaleBytes);
      const uint32_t lb0 = (uint32_t)(uintptr_t)(const MM3_AS3 uint8_t*)(smem + kPfFp4Lut);
      uint32_t w0a = nb0 + nl * (kDim / 2) + 16 * ((2 * kg) ^ sw);
      uint32_t w1a = nb0 + nl * (kDim / 2) + 16 * ((2 * kg + 1) ^ sw);
      uint32_t sa = sb0 + nl * (kDim / 16) + 4 * kg;
      asm volatile("" : "+v"(w0a), "+v"(w1a), "+v"(sa));
      auto ldw = [&](uint32_t base, int tt) {
        return *(const MM3_AS3 u32x4*)(uintptr_t)(base + tt * 32 * (kDim / 2));
      };
      auto lds = [&](int tt) { return *(const MM3_AS3 uint32_t*)(uintptr_t)(sa + tt * 32 * (kDim / 16)); };
      auto ldl = [&](uint32_t sword, int p) {
        return *(const MM3_AS3 u32x2*)(uintptr_t)(lb0 + 8 * ((sword >> (8 * p)) & 0xFFu));
      };
      u32x4 W0 = ldw(w0a, 0), W1 = ldw(w1a, 0);
      uint32_t S = lds(0), Sn = 0;
      // L[g & 1]: the entry of k-step pair g (k-steps 2g, 2g + 1 of the 32)
      u32x2 L[2];
      L[0] = ldl(S, 0);
      L[1] = ldl(S, 1);
      bf16x8 D = as_bf16x8(fp4x8_to_bf16(W0[0], L[0]));
#pragma unroll
      for (int st = 0; st < 32; ++st) {
        const int tt = st >> 3, kk = st & 7;
        if (kk == 0 && tt > 0) W1 = ldw(w1a, tt);
        if (kk == 0 && tt + 1 < 4) Sn = lds(tt + 1);
        if (kk == 4 && tt + 1 < 4) W0 = ldw(w0a, tt + 1);
        // the entry of the pair that starts at k-step st + 3
        if (((st + 3) & 1) == 0 && st + 3 < 32) {
          const int t3 = st + 3;
          L[(t3 >> 1) & 1] = ldl((t3 >> 3) == tt ? S : Sn, (t3 & 7) >> 1);
        }
        bf16x8 Dn = D;
        if (st + 1 < 32) {
          const int k1 = (st + 1) & 7;
          const uint32_t x = k1 < 4 ? W0[k1 & 3] : W1[k1 & 3];
          Dn = as_bf16x8(fp4x8_to_bf16(x, L[((st + 1) >> 1) & 1]));
        }
        multiply(D, kk);
        // reads first, then each multiply followed by a share of the decode
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int q = 0; q < kPfQt; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
        if (kk == 7) tile_max(tt);
        if (kk == 7) S = Sn;
        D = Dn;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int qt = 0; qt < kPfQt; ++qt) m[qt] = wave_max_xor32(m[qt]);
    // both lane halves now hold every tile's row maxima: lane (nl, kg) stages
    // row 32 qt + nl of tiles qt = kPfQt/2 kg .. kPfQt/2 kg + kPfQt/2 - 1
#pragma unroll
    for (int u = 0; u < kPfQt / 2; ++u) {
      const int qt = (kPfQt / 2) * kg + u, r = 32 * qt + nl;
      stage[r * kPfStage + ((((col >> 2) ^ (r & 1)) << 2) | (col & 3))] =
          (kg ? m[kPfQt / 2 + u] : m[u]) * a.sm_scale;
    }
  };

  // Write the staged blocks bfirst .. bfirst + nst - 1 of the wave's rows (all
  // in one group of eight, 8k .. 8k + 7; block b sits in stage column b & 7);
  // only visible (row, block) entries are written.  Lane l takes column group
  // g = l % 2 (columns 4g .. 4g + 3) of rows l / 2 + 32k, k = 0..3: a whole
  // group goes out as one 16-byte store when its four blocks are staged and
  // visible and the score layout is 16-byte aligned, else entry by entry.
  // Thirty-two rows further on, a row's position, head and score offset move
  // by fixed amounts (one carry when the head wraps), so the loop needs no
  // division and no 64-bit multiply.
  const bool vec_ok = (a.s_row & 3) == 0 && (a.s_head & 3) == 0 && ((uintptr_t)a.scores & 15) == 0;
  auto flush = [&](int bfirst, int nst) __attribute__((always_inline)) {
    const int g = lane & 1, rr = lane >> 1;
    const int bb = (bfirst & ~7) + 4 * g;  // block of the group's column 0
    const int q0 = max((bfirst & 7) - 4 * g, 0), q1s = min((bfirst & 7) + nst - 4 * g, 4);
    const int HQ = H * cur.n;
    const int i0 = cur.x * kPrefillRows + kPfWaveRows * wave + rr;
    int j = i0 / H, h = i0 - j * H;           // row i0: position p0 + j, head h
    const int dj = 32 / H, dh = 32 - dj * H;  // the step of 32 rows
    int64_t off = (int64_t)h * a.s_head + (int64_t)(cur.row0 + j) * a.s_row + bb;
    const int64_t doff = (int64_t)dh * a.s_head + (int64_t)dj * a.s_row;
    const int64_t wrap = a.s_row - (int64_t)H * a.s_head;
    // row rr + 32k: its group g at 8 (rr + 32k) + 4 (g ^ (rr & 1))
    const float* sv = stage + rr * kPfStage + ((g ^ (rr & 1)) << 2);
    // all reads first: left next to their stores, each would wait out the
    // LDS latency inside its own branch
    f32x4 v[kPfWaveRows / 32];
#pragma unroll
    for (int k = 0; k < kPfWaveRows / 32; ++k) v[k] = *reinterpret_cast<const f32x4*>(sv + 32 * kPfStage * k);
#pragma unroll
    for (int k = 0; k < kPfWaveRows / 32; ++k) asm volatile("" : "+v"(v[k]));
#pragma unroll
    for (int k = 0; k < kPfWaveRows / 32; ++k) {
      if (i0 + 32 * k < HQ) {
        const int pos = cur.p0 + j;
        // columns q with block bb + q <= pos / 128 are visible
        const int q1 = min(q1s, pos < 0 ? 0 : (pos >> 7) + 1 - bb);
        if (vec_ok && q0 == 0 && q1 == 4) {
          *reinterpret_cast<f32x4*>(a.scores + off) = v[k];
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (q >= q0 && q < q1) a.scores[off + q] = v[k][q];
        }
      }
      j += dj;
      h += dh;
      off += doff;
      if (h >= H) {
        h -= H;
        ++j;
        off += wrap;
      }
    }
  };

  // ---- fused selection.  ctr[u]: steps of tile u scored so far, counted
  // per wave; ctr[units + u]: the workgroup that completed it (-1 before).
  // A wave at the end of its part of tile cur.u (`done` steps).
  auto tile_part_done = [&](int done) __attribute__((always_inline)) {
    // this wave's score stores become visible device-wide before the count
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    int old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(ctr + cur.u, done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old + done == kPfWaves * cur.nv && lane == 0)
      __hip_atomic_store(ctr + units + cur.u, (int)blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // After the share: select the rows of the tiles in [u_first, u_last] this
  // workgroup owns, with the page buffers as the waves' scratch.
  auto select_owned = [&](int u_first, int u_last) __attribute__((always_inline)) {
    constexpr int kSplit = SEL > 0 ? SEL : 1;  // (SEL == 0 never calls this)
    wait_vmcnt<0>();  // this wave's owner stores are complete
    __syncthreads();  // ... and every wave's; the LDS is idle
    float* const trw = reinterpret_cast<float*>(smem) + wave * (64 * kLaneRowFloats);
    for (int u = u_first; u <= u_last; ++u) {
      const int owner = __hip_atomic_load(ctr + units + u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__builtin_amdgcn_readfirstlane(owner) != (int)blockIdx.x) continue;
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the other parts' score stores
      PfCursor t;
      unit_at(t, u);
      // the tile's flattened rows [i0, i1): position j = i / H, head h =
      // i % H; per head, one lane-selector pass per 64 / SEL consecutive
      // rows, the passes dealt round-robin to the waves
      const int i0 = t.x * kPrefillRows, i1 = min(H * t.n, i0 + kPrefillRows);
      int pass = 0;
      for (int h = 0; h < H; ++h) {
        const int jlo = (i0 - h + H - 1) / H;                         // first j with j H + h >= i0
        const int jend = i1 - 1 - h >= 0 ? (i1 - 1 - h) / H + 1 : 0;  // past the last
        for (int j = jlo; j < jend; j += 64 / kSplit, ++pass)
          if (pass % kPfWaves == wave)
            lane_select<kLaneChunks, false, kSplit>(sel, h, t.row0 + j, t.row0 + jend, trw);
      }
    }
  };

  // ---- the ring: block of step i sits in buffer i & 1; the copy of step
  // i + 1 is started once every wave is past step i - 1.
  if constexpr (KFMT == 1) {
    if (threadIdx.x < 256) fill_lut(lut);  // read after the first ring barrier
  }
  // the first page is on its way while the query rows load
  {
    const int64_t pg0 = bt_s[(int64_t)cur.r * a.bt_stride + cur.b];
    if constexpr (KFMT == 0) {
#pragma unroll
      for (int k = 0; k < kPfCopies; ++k) copy_one(wave_slot(kbuf0), page_bytes(pg0), k);
    } else {
      copy_fp4(0, pg0);
    }
  }
  // nn: the step two after the current one (page id in pg_next, loaded
  // during the step before)
  PfCursor nn = cur;
  int pg_next = 0;
  if (nsteps > 1) {
    advance(nn);
    pg_next = page_load(nn);
  }
  load_q();
  // Two workgroups share each CU, and at equal priority the SIMDs favour the
  // older one's waves, so left alone the first-dispatched workgroup runs
  // ahead and the other finishes its share alone, which keeps only half of
  // the CU's waves busy (0.24 instead of 0.31 steps per us).  Priority
  // falling with the progress through the share lets the one behind catch up
  // at each band, so the two finish close together.  Step i is below b% of
  // the share iff 100 i < b nsteps, i.e. i < ceil(b nsteps / 100).
  auto band = [&](int b) { return (int)(((int64_t)b * nsteps + 99) / 100); };
  const int band70 = band(70), band85 = band(85), band95 = band(95);
  int bfirst = cur.b, nst = 0, tile_done = 0;
  // A stage group completed (block 8k + 7) in the middle of a tile is written
  // out after the next step's barrier, not before it: that barrier waits for all of the wave's
  // vector memory operations, and stores issued just before it would hold
  // every wave of the workgroup there for their completion.
  bool flush_due = false;
  const int u_first = cur.u;
  for (int i = 0; i < nsteps; ++i) {
    uint8_t* const kl = (KFMT == 0 && (i & 1)) ? kbuf1 : kbuf0;
    ring_sync();
    {
      if (i < band70)
        __builtin_amdgcn_s_setprio(3);
      else if (i < band85)
        __builtin_amdgcn_s_setprio(2);
      else if (i < band95)
        __builtin_amdgcn_s_setprio(1);
      else
        __builtin_amdgcn_s_setprio(0);
    }
    if (i + 1 < nsteps) {
      // page of step i + 1 (its load has landed: the barrier waited for it)
      asm volatile("" : "+v"(pg_next));
      const int64_t pg = __builtin_amdgcn_readfirstlane(pg_next);
      if (i + 2 < nsteps) {
        advance(nn);
        pg_next = page_load(nn);
      }
      if constexpr (KFMT == 0) {
        const uint32_t l0 = wave_slot((i & 1) ? kbuf0 : kbuf1);
#pragma unroll
        for (int k = 0; k < kPfCopies; ++k) copy_one(l0, page_bytes(pg), k);
      } else {
        copy_fp4((i + 1) & 1, pg);
      }
    }
    if (flush_due) {
      // blocks bfirst .. bfirst + nst - 1 of the current tile, up to a block
      // 8k + 7; cur is already at the next block of the same tile
      flush(bfirst, nst);
      nst = 0;
      bfirst = cur.b;
      flush_due = false;
    }
    compute(kl, i & 1, cur.b, cur.b & (kPfStage - 1));
    ++nst;
    const bool last = i + 1 == nsteps;
    const bool tile_end = cur.b + 1 == cur.nv;
    if constexpr (SEL == 0) {
      if (tile_end || last) {
        flush(bfirst, nst);
        nst = 0;
        bfirst = cur.b + 1;
      } else if ((cur.b & (kPfStage - 1)) == kPfStage - 1) {
        flush_due = true;
      }
      if (!last) {
        advance(cur);
        if (cur.b == 0) {
          bfirst = 0;
          load_q();
        }
      }
    } else {
      ++tile_done;
      if ((cur.b & (kPfStage - 1)) == kPfStage - 1 || tile_end || last) {
        flush(bfirst, nst);
        nst = 0;
        bfirst = cur.b + 1;
      }
      if (tile_end || last) {
        tile_part_done(tile_done);
        tile_done = 0;
      }
      if (!last) {
        advance(cur);
        if (cur.b == 0) {
          bfirst = 0;
          load_q();
        }
      }
    }
  }
  if constexpr (SEL > 0) select_owned(u_first, cur.u);
}

// Ahead of the fused scorer: resets the tile counters (0) and owners (-1)
// -- ctr holds 2 * units words -- and writes the ids of the tiles that have
// no steps (rows that all sit before position 0 see no block: all -1), which
// no workgroup completes.  One wave per unit.
__global__ __launch_bounds__(256) void fused_reset_kernel(int32_t* ctr, int units, int tiles, ScoreArgs a,
                                                          TopkArgs sel) {
  const int gt = blockIdx.x * 256 + threadIdx.x;
  for (int i = gt; i < 2 * units; i += gridDim.x * 256) ctr[i] = i < units ? 0 : -1;
  const int lane = threadIdx.x & 63;
  const int H = a.heads;
  for (int u = gt >> 6; u < units; u += gridDim.x * 4) {
    const int r = u / tiles, x = u - r * tiles;
    const ReqRows q = req_rows(a.rows, r);
    if (x * kPrefillRows >= H * q.n || tile_blocks(q.p0, q.n, x, H) > 0) continue;
    const int i0 = x * kPrefillRows, i1 = min(H * q.n, i0 + kPrefillRows);
    for (int e = lane; e < (i1 - i0) * sel.topk; e += 64) {
      const int i = i0 + e / sel.topk, k = e - (e / sel.topk) * sel.topk;
      const int j = i / H, h = i - j * H;
      sel.out[(int64_t)h * sel.o_head + (int64_t)(q.row0 + j) * sel.o_row + k] = -1;
    }
  }
}

// Persistent grid: workgroups that fit the chip at once, cached per device
// and kernel.
template <int KFMT, int SEL>
static int prefill_grid() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  int g = dev < 64 ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (g <= 0) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, prefill_score_kernel<KFMT, true, SEL>, kPfThreads,
                                                     0) != hipSuccess ||
        per_cu <= 0)
      per_cu = 1;
    g = device_cus() * per_cu;
    if (dev < 64) cache[dev].store(g, std::memory_order_relaxed);
  }
  return g;
}

// (request, row tile) units of a batch: the tiles a request of up to
// query_len rows has, for every request.
static int64_t prefill_units(const ScoreArgs& a, int* tiles) {
  *tiles = (a.heads * a.rows.qlen + kPrefillRows - 1) / kPrefillRows;  // per request, at most
  return (int64_t)a.rows.num_reqs * *tiles;
}

static bool prefill_balanced(const ScoreArgs& a) {
  int tiles = 0;
  const int64_t units = prefill_units(a, &tiles);
  // the scan counts steps in 32-bit integers
  return units <= kPfBalancedMaxUnits && units * a.nb_max <= INT32_MAX;
}

template <int KFMT, int SEL>
static void launch_prefill_t(const ScoreArgs& a, const TopkArgs& sel, int32_t* ctr, hipStream_t s) {
  int tiles = 0;
  const int units = (int)prefill_units(a, &tiles);
  hipLaunchKernelGGL((prefill_score_kernel<KFMT, true, SEL>), dim3(prefill_grid<KFMT, SEL>()), dim3(kPfThreads), 0,
                     s, a, units, tiles, sel, ctr);
}

template <int KFMT>
static hipError_t launch_prefill(const ScoreArgs& a, hipStream_t s) {
  int tiles = 0;
  const int64_t units = prefill_units(a, &tiles);
  if (prefill_balanced(a)) {
    launch_prefill_t<KFMT, 0>(a, TopkArgs{}, nullptr, s);
  } else {
    hipLaunchKernelGGL((prefill_score_kernel<KFMT, false, 0>), dim3((unsigned)units), dim3(kPfThreads), 0, s, a,
                       (int)units, tiles, TopkArgs{}, (int32_t*)nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_score_bf16(const ScoreArgs& a, hipStream_t s) { return launch_prefill<0>(a, s); }

hipError_t launch_prefill_score_nvfp4(const ScoreArgs& a, hipStream_t s) { return launch_prefill<1>(a, s); }

int prefill_select_counters(const ScoreArgs& a, const TopkArgs& sel) {
  if (sel.topk > kLaneTop || a.nb_max > 16 * kLaneChunks * 8 || !prefill_balanced(a) || !lanes_layout_ok(sel))
    return 0;
  int tiles = 0;
  return 2 * (int)prefill_units(a, &tiles);
}

hipError_t launch_prefill_score_select(const ScoreArgs& a, int kfmt, const TopkArgs& sel, int32_t* ctr,
                                       hipStream_t s) {
  int tiles = 0;
  const int units = (int)prefill_units(a, &tiles);
  hipLaunchKernelGGL(fused_reset_kernel, dim3(min(1024, (units + 3) / 4)), dim3(256), 0, s, ctr, units, tiles, a,
                     sel);
  int split = 1;
  while (16 * kLaneChunks * split < a.nb_max) split *= 2;
  const bool nv4 = kfmt == 1;
  switch (split) {
    case 1: nv4 ? launch_prefill_t<1, 1>(a, sel, ctr, s) : launch_prefill_t<0, 1>(a, sel, ctr, s); break;
    case 2: nv4 ? launch_prefill_t<1, 2>(a, sel, ctr, s) : launch_prefill_t<0, 2>(a, sel, ctr, s); break;
    case 4: nv4 ? launch_prefill_t<1, 4>(a, sel, ctr, s) : launch_prefill_t<0, 4>(a, sel, ctr, s); break;
    case 8: nv4 ? launch_prefill_t<1, 8>(a, sel, ctr, s) : launch_prefill_t<0, 8>(a, sel, ctr, s); break;
    default: return hipErrorInvalidValue;  // prefill_select_counters admits no such batch
  }
  return hipGetLastError();
}

}  // namespace mm3
