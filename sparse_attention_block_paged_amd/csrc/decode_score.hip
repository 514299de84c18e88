// decode_score.hip -- split-K decode block scorer for gfx950.
//
// What it computes (page "vllm.models.minimax_m3.amd.ops.index_topk", module
// docstring and minimax_m3_index_decode): for each request, its H*Q index
// query rows (H heads x Q decode positions, <= 16) score every visible
// 128-token block of the paged, shared index-K cache as the maximum over the
// block's causally visible tokens of sm_scale * (q . k).
//
// Design.  Decode is a bandwidth-bound GEMV: every key (256 B bf16, 72 B
// NVFP4) is read once and serves all H*Q rows of its request.  One wavefront
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
// The grid is (block chunks, requests), sized from max_seq_len so it is
// fixed under graph capture; chunks past a request's end return at once.
// Unlike the pages' Triton split-K kernel there is no per-chunk partial
// result: a block's score is complete inside one wave, so the split needs no
// merge.
#include "mm3_device.h"
#include "mm3_launch.h"

namespace mm3 {

// ---------------------------------------------------------------- NVFP4 LUT
//
// Key element value = e4m3_rn_satfinite(e2m1(nibble) * e4m3(scale)) (page
// "vllm.models.minimax_m3.amd.indexer_nvfp4", module docstring).  For every
// scale byte the table holds the E4M3 codes of the 8 non-negative E2M1
// magnitudes times that scale, rounded to nearest-even and saturated at 448;
// the nibble's sign is XORed in at run time.  Built at compile time.

struct Fp4Lut {
  uint32_t w[256][2];
};

// e4m3 value of a non-negative code, in units of 2^-9
constexpr int64_t e4m3_units9(int c) {
  int e = (c >> 3) & 15, m = c & 7;
  return e == 0 ? m : (int64_t)(8 + m) << (e - 1);
}

// E4M3 code (no sign) nearest to p * 2^-10, ties to even code, saturating.
constexpr int e4m3_code_from_units10(int64_t p) {
  int code;
  if (p < 16) {  // below the smallest normal: grid step 2 units
    int64_t q = p >> 1;
    if (p & 1) q += (q & 1);
    code = (int)q;
  } else {
    int lg = 0;
    while ((p >> (lg + 1)) != 0) ++lg;  // floor(log2 p) >= 4
    int e = lg - 3;                     // p in [2^(e+3), 2^(e+4)), step 2^e
    int64_t q = p >> e, rem = p & ((int64_t(1) << e) - 1), half = int64_t(1) << (e - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
    code = (e << 3) + (int)(q - 8);
  }
  return code > 0x7E ? 0x7E : code;
}

constexpr Fp4Lut make_fp4_lut() {
  Fp4Lut t{};
  const int mag2[8] = {0, 1, 2, 3, 4, 6, 8, 12};  // e2m1 magnitudes x 2
  for (int s = 0; s < 256; ++s) {
    int a = s & 0x7F;
    uint32_t lo = 0, hi = 0;
    for (int j = 0; j < 8; ++j) {
      int code = 0;
      if (a != 0x7F)  // NaN scale: unspecified, mapped to +-0
        code = e4m3_code_from_units10(mag2[j] * e4m3_units9(a));
      code |= (s & 0x80);
      if (j < 4)
        lo |= (uint32_t)code << (8 * j);
      else
        hi |= (uint32_t)code << (8 * (j - 4));
    }
    t.w[s][0] = lo;
    t.w[s][1] = hi;
  }
  return t;
}

__device__ const Fp4Lut kFp4Lut = make_fp4_lut();

// 8 NVFP4 elements (one dword of nibbles, element 2i in the low nibble of
// byte i) -> 4 dwords of bf16 pairs in the element order
// {0,2 | 4,6 | 1,3 | 5,7}; tab = the 8 E4M3 codes for this group's scale.
__device__ __forceinline__ u32x4 fp4x8_to_bf16(uint32_t x, u32x2 tab) {
  uint32_t c_even = __builtin_amdgcn_perm(tab.y, tab.x, x & 0x07070707u) ^
                    ((x << 4) & 0x80808080u);
  uint32_t c_odd = __builtin_amdgcn_perm(tab.y, tab.x, (x >> 4) & 0x07070707u) ^
                   (x & 0x80808080u);
  u32x4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c_even, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c_even, 1.0f, true));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c_odd, 1.0f, false));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c_odd, 1.0f, true));
  return r;
}

// ------------------------------------------------------------------ scorer

template <int KFMT>
__global__ __launch_bounds__(256) void decode_score_kernel(ScoreArgs a) {
  __shared__ u32x2 lut[KFMT == 1 ? 256 : 1];
  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int seq = a.seq_lens[r];
  if (seq <= 0) return;
  const int nb = (seq - 1) / kBlock + 1;  // blocks the request's last row sees
  const int b_begin = blockIdx.x * a.blocks_per_wg;
  if (b_begin >= nb) return;
  const int b_end = min(nb, b_begin + a.blocks_per_wg);

  if (KFMT == 1) {
    lut[threadIdx.x].x = kFp4Lut.w[threadIdx.x][0];
    lut[threadIdx.x].y = kFp4Lut.w[threadIdx.x][1];
    __syncthreads();
  }

  // Query rows: MFMA column n is row c = j*H + h of this request.
  const int H = a.heads, Q = a.qlen, HQ = H * Q;
  int pos_n = -1, t_n = 0, h_n = 0;
  bf16x8 qb[4];
  if (n < HQ) {
    const int j = n / H;
    h_n = n - j * H;
    t_n = r * Q + j;
    pos_n = seq - Q + j;
    const uint16_t* qp = a.q + (int64_t)t_n * a.q_tok + (int64_t)h_n * a.q_head;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      if (KFMT == 0) {
        // k-group g, step kc covers d = 32*kc + 8*g .. +8 (natural order)
        qb[kc] = as_bf16x8(ld16(qp + 32 * kc + 8 * g));
      } else {
        // NVFP4 tiles hand lane group g the 32 dims [32g, 32g+32); step kc
        // covers 8 of them in the order {0,2,4,6,1,3,5,7}
        u32x4 v = ld16(qp + 32 * g + 8 * kc);
        u32x4 p;
        p.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);  // e0, e2
        p.y = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);  // e4, e6
        p.z = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);  // e1, e3
        p.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);  // e5, e7
        qb[kc] = as_bf16x8(p);
      }
    }
  } else {
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) qb[kc] = as_bf16x8(u32x4{0, 0, 0, 0});
  }
  const int min_pos = seq - Q;  // position of the request's first row
  const int32_t* bt_row = a.bt + (int64_t)r * a.bt_stride;

  for (int b = b_begin + wave; b < b_end; b += 4) {
    const int64_t page = bt_row[b];
    f32x4 acc[8];
    if (KFMT == 0) {
      const uint8_t* kp = a.kdata + page * (kBlock * kDim * 2);
      u32x4 kr[8][4];
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
          kr[tt][kc] = ld16(kp + ((16 * tt + n) * kDim + 32 * kc + 8 * g) * 2);
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) acc[tt] = mfma16(as_bf16x8(kr[tt][kc]), qb[kc], acc[tt]);
      }
    } else {
      const uint8_t* kn = a.kdata + page * (kBlock * kDim / 2);
      const uint8_t* ks = a.kscales + page * (kBlock * kDim / 16);
      u32x4 nib[8];
      uint32_t sc[8];
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        nib[tt] = ld16(kn + (16 * tt + n) * (kDim / 2) + 16 * g);
        sc[tt] = *reinterpret_cast<const uint16_t*>(ks + (16 * tt + n) * (kDim / 16) + 2 * g);
      }
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const u32x2 t0 = lut[sc[tt] & 0xFF];
        const u32x2 t1 = lut[sc[tt] >> 8];
        acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc[tt] = mfma16(as_bf16x8(fp4x8_to_bf16(nib[tt].x, t0)), qb[0], acc[tt]);
        acc[tt] = mfma16(as_bf16x8(fp4x8_to_bf16(nib[tt].y, t0)), qb[1], acc[tt]);
        acc[tt] = mfma16(as_bf16x8(fp4x8_to_bf16(nib[tt].z, t1)), qb[2], acc[tt]);
        acc[tt] = mfma16(as_bf16x8(fp4x8_to_bf16(nib[tt].w, t1)), qb[3], acc[tt]);
      }
    }
    // acc[tt][i] = dot of token 16*tt + 4*g + i with row n
    float m = -INFINITY;
    if (kBlock * b + (kBlock - 1) <= min_pos) {
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
        m = fmaxf(m, fmaxf(fmaxf(acc[tt][0], acc[tt][1]), fmaxf(acc[tt][2], acc[tt][3])));
    } else {
      const int lim = pos_n - kBlock * b;  // token s visible iff s <= lim
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * tt + 4 * g + i <= lim) m = fmaxf(m, acc[tt][i]);
    }
    m = wave_max_xor(m, 16);
    m = wave_max_xor(m, 32);
    if (g == 0 && n < HQ && pos_n >= kBlock * b)
      a.scores[(int64_t)h_n * a.s_head + (int64_t)t_n * a.s_row + b] = m * a.sm_scale;
  }
}

static dim3 decode_grid(const ScoreArgs& a) {
  const int chunks = (a.nb_max + a.blocks_per_wg - 1) / a.blocks_per_wg;
  return dim3(chunks, a.num_reqs, 1);
}

hipError_t launch_decode_score_bf16(const ScoreArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(decode_score_kernel<0>, decode_grid(a), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_score_nvfp4(const ScoreArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(decode_score_kernel<1>, decode_grid(a), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mm3
