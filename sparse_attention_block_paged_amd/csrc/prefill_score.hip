// prefill_score.hip -- MFMA block scorer for chunked prefill on gfx950.
//
// What it computes (page "vllm.models.minimax_m3.amd.ops.index_topk",
// minimax_m3_index_score: per query token and head, "the max over a 128-token
// index-K block" for each visible block; causal within the chunk).
//
// Design.  With many query rows per request the score is a dense product
// [rows x 128] . [128 x keys] followed by a max over each 128-key block, so it
// runs on the bf16 matrix cores:
//   * a workgroup owns 256 flattened (position, head) rows of one request --
//     all heads of a position share its causal bound -- and a range of key
//     blocks; wave w owns rows 64w..64w+63 as two 32-row MFMA B tiles held in
//     registers (the queries are read once per workgroup);
//   * each key page (32 KiB) is staged once per workgroup in LDS, double
//     buffered, with a 16-byte-chunk XOR swizzle (chunk c of token s at
//     c ^ (s & 15)) so the A-operand reads of 32 tokens x 16 B are free of
//     bank conflicts;
//   * v_mfma_f32_32x32x16_bf16 with keys as A (rows = tokens) and queries as
//     B (columns = rows): each lane holds one query row and 16 tokens per
//     tile, so the block max is an in-register max over 4 tiles x 16 values
//     plus one cross-lane step (l ^ 32), fused into the epilogue; the causal
//     mask is applied only on blocks that cross a row's position.
// Work splits by (row tile, request, block range); every (row, block) score
// is complete inside one workgroup, so splits need no merge.
#include "mm3_device.h"
#include "mm3_launch.h"

namespace mm3 {

constexpr int kPageBytes = kBlock * kDim * 2;  // 32 KiB
constexpr int kPrefillBlocksPerSplit = 32;

__device__ __forceinline__ int swz(int tok, int chunk) {
  return tok * (kDim * 2) + ((chunk ^ (tok & 15)) << 4);
}

__global__ __launch_bounds__(256, 2) void prefill_score_kernel(ScoreArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t kl[2][kPageBytes];
  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int seq = a.seq_lens[r];
  const int H = a.heads, Q = a.qlen, HQ = H * Q;
  const int row0 = blockIdx.x * kPrefillRows;  // first flattened row of the tile
  const int row_last = min(HQ, row0 + kPrefillRows) - 1;
  const int pos_first = seq - Q + row0 / H;
  const int pos_last = seq - Q + row_last / H;
  if (pos_last < 0) return;
  const int nv_tile = pos_last / kBlock + 1;
  const int b_begin = blockIdx.z * kPrefillBlocksPerSplit;
  if (b_begin >= nv_tile) return;
  const int b_end = min(nv_tile, b_begin + kPrefillBlocksPerSplit);

  // This lane's two query rows (one per 32-row tile) and their B operands.
  const int nl = lane & 31, kg = lane >> 5;
  int pos_q[2], t_q[2], h_q[2];
  bool ok_q[2];
  bf16x8 qb[2][8];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int i = row0 + 64 * wave + 32 * qt + nl;
    ok_q[qt] = i < HQ;
    const int ic = ok_q[qt] ? i : HQ - 1;
    const int j = ic / H;
    h_q[qt] = ic - j * H;
    t_q[qt] = r * Q + j;
    pos_q[qt] = ok_q[qt] ? seq - Q + j : -1;
    const uint16_t* qp = a.q + (int64_t)t_q[qt] * a.q_tok + (int64_t)h_q[qt] * a.q_head;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qb[qt][kk] = as_bf16x8(ld16(qp + 16 * kk + 8 * kg));
  }
  // smallest position among this wave's rows (rows are position-ordered)
  const int wave_row0 = row0 + 64 * wave;
  const int wave_pos_min = seq - Q + min(wave_row0, HQ - 1) / H;
  const int wave_pos_max = seq - Q + min(wave_row0 + 63, HQ - 1) / H;
  const bool wave_live = wave_row0 < HQ;

  const int32_t* bt_row = a.bt + (int64_t)r * a.bt_stride;

  // staging: thread th moves 16-byte chunks th + 256*u, u < 8
  u32x4 stage[8];
  auto gload = [&](int b) {
    const uint8_t* kp = a.kdata + (int64_t)bt_row[b] * kPageBytes;
#pragma unroll
    for (int u = 0; u < 8; ++u) stage[u] = ld16(kp + (threadIdx.x + 256 * u) * 16);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = threadIdx.x + 256 * u;
      *reinterpret_cast<u32x4*>(&kl[buf][swz(c >> 4, c & 15)]) = stage[u];
    }
  };

  gload(b_begin);
  lstore(0);
  __syncthreads();

  for (int b = b_begin; b < b_end; ++b) {
    const int buf = (b - b_begin) & 1;
    if (b + 1 < b_end) gload(b + 1);
    if (wave_live && wave_pos_max >= kBlock * b) {
      const bool full = kBlock * b + (kBlock - 1) <= wave_pos_min;
      float m[2] = {-INFINITY, -INFINITY};
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const int tok = 32 * tt + nl;
          const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(&kl[buf][swz(tok, 2 * kk + kg)]));
          acc[0] = mfma32(ka, qb[0][kk], acc[0]);
          acc[1] = mfma32(ka, qb[1][kk], acc[1]);
        }
        // acc[qt][i]: token 32*tt + 8*(i/4) + 4*kg + i%4 against row nl of tile qt
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          if (full) {
#pragma unroll
            for (int i = 0; i < 16; ++i) m[qt] = fmaxf(m[qt], acc[qt][i]);
          } else {
            const int lim = pos_q[qt] - kBlock * b;
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (32 * tt + 8 * (i >> 2) + 4 * kg + (i & 3) <= lim) m[qt] = fmaxf(m[qt], acc[qt][i]);
          }
        }
      }
      m[0] = wave_max_xor(m[0], 32);
      m[1] = wave_max_xor(m[1], 32);
      // lanes 0..31 write tile 0's rows, lanes 32..63 tile 1's
      const int qt = kg;
      const float v = qt ? m[1] : m[0];
      if (ok_q[qt] && pos_q[qt] >= kBlock * b)
        a.scores[(int64_t)h_q[qt] * a.s_head + (int64_t)t_q[qt] * a.s_row + b] = v * a.sm_scale;
    }
    if (b + 1 < b_end) lstore(buf ^ 1);
    __syncthreads();
  }
}

hipError_t launch_prefill_score_bf16(const ScoreArgs& a, hipStream_t s) {
  const int row_tiles = (a.heads * a.qlen + kPrefillRows - 1) / kPrefillRows;
  const int splits = (a.nb_max + kPrefillBlocksPerSplit - 1) / kPrefillBlocksPerSplit;
  hipLaunchKernelGGL(prefill_score_kernel, dim3(row_tiles, a.num_reqs, splits), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mm3
