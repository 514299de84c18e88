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
//   * each key page (32 KiB) is copied once per workgroup into LDS by direct
//     global->LDS DMA (no registers), double buffered, with a 16-byte-chunk
//     XOR swizzle (chunk c of token s at c ^ (s & 15)) so the A-operand reads
//     of 32 tokens x 16 B are free of bank conflicts;
//   * v_mfma_f32_32x32x16_bf16 with keys as A (rows = tokens) and queries as
//     B (columns = rows): each lane holds one query row and 16 tokens per
//     tile, so the block max is an in-register max over 4 tiles x 16 values
//     plus one cross-lane step (l ^ 32), fused into the epilogue; the causal
//     mask is applied only on blocks that cross a row's position.
// Work splits by (row tile, request, block range); every (row, block) score
// is complete inside one workgroup, so splits need no merge.  Scores are
// staged in LDS and written at the end as row-contiguous runs of 16 blocks:
// storing each (row, block) value as it is produced scatters 4-byte writes
// over 64 rows per instruction, which costs several times the score volume
// in partial-line write-backs.
#include "mm3_device.h"
#include "mm3_launch.h"

namespace mm3 {

constexpr int kPageBytes = kBlock * kDim * 2;  // 32 KiB
constexpr int kPrefillBlocksPerSplit = 16;


__device__ __forceinline__ int swz(int tok, int chunk) {
  return tok * (kDim * 2) + ((chunk ^ (tok & 15)) << 4);
}

// Copy key page `page` into LDS buffer kl with the chunk swizzle of swz():
// DMA instruction u of wave w fills LDS bytes [(4u + w) KiB, +1 KiB), lane l
// the 16-byte slot of token t = 4(4u + w) + l/16 at position l%16, which
// holds chunk (l%16) ^ (t & 15) of that token.  No registers are involved.
__device__ __forceinline__ void dma_page(uint8_t* kl, const uint8_t* kdata, int64_t page, int wave, int lane) {
  const uint8_t* kp = kdata + page * kPageBytes;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int t = 4 * (4 * u + wave) + (lane >> 4);
    const int c = (lane & 15) ^ (t & 15);
    __builtin_amdgcn_global_load_lds((const void*)(kp + t * (kDim * 2) + c * 16),
                                     (__attribute__((address_space(3))) void*)(kl + (4 * u + wave) * 1024), 16,
                                     0, 0);
  }
}

__global__ __launch_bounds__(256, 2) void prefill_score_kernel(ScoreArgs a) {
  // two page buffers as separate arrays, so reads of one never wait on the
  // copy into the other
  __shared__ __attribute__((aligned(16))) uint8_t kl0[kPageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t kl1[kPageBytes];
  // block scores of the tile's rows, written out row-contiguous at the end;
  // column j of row i sits at j ^ (i & 15) (spreads one column over banks)
  __shared__ float sstage[kPrefillRows * kPrefillBlocksPerSplit];
  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int seq = a.seq_lens[r];
  const int H = a.heads, Q = a.qlen, HQ = H * Q;
  const int row0 = blockIdx.x * kPrefillRows;  // first flattened row of the tile
  const int row_last = min(HQ, row0 + kPrefillRows) - 1;
  const int pos_last = seq - Q + row_last / H;
  if (pos_last < 0) return;
  const int nv_tile = pos_last / kBlock + 1;
  const int b_begin = blockIdx.z * kPrefillBlocksPerSplit;
  if (b_begin >= nv_tile) return;
  const int b_end = min(nv_tile, b_begin + kPrefillBlocksPerSplit);

  // This lane's two query rows (one per 32-row tile) and their B operands.
  const int nl = lane & 31, kg = lane >> 5;
  int pos_q[2];
  bf16x8 qb[2][8];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int i = row0 + 64 * wave + 32 * qt + nl;
    const bool ok = i < HQ;
    const int ic = ok ? i : HQ - 1;
    const int j = ic / H, h = ic - (ic / H) * H;
    pos_q[qt] = ok ? seq - Q + j : -1;
    const uint16_t* qp = a.q + (int64_t)(r * Q + j) * a.q_tok + (int64_t)h * a.q_head;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qb[qt][kk] = as_bf16x8(ld16(qp + 16 * kk + 8 * kg));
  }
  // smallest / largest position among this wave's rows (rows are position-ordered)
  const int wave_row0 = row0 + 64 * wave;
  const int wave_pos_min = seq - Q + min(wave_row0, HQ - 1) / H;
  const int wave_pos_max = seq - Q + min(wave_row0 + 63, HQ - 1) / H;
  const bool wave_live = wave_row0 < HQ;
  const int32_t* bt_row = a.bt + (int64_t)r * a.bt_stride;

  auto compute = [&](const uint8_t* kl, int b) {
    if (!(wave_live && wave_pos_max >= kBlock * b)) return;
    const bool full = kBlock * b + (kBlock - 1) <= wave_pos_min;
    float m[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int tok = 32 * tt + nl;
        const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(&kl[swz(tok, 2 * kk + kg)]));
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
    // lanes 0..31 stage tile 0's rows, lanes 32..63 tile 1's
    const float v = kg ? m[1] : m[0];
    const int srow = 64 * wave + 32 * kg + nl;
    sstage[srow * kPrefillBlocksPerSplit + ((b - b_begin) ^ (srow & 15))] = v * a.sm_scale;
  };

  dma_page(kl0, a.kdata, bt_row[b_begin], wave, lane);
  __syncthreads();
  for (int b = b_begin; b < b_end; b += 2) {
    if (b + 1 < b_end) dma_page(kl1, a.kdata, bt_row[b + 1], wave, lane);
    compute(kl0, b);
    __syncthreads();  // also waits for the copy into kl1
    if (b + 1 < b_end) {
      if (b + 2 < b_end) dma_page(kl0, a.kdata, bt_row[b + 2], wave, lane);
      compute(kl1, b + 1);
      __syncthreads();
    }
  }
  // Write the staged scores: 16 consecutive blocks of a row per 16 lanes.
  // Only visible (row, block) entries are written.
  const int nbl = b_end - b_begin;
  for (int k = 0; k < kPrefillRows * kPrefillBlocksPerSplit / 256; ++k) {
    const int e = 256 * k + threadIdx.x;
    const int row = e / kPrefillBlocksPerSplit, j = e % kPrefillBlocksPerSplit;
    const int i = row0 + row;
    if (j < nbl && i < HQ) {
      const int jq = i / H, h = i - jq * H;
      const int pos = seq - Q + jq;
      const int b = b_begin + j;
      if (pos >= kBlock * b)
        a.scores[(int64_t)h * a.s_head + (int64_t)(r * Q + jq) * a.s_row + b] =
            sstage[row * kPrefillBlocksPerSplit + (j ^ (row & 15))];
    }
  }
}

hipError_t launch_prefill_score_bf16(const ScoreArgs& a, hipStream_t s) {
  const int row_tiles = (a.heads * a.qlen + kPrefillRows - 1) / kPrefillRows;
  const int splits = (a.nb_max + kPrefillBlocksPerSplit - 1) / kPrefillBlocksPerSplit;
  hipLaunchKernelGGL(prefill_score_kernel, dim3(row_tiles, a.num_reqs, splits), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mm3
