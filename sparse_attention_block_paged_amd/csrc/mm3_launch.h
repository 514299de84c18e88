// mm3_launch.h -- internal kernel argument blocks and launchers.  The C ABI
// (mm3_abi.cpp) validates every host-visible rule before calling these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mm3 {

// The batch's rows.  Uniform (cu == nullptr): request r owns rows
// [r*qlen, (r+1)*qlen) and its row j sits at seq_lens[r] - qlen + j.
// Ragged: rows [cu[r], cu[r+1]); row j at prefix[r] + j, or at
// seq_lens[r] - n_r + j without prefix.  qlen bounds every n_r.
struct Rows {
  const int32_t* seq_lens;
  const int32_t* cu;
  const int32_t* prefix;
  int32_t num_reqs;
  int32_t qlen;
  int32_t tokens;
};

// Which requests a scorer launch takes (a ragged batch may need both).
enum Route : int32_t {
  kRouteAll = 0,      // every request
  kRouteDecode = 1,   // requests with heads * n_r <= kDecodeRows
  kRoutePrefill = 2,  // requests with heads * n_r > kDecodeRows
};

// Everything a scorer reads.  Strides in elements.
struct ScoreArgs {
  const uint16_t* q;        // bf16 bits [T, H, 128]
  int64_t q_tok;
  int64_t q_head;
  const uint8_t* kdata;     // bf16 [P,128,128] or nvfp4 nibbles [P,128,64]
  const uint8_t* kscales;   // nvfp4 e4m3 scales [P,128,8]
  const int32_t* bt;
  int64_t bt_stride;
  Rows rows;                // qlen: rows per request this launch handles at most
  float* scores;            // [H, T, >=nb] fp32
  int64_t s_head;
  int64_t s_row;
  int32_t heads;
  int32_t route;            // Route
  int32_t nb_max;           // cdiv(max_seq_len, 128)
  int32_t blocks_per_wg;    // decode: blocks one workgroup covers
  int32_t s_bytes;          // bytes from scores to one past its last element
                            // (0 when that exceeds 2^31 - 64)
  float sm_scale;
};

// Sparse block-table output (one index head).
struct SparseOut {
  const int32_t* abt;
  int64_t abt_row;
  int32_t* table;
  int64_t st_row;
  int32_t* ctx_lens;
  int32_t pages_per_block;
  int32_t block_page_stride;
};

struct TopkArgs {
  const float* scores;
  int64_t s_head;
  int64_t s_row;
  int32_t s_width;  // columns of a score row (reads stay below it)
  Rows rows;
  int32_t* out;
  int64_t o_head;
  int64_t o_row;
  int32_t heads;
  int32_t topk;
  int32_t init_blocks;
  int32_t local_blocks;
  int32_t nb_max;
  SparseOut sp;   // used when sparse != 0 (heads == 1)
  int32_t sparse;
  const int32_t* row_blocks;  // when set: nv per row, instead of rows' positions
  int32_t s_bytes;            // bytes from scores to one past its last element
                              // (0 when that exceeds 2^31 - 64)
};

struct SparseTableArgs {
  const int32_t* topk_idx;
  int64_t o_row;
  Rows rows;
  SparseOut sp;
  int32_t topk;
};

// Each returns hipSuccess or the launch error.
hipError_t launch_decode_score_bf16(const ScoreArgs& a, hipStream_t s);
hipError_t launch_decode_score_nvfp4(const ScoreArgs& a, hipStream_t s);
// Scores and selection in one launch, one workgroup per request, for
// batches whose requests see at most kSmallBlocks blocks and hold at most
// kDecodeRows rows each; no sparse table.  a.scores / a.s_bytes: where the
// scores also go (s_bytes 0: nowhere).
hipError_t launch_decode_small(const ScoreArgs& a, const TopkArgs& t, int kfmt, hipStream_t s);
hipError_t launch_prefill_score_bf16(const ScoreArgs& a, hipStream_t s);
hipError_t launch_prefill_score_nvfp4(const ScoreArgs& a, hipStream_t s);
// The prefill scorer with the selection fused in (every request of the batch
// must go to the prefill scorer).  prefill_select_counters: the int32
// words of device memory (any contents; the launch resets them) the fused
// launch needs -- a counter and an owner per row tile -- or 0 when the batch
// cannot take it (topk above 16, rows past 512 blocks, more row tiles than
// the balanced grid takes, a score layout the lane selector cannot read).
int prefill_select_counters(const ScoreArgs& a, const TopkArgs& sel);
hipError_t launch_prefill_score_select(const ScoreArgs& a, int kfmt, const TopkArgs& sel, int32_t* ctr,
                                       hipStream_t s);
// Whether a score tensor's layout suits the lane selector's 16-byte row loads.
bool lanes_layout_ok(const TopkArgs& a);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
// The selector kernel launch_topk runs for these arguments, as its name and
// template arguments (host only; the string lives until the thread's next call).
const char* topk_kernel_name(const TopkArgs& a);
hipError_t launch_sparse_table(const SparseTableArgs& a, hipStream_t s);

// Rows one decode-scorer MFMA tile holds (heads * query_len must fit).
constexpr int kDecodeRows = 16;
// Most blocks a request may see, and most requests, for the single-launch
// small-batch path.
constexpr int kSmallBlocks = 16;
constexpr int kSmallMaxReqs = 256;
// Flattened (token, head) rows of one prefill row tile.
constexpr int kPrefillRows = 512;

// Compute units of the current device (cached per device).
int device_cus();

}  // namespace mm3
