// Internal interface between the C-ABI host layer (pdattn.hip) and the
// gfx950 kernels (decode_kernels.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pdattn {

// Entries of one split's block-table slice staged in LDS. The planner keeps
// ceil(split_tokens / page_size) + 1 within this bound.
constexpr int kMaxPageList = 1024;
// Waves per workgroup of the partial kernel; each wave owns every
// kWaves-th 16-token tile of the workgroup's split.
constexpr int kWaves = 4;
// Tokens per tile: the M extent of one 16x16x32 MFMA.
constexpr int kTileTokens = 16;
// Stages of each wave's direct-to-LDS load ring (tiles in flight).
constexpr int kStages = 2;

struct DecodeParams {
  const uint16_t* q;          // bf16 bits [B][Hq][D]
  const uint8_t* k;           // pool bytes [num_pages][P][Hkv][D * esize]
  const uint8_t* v;
  const float* k_scale;       // fp8 pools: [num_pages][P][Hkv]
  const float* v_scale;
  const int32_t* block_table; // [B][max_pages_per_seq]
  const int32_t* context_lens;
  float* out;                 // [B][Hq][D]
  float* lse;                 // [B][Hq] or null
  float* part_acc;            // [B][Hq][max_splits][D]
  float* part_ml;             // [B][Hq][max_splits][2] = (m, l), base-2 units
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t page_log2;
  int32_t max_pages_per_seq;
  int32_t num_pages;
  int32_t split_tokens;
  int32_t max_splits;
  int32_t num_units;          // B * max_splits
  float qk_scale_log2;        // softmax scale * log2(e)
};

struct ReduceParams {
  const float* part_acc;
  const float* part_ml;
  const int32_t* context_lens;
  float* out;
  float* lse;
  int32_t num_q_heads;
  int32_t page_log2;
  int32_t max_pages_per_seq;
  int32_t split_tokens;
  int32_t max_splits;
};

// Returns hipErrorInvalidValue for an instantiation that is not built.
hipError_t launch_partial(const DecodeParams& p, int head_dim, int group, bool fp8, uint32_t grid,
                          hipStream_t stream);
hipError_t launch_reduce(const ReduceParams& p, int head_dim, uint32_t grid, hipStream_t stream);

}  // namespace pdattn
