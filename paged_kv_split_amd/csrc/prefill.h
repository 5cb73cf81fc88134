// Internal interface between the C-ABI host layer (pdattn.hip) and the
// ragged paged prefill kernel (prefill.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pdattn {

// (query row, head) columns one prefill workgroup computes: 4 waves of two
// 16-column blocks (one block for head_dim 256).
constexpr int prefill_columns(int head_dim) { return head_dim == 256 ? 64 : 128; }
// Tokens of the kernel's K/V tiles.
constexpr int prefill_kv_tile(int head_dim) { return head_dim == 256 ? 32 : 64; }
// Floats of one part record of a split tile (per kv head): the unnormalised
// accumulators of every column, then each column's (m, l).
constexpr int64_t prefill_record_floats(int head_dim) { return (int64_t)prefill_columns(head_dim) * (head_dim + 2); }

struct PrefillParams {
  const uint16_t* q;          // bf16 bits [total_q][Hq][D]
  const int32_t* qo_indptr;   // [B + 1]
  const int32_t* tile_batch;  // [num_tiles]: request of each query tile
  const int32_t* tile_index;  // [num_tiles]: its tile index inside that request
  const uint8_t* k;           // pool bytes, rows as in the decode kernels (inline fp8: D + 4 bytes each)
  const uint8_t* v;
  const float* k_scale;       // separate-scale fp8 pools: one per row
  const float* v_scale;
  const int32_t* block_table; // [B][max_pages_per_seq]
  const int32_t* context_lens;
  float* out;                 // [total_q][Hq][D]
  float* lse;                 // [total_q][Hq] or null
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t heads_per_kv;       // G (any value 1..16)
  int32_t rows_per_tile;      // prefill_columns(D) / G
  int32_t page_log2;
  int32_t max_pages_per_seq;
  int32_t num_pages;
  int32_t slot_stride;        // row index = page * P * Hkv + slot * slot_stride + kvh * head_stride
  int32_t head_stride;
  int32_t causal;
  float qk_scale_log2;        // softmax scale * log2(e)
  // split tiles (null tile_kv: every tile whole)
  const int32_t* tile_kv;     // [num_tiles][4]: first position, end position, first slot (-1: whole), part | parts << 16
  float* part_rec;            // [num_slots][num_kv_heads][prefill_record_floats]
  uint32_t* part_ctr;         // [num_slots][num_kv_heads]: parts finished (low 16 bits) and poisoned (high)
  int32_t num_slots;
};

// Pool kinds of the prefill kernel.
constexpr int kPrefillBf16 = 0, kPrefillFp8 = 1, kPrefillFp8Inline = 2;

// grid: num_tiles * num_kv_heads workgroups of 256 threads.
hipError_t launch_prefill(const PrefillParams& p, int head_dim, int pool, uint32_t grid, hipStream_t stream);
// Resident prefill workgroups per compute unit (0 when the runtime cannot say).
int prefill_wgs_per_cu(int head_dim, int pool);

}  // namespace pdattn
