// Internal interface between the C-ABI host layer (pdattn.hip) and the TQ4
// kernels (tq4.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pdattn {

// Waves per workgroup of the TQ4 decode kernel (they share the two
// centroid tables in LDS).
constexpr int kTq4Waves = 8;
// Fewest tiles the planner puts in one work item.
constexpr int kTq4MinChunkTiles = 4;

// Floats of one work item's record: m[G], l[G] padded to a multiple of 4,
// then G accumulators of D floats (16-byte aligned throughout).
__host__ __device__ constexpr int tq4_record_header(int group) { return (2 * group + 3) / 4 * 4; }
__host__ __device__ constexpr long long tq4_record_floats(int group, int head_dim) {
  return tq4_record_header(group) + (long long)group * head_dim;
}

// Compress-and-scatter (one wave per (token, kv head)).
struct Tq4AppendParams {
  const uint16_t* k_new;       // bf16 bits [T][Hkv][D]
  const uint16_t* v_new;
  const int32_t* token_seq;    // [T]
  const int32_t* token_pos;    // [T]
  const int32_t* block_table;  // [B][max_pages_per_seq]
  const float* rotation;       // [D][D] row-major: y = R x
  const float* k_bounds;       // [15] sorted
  const float* v_bounds;
  uint8_t* cache;              // [num_pages][Hkv][P][D + 8]
  int32_t num_tokens;
  int32_t batch;
  int32_t num_kv_heads;
  int32_t page_log2;
  int32_t max_pages_per_seq;
  int32_t num_pages;
};

// Decode: q rotation, the chunk kernel, the merge with the back-rotation.
struct Tq4DecodeParams {
  const uint16_t* q;           // bf16 bits [B][Hq][D], model space; with q_rotated: fp16 bits, y = R q
  uint16_t* q_seq;             // workspace: fp16 [B][Hq][D], rotated, sequential order
  const uint8_t* cache;        // [num_pages][Hkv][P][D + 8]
  const float* rotation;       // [D][D]
  const float* k_cent;         // [16]
  const float* v_cent;
  const int32_t* block_table;
  const int32_t* context_lens;
  float* rec;                  // workspace: [max_chunks][B * Hkv][tq4_record_floats(G, D)]
  float* out;                  // [B][Hq][D]
  float* lse;                  // [B][Hq] or null
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t heads_per_kv;        // G
  int32_t page_log2;
  int32_t max_pages_per_seq;
  int32_t num_pages;
  int32_t chunk_tiles;         // planned tiles per work item (a pair has ceil(tiles / chunk_tiles) items,
  int32_t max_chunks;          //  at most max_chunks, splitting its tiles evenly)
  int32_t num_waves;           // waves of the decode grid
  float qk_scale_log2;         // softmax scale * log2(e)
  int32_t q_rotated;           // 1: q arrives rotated (natural order) and out stays rotated (no rotation kernels)
};

// Resident decode workgroups per compute unit (runtime occupancy query),
// 0 when it cannot be asked.
int tq4_decode_wgs_per_cu(int head_dim);
hipError_t launch_tq4_append(const Tq4AppendParams& p, int head_dim, uint32_t grid, hipStream_t stream);
// The decode launches on one stream: three, or two with q_rotated.
hipError_t launch_tq4_decode(const Tq4DecodeParams& p, int head_dim, uint32_t decode_grid, hipStream_t stream);

}  // namespace pdattn
