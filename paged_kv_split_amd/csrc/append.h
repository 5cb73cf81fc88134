// Internal interface between the C-ABI host layer (pdattn.hip) and the KV
// append kernels (kv_append.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pdattn {

// The KV append (one wave per new token).
struct AppendParams {
  const uint16_t* k_new;      // bf16 bits [num_tokens][Hkv][D]
  const uint16_t* v_new;
  const int32_t* token_seq;   // [num_tokens]
  const int32_t* token_pos;   // [num_tokens]
  const int32_t* block_table; // [B][max_pages_per_seq]
  void* k_pages;              // pool rows of D * esize bytes (D + 4 with inline scales)
  void* v_pages;
  float* k_scale;             // fp8 pools with separate scales: one per row
  float* v_scale;
  int32_t num_tokens;
  int32_t batch;
  int32_t num_kv_heads;
  int32_t page_log2;
  int32_t max_pages_per_seq;
  int32_t num_pages;
  int32_t pow2_scales;        // fp8: power-of-two scales instead of absmax / 448
  int32_t inline_scales;      // fp8: rows of D codes then the fp32 scale (D + 4 bytes apart)
  int32_t slot_stride;        // row index = page * P * Hkv + slot * slot_stride + kvh * head_stride
  int32_t head_stride;
};

hipError_t launch_kv_append(const AppendParams& p, int head_dim, bool fp8, uint32_t grid, hipStream_t stream);
hipError_t launch_fp8_conversion_check(unsigned long long* mismatches, hipStream_t stream);

}  // namespace pdattn
