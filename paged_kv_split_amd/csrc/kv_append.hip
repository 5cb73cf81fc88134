// KV append: new tokens' K and V rows written into the paged cache, with the
// FP8 quantise-and-scatter for e4m3fn pools (FlashQuant wiki "CUDA Kernels",
// paged_decode.cu Page Table Addressing; Atlas "CUDA Kernel Engineering",
// kernel inventory: per-token K/V write into the paged cache; OASR "Kernel
// Layer", FP8 KV variants: the quantise-and-scatter that fills the cache,
// with power-of-two scales).
//
// One wave per (token, kv head) row: lanes 0..31 carry the K row, lanes
// 32..63 the V row, D/32 elements each, so a row is one coalesced load and
// one coalesced store per half-wave. An fp8 row's absolute maximum is a
// 5-step butterfly inside its half-wave; the scale and the codes follow from
// it in fp32 with correctly rounded divisions.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace pdattn {
namespace {

constexpr float kE4m3Max = 448.0f;

template <int E>
struct Lane;  // E bf16 elements = E/2 words
template <>
struct Lane<2> {
  typedef uint32_t W;
  static constexpr int kWords = 1;
  __device__ static uint32_t word(W w, int) { return w; }
};
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <>
struct Lane<4> {
  typedef u32x2 W;
  static constexpr int kWords = 2;
  __device__ static uint32_t word(W w, int i) { return i == 0 ? w.x : w.y; }
};

// Nearest E4M3FN code of an fp32 y with |y| <= 448, ties to the even code,
// sign bit from y. The format: 1 sign bit, 4 exponent bits with bias 7 and 3
// mantissa bits; exponent field 0 holds the subnormals m * 2^-9. Below 2^-6
// the code is the integer nearest to |y| * 2^9 (a code of 8 is 2^-6, the
// smallest normal); above, the fp32 mantissa is cut to 3 bits with round to
// nearest even, a carry moving into the exponent, and the fp32 exponent bias
// 127 is re-based to 7. |y| <= 448 never reaches the NaN code 0x7F.
__device__ inline uint32_t e4m3fn_code(float y) {
  const uint32_t bits = __float_as_uint(y);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t abits = bits & 0x7FFFFFFFu;
  uint32_t mag;
  if (abits < 0x3C800000u) {  // 2^-6
    mag = (uint32_t)rintf(__uint_as_float(abits) * 512.0f);
  } else {
    const uint32_t r = abits + 0x7FFFFu + ((abits >> 20) & 1u);
    mag = (r >> 20) - (120u << 3);
  }
  return sign | mag;
}

// The smallest power of two s with 448 * s >= amax (amax > 0, finite).
// With amax = m * 2^k, m in [0.5, 1): 448 * 2^(k-9) = 0.875 * 2^k covers
// amax exactly when m <= 0.875, and 448 * 2^(k-10) never does.
__device__ inline float pow2_scale(float amax) {
  int k;
  const float m = frexpf(amax, &k);
  return ldexpf(1.0f, m <= 0.875f ? k - 9 : k - 8);
}

template <int D, bool FP8>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p) {
  constexpr int E = D / 32;
  typedef Lane<E> L;
  const int lane = threadIdx.x & 63;
  const int sub = lane & 31;
  const bool is_v = lane >= 32;
  const int64_t rows = (int64_t)p.num_tokens * p.num_kv_heads;
  const int64_t stride = (int64_t)gridDim.x * 4;
  const int64_t cap = (int64_t)p.max_pages_per_seq << p.page_log2;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += stride) {
    const int64_t tok = row / p.num_kv_heads;
    const int kvh = (int)(row - tok * p.num_kv_heads);
    const int b = p.token_seq[tok];
    const int t = p.token_pos[tok];
    if (b < 0 || b >= p.batch || t < 0 || (int64_t)t >= cap) continue;
    const int page = p.block_table[(int64_t)b * p.max_pages_per_seq + (t >> p.page_log2)];
    if (page < 0 || page >= p.num_pages) continue;
    const int64_t dst = ((((int64_t)page << p.page_log2) | (t & ((1 << p.page_log2) - 1))) * p.num_kv_heads + kvh);

    const uint16_t* src = (is_v ? p.v_new : p.k_new) + row * D + sub * E;
    const typename L::W w = __builtin_nontemporal_load(reinterpret_cast<const typename L::W*>(src));
    if constexpr (!FP8) {
      uint16_t* out = static_cast<uint16_t*>(is_v ? p.v_pages : p.k_pages) + dst * D + sub * E;
      *reinterpret_cast<typename L::W*>(out) = w;
    } else {
      float x[E];
#pragma unroll
      for (int i = 0; i < L::kWords; ++i) {
        const uint32_t u = L::word(w, i);
        x[2 * i] = __uint_as_float(u << 16);
        x[2 * i + 1] = __uint_as_float(u & 0xFFFF0000u);
      }
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < E; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
      const float s = amax == 0.0f ? 1.0f : (p.pow2_scales ? pow2_scale(amax) : amax / kE4m3Max);
      uint32_t codes = 0;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const float y = fminf(fmaxf(x[i] / s, -kE4m3Max), kE4m3Max);
        codes |= e4m3fn_code(y) << (8 * i);
      }
      uint8_t* out = static_cast<uint8_t*>(is_v ? p.v_pages : p.k_pages) + dst * D + sub * E;
      if constexpr (E == 4) {
        *reinterpret_cast<uint32_t*>(out) = codes;
      } else {
        *reinterpret_cast<uint16_t*>(out) = (uint16_t)codes;
      }
      if (sub == 0) (is_v ? p.v_scale : p.k_scale)[dst] = s;
    }
  }
}

template <int D>
hipError_t launch_d(const AppendParams& p, bool fp8, uint32_t grid, hipStream_t stream) {
  if (fp8)
    hipLaunchKernelGGL((kv_append_kernel<D, true>), dim3(grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((kv_append_kernel<D, false>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_append(const AppendParams& p, int head_dim, bool fp8, uint32_t grid, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_d<64>(p, fp8, grid, stream);
    case 128: return launch_d<128>(p, fp8, grid, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pdattn
