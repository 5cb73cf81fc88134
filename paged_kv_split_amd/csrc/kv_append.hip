// KV append: new tokens' K and V rows written into the paged cache, with the
// FP8 quantise-and-scatter for e4m3fn pools (FlashQuant wiki "CUDA Kernels",
// paged_decode.cu Page Table Addressing; Atlas "CUDA Kernel Engineering",
// kernel inventory: per-token K/V write into the paged cache; OASR "Kernel
// Layer", FP8 KV variants: the quantise-and-scatter that fills the cache,
// with power-of-two scales).
//
// One wave per new token moves that token's K and V rows for every kv head
// (each a contiguous chunk on both sides) with 16-byte lanes. An fp8 row's
// absolute maximum is a butterfly over the D/8 lanes that hold it; the scale
// and the codes follow from it in fp32 with correctly rounded divisions.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "append.h"

namespace pdattn {
namespace {

constexpr float kE4m3Max = 448.0f;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte chunks of a token's K (or V) rows one wave moves per step, per
// lane; each lane keeps kBatch chunks of K and of V in flight.
constexpr int kBatch = 2;

// Max over aligned groups of L lanes (L = 8, 16 or 32) with DPP lane moves:
// swap neighbours, swap pairs, mirror each 8-lane half, mirror each 16-lane
// row; then (L = 32) the neighbouring 16-lane row.
template <int Ctrl>
__device__ inline float dpp_move(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), Ctrl, 0xF, 0xF, false));
}

template <int L>
__device__ inline float group_max(float v) {
  v = fmaxf(v, dpp_move<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp_move<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  v = fmaxf(v, dpp_move<0x141>(v));  // row_half_mirror
  if constexpr (L >= 16) v = fmaxf(v, dpp_move<0x140>(v));  // row_mirror
  if constexpr (L == 32) v = fmaxf(v, __shfl_xor(v, 16));     // the neighbouring row
  return v;
}

// Quantise one lane's 8 bf16 values (a 16-byte chunk of one row; the D/8
// lanes of a row are an aligned lane group). Returns the 8 codes and the
// row's scale. The quotients y = x / s are the correctly rounded fp32
// quotients wherever they can decide a code:
//   * power-of-two s = 2^e: y = x * 2^-e, exact (or rounded below 2^-126,
//     where every y gives a zero code);
//   * s = absmax / 448 with absmax >= 2^-82: r = 1/s once per row, then
//     q = x * r refined by the residual x - q * s (Markstein's correction
//     with fused multiply-adds). For every pair of bf16 values x and absmax
//     >= |x| in this range this equals the correctly rounded quotient
//     whenever |x / s| >= 2^-11, and stays <= 2^-10 (a zero code) below;
//   * smaller absmax: the correctly rounded division itself.
// Every y carries the sign of x (s > 0), also where it is zero, and is
// clamped to [-448, 448] (a plain s rounded down can put |x / s| a hair above
// 448; a power-of-two s cannot).
template <int D>
__device__ inline u32x2 quantise_chunk(u32x4 w, bool pow2, float* scale_out) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = group_max<D / 8>(amax);
  float y[8];
  float s;
  if (amax == 0.0f) {
    s = 1.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = x[i];  // +-0
  } else if (pow2) {
    // the smallest e with 448 * 2^e >= amax: with amax = m * 2^k, m in
    // [0.5, 1), 448 * 2^(k-9) = 0.875 * 2^k covers amax exactly when
    // m <= 0.875, and 448 * 2^(k-10) never does
    int k;
    const float m = frexpf(amax, &k);
    const int e = m <= 0.875f ? k - 9 : k - 8;
    s = ldexpf(1.0f, e);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = ldexpf(x[i], -e);
  } else {
    s = amax / kE4m3Max;
    if (amax >= 0x1p-82f) {
      const float r = 1.0f / s;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float q = __fmul_rn(x[i], r);
        const float a = fminf(fabsf(__builtin_fmaf(__builtin_fmaf(-q, s, x[i]), r, q)), kE4m3Max);
        y[i] = __uint_as_float(__float_as_uint(a) | (__float_as_uint(x[i]) & 0x80000000u));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = fminf(fmaxf(x[i] / s, -kE4m3Max), kE4m3Max);
    }
  }
  *scale_out = s;
  // the hardware conversion rounds to the nearest code, ties to even, and
  // takes the sign of its operand (checked against the format definition
  // for every fp32 magnitude <= 448 by the conversion check below)
  u32x2 r;
  r.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  r.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], (int)r.x, true);
  r.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  r.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], (int)r.y, true);
  return r;
}

// One wave per new token. The token's K rows for all kv heads are one
// contiguous chunk of Hkv * D bf16 values in k_new, and so are its V rows: a
// step moves 1 KB of each with 16-byte lanes into the token's rows (adjacent
// in an NHD pool, P rows apart in an HND pool), and the first loads are
// issued before the token's slot is resolved, so the block-table round
// trip overlaps them.
template <int D, bool FP8>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p) {
  const int lane = threadIdx.x & 63;
  const int chunk = p.num_kv_heads * D * 2;  // bytes of one token's K (or V) rows, a multiple of 128
  const int steps = (chunk + 1023) >> 10;
  const int64_t cap = (int64_t)p.max_pages_per_seq << p.page_log2;
  const int first = __builtin_amdgcn_readfirstlane((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6));
  for (int64_t tok = first; tok < p.num_tokens; tok += (int64_t)gridDim.x * 4) {
    const int b = p.token_seq[tok];
    const int t = p.token_pos[tok];
    const unsigned char* ksrc = reinterpret_cast<const unsigned char*>(p.k_new) + tok * chunk;
    const unsigned char* vsrc = reinterpret_cast<const unsigned char*>(p.v_new) + tok * chunk;
    u32x4 kx[kBatch], vx[kBatch];
    // every lane loads (lanes past the chunk re-read its last 16 bytes and
    // store nothing), so the loads need no branch and issue at once
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int o = min(u * 1024 + lane * 16, chunk - 16);
      kx[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ksrc + o));
      vx[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vsrc + o));
    }
    // the slot, without a branch: an unresolved token reads block-table
    // entry 0 and is dropped below
    bool ok = b >= 0 && b < p.batch && t >= 0 && (int64_t)t < cap;
    const int page = p.block_table[ok ? (int64_t)b * p.max_pages_per_seq + (t >> p.page_log2) : 0];
    ok = ok && page >= 0 && page < p.num_pages;
    if (!ok) {
      // an empty use of the loaded chunks on this path keeps their loads
      // ahead of the branch instead of sunk below it
#pragma unroll
      for (int u = 0; u < kBatch; ++u) asm volatile("" ::"v"(kx[u]), "v"(vx[u]));
      continue;
    }
    // the token's row for kv head h: base + h * head_stride
    const int64_t base = ((int64_t)page << p.page_log2) * p.num_kv_heads +
                         (int64_t)(t & ((1 << p.page_log2) - 1)) * p.slot_stride;
    unsigned char* kpool = static_cast<unsigned char*>(p.k_pages);
    unsigned char* vpool = static_cast<unsigned char*>(p.v_pages);
    for (int j0 = 0; j0 < steps; j0 += kBatch) {
      if (j0 > 0) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int o = min((j0 + u) * 1024 + lane * 16, chunk - 16);
          kx[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ksrc + o));
          vx[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vsrc + o));
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int o = (j0 + u) * 1024 + lane * 16;
        // a 16-byte lane chunk lies inside one row: kv head o / (2 D)
        const int64_t r = base + (int64_t)(o / (2 * D)) * p.head_stride;
        const int within = o & (2 * D - 1);
        if constexpr (!FP8) {
          if (o < chunk) {
            *reinterpret_cast<u32x4*>(kpool + r * (2 * D) + within) = kx[u];
            *reinterpret_cast<u32x4*>(vpool + r * (2 * D) + within) = vx[u];
          }
        } else {
          // whole rows are in or out of range together, so every lane of a
          // row takes part in its reduction; lanes past the chunk reduce
          // zeros among themselves and store nothing
          const bool in = o < chunk;
          float ks, vs;
          const u32x2 kc = quantise_chunk<D>(in ? kx[u] : u32x4{0, 0, 0, 0}, p.pow2_scales, &ks);
          const u32x2 vc = quantise_chunk<D>(in ? vx[u] : u32x4{0, 0, 0, 0}, p.pow2_scales, &vs);
          if (in && p.inline_scales) {
            // rows D + 4 bytes apart are 4-byte aligned: dword stores; the
            // row's first lane also writes its scale after the codes
            unsigned char* kr = kpool + r * (D + 4);
            unsigned char* vr = vpool + r * (D + 4);
            reinterpret_cast<uint32_t*>(kr + within / 2)[0] = kc.x;
            reinterpret_cast<uint32_t*>(kr + within / 2)[1] = kc.y;
            reinterpret_cast<uint32_t*>(vr + within / 2)[0] = vc.x;
            reinterpret_cast<uint32_t*>(vr + within / 2)[1] = vc.y;
            if ((lane & (D / 8 - 1)) == 0) {
              *reinterpret_cast<float*>(kr + D) = ks;
              *reinterpret_cast<float*>(vr + D) = vs;
            }
          } else if (in) {
            *reinterpret_cast<u32x2*>(kpool + r * D + within / 2) = kc;
            *reinterpret_cast<u32x2*>(vpool + r * D + within / 2) = vc;
            if ((lane & (D / 8 - 1)) == 0) {
              p.k_scale[r] = ks;
              p.v_scale[r] = vs;
            }
          }
        }
      }
    }
  }
}

// The format definition of the E4M3FN code of |y| <= 448 (1 sign bit, 4
// exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
// subnormals m * 2^-9), written out in integer steps: below 2^-6 the code is
// the integer nearest to |y| * 2^9, ties to even (a code of 8 is 2^-6, the
// smallest normal); above, the fp32 mantissa is cut to 3 bits with round to
// nearest even, a carry moving into the exponent, and the exponent bias 127
// re-based to 7.
__device__ inline uint32_t e4m3fn_code_by_definition(float y) {
  const uint32_t b = __float_as_uint(y);
  const uint32_t a = b & 0x7FFFFFFFu;
  uint32_t m;
  if (a < 0x3C800000u) {  // 2^-6
    m = (uint32_t)rintf(__uint_as_float(a) * 512.0f);
  } else {
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    m = (r >> 20) - (120u << 3);
  }
  return ((b >> 24) & 0x80u) | m;
}

// Every fp32 bit pattern with |y| <= 448, both signs, through the hardware
// conversion and through the definition; mismatches are counted.
__global__ __launch_bounds__(256) void fp8_conversion_check_kernel(unsigned long long* mismatches) {
  constexpr uint64_t kLim = 0x43E00001ull;  // bit patterns 0 .. 448
  const uint64_t n = (uint64_t)gridDim.x * 256;
  unsigned long long c = 0;
  for (uint64_t u = (uint64_t)blockIdx.x * 256 + threadIdx.x; u < 2 * kLim; u += n) {
    const uint32_t b = u < kLim ? (uint32_t)u : (0x80000000u | (uint32_t)(u - kLim));
    const float y = __uint_as_float(b);
    const uint32_t hw = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, -y, 0, false);
    const uint32_t want = e4m3fn_code_by_definition(y) | (e4m3fn_code_by_definition(-y) << 8);
    c += (hw & 0xFFFFu) != want;
  }
  if (c) atomicAdd(mismatches, c);
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

hipError_t launch_fp8_conversion_check(unsigned long long* mismatches, hipStream_t stream) {
  hipLaunchKernelGGL(fp8_conversion_check_kernel, dim3(4096), dim3(256), 0, stream, mismatches);
  return hipGetLastError();
}

hipError_t launch_kv_append(const AppendParams& p, int head_dim, bool fp8, uint32_t grid, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_d<64>(p, fp8, grid, stream);
    case 128: return launch_d<128>(p, fp8, grid, stream);
    case 256: return launch_d<256>(p, fp8, grid, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pdattn
