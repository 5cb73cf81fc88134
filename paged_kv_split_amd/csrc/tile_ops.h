// Device building blocks shared by the gfx950 decode kernels: the direct-to-
// LDS tile loads, the per-tile q.K / online-softmax / p.V step on one wave,
// and the partial-record layout. Internal; included by the kernel sources.
//
// One tile is 16 consecutive tokens of one (sequence, kv head) pair. A wave
// computes all G query heads of the kv head at once (AstrAI "CUDA Kernels",
// GQA head packing; FlashQuant wiki "CUDA Kernels", GQA Support):
//   * S = K_tile (16 tokens x d) . Q^T (d x 16, the G heads zero-padded) on
//     v_mfma_f32_16x16x32_bf16. The K tile lands in LDS already in A-operand
//     lane order; the head_dim order inside a fragment is the same for Q and
//     K, so the contraction is exact.
//   * online softmax (FlashQuant wiki, flash_attention.cu, Online Softmax) in
//     base 2 with the scale pre-multiplied by log2(e) (same page, utils.cuh):
//     lane (row r, column g) holds head g for tokens r, r+4, r+8, r+12; the
//     tile max comes from a local max and two cross-row exchanges.
//   * p . V on the matrix cores (v_mfma_f32_16x16x32_bf16, fp32
//     accumulation), for any group size: the G columns (padded to 16) x 16
//     tokens x d product. Its operands need no data movement: the k index of
//     the product is chosen so that k <-> token r + 4 j, which is where lane
//     (r, c) already holds column c's weights (A operand) and its V chunk
//     rows (B operand, V element e of the lane's chunk: n = c stands for
//     d = c VE + e). Each weight enters as two bf16 terms (hi and the
//     bf16 of its remainder), so the product carries it to 2^-18 relative;
//     the normaliser l and lse stay fp32. (On the VALU this product costs
//     G x d/16 x 4 FMAs per lane per tile, which lengthened every tile
//     step.)
//   * the running maximum moves lazily (by more than kRescaleSlack, base
//     2), so the accumulators are rescaled only when a score jumps.
// fp8 pools: e4m3fn bytes widen exactly in registers (to bf16 for both MFMA
// operands) and the per-(token, kv head) scales multiply the score (k) and
// the weight (v) (OASR "Kernel Layer", FP8 KV variants).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "kernels.h"

namespace pdattn {
namespace dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994530942f;

// Base-2 headroom of the lazily raised running maximum (weights < 2^8).
constexpr float kRescaleSlack = 8.0f;

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Eight e4m3fn bytes (w0 holds bytes 0..3, w1 bytes 4..7, memory order) as
// eight bf16 values in the same order, by gfx950's fp8 -> bf16 pair convert
// with unit scale. The widening is exact: an e4m3 value has 4 significant
// bits and an exponent inside bf16's range.
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  return r;
}

template <int VB>
struct VChunk;
template <>
struct VChunk<32> { using type = u32x8; };
template <>
struct VChunk<16> { using type = u32x4; };
template <>
struct VChunk<8> { using type = u32x2; };
template <>
struct VChunk<4> { using type = uint32_t; };

// Dword w of a V chunk.
template <typename T>
__device__ __forceinline__ uint32_t dword(const T& x, int w) {
  if constexpr (std::is_same_v<T, uint32_t>) {
    return x;
  } else {
    return x[w];
  }
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8), followed by a
// compiler barrier so that no LDS access is moved across it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(n) for a wave-uniform n (clamped to 63: waiting for fewer
// outstanding operations than allowed is always safe), by a binary dispatch
// over the immediate forms.
template <int LO = 0, int HI = 63>
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  if constexpr (LO == HI) {
    wait_vmcnt<LO>();
  } else {
    constexpr int MID = (LO + HI + 1) / 2;
    if (n >= MID) wait_vmcnt_le<MID, HI>(n);
    else wait_vmcnt_le<LO, MID - 1>(n);
  }
}

// Wait until at most `ahead` tiles of C loads each are still in flight (the
// loads of a wave return in issue order).
template <int C, int S>
__device__ __forceinline__ void wait_tiles(int ahead) {
  if constexpr (S >= 4) {
    if (ahead >= 3) { wait_vmcnt<3 * C>(); return; }
  }
  if constexpr (S >= 3) {
    if (ahead >= 2) { wait_vmcnt<2 * C>(); return; }
  }
  if (ahead >= 1) { wait_vmcnt<C>(); return; }
  wait_vmcnt<0>();
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Cache policy of the K/V stream: non-temporal. Each KV byte is read once
// per call, so it is not kept in L2 or the Infinity Cache; on MI355X this
// lifts a streaming read from about 4.7 to about 6.9 TB/s.
constexpr int kStreamPolicy = 2;  // nt

// Direct-to-LDS loads: lane i's `bytes` bytes from g land at lds + i * bytes
// (lds is the wave-uniform base).
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds, 16, 0, kStreamPolicy);
}
__device__ __forceinline__ void dma4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds, 4, 0, kStreamPolicy);
}
// Same, cached (small metadata reused by many waves: block-table windows).
__device__ __forceinline__ void dma4_cached(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds, 4, 0, 0);
}

// LDS byte address of a generic pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Read one ring stage into registers: the lane's K fragments (kf), its four
// V chunks (V rows row + 4 j; vp points at row `row`) and, for fp8, the k / v
// scales of its four tokens. One inline-assembly block issues the reads and
// waits for them (lgkmcnt(0)), so every destination is defined only once
// its data has landed and no use or copy can be scheduled earlier; the
// compiler also adds no wait of its own for the ring's direct-to-LDS loads
// (the caller has waited for them).
template <int D, bool FP8, typename VVec, int K_LD>
__device__ __forceinline__ void read_stage(const unsigned char* kp, const unsigned char* vp, const unsigned char* sp,
                                           u32x4 (&kf)[K_LD], VVec (&vf)[4], float (&ks)[4], float (&vs)[4]) {
  const uint32_t ka = lds_addr(kp), va = lds_addr(vp), sa = lds_addr(sp);
  if constexpr (!FP8 && D == 128) {  // row 256 B: 4 K fragments, V rows 1024 B apart
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:1024\n\t"
        "ds_read_b128 %2, %8 offset:2048\n\t"
        "ds_read_b128 %3, %8 offset:3072\n\t"
        "ds_read_b128 %4, %9\n\t"
        "ds_read_b128 %5, %9 offset:1024\n\t"
        "ds_read_b128 %6, %9 offset:2048\n\t"
        "ds_read_b128 %7, %9 offset:3072\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(kf[0]), "=&v"(kf[1]), "=&v"(kf[2]), "=&v"(kf[3]), "=&v"(vf[0]), "=&v"(vf[1]), "=&v"(vf[2]),
          "=&v"(vf[3])
        : "v"(ka), "v"(va)
        : "memory");
  } else if constexpr (!FP8 && D == 256) {  // row 512 B: 8 K fragments, 32-byte V chunks 2048 B apart
    u32x4 h[8];
    asm volatile(
        "ds_read_b128 %0, %16\n\t"
        "ds_read_b128 %1, %16 offset:1024\n\t"
        "ds_read_b128 %2, %16 offset:2048\n\t"
        "ds_read_b128 %3, %16 offset:3072\n\t"
        "ds_read_b128 %4, %16 offset:4096\n\t"
        "ds_read_b128 %5, %16 offset:5120\n\t"
        "ds_read_b128 %6, %16 offset:6144\n\t"
        "ds_read_b128 %7, %16 offset:7168\n\t"
        "ds_read_b128 %8, %17\n\t"
        "ds_read_b128 %9, %17 offset:16\n\t"
        "ds_read_b128 %10, %17 offset:2048\n\t"
        "ds_read_b128 %11, %17 offset:2064\n\t"
        "ds_read_b128 %12, %17 offset:4096\n\t"
        "ds_read_b128 %13, %17 offset:4112\n\t"
        "ds_read_b128 %14, %17 offset:6144\n\t"
        "ds_read_b128 %15, %17 offset:6160\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(kf[0]), "=&v"(kf[1]), "=&v"(kf[2]), "=&v"(kf[3]), "=&v"(kf[4]), "=&v"(kf[5]), "=&v"(kf[6]),
          "=&v"(kf[7]), "=&v"(h[0]), "=&v"(h[1]), "=&v"(h[2]), "=&v"(h[3]), "=&v"(h[4]), "=&v"(h[5]), "=&v"(h[6]),
          "=&v"(h[7])
        : "v"(ka), "v"(va)
        : "memory");
#pragma unroll
    for (int j = 0; j < 4; ++j) vf[j] = __builtin_shufflevector(h[2 * j], h[2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
  } else if constexpr (FP8 && D == 256) {  // row 256 B: 4 K fragments, 16-byte V chunks 1024 B apart, scales
    f32x4 a, c;
    asm volatile(
        "ds_read_b128 %0, %10\n\t"
        "ds_read_b128 %1, %10 offset:1024\n\t"
        "ds_read_b128 %2, %10 offset:2048\n\t"
        "ds_read_b128 %3, %10 offset:3072\n\t"
        "ds_read_b128 %4, %11\n\t"
        "ds_read_b128 %5, %11 offset:1024\n\t"
        "ds_read_b128 %6, %11 offset:2048\n\t"
        "ds_read_b128 %7, %11 offset:3072\n\t"
        "ds_read_b128 %8, %12\n\t"
        "ds_read_b128 %9, %12 offset:64\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(kf[0]), "=&v"(kf[1]), "=&v"(kf[2]), "=&v"(kf[3]), "=&v"(vf[0]), "=&v"(vf[1]), "=&v"(vf[2]),
          "=&v"(vf[3]), "=&v"(a), "=&v"(c)
        : "v"(ka), "v"(va), "v"(sa)
        : "memory");
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      ks[v] = a[v];
      vs[v] = c[v];
    }
  } else if constexpr (!FP8 && D == 64) {  // row 128 B: 2 K fragments, 8-byte V chunks 512 B apart
    asm volatile(
        "ds_read_b128 %0, %6\n\t"
        "ds_read_b128 %1, %6 offset:1024\n\t"
        "ds_read_b64 %2, %7\n\t"
        "ds_read_b64 %3, %7 offset:512\n\t"
        "ds_read_b64 %4, %7 offset:1024\n\t"
        "ds_read_b64 %5, %7 offset:1536\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(kf[0]), "=&v"(kf[1]), "=&v"(vf[0]), "=&v"(vf[1]), "=&v"(vf[2]), "=&v"(vf[3])
        : "v"(ka), "v"(va)
        : "memory");
  } else if constexpr (FP8 && D == 128) {  // row 128 B, plus two scale quads
    f32x4 a, c;
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:1024\n\t"
        "ds_read_b64 %2, %9\n\t"
        "ds_read_b64 %3, %9 offset:512\n\t"
        "ds_read_b64 %4, %9 offset:1024\n\t"
        "ds_read_b64 %5, %9 offset:1536\n\t"
        "ds_read_b128 %6, %10\n\t"
        "ds_read_b128 %7, %10 offset:64\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(kf[0]), "=&v"(kf[1]), "=&v"(vf[0]), "=&v"(vf[1]), "=&v"(vf[2]), "=&v"(vf[3]), "=&v"(a), "=&v"(c)
        : "v"(ka), "v"(va), "v"(sa)
        : "memory");
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      ks[v] = a[v];
      vs[v] = c[v];
    }
  } else {  // fp8, D == 64: row 64 B: 1 K fragment, 4-byte V chunks 256 B apart
    static_assert(FP8 && D == 64, "layout");
    f32x4 a, c;
    asm volatile(
        "ds_read_b128 %0, %7\n\t"
        "ds_read_b32 %1, %8\n\t"
        "ds_read_b32 %2, %8 offset:256\n\t"
        "ds_read_b32 %3, %8 offset:512\n\t"
        "ds_read_b32 %4, %8 offset:768\n\t"
        "ds_read_b128 %5, %9\n\t"
        "ds_read_b128 %6, %9 offset:64\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(kf[0]), "=&v"(vf[0]), "=&v"(vf[1]), "=&v"(vf[2]), "=&v"(vf[3]), "=&v"(a), "=&v"(c)
        : "v"(ka), "v"(va), "v"(sa)
        : "memory");
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      ks[v] = a[v];
      vs[v] = c[v];
    }
  }
}

// 4-byte LDS reads at immediate offsets from one address and the wait for
// them, in one asm block (as read_stage: no destination is touched before
// its data lands, and no wait is added for the ring's direct-to-LDS loads).
template <int... O>
__device__ __forceinline__ void lds_b32(uint32_t (&r)[sizeof...(O)], uint32_t a) {
  constexpr int o[] = {O...};
  constexpr int N = sizeof...(O);
  if constexpr (N == 4) {
    asm volatile(
        "ds_read_b32 %0, %4 offset:%5\n\t"
        "ds_read_b32 %1, %4 offset:%6\n\t"
        "ds_read_b32 %2, %4 offset:%7\n\t"
        "ds_read_b32 %3, %4 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(a), "i"(o[0]), "i"(o[1]), "i"(o[2]), "i"(o[3])
        : "memory");
  } else {
    static_assert(N == 8, "read count");
    asm volatile(
        "ds_read_b32 %0, %8 offset:%9\n\t"
        "ds_read_b32 %1, %8 offset:%10\n\t"
        "ds_read_b32 %2, %8 offset:%11\n\t"
        "ds_read_b32 %3, %8 offset:%12\n\t"
        "ds_read_b32 %4, %8 offset:%13\n\t"
        "ds_read_b32 %5, %8 offset:%14\n\t"
        "ds_read_b32 %6, %8 offset:%15\n\t"
        "ds_read_b32 %7, %8 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(a), "i"(o[0]), "i"(o[1]), "i"(o[2]), "i"(o[3]), "i"(o[4]), "i"(o[5]), "i"(o[6]), "i"(o[7])
        : "memory");
  }
}

// Reads dwords FIRST .. FIRST + N - 1 of a list whose dword i sits at byte
// 4 * (i mod W) + STRIDE * (i / W) from the base (W dwords per group).
template <int W, int STRIDE, int FIRST, size_t... I>
__device__ __forceinline__ void lds_b32_groups(uint32_t (&r)[sizeof...(I)], uint32_t a, std::index_sequence<I...>) {
  lds_b32<(int)(4 * ((FIRST + I) % W) + STRIDE * ((FIRST + I) / W))...>(r, a);
}

// 16-byte LDS reads at immediate offsets from one address, and the wait for
// them, in one asm block (as read_stage).
template <int... O>
__device__ __forceinline__ void lds_b128(u32x4 (&r)[sizeof...(O)], uint32_t a) {
  constexpr int o[] = {O...};
  constexpr int N = sizeof...(O);
  if constexpr (N == 2) {
    asm volatile(
        "ds_read_b128 %0, %2 offset:%3\n\t"
        "ds_read_b128 %1, %2 offset:%4\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1])
        : "v"(a), "i"(o[0]), "i"(o[1])
        : "memory");
  } else if constexpr (N == 4) {
    asm volatile(
        "ds_read_b128 %0, %4 offset:%5\n\t"
        "ds_read_b128 %1, %4 offset:%6\n\t"
        "ds_read_b128 %2, %4 offset:%7\n\t"
        "ds_read_b128 %3, %4 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(a), "i"(o[0]), "i"(o[1]), "i"(o[2]), "i"(o[3])
        : "memory");
  } else {
    static_assert(N == 8, "read count");
    asm volatile(
        "ds_read_b128 %0, %8 offset:%9\n\t"
        "ds_read_b128 %1, %8 offset:%10\n\t"
        "ds_read_b128 %2, %8 offset:%11\n\t"
        "ds_read_b128 %3, %8 offset:%12\n\t"
        "ds_read_b128 %4, %8 offset:%13\n\t"
        "ds_read_b128 %5, %8 offset:%14\n\t"
        "ds_read_b128 %6, %8 offset:%15\n\t"
        "ds_read_b128 %7, %8 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(a), "i"(o[0]), "i"(o[1]), "i"(o[2]), "i"(o[3]), "i"(o[4]), "i"(o[5]), "i"(o[6]), "i"(o[7])
        : "memory");
  }
}

// One dword of LDS at a wave-uniform address, read in an asm block that also
// waits for it, returned as a wave-uniform value.
__device__ __forceinline__ int lds_uniform_i32(const void* p) {
  int r;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(lds_addr(p)) : "memory");
  return __builtin_amdgcn_readfirstlane(r);
}

// Token order inside a 16-token tile. MFMA A-row m carries token
// tile_token(m) = m / 4 + 4 (m mod 4), so the result row 4 r + v held by
// 16-lane row r is token r + 4 v: every 16-lane row owns the tokens
// congruent to r mod 4, for the scores as well as for the V rows it reads.
__device__ __forceinline__ int tile_token(int m) { return (m >> 2) + 4 * (m & 3); }

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ long long wave_incl_scan(long long v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ long long uniform64(long long x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(x & 0xffffffffll));
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((unsigned long long)x >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// The per-wave tile machinery for head_dim D, group size G and pool type.
// INL (fp8 only) != 0: each pool row holds its D codes and then its fp32
// scale (DeepGEMM documentation 6.1, the paged cache with the scale fused
// per token), D + 4 bytes, so rows are only 4-byte aligned.
//   INL 1 (any row order): the tile is fetched with 4-byte direct-to-LDS
//     loads into the same LDS image as the 16-byte loads of separate-scale
//     pools build; everything after the loads is shared.
//   INL 2 (head-major pools, rows [page][kv head][slot]): the tile's 16 rows
//     are one contiguous 16-byte-aligned block (two of 8 rows when P = 8),
//     fetched with 16-byte loads as raw rows; the operands are read back
//     with 4-byte LDS reads at the rows' offsets into the same registers.
template <int D, int G, bool FP8, int INL = 0>
struct Tile {
  static_assert(INL == 0 || FP8, "inline scales are an fp8 layout");
  static constexpr int ESZ = FP8 ? 1 : 2;             // bytes per stored element
  static constexpr int ROW_BYTES = D * ESZ;           // one (token, kv head) row's values
  static constexpr int PITCH = ROW_BYTES + (INL ? 4 : 0);  // pool bytes per row
  static constexpr int KSTEPS = D / 32;               // MFMA k-steps over head_dim
  static constexpr int K_LD = ROW_BYTES / 64;         // 16-byte loads per lane per tile, K
  static constexpr int V_LD = ROW_BYTES / 64;         // and V (a tile is 16 rows)
  static constexpr int BLK = kTileTokens * PITCH;     // INL 2: bytes of a tile's raw rows
  static constexpr int BLK_LD = (BLK / 16 + 63) / 64; // INL 2: 16-byte loads per lane per block
  // direct-to-LDS loads per tile: each 16-byte load is four 4-byte ones
  // with INL 1; INL 2 loads the two raw blocks (scales inside)
  static constexpr int C = INL == 2 ? 2 * BLK_LD : (INL ? 4 : 1) * (K_LD + V_LD) + (FP8 ? 1 : 0);
  static constexpr int VE = D / 16;                   // V elements per lane per row
  static constexpr int VB = VE * ESZ;                 // V bytes per lane per row
  // one ring stage: K tile in MFMA-operand lane order, V tile row-major,
  // then (fp8) 64 scale slots: k scales 0..15, v scales 16..31
  static constexpr int K_TILE = INL == 2 ? BLK : kTileTokens * ROW_BYTES;
  static constexpr int V_TILE = K_TILE;
  static constexpr int STAGE = K_TILE + V_TILE + (FP8 && INL != 2 ? 256 : 0);
  static_assert(BLK % 16 == 0, "raw blocks are 16-byte multiples");
  static constexpr int RF = (int)record_floats(D, G);
  static constexpr int EPL = G * D / 64;  // accumulator elements per lane in the merge layout
  using VVec = typename VChunk<VB>::type;
  // buffer stores of one finished pair (out and lse) and of one record
  // (acc, then m and l): a fixed count, whatever the lanes that write
  static constexpr int N_OUT_STORES = VE + 1;
  static constexpr int N_REC_STORES = VE + 2;
  static_assert(K_LD >= 1 && (D == 64 || D == 128 || D == 256), "head_dim");
  static_assert(G >= 1 && G <= 16, "group size");
  static_assert(EPL >= 1 && D % EPL == 0, "merge lane slice");

  // Online-softmax state of one piece: running max m (base 2) and sum l of
  // column `col` (every row holds the same after reduce_rows), and
  // cacc[e][v]: column 4 row + v at d = col * VE + e, summed over all tokens
  // of the piece by the matrix cores.
  struct State {
    float m, l;
    f32x4 cacc[VE];
  };
  // One stage read back into registers.
  struct Frag {
    u32x4 kf[K_LD];
    VVec vf[4];
    float ks[4], vs[4];
  };

  __device__ static void reset(State& s) {
    s.m = -__builtin_inff();
    s.l = 0.0f;
#pragma unroll
    for (int e = 0; e < VE; ++e) s.cacc[e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // Value of x in lane (row, 4 row + v): column 4 row + v's copy of a
  // per-column quantity (m, l, alpha: every row holds the same).
  __device__ static float col_of_row(float x, int row, int v) { return __shfl(x, 20 * row + v); }

  // The MFMA B operands of the lane's four V chunk rows (rows row + 4 j):
  // operand e holds element e of each, as bf16 (fp8 codes widen exactly).
  // Two source dwords are interleaved by one byte permute (v_perm_b32:
  // selector bytes 0-3 pick bytes of the second source, 4-7 of the first).
  __device__ static void v_operands(const Frag& f, bf16x4 (&b)[VE]) {
    if constexpr (FP8) {
      // elements e, e + 1 (e even) sit in bytes e & 3, (e & 3) + 1 of dword
      // e / 4; one permute gathers them from two rows, then two converts
      // widen the low and the high byte pairs
#pragma unroll
      for (int e = 0; e < VE; e += 2) {
        const uint32_t x = e & 3;
        const uint32_t sel = x | ((4 + x) << 8) | ((x + 1) << 16) | ((5 + x) << 24);
        const uint32_t a01 = __builtin_amdgcn_perm(dword(f.vf[1], e >> 2), dword(f.vf[0], e >> 2), sel);
        const uint32_t a23 = __builtin_amdgcn_perm(dword(f.vf[3], e >> 2), dword(f.vf[2], e >> 2), sel);
        const uint32_t l0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a01, 1.0f, false));
        const uint32_t l1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a23, 1.0f, false));
        const uint32_t h0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a01, 1.0f, true));
        const uint32_t h1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a23, 1.0f, true));
        b[e] = __builtin_bit_cast(bf16x4, u32x2{l0, l1});
        b[e + 1] = __builtin_bit_cast(bf16x4, u32x2{h0, h1});
      }
    } else {
      // element e is the low (e even) or high half of dword e / 2
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t lo = __builtin_amdgcn_perm(dword(f.vf[1], e >> 1), dword(f.vf[0], e >> 1), sel);
        const uint32_t hi = __builtin_amdgcn_perm(dword(f.vf[3], e >> 1), dword(f.vf[2], e >> 1), sel);
        b[e] = __builtin_bit_cast(bf16x4, u32x2{lo, hi});
      }
    }
  }

  // head_dim position of element 0 of lane (row, ·)'s fragment at k-step kk;
  // the K fragments follow the same order
  __device__ static int dpos(int kk, int row) {
    if constexpr (FP8) return (kk >> 1) * 64 + row * 16 + (kk & 1) * 8;
    else return kk * 32 + row * 8;
  }

  // Q as the MFMA B operand: lane (row, col) holds column col's query row
  // (zero for col >= ncols: padding columns) at 8 head_dim positions per
  // k-step. qrow points at that column's query row (any valid row for a
  // padding column).
  __device__ static void load_q(bf16x8 (&qop)[KSTEPS], const uint16_t* qrow, int row, int col, int ncols) {
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      u32x4 raw = *reinterpret_cast<const u32x4*>(qrow + dpos(kk, row));
      if (col >= ncols) raw = u32x4{0u, 0u, 0u, 0u};
      qop[kk] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // Issue the C direct-to-LDS loads of the tile starting at token tb of one
  // pair into stage st. row_of(pos) gives the (token, kv head) row index of
  // sequence position pos; rows past `last` (the pair's last token) are
  // clamped onto it (finite data, masked in the softmax).
  template <typename RowOf>
  __device__ static void issue(unsigned char* st, const uint8_t* k, const uint8_t* v, const float* k_scale,
                               const float* v_scale, RowOf&& row_of, int tb, int last, int lane, int row,
                               int col) {
    if constexpr (INL == 2) {
      // raw rows: byte x of the tile's block is byte x mod (8 PITCH) of the
      // 8-row run starting at row ra (x < 8 PITCH) or rb; with P >= 16 the
      // 16 rows are one run (rb = ra + 8). Rows past `last` are read as they
      // are (inside an allocated page) and never used: their scores are
      // masked and read() zeroes their V values and v scales.
      const long long ra = row_of(tb);
      const long long rb = tb + 8 <= last ? row_of(tb + 8) : ra;
#pragma unroll
      for (int i = 0; i < BLK_LD; ++i) {
        const int x = (i * 64 + lane) * 16;
        if (i < BLK_LD - 1 || x < BLK) {
          const long long off = x < 8 * PITCH ? ra * PITCH + x : rb * PITCH + (x - 8 * PITCH);
          dma16(k + off, st + i * 1024);
          dma16(v + off, st + K_TILE + i * 1024);
        }
      }
      return;
    } else if constexpr (INL == 1) {
      // Same LDS image from 4-byte loads: load (jj, q) fills bytes
      // [jj * 1024 + q * 256, +256), lane i the dword at + 4 i.
      // K: that dword is dword i mod 4 of the 16-byte fragment of MFMA lane
      // 16 q + i / 4, i.e. row q, column i / 4: token tile_token(i / 4),
      // bytes 64 jj + 16 q + 4 (i mod 4) of its row
      {
        const int pos = min(tb + tile_token(lane >> 2), last);
        const unsigned char* src = k + row_of(pos) * PITCH + 4 * (lane & 3);
#pragma unroll
        for (int jj = 0; jj < K_LD; ++jj)
#pragma unroll
          for (int q = 0; q < 4; ++q) dma4(src + jj * 64 + q * 16, st + jj * 1024 + q * 256);
      }
      // V: row-major, the dword at byte b of the tile is byte b mod ROW of
      // token b / ROW
#pragma unroll
      for (int jj = 0; jj < V_LD; ++jj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int byte = jj * 1024 + q * 256 + lane * 4;
          const int pos = min(tb + byte / ROW_BYTES, last);
          dma4(v + row_of(pos) * PITCH + (byte % ROW_BYTES), st + K_TILE + jj * 1024 + q * 256);
        }
      // scales: slot m < 16 the k scale of token tile_token(m), 16 + m its
      // v scale (the dword after the row's codes); lanes 32..63 repeat
      {
        const int m = lane & 15;
        const int pos = min(tb + tile_token(m), last);
        dma4(((lane & 16) ? v : k) + row_of(pos) * PITCH + ROW_BYTES, st + K_TILE + V_TILE);
      }
      return;
    }
    {
      // K: lane (row, col) fetches bytes [j*64 + row*16, +16) of token
      // tile_token(col); it lands at j*1024 + lane*16, the lane's own
      // A-operand fragment for k-steps 2j, 2j+1 (fp8) or j (bf16).
      const int pos = min(tb + tile_token(col), last);
      const unsigned char* src = k + row_of(pos) * ROW_BYTES + row * 16;
#pragma unroll
      for (int jj = 0; jj < K_LD; ++jj) dma16(src + jj * 64, st + jj * 1024);
    }
#pragma unroll
    for (int jj = 0; jj < V_LD; ++jj) {
      // V: row-major tile, 64 lanes x 16 bytes per load
      const int byte = jj * 1024 + lane * 16;
      const int pos = min(tb + byte / ROW_BYTES, last);
      dma16(v + row_of(pos) * ROW_BYTES + (byte % ROW_BYTES), st + K_TILE + jj * 1024);
    }
    if constexpr (FP8) {
      // scale slot m < 16 holds k_scale of token tile_token(m); slot 16 + m
      // holds its v_scale; lanes 32..63 repeat lanes 0..31
      const int m = lane & 15;
      const int pos = min(tb + tile_token(m), last);
      const float* src = ((lane & 16) ? v_scale : k_scale) + row_of(pos);
      dma4(src, st + K_TILE + V_TILE);
    }
  }

  // Issue for a tile whose 16 rows lie in one page and all belong to the
  // piece: row0 (wave-uniform) is the row index of its first token, and
  // consecutive tokens are slot_stride rows apart. The same LDS image as
  // issue(), from one scalar base plus per-lane offsets that do not change
  // from tile to tile.
  __device__ static void issue_rows(unsigned char* st, const uint8_t* k, const uint8_t* v, const float* k_scale,
                                    const float* v_scale, long long row0, int slot_stride, int lane, int row,
                                    int col) {
    static_assert(INL == 0, "separate-scale or bf16 pools");
    const uint32_t rs = (uint32_t)slot_stride * ROW_BYTES;  // bytes between consecutive tokens
    const long long base = row0 * ROW_BYTES;
    {
      // K: lane (row, col) fetches bytes [jj * 64 + row * 16, +16) of token
      // tile_token(col)
      const uint8_t* kb = k + base;
      const uint32_t ko = (uint32_t)tile_token(col) * rs + (uint32_t)row * 16u;
#pragma unroll
      for (int jj = 0; jj < K_LD; ++jj) dma16(kb + ko + jj * 64, st + jj * 1024);
    }
    {
      // V: byte jj * 1024 + lane * 16 of the row-major tile
      constexpr int TPJ = 1024 / ROW_BYTES;  // tokens per 1024 bytes
      const uint8_t* vb = v + base;
      const uint32_t lb = (uint32_t)lane * 16u;
      const uint32_t vo = (lb / ROW_BYTES) * rs + lb % ROW_BYTES;
#pragma unroll
      for (int jj = 0; jj < V_LD; ++jj) dma16(vb + vo + (uint32_t)(jj * TPJ) * rs, st + K_TILE + jj * 1024);
    }
    if constexpr (FP8) {
      // scale slot m < 16: k_scale of token tile_token(m); 16 + m: its v_scale
      const int m = lane & 15;
      const float* src = ((lane & 16) ? v_scale : k_scale) + row0 + (long long)tile_token(m) * slot_stride;
      dma4(src, st + K_TILE + V_TILE);
    }
  }

  // issue_rows for the pair's last tile when it is partial: tokens past
  // `last` (0..15, the last valid token of the tile) are fetched as the
  // last valid one (finite data, masked by the softmax), all inside the
  // tile's page.
  __device__ static void issue_rows_clamped(unsigned char* st, const uint8_t* k, const uint8_t* v, const float* k_scale,
                                            const float* v_scale, long long row0, int slot_stride, int last, int lane,
                                            int row, int col) {
    static_assert(INL == 0, "separate-scale or bf16 pools");
    const uint32_t rs = (uint32_t)slot_stride * ROW_BYTES;
    const long long base = row0 * ROW_BYTES;
    {
      const uint8_t* kb = k + base;
      const uint32_t ko = (uint32_t)min(tile_token(col), last) * rs + (uint32_t)row * 16u;
#pragma unroll
      for (int jj = 0; jj < K_LD; ++jj) dma16(kb + ko + jj * 64, st + jj * 1024);
    }
    {
      constexpr int TPJ = 1024 / ROW_BYTES;
      const uint8_t* vb = v + base;
      const int lb = lane * 16;
#pragma unroll
      for (int jj = 0; jj < V_LD; ++jj) {
        const uint32_t tok = (uint32_t)min(jj * TPJ + lb / ROW_BYTES, last);
        dma16(vb + tok * rs + (uint32_t)(lb % ROW_BYTES), st + K_TILE + jj * 1024);
      }
    }
    if constexpr (FP8) {
      const int m = lane & 15;
      const float* src =
          ((lane & 16) ? v_scale : k_scale) + row0 + (long long)min(tile_token(m), last) * slot_stride;
      dma4(src, st + K_TILE + V_TILE);
    }
  }

  // A pair's query rows as direct-to-LDS loads into a slot of QSLOT bytes:
  // column c's row lands at slot + c * D * 2 (padding columns fetch a valid
  // row; q_read zeroes them). qrow_of(c) is column c's query row index.
  static constexpr int Q_LPR = D * 2 / 16;                 // lanes per query row
  static constexpr int Q_RPL = 64 / Q_LPR;                 // rows per load
  static constexpr int CQ = (G + Q_RPL - 1) / Q_RPL;       // loads per pair
  static constexpr int QSLOT = CQ * 1024;
  template <typename QRowOf>
  __device__ static void q_issue(unsigned char* slot, const uint16_t* q, QRowOf&& qrow_of, int ncols, int lane) {
#pragma unroll
    for (int i = 0; i < CQ; ++i) {
      const int c = min(i * Q_RPL + lane / Q_LPR, ncols - 1);
      dma16(reinterpret_cast<const unsigned char*>(q + qrow_of(c) * D) + (lane % Q_LPR) * 16, slot + i * 1024);
    }
  }
  // Q as the MFMA B operand from a slot (as load_q).
  __device__ static void q_read(bf16x8 (&qop)[KSTEPS], const unsigned char* slot, int row, int col, int ncols) {
    // byte offset of dpos(kk, row): row * RS + QO(kk)
    constexpr int RS = FP8 ? 32 : 16;
    const uint32_t a = lds_addr(slot) + (uint32_t)(min(col, G - 1) * D * 2 + row * RS);
    u32x4 r[KSTEPS];
    if constexpr (FP8) {
      if constexpr (KSTEPS == 2) lds_b128<0, 16>(r, a);
      else if constexpr (KSTEPS == 4) lds_b128<0, 16, 128, 144>(r, a);
      else lds_b128<0, 16, 128, 144, 256, 272, 384, 400>(r, a);
    } else {
      if constexpr (KSTEPS == 2) lds_b128<0, 64>(r, a);
      else if constexpr (KSTEPS == 4) lds_b128<0, 64, 128, 192>(r, a);
      else lds_b128<0, 64, 128, 192, 256, 320, 384, 448>(r, a);
    }
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
      qop[kk] = __builtin_bit_cast(bf16x8, col < ncols ? r[kk] : u32x4{0u, 0u, 0u, 0u});
  }

  // `valid`: tokens of the tile that exist in the piece (INL 2 zeroes the V
  // values and v scales of the others; the other modes load clamped rows)
  __device__ static void read(Frag& f, const unsigned char* st, int lane, int row, int col,
                              int valid = kTileTokens) {
    if constexpr (INL == 2) {
      const uint32_t kb = lds_addr(st), vb = lds_addr(st + K_TILE);
      // K fragment jj: dwords q of bytes 64 jj + 16 row of token tile_token(col)
      {
        const uint32_t ak = kb + tile_token(col) * PITCH + 16 * row;
        uint32_t r[4 * K_LD];
        static_for<0, (4 * K_LD + 7) / 8>([&](auto hc) {
          constexpr int h = decltype(hc)::value;
          constexpr int n = 4 * K_LD - 8 * h < 8 ? 4 * K_LD - 8 * h : 8;
          uint32_t t[n];
          lds_b32_groups<4, 64, 8 * h>(t, ak, std::make_index_sequence<n>{});
#pragma unroll
          for (int i = 0; i < n; ++i) r[8 * h + i] = t[i];
        });
#pragma unroll
        for (int jj = 0; jj < K_LD; ++jj) f.kf[jj] = u32x4{r[4 * jj], r[4 * jj + 1], r[4 * jj + 2], r[4 * jj + 3]};
      }
      // V chunk j: token row + 4 j, bytes col * VB .. + VB
      {
        constexpr int W = VB / 4;
        const uint32_t av = vb + row * PITCH + col * VB;
        uint32_t r[4 * W];
        static_for<0, (4 * W + 7) / 8>([&](auto hc) {
          constexpr int h = decltype(hc)::value;
          constexpr int n = 4 * W - 8 * h < 8 ? 4 * W - 8 * h : 8;
          uint32_t t[n];
          lds_b32_groups<W, 4 * PITCH, 8 * h>(t, av, std::make_index_sequence<n>{});
#pragma unroll
          for (int i = 0; i < n; ++i) r[8 * h + i] = t[i];
        });
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (W == 1) {
            f.vf[j] = r[j];
          } else {
#pragma unroll
            for (int w = 0; w < W; ++w) f.vf[j][w] = r[W * j + w];
          }
        }
      }
      // scales: tokens row + 4 v, the dword after the codes
      {
        uint32_t rk[4], rv[4];
        lds_b32_groups<1, 4 * PITCH, 0>(rk, kb + row * PITCH + ROW_BYTES, std::make_index_sequence<4>{});
        lds_b32_groups<1, 4 * PITCH, 0>(rv, vb + row * PITCH + ROW_BYTES, std::make_index_sequence<4>{});
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          f.ks[v] = __uint_as_float(rk[v]);
          f.vs[v] = __uint_as_float(rv[v]);
        }
      }
      // rows past the piece were loaded raw: their weights are exactly 0,
      // and 0 times a NaN left in an unused slot would not be
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (row + 4 * v >= valid) {
          f.vs[v] = 0.0f;
          if constexpr (VB / 4 == 1) {
            f.vf[v] = 0u;
          } else {
#pragma unroll
            for (int w = 0; w < VB / 4; ++w) f.vf[v][w] = 0u;
          }
        }
      }
      return;
    }
    read_stage<D, FP8>(st + lane * 16, st + K_TILE + row * ROW_BYTES + col * VB, st + K_TILE + V_TILE + row * 16,
                       f.kf, f.vf, f.ks, f.vs);
  }

  // One tile of the online softmax: tokens tb .. tb+15 of the pair, those
  // at or past L masked (L may differ between columns: lane (row, col)
  // passes its column's limit). FULL: every token of the tile is visible to
  // every column (no masking).
  //
  // The running maximum moves lazily: it is raised (and the accumulators
  // rescaled) only when a score exceeds it by more than kRescaleSlack (base
  // 2), so weights stay below 2^kRescaleSlack; m, l and acc stay mutually
  // consistent, which is all the final division and the merge need.
  template <bool FULL = false>
  __device__ static void compute(State& s, const Frag& f, const bf16x8 (&qop)[KSTEPS], int tb, int L,
                                 float qk_scale_log2, int row) {
    // S[t][g]: lane (row, col) holds head col for tokens row + 4 v
    f32x4 Sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      u32x4 kw;
      if constexpr (FP8) {
        const u32x4& c = f.kf[kk >> 1];
        kw = fp8x8_to_bf16x8(c[(kk & 1) * 2], c[(kk & 1) * 2 + 1]);
      } else {
        kw = f.kf[kk];
      }
      Sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kw), qop[kk], Sacc, 0, 0, 0);
    }
    float sc[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float x = Sacc[v] * qk_scale_log2;
      if constexpr (FP8) x *= f.ks[v];
      if constexpr (FULL) sc[v] = x;
      else sc[v] = (tb + row + 4 * v < L) ? x : -__builtin_inff();
    }
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // a column that has seen no score keeps m = -inf (and never grows on an
    // all-masked tile: -inf > -inf + slack is false)
    const bool grow = mx > s.m + kRescaleSlack;
    if (__any(grow)) {
      const float m_new = grow ? mx : s.m;
      const float alpha = grow ? __builtin_amdgcn_exp2f(s.m - m_new) : 1.0f;  // exp2(-inf) = 0
      s.l *= alpha;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float a = col_of_row(alpha, row, v);
#pragma unroll
        for (int e = 0; e < VE; ++e) s.cacc[e][v] *= a;
      }
      s.m = m_new;
    }
    // exponents against m, or against 0 while m = -inf (every weight is then
    // exactly 0: never -inf - -inf)
    const float m_ref = s.m == -__builtin_inff() ? 0.0f : s.m;
    float pr[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) pr[v] = __builtin_amdgcn_exp2f(sc[v] - m_ref);
    s.l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    if constexpr (FP8) {
#pragma unroll
      for (int v = 0; v < 4; ++v) pr[v] *= f.vs[v];
    }
    // p . V on the matrix cores. Each weight enters as two bf16 terms (hi
    // and the bf16 of its remainder: within 2^-18 relative). One 16x16x32
    // product per V element e: k = 8 row + j carries hi of token row + 4 j
    // and k = 8 row + 4 + j its remainder, against the same V element twice
    // (B: V element e of tokens row + 4 j, n = col <-> d = col * VE + e).
    bf16x4 vb[VE];
    v_operands(f, vb);
    const bf16x4 ph = {(__bf16)pr[0], (__bf16)pr[1], (__bf16)pr[2], (__bf16)pr[3]};
    const bf16x4 pm = {(__bf16)(pr[0] - (float)ph[0]), (__bf16)(pr[1] - (float)ph[1]), (__bf16)(pr[2] - (float)ph[2]),
                       (__bf16)(pr[3] - (float)ph[3])};
    const bf16x8 a8 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(ph, pm, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const bf16x8 b8 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vb[e], vb[e], 0, 1, 2, 3, 4, 5, 6, 7));
      s.cacc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, s.cacc[e], 0, 0, 0);
    }
  }

  // Sum l over the four rows (disjoint tokens); every row then holds the
  // total (the matrix cores already summed acc over the tile's tokens).
  __device__ static void reduce_rows(State& s) {
    s.l += __shfl_xor(s.l, 16);
    s.l += __shfl_xor(s.l, 32);
  }

  // A whole pair after reduce_rows: out = acc / l, lse = ln 2 (m + log2 l);
  // a column that saw no token (l = 0) gets out = 0, lse = -inf (a NaN l
  // stays NaN). Column c < ncols has its output row at o + row_of(c) * D and
  // its lse at lo[row_of(c)] (lo may be null); padding columns are not
  // written. Lane (row, col) holds columns 4 row + v at d = col * VE + e.
  template <typename RowOfCol>
  __device__ static void store_out(const State& s, float* o, float* lo, RowOfCol&& row_of, int ncols, bool poisoned,
                                   int row, int col) {
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float lg = col_of_row(s.l, row, v);
      const int c = 4 * row + v;
      if (c < ncols) {
        float* d = o + (long long)row_of(c) * D + col * VE;
#pragma unroll
        for (int e = 0; e < VE; ++e) d[e] = poisoned ? nan : (lg != 0.0f ? s.cacc[e][v] / lg : 0.0f);
      }
    }
    if (lo != nullptr && row == 0 && col < ncols)
      lo[row_of(col)] = poisoned ? nan : (s.l != 0.0f ? (s.m + log2f(s.l)) * kLn2 : -__builtin_inff());
  }

  // A partial record after reduce_rows: m[G], l[G], acc[G][D] (un-normalised).
  // A poisoned piece records m = 0, l = acc = NaN, so every merge it enters
  // gives NaN. COHERENT: device-scope atomic stores (visible to waves on
  // other XCDs once complete) instead of plain ones.
  template <bool COHERENT = false>
  __device__ static void store_record(const State& s, float* r, bool poisoned, int row, int col) {
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int c = 4 * row + v;
      if (c < G) {
#pragma unroll
        for (int e = 0; e < VE; ++e) put<COHERENT>(r + 2 * G + c * D + col * VE + e, poisoned ? nan : s.cacc[e][v]);
      }
    }
    if (row == 0 && col < G) {
      put<COHERENT>(r + col, poisoned ? 0.0f : s.m);
      put<COHERENT>(r + G + col, poisoned ? nan : s.l);
    }
  }

  // The same two stores as buffer stores whose count does not depend on the
  // data: exactly N_OUT_STORES (N_REC_STORES) instructions, every lane
  // taking part; a lane with nothing to write addresses past the buffer's
  // end, which the hardware drops. (The streaming kernel counts them in its
  // vmcnt waits.) out_rs / lse_rs cover the output and lse arrays (lse_rs
  // with no records when there is no lse), rec_rs the records; row_of(c) is
  // column c's row index, rec_off the record's float offset.
  template <typename RowOfCol>
  __device__ static void store_out_counted(const State& s, __amdgpu_buffer_rsrc_t out_rs, __amdgpu_buffer_rsrc_t lse_rs,
                                           RowOfCol&& row_of, int ncols, bool poisoned, int row, int col) {
    const float nan = __builtin_nanf("");
    constexpr uint32_t kDrop = 0x80000000u;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float lg = col_of_row(s.l, row, v);
      const int c = 4 * row + v;
      const uint32_t off = c < ncols ? (uint32_t)(row_of(c) * D + col * VE) * 4u : kDrop;
#pragma unroll
      for (int i = 0; i < VE / 4; ++i) {
        f32x4 x;
#pragma unroll
        for (int t = 0; t < 4; ++t) x[t] = poisoned ? nan : (lg != 0.0f ? s.cacc[4 * i + t][v] / lg : 0.0f);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), out_rs, off == kDrop ? kDrop : off + 16u * i,
                                               0, 0);
      }
    }
    const float ls = poisoned ? nan : (s.l != 0.0f ? (s.m + log2f(s.l)) * kLn2 : -__builtin_inff());
    const uint32_t loff = row == 0 && col < ncols ? (uint32_t)row_of(col) * 4u : kDrop;
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, ls), lse_rs, loff, 0, 0);
  }
  __device__ static void store_record_counted(const State& s, __amdgpu_buffer_rsrc_t rec_rs, uint32_t rec_off,
                                              bool poisoned, int row, int col) {
    const float nan = __builtin_nanf("");
    constexpr uint32_t kDrop = 0x80000000u;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int c = 4 * row + v;
      const uint32_t off = c < G ? (rec_off + 2 * G + c * D + col * VE) * 4u : kDrop;
#pragma unroll
      for (int i = 0; i < VE / 4; ++i) {
        f32x4 x;
#pragma unroll
        for (int t = 0; t < 4; ++t) x[t] = poisoned ? nan : s.cacc[4 * i + t][v];
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rec_rs, off == kDrop ? kDrop : off + 16u * i,
                                               0, 0);
      }
    }
    const bool w = row == 0 && col < G;
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, poisoned ? 0.0f : s.m), rec_rs,
                                          w ? (rec_off + col) * 4u : kDrop, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, poisoned ? nan : s.l), rec_rs,
                                          w ? (rec_off + G + col) * 4u : kDrop, 0, 0);
  }
  template <bool COHERENT>
  __device__ static void put(float* a, float v) {
    if constexpr (COHERENT) __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *a = v;
  }
};

}  // namespace dev
}  // namespace pdattn
