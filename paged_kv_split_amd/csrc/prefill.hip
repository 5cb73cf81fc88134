// Ragged paged prefill attention on gfx950.
//
// The operation (AstrAI "CUDA Kernels": the paged prefill entry over a
// ragged batch, section "Q Scheduling and KV Addressing"; attention itself as
// in the decode kernels): request b owns the packed query rows
// qo_indptr[b] .. qo_indptr[b+1] - 1 (n of them), the last n positions of its
// context of L positions; with the causal mask query row i sees the positions
// t < L - n + i + 1, without it all t < L.
//
// Work decomposition. A host-built map gives every query tile its request
// and its index inside the request in O(1) (same section). One workgroup
// computes one (query tile, kv head): its 4 waves hold 16 NB (query row,
// head) columns each (the G query heads of the kv head packed with the rows,
// GQA head packing as on the same page), and share every K/V tile through a
// two-stage LDS ring, so each K/V byte fetched serves 64 NB columns.
//
// Per KV tile of NT tokens, on each wave:
//   * S^T = K_tile . Q^T on v_mfma_f32_16x16x32_bf16 (A: 16 tokens x 32 d,
//     staged in LDS in operand order by the direct-to-LDS loads; B: the
//     wave's columns, held in registers for the whole call);
//   * online softmax per column in base 2 (FlashQuant wiki "CUDA Kernels",
//     flash_attention.cu, Online Softmax): a lane holds 4 M-blocks x 4 rows of
//     its column, the tile max needs two cross-row exchanges;
//   * O^T += V^T . P on the same MFMA: the probabilities sit, after the
//     softmax, exactly where the B operand wants them (k = 8 r + j is
//     M-block 2 p + j / 4, row 4 r + j mod 4), and the V^T operand is
//     gathered from LDS with the same k -> token order; O^T's columns are
//     the lane's own, so the rescale by exp2(m_old - m_new) is per lane.
// Tiles entirely below every column's causal limit skip the mask; tiles past
// the last row's limit are not read (causal tile skipping, same page,
// Causal Masking with Tile-Skipping).
//
// fp8 pools: the staged codes are widened once per tile, by the whole
// workgroup, into a bf16 image laid out as a bf16 tile is (exact: an e4m3
// value fits bf16), which the products then read as for bf16 pools; the k
// scale multiplies the score, the v scale the probability (OASR "Kernel
// Layer", FP8 KV variants), as in the decode kernels. Pools with the scale inline
// (each row's D codes followed by its fp32 scale, DeepGEMM documentation
// 6.1) are fetched with 4-byte loads into the same LDS image.

#include "prefill.h"
#include "tile_ops.h"

namespace pdattn {
namespace {

using dev::bf16x8;
using dev::f32x4;
using dev::u32x2;
using dev::u32x4;
using dev::u32x8;

template <int D, bool FP8>
struct Cfg {
  static constexpr int ESZ = FP8 ? 1 : 2;
  static constexpr int NB = D == 256 ? 1 : 2;       // 16-column blocks per wave
  static constexpr int NT = D == 256 ? 32 : 64;     // tokens per K/V tile
  static constexpr int MB = NT / 16;                // 16-token M-blocks per tile
  static constexpr int KS = D / 32;                 // k-steps of q.K
  static constexpr int DB = D / 16;                 // 16-row d-blocks of O^T
  static constexpr int PS = NT / 32;                // k-steps of p.V
  static constexpr int ROW = D * ESZ;               // bytes of one (token, kv head) row
  static constexpr int QK = ROW / 64;               // 16-byte K chunks per lane per M-block
  static constexpr int K_T = NT * ROW;
  static constexpr int V_T = NT * ROW;
  static constexpr int SC_T = FP8 ? MB * 128 : 0;   // per M-block: 16 k scales, 16 v scales
  static constexpr int STAGE = K_T + V_T + SC_T;
  static constexpr int KI = K_T / (kWaves * 64 * 16);  // K loads per lane per tile
  static constexpr int VI = V_T / (kWaves * 64 * 16);
  static constexpr int VR = DB * ESZ;               // bytes of a lane's V piece of one token
  static constexpr int COLS = kWaves * 16 * NB;
  // bf16 d 128: V^T operands by transposing LDS reads from a chunk-swizzled
  // V tile (16-byte chunk s of tile row t holds the row's chunk s ^ 2 (t mod
  // 8)); d-block e of O^T is then d 16 e .. 16 e + 15
  static constexpr bool TRV = !FP8 && D == 128;
  static constexpr int CPR = ROW / 16;                     // 16-byte chunks per row
  // fp8: the bf16 image of one tile after the two stages
  static constexpr int IMG = FP8 ? 2 * NT * D * 2 : 0;
  static constexpr int SMEM = 2 * STAGE + IMG;
  static_assert(COLS == prefill_columns(D), "columns");
  static_assert(NT == prefill_kv_tile(D), "kv tile");
  static_assert(KI >= 1 && QK % KI == 0 && VI >= 1, "load split");
  static_assert(MB * QK == kWaves * KI, "K image");
};

// LDS reads at immediate offsets from one address, and the wait for all of
// them, in one asm block: no destination is copied or used before its data
// has landed, and the compiler inserts no wait of its own for the direct-to-
// LDS loads of the next tile that are in flight meanwhile.
template <int... O>
__device__ __forceinline__ void lds_b128(u32x4 (&r)[sizeof...(O)], uint32_t a) {
  constexpr int o[] = {O...};
  constexpr int N = sizeof...(O);
  if constexpr (N == 1) {
    asm volatile("ds_read_b128 %0, %1 offset:%2\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r[0]) : "v"(a), "i"(o[0]) : "memory");
  } else if constexpr (N == 2) {
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

// Eight transposing 8-byte LDS reads (ds_read_b64_tr_b16: in each 16-lane
// group, lanes 4 r .. 4 r + 3 supply row r of a 4 x 16 block of 16-bit
// values, 8 bytes each, and lane i receives column i: the four rows' values
// of it), from eight base addresses at one immediate offset. WAIT closes the
// block with the wait for every LDS read issued so far.
template <int OFF, bool WAIT>
__device__ __forceinline__ void lds_tr8(u32x2 (&r)[8], const uint32_t (&a)[8]) {
  if constexpr (WAIT) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%16\n\t"
        "ds_read_b64_tr_b16 %1, %9 offset:%16\n\t"
        "ds_read_b64_tr_b16 %2, %10 offset:%16\n\t"
        "ds_read_b64_tr_b16 %3, %11 offset:%16\n\t"
        "ds_read_b64_tr_b16 %4, %12 offset:%16\n\t"
        "ds_read_b64_tr_b16 %5, %13 offset:%16\n\t"
        "ds_read_b64_tr_b16 %6, %14 offset:%16\n\t"
        "ds_read_b64_tr_b16 %7, %15 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "i"(OFF)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%16\n\t"
        "ds_read_b64_tr_b16 %1, %9 offset:%16\n\t"
        "ds_read_b64_tr_b16 %2, %10 offset:%16\n\t"
        "ds_read_b64_tr_b16 %3, %11 offset:%16\n\t"
        "ds_read_b64_tr_b16 %4, %12 offset:%16\n\t"
        "ds_read_b64_tr_b16 %5, %13 offset:%16\n\t"
        "ds_read_b64_tr_b16 %6, %14 offset:%16\n\t"
        "ds_read_b64_tr_b16 %7, %15 offset:%16"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "i"(OFF)
        : "memory");
  }
}

template <int... O>
__device__ __forceinline__ void lds_b64x8(u32x2 (&r)[8], uint32_t a) {
  constexpr int o[] = {O...};
  static_assert(sizeof...(O) == 8, "read count");
  asm volatile(
      "ds_read_b64 %0, %8 offset:%9\n\t"
      "ds_read_b64 %1, %8 offset:%10\n\t"
      "ds_read_b64 %2, %8 offset:%11\n\t"
      "ds_read_b64 %3, %8 offset:%12\n\t"
      "ds_read_b64 %4, %8 offset:%13\n\t"
      "ds_read_b64 %5, %8 offset:%14\n\t"
      "ds_read_b64 %6, %8 offset:%15\n\t"
      "ds_read_b64 %7, %8 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(a), "i"(o[0]), "i"(o[1]), "i"(o[2]), "i"(o[3]), "i"(o[4]), "i"(o[5]), "i"(o[6]), "i"(o[7])
      : "memory");
}

// N 16-byte LDS reads from N addresses, and their wait.
template <int N>
__device__ __forceinline__ void lds_b128_at(u32x4 (&r)[N], const uint32_t (&a)[N]) {
  if constexpr (N == 2) {
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1])
        : "v"(a[0]), "v"(a[1])
        : "memory");
  } else {
    static_assert(N == 4, "read count");
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
  }
}

// Two 16-byte LDS writes, at a and a + OFF. Issued from asm like the reads,
// so the compiler neither orders them behind the direct-to-LDS loads in
// flight nor counts them: the caller waits (lgkmcnt) before its barrier.
template <int OFF>
__device__ __forceinline__ void lds_write2_b128(uint32_t a, const u32x4& x, const u32x4& y) {
  asm volatile(
      "ds_write_b128 %0, %1\n\t"
      "ds_write_b128 %0, %2 offset:%3"
      :
      : "v"(a), "v"(x), "v"(y), "i"(OFF)
      : "memory");
}

// The K chunks of M-block MB_ and the ones after it (QK 16-byte reads from
// the lane's slot per M-block, one LDS wait for all of them).
template <typename C, int MB_, size_t... I>
__device__ __forceinline__ void read_k(u32x4 (&r)[sizeof...(I)], uint32_t ak, std::index_sequence<I...>) {
  lds_b128<(int)((MB_ * C::QK + I) * 1024)...>(r, ak);
}

// Byte offset (from the lane's V base, which already holds its 4 r rows and
// its d piece) of the token in k slot j of p.V k-step P_.
template <typename C, int P_, int J>
constexpr int v_off() { return (32 * P_ + 16 * (J >> 2) + (J & 3)) * C::ROW; }

// The lane's V pieces of p.V k-step P_: for k slot j (j = 0..7), the DB
// elements of its d range, as dwords.
template <typename C, int P_>
struct VPieces {
  static constexpr int WORDS = C::VR / 4 > 0 ? C::VR / 4 : 1;
  uint32_t w[8][WORDS];
};

template <typename C, int P_>
__device__ __forceinline__ void read_v(VPieces<C, P_>& v, uint32_t av) {
  if constexpr (C::VR == 32) {
    u32x4 a[8], b[8];
    lds_b128<v_off<C, P_, 0>(), v_off<C, P_, 1>(), v_off<C, P_, 2>(), v_off<C, P_, 3>(), v_off<C, P_, 4>(),
             v_off<C, P_, 5>(), v_off<C, P_, 6>(), v_off<C, P_, 7>()>(a, av);
    lds_b128<v_off<C, P_, 0>() + 16, v_off<C, P_, 1>() + 16, v_off<C, P_, 2>() + 16, v_off<C, P_, 3>() + 16,
             v_off<C, P_, 4>() + 16, v_off<C, P_, 5>() + 16, v_off<C, P_, 6>() + 16, v_off<C, P_, 7>() + 16>(b, av);
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        v.w[j][x] = a[j][x];
        v.w[j][4 + x] = b[j][x];
      }
  } else {
    static_assert(C::VR == 8, "V piece");
    u32x2 a[8];
    lds_b64x8<v_off<C, P_, 0>(), v_off<C, P_, 1>(), v_off<C, P_, 2>(), v_off<C, P_, 3>(), v_off<C, P_, 4>(),
              v_off<C, P_, 5>(), v_off<C, P_, 6>(), v_off<C, P_, 7>()>(a, av);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v.w[j][0] = a[j][0];
      v.w[j][1] = a[j][1];
    }
  }
}

// The V^T operand of d-block e: element e of the eight k slots' pieces,
// gathered with byte permutes (perm(s0, s1, sel): selector bytes 0-3 pick
// bytes of s1, 4-7 bytes of s0).
template <typename VP>
__device__ __forceinline__ bf16x8 v_operand(const VP& v, int e) {
  const int wd = e >> 1;
  const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;  // high or low halves of s1 then s0
  u32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = __builtin_amdgcn_perm(v.w[2 * q + 1][wd], v.w[2 * q][wd], sel);
  return __builtin_bit_cast(bf16x8, r);
}

// Maximum over the four 16-lane rows, for every lane (the lane's column
// in each row): gfx950's row swaps (permlane16 pairs rows 0-1 and 2-3,
// permlane32 the two halves; with both operands x, the two results of a
// lane are its own value and its partner's), plain VALU, no LDS trip.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ float max_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats as bf16 (round to nearest even), a in the low half: one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

// Part records cross workgroups on different XCDs. They are written and
// read with device-scope (sc1) 16-byte buffer accesses, coherent at device
// level without a write-back or invalidation of a whole L2; the writer's
// stores complete before the counter update that publishes them.
constexpr int kBufferWord3 = 0x00020000;  // word 3 of a raw buffer resource (gfx9 family)
constexpr int kDeviceScope = 16;          // cache policy: sc1

// One part of a split tile: store its record (the lane's accumulators in
// its own layout, then per column m and the row-summed l), count the part
// in, and return false unless it is the last to finish. The last one merges
// every part's record in part order (its own from registers), so the result
// does not depend on which part finished last, leaves the merged state in
// acc, m, l, and resets the counter for the next call. A part that saw a bad
// page poisons the tile through the counter's high half.
template <int D, bool FP8>
__device__ __forceinline__ bool merge_parts(const PrefillParams& p, uint32_t& s_count,
                                            f32x4 (&acc)[Cfg<D, FP8>::NB][Cfg<D, FP8>::DB],
                                            float (&m)[Cfg<D, FP8>::NB], float (&l)[Cfg<D, FP8>::NB], bool& poisoned,
                                            int slot0, int part, int parts, int kvh, int w, int lane) {
  using C = Cfg<D, FP8>;
  constexpr long long RF = prefill_record_floats(D);
  const int n = lane & 15, g = lane >> 4;
  auto rec_of = [&](int q) {
    return __builtin_amdgcn_make_buffer_rsrc(p.part_rec + ((long long)(slot0 + q) * p.num_kv_heads + kvh) * RF, 0,
                                             (int)(RF * 4), kBufferWord3);
  };
  // byte offsets: accumulators [wave][block][d-block][lane][4], then
  // [wave][block][column][m, l]
  auto acc_off = [&](int bb, int e) { return (uint32_t)((((w * C::NB + bb) * C::DB + e) * 64 + lane) * 16); };
  auto ml_off = [&](int bb) { return (uint32_t)((C::COLS * D + ((w * C::NB + bb) * 16 + n) * 2) * 4); };
  {
    const auto r = rec_of(part);
#pragma unroll
    for (int bb = 0; bb < C::NB; ++bb)
#pragma unroll
      for (int e = 0; e < C::DB; ++e)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[bb][e]), r, acc_off(bb, e), 0,
                                               kDeviceScope);
    if (g == 0) {
#pragma unroll
      for (int bb = 0; bb < C::NB; ++bb)
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(m[bb]), __float_as_uint(l[bb])}, r, ml_off(bb),
                                              0, kDeviceScope);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  uint32_t* ctr = p.part_ctr + (long long)slot0 * p.num_kv_heads + kvh;
  if (threadIdx.x == 0)
    s_count = __hip_atomic_fetch_add(ctr, 1u + (poisoned ? 0x10000u : 0u), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint32_t before = s_count;
  if ((int)(before & 0xffffu) + 1 < parts) return false;
  if (threadIdx.x == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  poisoned = poisoned || (before >> 16) != 0;
#pragma unroll
  for (int bb = 0; bb < C::NB; ++bb) {
    float M = m[bb];
    for (int q = 0; q < parts; ++q) {
      if (q == part) continue;
      const u32x2 ml = __builtin_amdgcn_raw_buffer_load_b64(rec_of(q), ml_off(bb), 0, kDeviceScope);
      M = fmaxf(M, __uint_as_float(ml[0]));
    }
    // parts that saw nothing keep m = -inf, l = 0, acc = 0 and weigh 0
    const float m_ref = M == -__builtin_inff() ? 0.0f : M;
    f32x4 R[C::DB];
#pragma unroll
    for (int e = 0; e < C::DB; ++e) R[e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float L = 0.0f;
    for (int q = 0; q < parts; ++q) {
      float mq, lq;
      f32x4 a[C::DB];
      if (q == part) {
        mq = m[bb];
        lq = l[bb];
#pragma unroll
        for (int e = 0; e < C::DB; ++e) a[e] = acc[bb][e];
      } else {
        const auto r = rec_of(q);
        const u32x2 ml = __builtin_amdgcn_raw_buffer_load_b64(r, ml_off(bb), 0, kDeviceScope);
        mq = __uint_as_float(ml[0]);
        lq = __uint_as_float(ml[1]);
#pragma unroll
        for (int e = 0; e < C::DB; ++e)
          a[e] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, acc_off(bb, e), 0, kDeviceScope));
      }
      const float sc = __builtin_amdgcn_exp2f(mq - m_ref);
      L = fmaf(lq, sc, L);
#pragma unroll
      for (int e = 0; e < C::DB; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j) R[e][j] = fmaf(a[e][j], sc, R[e][j]);
    }
#pragma unroll
    for (int e = 0; e < C::DB; ++e) acc[bb][e] = R[e];
    l[bb] = L;
    m[bb] = M;
  }
  return true;
}

// One map entry (a whole query tile, or one part of a split one) for kv
// head kvh, on the whole workgroup. INL: fp8 rows with their scale inline.
template <int D, bool FP8, bool INL>
__device__ __forceinline__ void prefill_item(const PrefillParams& p, const int tile, const int kvh,
                                             unsigned char (&smem)[Cfg<D, FP8>::SMEM], uint32_t& s_count) {
  using C = Cfg<D, FP8>;     // the staged tiles (loads, fp8 scales)
  using CC = Cfg<D, false>;  // the bf16 tile the products read (fp8: the widened image)
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, n = lane & 15;
  const int b = p.tile_batch[tile];
  if (b < 0 || b >= p.batch) return;
  const int row_base = p.tile_index[tile] * p.rows_per_tile;
  const int q0 = p.qo_indptr[b];
  const int nreq = p.qo_indptr[b + 1] - q0;
  if (row_base < 0 || row_base >= nreq) return;
  const int L = p.context_lens[b];
  const bool bad_len = L < 0 || L > (p.max_pages_per_seq << p.page_log2);
  const int G = p.heads_per_kv;
  const int last_row = min(row_base + p.rows_per_tile, nreq) - 1;

  // the lane's columns: block bb holds column c = 16 (NB w + bb) + n, the
  // (tile row c / G, head c mod G) pair; lim = positions it may see
  int lim[C::NB];
  long long orow[C::NB];  // output row (packed query row * Hq + head), -1 if none
#pragma unroll
  for (int bb = 0; bb < C::NB; ++bb) {
    const int c = 16 * (C::NB * w + bb) + n;
    const int rr = c / G;
    const int i = row_base + rr;
    const bool valid = rr < p.rows_per_tile && i < nreq;
    int li = p.causal ? L - nreq + i + 1 : L;
    li = li < 0 ? 0 : (li > L ? L : li);
    lim[bb] = valid && !bad_len ? li : 0;
    orow[bb] = valid ? (long long)(q0 + i) * p.num_q_heads + (long long)kvh * G + (c - rr * G) : -1;
  }
  const float nan = __builtin_nanf("");
  if (bad_len) {
#pragma unroll
    for (int bb = 0; bb < C::NB; ++bb) {
      if (orow[bb] < 0) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < C::DB; ++e) p.out[orow[bb] * D + (4 * g + j) * C::DB + e] = nan;
      if (p.lse != nullptr && g == 0) p.lse[orow[bb]] = nan;
    }
    return;
  }
  int kv_end = p.causal ? L - nreq + last_row + 1 : L;
  kv_end = kv_end < 0 ? 0 : (kv_end > L ? L : kv_end);
  int mask_from = p.causal ? L - nreq + row_base + 1 : L;
  mask_from = mask_from < 0 ? 0 : (mask_from > L ? L : mask_from);
  const int T = (kv_end + C::NT - 1) / C::NT;
  // The tiles [it0, it1) this workgroup reads: all T, or the range of one
  // part of a split tile. A part keeps its (m, l, acc) in a record; the last
  // part to finish merges the records and writes the rows. An entry that
  // does not fit the workspace poisons the tile instead.
  int it0 = 0, it1 = T, slot0 = -1, part = 0, parts = 1;
  bool bad_map = false;
  if (p.tile_kv != nullptr) {
    const int32_t* kv = p.tile_kv + 4 * (long long)tile;
    const int kv_first = kv[0], kv_last = kv[1], s0 = kv[2], pq = kv[3];
    it0 = kv_first <= 0 ? 0 : min(kv_first / C::NT, T);
    it1 = kv_last <= 0 ? it0 : max(it0, min((int)(((long long)kv_last + C::NT - 1) / C::NT), T));
    if (s0 >= 0) {
      parts = pq >> 16;
      part = pq & 0xffff;
      if (parts < 2 || part >= parts || s0 > p.num_slots - parts) {
        bad_map = true;
        it1 = it0;
      } else {
        slot0 = s0;
      }
    }
  }

  // Q as the B operand of q.K, zero for columns without a row; the head_dim
  // order inside a k-step matches the K chunks (32 ks + 8 r + j)
  bf16x8 qop[C::NB][C::KS];
#pragma unroll
  for (int bb = 0; bb < C::NB; ++bb) {
    const uint16_t* qrow = p.q + (orow[bb] >= 0 ? orow[bb] * D : 0);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int d0 = 32 * ks + 8 * g;
      u32x4 raw = *reinterpret_cast<const u32x4*>(qrow + d0);
      if (orow[bb] < 0) raw = u32x4{0u, 0u, 0u, 0u};
      qop[bb][ks] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // Page entries. Every position a wave loads for the tile at tb lies in its
  // 16-token group [first, first + 15] (clamped to L - 1), so on at most two
  // pages (P >= 8, groups 16-aligned). The block table is read-only for the
  // whole call: through the constant address space these wave-uniform
  // entries load with scalar loads, which the tiles' vector-memory waits do
  // not count.
  typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
  const const_i32_ptr bt = (const_i32_ptr)(p.block_table + (long long)b * p.max_pages_per_seq);
  const int mbK = w * C::KI / C::QK;
  bool bad_page = false;
  auto group_first = [&](int tb) { return min(tb + 16 * mbK, L - 1); };
  // loaded one tile ahead and checked only when used, so that the load's
  // latency hides behind a tile of compute
  auto load_pages = [&](int tb, int& e0, int& e1) {
    const int first = group_first(tb);
    const int lastp = min(first + 15, L - 1);
    e0 = bt[first >> p.page_log2];
    e1 = bt[lastp >> p.page_log2];
  };
  auto check_page = [&](int e) {
    const bool ok = e >= 0 && e < p.num_pages;
    bad_page |= !ok;
    return ok ? e : 0;
  };
  const int P = 1 << p.page_log2;
  auto row_of = [&](int pos, int first, int e0, int e1) -> long long {
    const int page = (pos >> p.page_log2) == (first >> p.page_log2) ? e0 : e1;
    return ((long long)page * P * p.num_kv_heads) + (long long)(pos & (P - 1)) * p.slot_stride +
           (long long)kvh * p.head_stride;
  };
  // Per-lane byte offsets of the loads inside the wave's 16-token group,
  // fixed for the whole call: the group's token x sits x * slot_stride rows
  // after the group's first row, when the group lies in one page.
  const uint32_t slot_bytes = (uint32_t)p.slot_stride * C::ROW;
  uint32_t koff[C::KI], voff[C::VI];
#pragma unroll
  for (int i = 0; i < C::KI; ++i) koff[i] = n * slot_bytes + 16 * g + 64 * ((w * C::KI + i) % C::QK);
#pragma unroll
  for (int i = 0; i < C::VI; ++i) {
    const int cv = (w * C::VI + i) * 64 + lane;
    const int chunk = C::TRV ? (cv % C::CPR) ^ (2 * ((cv / C::CPR) % 8)) : cv % C::CPR;
    voff[i] = (uint32_t)(cv * 16 / C::ROW - 16 * mbK) * slot_bytes + chunk * 16;
  }
  const uint32_t soff = (uint32_t)((lane & 15) * p.slot_stride) * 4u;
  // inline-scale rows (D + 4 bytes): the lane's K dword (token lane / 4 of
  // the group, dword lane mod 4 of a fragment), its V dword (byte 4 lane of
  // a 256-byte run of row-major rows) and its scale (token lane mod 16)
  const uint32_t inl_slot = (uint32_t)p.slot_stride * (D + 4);
  const uint32_t inl_k = (uint32_t)(lane >> 2) * inl_slot + 4 * (lane & 3);
  const uint32_t inl_v = (uint32_t)(4 * lane / C::ROW) * inl_slot + (4 * lane) % C::ROW;
  const uint32_t inl_s = (uint32_t)(lane & 15) * inl_slot + D;
  const float* sbase_lane = lane < 16 ? p.k_scale : p.v_scale;
  auto issue = [&](int tb, int stage, int raw0, int raw1) {
    const int e0 = check_page(raw0), e1 = check_page(raw1);
    unsigned char* st = smem + stage * C::STAGE;
    const int first = group_first(tb);
    if constexpr (INL) {
      // rows of D codes and the row's fp32 scale, D + 4 bytes apart and so
      // only 4-byte aligned: load (i, qq) fills bytes [qq * 256, +256) of
      // the wave's 1 KB piece i, lane x the dword at + 4 x
      constexpr int PITCH = D + 4;
      if (P >= 16 && tb + C::NT <= L) {
        // the group inside one page, every position < L: a wave-uniform row
        // base, the two fixed lane offsets and constant ones per load
        const int tg = tb + 16 * mbK;
        const long long rb = (long long)e0 * P * p.num_kv_heads + (long long)(tg & (P - 1)) * p.slot_stride +
                             (long long)kvh * p.head_stride;
        const uint8_t* kb = p.k + rb * PITCH + inl_k;
        const uint8_t* vb = p.v + rb * PITCH + inl_v;
#pragma unroll
        for (int i = 0; i < C::KI; ++i) {
          const int q = w * C::KI + i;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) dev::dma4(kb + 64 * (q % C::QK) + 16 * qq, st + q * 1024 + qq * 256);
        }
#pragma unroll
        for (int i = 0; i < C::VI; ++i)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const int t = ((w * C::VI + i) * 1024 + qq * 256) / C::ROW - 16 * mbK;
            dev::dma4(vb + (uint32_t)t * inl_slot, st + C::K_T + (w * C::VI + i) * 1024 + qq * 256);
          }
        if ((w * C::KI) % C::QK == 0 && lane < 32)
          dev::dma4((lane < 16 ? p.k : p.v) + rb * PITCH + inl_s, st + C::K_T + C::V_T + mbK * 128);
        return;
      }
      {
        // K: that dword is dword x mod 4 of the 16-byte operand fragment of
        // lane 16 qq + x / 4, i.e. token x / 4 of the group, row bytes
        // 64 (piece mod QK) + 16 qq + 4 (x mod 4)
        const int pos = min(tb + 16 * mbK + (lane >> 2), L - 1);
        const uint8_t* src = p.k + row_of(pos, first, e0, e1) * PITCH + 4 * (lane & 3);
#pragma unroll
        for (int i = 0; i < C::KI; ++i) {
          const int q = w * C::KI + i;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) dev::dma4(src + 64 * (q % C::QK) + 16 * qq, st + q * 1024 + qq * 256);
        }
      }
      // V, row-major: byte y of the tile is byte y mod ROW of token y / ROW
#pragma unroll
      for (int i = 0; i < C::VI; ++i)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int y = (w * C::VI + i) * 1024 + qq * 256 + 4 * lane;
          const int pos = min(tb + y / C::ROW, L - 1);
          dev::dma4(p.v + row_of(pos, first, e0, e1) * PITCH + y % C::ROW,
                    st + C::K_T + (w * C::VI + i) * 1024 + qq * 256);
        }
      // the first wave of each M-block group stages its 16 k and 16 v
      // scales, the dwords after the rows' codes
      if ((w * C::KI) % C::QK == 0 && lane < 32) {
        const int pos = min(tb + 16 * mbK + (lane & 15), L - 1);
        dev::dma4((lane < 16 ? p.k : p.v) + row_of(pos, first, e0, e1) * PITCH + D,
                  st + C::K_T + C::V_T + mbK * 128);
      }
      return;
    }
    if (P >= 16 && tb + C::NT <= L) {
      // the group is 16-aligned and inside one page, every position < L:
      // a wave-uniform row base plus the fixed lane offsets
      const int tg = tb + 16 * mbK;
      const long long rb = (long long)e0 * P * p.num_kv_heads + (long long)(tg & (P - 1)) * p.slot_stride +
                           (long long)kvh * p.head_stride;
      const uint8_t* kb = p.k + rb * C::ROW;
      const uint8_t* vb = p.v + rb * C::ROW;
#pragma unroll
      for (int i = 0; i < C::KI; ++i) dev::dma16(kb + koff[i], st + (w * C::KI + i) * 1024);
#pragma unroll
      for (int i = 0; i < C::VI; ++i) dev::dma16(vb + voff[i], st + C::K_T + (w * C::VI + i) * 1024);
      if constexpr (FP8) {
        if ((w * C::KI) % C::QK == 0 && lane < 32)
          dev::dma4(reinterpret_cast<const uint8_t*>(sbase_lane + rb) + soff, st + C::K_T + C::V_T + mbK * 128);
      }
      return;
    }
    {
      const int pos = min(tb + 16 * mbK + n, L - 1);
      const uint8_t* src = p.k + row_of(pos, first, e0, e1) * C::ROW + 16 * g;
#pragma unroll
      for (int i = 0; i < C::KI; ++i) {
        const int q = w * C::KI + i;
        dev::dma16(src + 64 * (q % C::QK), st + q * 1024);
      }
    }
#pragma unroll
    for (int i = 0; i < C::VI; ++i) {
      const int cv = (w * C::VI + i) * 64 + lane;
      const int pos = min(tb + cv * 16 / C::ROW, L - 1);
      const int chunk = C::TRV ? (cv % C::CPR) ^ (2 * ((cv / C::CPR) % 8)) : cv % C::CPR;
      dev::dma16(p.v + row_of(pos, first, e0, e1) * C::ROW + chunk * 16, st + C::K_T + (w * C::VI + i) * 1024);
    }
    if constexpr (FP8) {
      // the first wave of each M-block group stages its 16 k and 16 v scales
      if ((w * C::KI) % C::QK == 0 && lane < 32) {
        const int pos = min(tb + 16 * mbK + (lane & 15), L - 1);
        const float* src = (lane < 16 ? p.k_scale : p.v_scale) + row_of(pos, first, e0, e1);
        dev::dma4(src, st + C::K_T + C::V_T + mbK * 128);
      }
    }
  };

  // transposing V reads: lane 4 r + q of 16-lane group g supplies tile row
  // 4 g + r (+ 32 pp + 16 h, at the immediate offset), d 16 e + 4 q .. + 3,
  // whose 32-byte pair e sits at pair slot e ^ ((4 g + r) mod 8)
  uint32_t trv_off[8];
  if constexpr (CC::TRV) {
    const int tr_r = n >> 2, tr_q = n & 3;
    const int tr_x = (4 * g + tr_r) % 8;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      trv_off[e] = (uint32_t)(CC::K_T + (4 * g + tr_r) * CC::ROW + 32 * (e ^ tr_x) + 8 * tr_q);
  }
  float m[C::NB], l[C::NB];
  f32x4 acc[C::NB][C::DB];
#pragma unroll
  for (int bb = 0; bb < C::NB; ++bb) {
    m[bb] = -__builtin_inff();
    l[bb] = 0.0f;
#pragma unroll
    for (int e = 0; e < C::DB; ++e) acc[bb][e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  const uint32_t lds0 = dev::lds_addr(smem);
  // fp8: thread t widens 16-byte pieces u = t + 256 i (i < WP) of the staged
  // K tile and as many of V. K piece u is lane (g', n') of chunk u / 64,
  // M-block (u / 64) / QK: token n', d 64 ((u / 64) mod QK) + 16 g' .. + 15,
  // which in bf16 is k-step 2 ((u / 64) mod QK) + g' / 2, lane groups
  // 2 (g' mod 2) and the next (256 bytes on). V piece u is token u / (D / 16),
  // d 16 k .. + 15 with k = u mod (D / 16): bf16 chunks 2k and 2k + 1 of the
  // row, adjacent also where the image swizzles chunks (the swizzle is even).
  constexpr int WP = FP8 ? C::K_T / (kWaves * 64 * 16) : 1;
  static_assert(!FP8 || (C::K_T == C::V_T && C::K_T % (kWaves * 64 * 16) == 0 && (WP == 1 || WP == 2)), "pieces");
  const uint32_t img = lds0 + 2 * C::STAGE;
  uint32_t w_src[2 * WP], w_dst[2 * WP];
  if constexpr (FP8) {
#pragma unroll
    for (int i = 0; i < WP; ++i) {
      const int u = i * kWaves * 64 + (int)threadIdx.x;
      const int q = u >> 6, gg = (u >> 4) & 3, nn = u & 15;
      const int kq = 2 * (q % C::QK) + (gg >> 1);
      w_src[i] = (uint32_t)(u * 16);
      w_dst[i] = img + (uint32_t)((((q / C::QK) * CC::QK + kq) * 64 + 32 * (gg & 1) + nn) * 16);
      const int t = u / (D / 16), k = u % (D / 16);
      const int s0 = CC::TRV ? (2 * k) ^ (2 * (t % 8)) : 2 * k;
      w_src[WP + i] = (uint32_t)(C::K_T + u * 16);
      w_dst[WP + i] = img + (uint32_t)(CC::K_T + t * CC::ROW + s0 * 16);
    }
  }
  auto widen = [&](uint32_t stage) {
    uint32_t a[2 * WP];
#pragma unroll
    for (int i = 0; i < 2 * WP; ++i) a[i] = stage + w_src[i];
    u32x4 r[2 * WP];
    lds_b128_at<2 * WP>(r, a);
#pragma unroll
    for (int i = 0; i < 2 * WP; ++i) {
      const u32x4 lo = dev::fp8x8_to_bf16x8(r[i][0], r[i][1]);
      const u32x4 hi = dev::fp8x8_to_bf16x8(r[i][2], r[i][3]);
      if (i < WP) lds_write2_b128<256>(w_dst[i], lo, hi);
      else lds_write2_b128<16>(w_dst[i], lo, hi);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  int e0 = 0, e1 = 0;
  if (it0 < it1) {
    load_pages(it0 * C::NT, e0, e1);
    issue(it0 * C::NT, it0 & 1, e0, e1);
    if (it0 + 1 < it1) load_pages((it0 + 1) * C::NT, e0, e1);
  }
  // one K/V tile: wait for its loads, start the next tile's, then compute.
  // MASKED (a compile-time flag) applies the columns' limits; the tiles that
  // need it come last, in a loop of their own, so that neither loop merges
  // masked and unmasked scores before the max (a merge would make the
  // compiler re-canonicalise every score)
  auto tile_step = [&](int it, auto masked_c) {
    constexpr bool MASKED = decltype(masked_c)::value;
    dev::wait_vmcnt<0>();
    __syncthreads();  // every wave's loads of tile it landed; stage (it + 1) & 1 is free
    const int tb = it * C::NT;
    if (it + 1 < it1) {
      issue(tb + C::NT, (it + 1) & 1, e0, e1);
      if (it + 2 < it1) load_pages(tb + 2 * C::NT, e0, e1);
    }
    const uint32_t st_b = lds0 + (it & 1) * C::STAGE;
    if constexpr (FP8) {
      widen(st_b);
      __syncthreads();  // the image holds tile it
    }
    const uint32_t sb = FP8 ? img : st_b;  // the bf16 tile

    // the MFMA phases run at raised wave priority, so that the other waves
    // of the SIMD fill the VALU around them instead of competing for issue
    __builtin_amdgcn_s_setprio(1);
    // S^T = K . Q^T
    f32x4 S[C::MB][C::NB];
    constexpr int KG = 2 * CC::QK <= 8 ? 2 : 1;  // M-blocks per LDS wait
    u32x4 kcg[KG * CC::QK];
    dev::static_for<0, C::MB>([&](auto mbc) {
      constexpr int mb = decltype(mbc)::value;
      if constexpr (mb % KG == 0) read_k<CC, mb>(kcg, sb + lane * 16, std::make_index_sequence<KG * CC::QK>{});
      const u32x4* kc = kcg + (mb % KG) * CC::QK;
#pragma unroll
      for (int bb = 0; bb < C::NB; ++bb) S[mb][bb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kq = 0; kq < CC::QK; ++kq) {
        const bf16x8 k0 = __builtin_bit_cast(bf16x8, kc[kq]);
#pragma unroll
        for (int bb = 0; bb < C::NB; ++bb)
          S[mb][bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qop[bb][kq], S[mb][bb], 0, 0, 0);
      }
    });

    // The bf16 softmax reads the raw S registers with inline-asm v_max3,
    // and the compiler inserts no wait states between an MFMA and an asm
    // operand it writes (the matrix core does not interlock its results).
    // All of S passes through this block: every q.K product is issued
    // before it (no pass can sink one towards its use), 19 wait states
    // pass, and the reads below take its outputs.
    if constexpr (!FP8) {
      static_assert(C::MB * C::NB == 8 || C::MB * C::NB == 2, "S blocks");
      if constexpr (C::MB * C::NB == 8) {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 2"
                     : "+v"(S[0][0]), "+v"(S[0][1]), "+v"(S[1][0]), "+v"(S[1][1]), "+v"(S[2][0]), "+v"(S[2][1]),
                       "+v"(S[3][0]), "+v"(S[3][1]));
      } else {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 2" : "+v"(S[0][0]), "+v"(S[1][0]));
      }
    }
    __builtin_amdgcn_s_setprio(0);
    float ksc[C::MB][4], vsc[C::MB][4];
    if constexpr (FP8) {
      dev::static_for<0, C::MB>([&](auto mbc) {
        constexpr int mb = decltype(mbc)::value;
        u32x4 s2[2];
        lds_b128<mb * 128, mb * 128 + 64>(s2, st_b + C::K_T + C::V_T + 16 * g);
        // __uint_as_float: hipcc mistranslates __builtin_bit_cast applied
        // to one element of a vector (every element reads as element 0)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ksc[mb][j] = __uint_as_float(s2[0][j]) * p.qk_scale_log2;
          vsc[mb][j] = __uint_as_float(s2[1][j]);
        }
      });
    }

    // online softmax per column block in base 2; P as the B operand of
    // p.V. Scores x = q.k * scale * log2 e (fp8: times the k scale, folded
    // into the scale reads); the multiply also gives the max canonical
    // inputs, which a raw MFMA result is not known to be
    bf16x8 pop[C::NB][C::PS];
#pragma unroll
    for (int bb = 0; bb < C::NB; ++bb) {
      // fp8: scores scaled here (the k scale varies per token); bf16: raw
      // scores, the scale (positive) applied to their maximum and inside the
      // exponent's fma
      float x[C::MB][4];
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) x[mb][j] = FP8 ? S[mb][bb][j] * ksc[mb][j] : S[mb][bb][j];
      if constexpr (MASKED) {
        // only tiles that reach past some column's limit: token
        // tb + 16 mb + 4 r + j is visible iff 16 mb + j < rel
        const int rel = lim[bb] - (tb + 4 * g);
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (16 * mb + j >= rel) x[mb][j] = -__builtin_inff();
      }
      float mx = -__builtin_inff();
      if constexpr (FP8) {
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
          mx = fmaxf(fmaxf(mx, fmaxf(x[mb][0], x[mb][1])), fmaxf(x[mb][2], x[mb][3]));
      } else {
        // v_max3 on the raw MFMA results (fmaxf would first canonicalise
        // each); it skips quiet NaNs as fmaxf does
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) mx = max3(max3(mx, x[mb][0], x[mb][1]), x[mb][2], x[mb][3]);
      }
      mx = max_rows(mx);
      if constexpr (!FP8) mx *= p.qk_scale_log2;
      // the running max moves only when a column's max exceeds it by more
      // than 8 in the exponent (or it is still -inf): every weight stays
      // below 2^8, and since numerator and denominator are taken against
      // the same m the result does not depend on it. A NaN max leaves m
      // alone (and the NaN reaches l and the output through the weights)
      const float m_old = m[bb];
      const bool up = mx - m_old > 8.0f;
      const float m_new = up ? mx : m_old;
      // a column with nothing visible yet keeps m = -inf; its weights are
      // then taken against 0 and are exactly 0
      const float m_ref = m_new == -__builtin_inff() ? 0.0f : m_new;
      if (__any(up)) {
        const float alpha = __builtin_amdgcn_exp2f(m_old - m_ref);  // 1 where m stays
        l[bb] *= alpha;
#pragma unroll
        for (int e = 0; e < C::DB; ++e) acc[bb][e] *= alpha;
      }
      m[bb] = m_new;
      float sum = 0.0f;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[mb][j] = __builtin_amdgcn_exp2f(FP8 ? x[mb][j] - m_ref : fmaf(x[mb][j], p.qk_scale_log2, -m_ref));
          sum += x[mb][j];
        }
      l[bb] += sum;
#pragma unroll
      for (int pp = 0; pp < C::PS; ++pp) {
        float y[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          y[j] = x[2 * pp][j];
          y[4 + j] = x[2 * pp + 1][j];
          if constexpr (FP8) {
            y[j] *= vsc[2 * pp][j];
            y[4 + j] *= vsc[2 * pp + 1][j];
          }
        }
        const u32x4 pw = {pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), pack_bf16(y[4], y[5]),
                          pack_bf16(y[6], y[7])};
        pop[bb][pp] = __builtin_bit_cast(bf16x8, pw);
      }
    }

    __builtin_amdgcn_s_setprio(1);
    // O^T += V^T . P
    if constexpr (CC::TRV) {
      // d-block e, k slots 8 g + j: tokens 32 pp + 16 (j / 4) + 4 g + j mod 4
      // (the P operand's order); the two transposing reads of a block give
      // tokens 32 pp + 4 g .. + 3 and 32 pp + 16 + 4 g .. + 3 of d 16 e + n
      static_assert(C::DB == 8, "eight d-blocks");
      uint32_t ab[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ab[e] = sb + trv_off[e];
      dev::static_for<0, C::PS>([&](auto ppc) {
        constexpr int pp = decltype(ppc)::value;
        u32x2 t0[8], t1[8];
        lds_tr8<32 * pp * CC::ROW, false>(t0, ab);
        lds_tr8<(32 * pp + 16) * CC::ROW, true>(t1, ab);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const u32x4 vw = {t0[e][0], t0[e][1], t1[e][0], t1[e][1]};
          const bf16x8 va = __builtin_bit_cast(bf16x8, vw);
#pragma unroll
          for (int bb = 0; bb < C::NB; ++bb)
            acc[bb][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pop[bb][pp], acc[bb][e], 0, 0, 0);
        }
      });
    } else {
      const uint32_t av = sb + CC::K_T + 4 * g * CC::ROW + n * CC::VR;
      dev::static_for<0, C::PS>([&](auto ppc) {
        constexpr int pp = decltype(ppc)::value;
        VPieces<CC, pp> vp;
        read_v<CC, pp>(vp, av);
#pragma unroll
        for (int e = 0; e < C::DB; ++e) {
          const bf16x8 va = v_operand(vp, e);
#pragma unroll
          for (int bb = 0; bb < C::NB; ++bb)
            acc[bb][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pop[bb][pp], acc[bb][e], 0, 0, 0);
        }
      });
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // tiles entirely below every column's limit, then the rest
  const int T_open = min(it1, max(it0, mask_from / C::NT));
  int it = it0;
  for (; it < T_open; ++it) tile_step(it, std::false_type{});
  for (; it < it1; ++it) tile_step(it, std::true_type{});

  // totals over the four lane rows (disjoint tokens)
  bool poisoned = __syncthreads_or(bad_page || bad_map) != 0;
#pragma unroll
  for (int bb = 0; bb < C::NB; ++bb) {
    l[bb] += __shfl_xor(l[bb], 16);
    l[bb] += __shfl_xor(l[bb], 32);
  }
  if (slot0 >= 0 && !merge_parts<D, FP8>(p, s_count, acc, m, l, poisoned, slot0, part, parts, kvh, w, lane)) return;

  // the outputs: lane (r, c) holds d = (4 r + j) DB + e of its column
#pragma unroll
  for (int bb = 0; bb < C::NB; ++bb) {
    const float lt = l[bb];
    if (orow[bb] < 0) continue;
    float* o = p.out + orow[bb] * D;
    if constexpr (CC::TRV) {
      // lane (g, n) holds d 16 e + 4 g + j
      const float inv = lt != 0.0f ? 1.0f / lt : 0.0f;
#pragma unroll
      for (int e = 0; e < C::DB; ++e) {
        float r[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = poisoned ? nan : acc[bb][e][j] * inv;
        *reinterpret_cast<f32x4*>(o + 16 * e + 4 * g) = f32x4{r[0], r[1], r[2], r[3]};
      }
    } else {
      // lane (g, n) holds d (4 g + j) DB + e
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float r[C::DB];
#pragma unroll
        for (int e = 0; e < C::DB; ++e) r[e] = poisoned ? nan : (lt != 0.0f ? acc[bb][e][j] / lt : 0.0f);
#pragma unroll
        for (int e = 0; e < C::DB; e += 4)
          *reinterpret_cast<f32x4*>(o + (4 * g + j) * C::DB + e) = f32x4{r[e], r[e + 1], r[e + 2], r[e + 3]};
      }
    }
    if (p.lse != nullptr && g == 0)
      p.lse[orow[bb]] = poisoned ? nan : (lt != 0.0f ? (m[bb] + log2f(lt)) * dev::kLn2 : -__builtin_inff());
  }
}

// Workgroup (t, kv head) with t = blockIdx / Hkv: map entry t.
template <int D, bool FP8, bool INL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(const PrefillParams p) {
  using C = Cfg<D, FP8>;
  static_assert(FP8 || !INL, "inline scales are an fp8 layout");
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::SMEM];
  __shared__ uint32_t s_count;  // a split tile's parts counted in before this one
  prefill_item<D, FP8, INL>(p, blockIdx.x / p.num_kv_heads, blockIdx.x % p.num_kv_heads, smem, s_count);
}

template <int D, bool FP8, bool INL>
hipError_t launch_one(const PrefillParams& p, uint32_t grid, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_kernel<D, FP8, INL>), dim3(grid), dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool FP8, bool INL>
int wgs_one() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_kernel<D, FP8, INL>, kWaves * 64, 0) != hipSuccess)
    return 0;
  return n;
}

template <int D>
int wgs_of(int pool) {
  return pool == kPrefillFp8Inline ? wgs_one<D, true, true>()
         : pool == kPrefillFp8     ? wgs_one<D, true, false>()
                                   : wgs_one<D, false, false>();
}

template <int D>
hipError_t launch_of(const PrefillParams& p, int pool, uint32_t grid, hipStream_t stream) {
  return pool == kPrefillFp8Inline ? launch_one<D, true, true>(p, grid, stream)
         : pool == kPrefillFp8     ? launch_one<D, true, false>(p, grid, stream)
                                   : launch_one<D, false, false>(p, grid, stream);
}

}  // namespace

int prefill_wgs_per_cu(int head_dim, int pool) {
  if (head_dim == 64) return wgs_of<64>(pool);
  if (head_dim == 128) return wgs_of<128>(pool);
  if (head_dim == 256) return wgs_of<256>(pool);
  return 0;
}

hipError_t launch_prefill(const PrefillParams& p, int head_dim, int pool, uint32_t grid, hipStream_t stream) {
  if (head_dim == 64) return launch_of<64>(p, pool, grid, stream);
  if (head_dim == 128) return launch_of<128>(p, pool, grid, stream);
  if (head_dim == 256) return launch_of<256>(p, pool, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace pdattn
