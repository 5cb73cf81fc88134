// gfx950 kernels for paged split-KV GQA decode attention.
//
// partial_kernel: one workgroup per (sequence b, kv head, split) work item
// computes the split for all G query heads of the kv head, so each K/V row
// is read from HBM once per split rather than once per query head (AstrAI
// "CUDA Kernels", GQA head packing in paged prefill; FlashQuant wiki "CUDA
// Kernels", GQA Support). The split is cut into 16-token tiles; wave w of the
// workgroup owns tiles w, w + 4, w + 8, ... and keeps its own online-softmax
// state (FlashQuant wiki, flash_attention.cu, Online Softmax), in base 2
// with the softmax scale pre-multiplied by log2(e) (same page, utils.cuh,
// the exp2/log2(e) trick). The four waves merge their states through LDS at
// the end; a sequence with one split is finished there, otherwise (m, l, acc)
// partials go to the workspace (same page, paged_decode.cu, Partial Output).
//
// Per tile and wave:
//   * page gather: every lane issues 16-byte loads of its K row segment and
//     of its V row chunks, addressed through the block-table slice staged in
//     LDS (page = block_table[pos >> log2 P], slot = pos & (P - 1); same page,
//     paged_decode.cu, Page Table Addressing). The next tile of the wave is
//     loaded into a second register set while the current one is computed.
//   * S = K_tile (16 tokens x d) . Q^T (d x 16, the G heads zero-padded) on
//     v_mfma_f32_16x16x32_bf16: a 16-token x d x G contraction. The lane
//     mapping of the loads is chosen so that each lane's 16 loaded bytes are
//     its MFMA A-operand fragment directly; the head_dim order inside a
//     fragment is the same for Q and K, so the contraction is exact.
//   * softmax on the MFMA result layout (lane: one head, four tokens):
//     tile max by a 4-way local max and two cross-row exchanges, exp2.
//   * p . V on the VALU with fp32 accumulators: lane (row r, chunk c) owns
//     d-chunk c for tokens 4r..4r+3 of each tile; the probabilities of those
//     tokens for head g sit in lane g of the same 16-lane row and arrive with
//     a DPP row broadcast.
//
// fp8 pools: e4m3fn bytes are widened in registers (hardware convert; exact
// in bf16 for the K operand, fp32 for V); the per-(token, kv head) scales are
// folded into the score (k) and the probability (v) instead of being
// multiplied into the elements (OASR "Kernel Layer", FP8 KV variants: one
// fp32 scale per token and kv head).
//
// reduce_kernel: one workgroup of d threads per (b, h) of a multi-split
// sequence: M = max m_s, out = sum 2^(m_s - M) acc_s / sum 2^(m_s - M) l_s,
// lse = ln 2 (M + log2 sum 2^(m_s - M) l_s) (FlashQuant wiki, split_k_reduce.cu,
// Algorithm and Numerical Stability, on un-normalised accumulators).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "kernels.h"

namespace pdattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));

constexpr float kLn2 = 0.69314718055994530942f;

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Value of lane SRC of the caller's 16-lane row (DPP row_newbcast).
template <int SRC>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + SRC, 0xf, 0xf, false));
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

__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
  asm volatile("" ::: "memory");
}

// Wait until at most `ahead` tiles of C loads each are still in flight.
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

__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds, 16, 0, kStreamPolicy);
}
__device__ __forceinline__ void dma4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds, 4, 0, kStreamPolicy);
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
// (the caller has waited for them with wait_tiles).
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

// Token order inside a 16-token tile. MFMA A-row m carries token
// tile_token(m) = m / 4 + 4 (m mod 4), so the result row 4 r + v held by
// 16-lane row r is token r + 4 v: every 16-lane row owns the tokens
// congruent to r mod 4, for the scores as well as for the V rows it reads.
__device__ __forceinline__ int tile_token(int m) { return (m >> 2) + 4 * (m & 3); }

template <int D, int G, bool FP8>
__global__ __launch_bounds__(kWaves * 64) void partial_kernel(DecodeParams p) {
  constexpr int ESZ = FP8 ? 1 : 2;             // bytes per stored element
  constexpr int ROW_BYTES = D * ESZ;           // one (token, kv head) row
  constexpr int KSTEPS = D / 32;               // MFMA k-steps over head_dim
  constexpr int K_LD = ROW_BYTES / 64;         // 16-byte loads per lane per tile, K
  constexpr int V_LD = ROW_BYTES / 64;         // and V (a tile is 16 rows)
  constexpr int C = K_LD + V_LD + (FP8 ? 1 : 0);  // DMA instructions per tile
  constexpr int VE = D / 16;                   // V elements per lane per row
  constexpr int VB = VE * ESZ;                 // V bytes per lane per row
  constexpr int NT = kWaves * 64;
  constexpr int S = kStages;
  // one ring stage: K tile in MFMA-operand lane order, V tile row-major,
  // then (fp8) 64 scale slots: k scales 0..15, v scales 16..31
  constexpr int K_TILE = kTileTokens * ROW_BYTES;
  constexpr int V_TILE = kTileTokens * ROW_BYTES;
  constexpr int STAGE = K_TILE + V_TILE + (FP8 ? 256 : 0);
  constexpr int RING = kWaves * S * STAGE;
  constexpr int MERGE = kWaves * G * (D + 2) * 4;
  constexpr int UNION = RING > MERGE ? RING : MERGE;
  using VVec = typename VChunk<VB>::type;
  static_assert(K_LD >= 1 && (D == 64 || D == 128), "head_dim");
  static_assert(G >= 1 && G <= 16, "group size");
  static_assert(C * (S - 1) < 64, "vmcnt range");

  // LDS: per-wave load rings (reused for the cross-wave merge after the tile
  // loop), then the split's block-table slice.
  __shared__ __attribute__((aligned(16))) unsigned char s_mem[UNION];
  __shared__ int s_pages[kMaxPageList];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int col = lane & 15;   // MFMA column / V chunk index
  const int row = lane >> 4;   // 16-lane row

  // Work item. Hardware hands consecutive workgroup ids to the 8 XCDs in
  // turn; ids x, x + 8, x + 16, ... (one XCD) take the kv heads of one
  // (sequence, split), so the rows of one token that those heads share (the
  // fp8 scales, the block table, q) are fetched into one L2.
  const uint32_t bid = blockIdx.x;
  const uint32_t in_xcd = bid >> 3;
  const int kvh = (int)(in_xcd % (uint32_t)p.num_kv_heads);
  const uint32_t unit = (in_xcd / (uint32_t)p.num_kv_heads) * 8u + (bid & 7u);
  if (unit >= (uint32_t)p.num_units) return;
  const int b = (int)(unit / (uint32_t)p.max_splits);
  const int split = (int)(unit % (uint32_t)p.max_splits);
  const int Hq = p.num_q_heads;
  const int Hkv = p.num_kv_heads;
  const int h0 = kvh * G;
  const int lp = p.page_log2;
  const int P = 1 << lp;

  const int L = __builtin_amdgcn_readfirstlane(p.context_lens[b]);
  const int64_t cap = (int64_t)p.max_pages_per_seq << lp;
  const int nsplit = L > 0 ? (int)(((int64_t)L + p.split_tokens - 1) / p.split_tokens) : 0;
  if (L <= 0 || (int64_t)L > cap || nsplit > p.max_splits) {
    // empty sequence: out = 0, lse = -inf; a length the plan or the block
    // table cannot hold: NaN, and nothing is read.
    if (split == 0) {
      const bool bad = L != 0;
      const float fo = bad ? __builtin_nanf("") : 0.0f;
      const float fl = bad ? __builtin_nanf("") : -__builtin_inff();
      for (int i = tid; i < G * D; i += NT) p.out[((int64_t)b * Hq + h0 + i / D) * D + i % D] = fo;
      if (p.lse != nullptr && tid < G) p.lse[(int64_t)b * Hq + h0 + tid] = fl;
    }
    return;
  }
  if (split >= nsplit) return;

  const int s0 = split * p.split_tokens;
  const int s1 = min(L, s0 + p.split_tokens);
  const int ntiles = (s1 - s0 + kTileTokens - 1) / kTileTokens;
  const int pg0 = s0 >> lp;
  const int npg = ((s1 - 1) >> lp) - pg0 + 1;

  // Stage the block-table slice; an entry outside [0, num_pages) is replaced
  // by page 0 (never read through) and poisons this work item's output.
  int bad = npg > kMaxPageList;
  {
    const int32_t* bt = p.block_table + (int64_t)b * p.max_pages_per_seq + pg0;
    const int n = min(npg, kMaxPageList);
    for (int i = tid; i < n; i += NT) {
      int pg = bt[i];
      if ((unsigned)pg >= (unsigned)p.num_pages) {
        bad = 1;
        pg = 0;
      }
      s_pages[i] = pg;
    }
  }

  // Q as the MFMA B operand: lane (row, col) holds head col (zero for
  // col >= G) at 8 head_dim positions per k-step; dpos() is the order shared
  // with the K fragments.
  auto dpos = [&](int kk) -> int {
    if constexpr (FP8) return (kk >> 1) * 64 + row * 16 + (kk & 1) * 8;
    else return kk * 32 + row * 8;
  };
  bf16x8 qop[KSTEPS];
  {
    const uint16_t* qrow = p.q + ((int64_t)b * Hq + h0 + min(col, G - 1)) * D;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      u32x4 raw = *reinterpret_cast<const u32x4*>(qrow + dpos(kk));
      if (col >= G) raw = u32x4{0u, 0u, 0u, 0u};
      qop[kk] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  __syncthreads();

  auto page_of = [&](int pos) -> int {
    const int idx = min((pos >> lp) - pg0, kMaxPageList - 1);
    return s_pages[idx];
  };
  // (token, kv head) row index of sequence position pos
  auto row_of = [&](int pos) -> int64_t {
    return ((((int64_t)page_of(pos)) << lp) + (pos & (P - 1))) * Hkv + kvh;
  };

  unsigned char* ring = s_mem + wave * (S * STAGE);
  // this wave's tiles: i = wave + k * kWaves, k < nk
  const int nk = wave < ntiles ? (ntiles - 1 - wave) / kWaves + 1 : 0;

  // Issue the C direct-to-LDS loads of local tile k into stage k % S. Rows
  // past the split's last token are clamped onto that token (finite data,
  // masked in the softmax).
  auto issue = [&](int k) {
    unsigned char* st = ring + (k % S) * STAGE;
    const int tb = s0 + (wave + k * kWaves) * kTileTokens;
    {
      // K: lane (row, col) fetches bytes [j*64 + row*16, +16) of token
      // tile_token(col); it lands at j*1024 + lane*16, the lane's own
      // A-operand fragment for k-steps 2j, 2j+1 (fp8) or j (bf16).
      const int pos = min(tb + tile_token(col), s1 - 1);
      const unsigned char* src = p.k + row_of(pos) * ROW_BYTES + row * 16;
#pragma unroll
      for (int j = 0; j < K_LD; ++j) dma16(src + j * 64, st + j * 1024 + lane * 16);
    }
    {
      // V: row-major tile, 64 lanes x 16 bytes per load
#pragma unroll
      for (int j = 0; j < V_LD; ++j) {
        const int byte = j * 1024 + lane * 16;
        const int r = byte / ROW_BYTES;
        const int pos = min(tb + r, s1 - 1);
        dma16(p.v + row_of(pos) * ROW_BYTES + (byte % ROW_BYTES), st + K_TILE + j * 1024 + lane * 16);
      }
    }
    if constexpr (FP8) {
      // scale slot m < 16 holds k_scale of token tile_token(m); slot 16 + m
      // holds its v_scale; lanes 32..63 repeat lanes 0..31
      const int m = lane & 15;
      const int pos = min(tb + tile_token(m), s1 - 1);
      const float* src = ((lane & 16) ? p.v_scale : p.k_scale) + row_of(pos);
      dma4(src, st + K_TILE + V_TILE + lane * 4);
    }
  };

  float m_run = -__builtin_inff();
  float l_run = 0.0f;
  float acc[G][VE];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[g][e] = 0.0f;

  // prologue: fill the ring
#pragma unroll
  for (int k = 0; k < S; ++k)
    if (k < nk) issue(k);

  for (int k = 0; k < nk; ++k) {
    // tiles k+1 .. min(k+S-1, nk-1) may stay in flight
    wait_tiles<C, S>(min(S - 1, nk - 1 - k));
    const unsigned char* st = ring + (k % S) * STAGE;
    u32x4 kf[K_LD];
    VVec vf_raw[4];
    float ks[4], vs[4];
    read_stage<D, FP8>(
        st + lane * 16, st + K_TILE + row * ROW_BYTES + col * VB, st + K_TILE + V_TILE + row * 16, kf, vf_raw,
        ks, vs);
    // the stage's reads have returned (read_stage waits for them): refill it
    if (k + S < nk) issue(k + S);

    const int tb = s0 + (wave + k * kWaves) * kTileTokens;
    // S[t][g]: lane (row, col) holds head col for tokens row + 4 v
    f32x4 Sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      u32x4 kw;
      if constexpr (FP8) {
        const u32x4& c = kf[kk >> 1];
        kw = fp8x8_to_bf16x8(c[(kk & 1) * 2], c[(kk & 1) * 2 + 1]);
      } else {
        kw = kf[kk];
      }
      Sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kw), qop[kk], Sacc, 0, 0, 0);
    }
    float s[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float x = Sacc[v] * p.qk_scale_log2;
      if constexpr (FP8) x *= ks[v];
      s[v] = (tb + row + 4 * v < s1) ? x : -__builtin_inff();
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float pr[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) pr[v] = __builtin_amdgcn_exp2f(s[v] - m_new);
    l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    const bool grew = m_new > m_run;
    m_run = m_new;
    if (__any(grew)) {
      static_for<0, G>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        const float a = row_bcast<g>(alpha);
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[g][e] *= a;
      });
    }
    if constexpr (FP8) {
#pragma unroll
      for (int v = 0; v < 4; ++v) pr[v] *= vs[v];
    }
    // p . V: lane (row, col) takes V row (token) row + 4 j, d-chunk col
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float vf[VE];
      if constexpr (FP8) {
#pragma unroll
        for (int w = 0; w < VB / 4; ++w) {
          const uint32_t x = dword(vf_raw[j], w);
          auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(x, false);
          auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(x, true);
          vf[4 * w + 0] = lo[0];
          vf[4 * w + 1] = lo[1];
          vf[4 * w + 2] = hi[0];
          vf[4 * w + 3] = hi[1];
        }
      } else {
#pragma unroll
        for (int w = 0; w < VB / 4; ++w) {
          const uint32_t x = dword(vf_raw[j], w);
          vf[2 * w + 0] = bf16_lo(x);
          vf[2 * w + 1] = bf16_hi(x);
        }
      }
      const float pj = pr[j];
      static_for<0, G>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        const float pg = row_bcast<g>(pj);
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[g][e] = fmaf(pg, vf[e], acc[g][e]);
      });
    }
  }

  // Sum l and acc over the four rows of the wave (they hold disjoint tokens).
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      float a = acc[g][e];
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      acc[g][e] = a;
    }
  // every wave has drained its ring (the last wait was vmcnt(0)); the ring
  // memory now holds the per-wave states: acc [wave][g][D], m, l [wave][g]
  __syncthreads();
  float* s_acc = reinterpret_cast<float*>(s_mem);
  float* s_m = s_acc + kWaves * G * D;
  float* s_l = s_m + kWaves * G;
  if (row == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < VE; ++e) s_acc[(wave * G + g) * D + col * VE + e] = acc[g][e];
    if (col < G) {
      s_m[wave * G + col] = m_run;
      s_l[wave * G + col] = l_run;
    }
  }
  const int any_bad = __syncthreads_or(bad);

  // Merge the waves' states (a wave without tiles has m = -inf, l = acc = 0).
  for (int idx = tid; idx < G * D; idx += NT) {
    const int g = idx / D;
    const int d = idx % D;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w * G + g]);
    float A = 0.0f, Ls = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(s_m[w * G + g] - M);
      A = fmaf(f, s_acc[(w * G + g) * D + d], A);
      Ls = fmaf(f, s_l[w * G + g], Ls);
    }
    const int64_t bh = (int64_t)b * Hq + h0 + g;
    const float nan = __builtin_nanf("");
    if (nsplit == 1) {
      p.out[bh * D + d] = any_bad ? nan : A / Ls;
      if (d == 0 && p.lse != nullptr) p.lse[bh] = any_bad ? nan : (M + log2f(Ls)) * kLn2;
    } else {
      const int64_t pi = bh * p.max_splits + split;
      p.part_acc[pi * D + d] = any_bad ? nan : A;
      if (d == 0) {
        p.part_ml[pi * 2 + 0] = any_bad ? 0.0f : M;
        p.part_ml[pi * 2 + 1] = any_bad ? nan : Ls;
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(D) void reduce_kernel(ReduceParams p) {
  const int64_t bh = blockIdx.x;
  const int b = (int)(bh / p.num_q_heads);
  const int d = threadIdx.x;
  const int L = p.context_lens[b];
  const int64_t cap = (int64_t)p.max_pages_per_seq << p.page_log2;
  if (L <= 0 || (int64_t)L > cap) return;
  const int nsplit = (int)(((int64_t)L + p.split_tokens - 1) / p.split_tokens);
  if (nsplit <= 1 || nsplit > p.max_splits) return;
  const float* ml = p.part_ml + bh * p.max_splits * 2;
  const float* pa = p.part_acc + bh * p.max_splits * D + d;
  float M = -__builtin_inff();
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[2 * s]);
  float A = 0.0f, Ls = 0.0f;
  for (int s = 0; s < nsplit; ++s) {
    const float f = __builtin_amdgcn_exp2f(ml[2 * s] - M);
    A = fmaf(f, pa[(int64_t)s * D], A);
    Ls = fmaf(f, ml[2 * s + 1], Ls);
  }
  p.out[bh * D + d] = A / Ls;
  if (d == 0 && p.lse != nullptr) p.lse[bh] = (M + log2f(Ls)) * kLn2;
}

template <int D, int G, bool FP8>
hipError_t launch_one(const DecodeParams& p, uint32_t grid, hipStream_t stream) {
  hipLaunchKernelGGL((partial_kernel<D, G, FP8>), dim3(grid), dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool FP8>
hipError_t launch_group(const DecodeParams& p, int group, uint32_t grid, hipStream_t stream) {
  switch (group) {
    case 1: return launch_one<D, 1, FP8>(p, grid, stream);
    case 2: return launch_one<D, 2, FP8>(p, grid, stream);
    case 4: return launch_one<D, 4, FP8>(p, grid, stream);
    case 8: return launch_one<D, 8, FP8>(p, grid, stream);
    case 16: return launch_one<D, 16, FP8>(p, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_partial(const DecodeParams& p, int head_dim, int group, bool fp8, uint32_t grid,
                          hipStream_t stream) {
  if (head_dim == 64) return fp8 ? launch_group<64, true>(p, group, grid, stream)
                                 : launch_group<64, false>(p, group, grid, stream);
  if (head_dim == 128) return fp8 ? launch_group<128, true>(p, group, grid, stream)
                                  : launch_group<128, false>(p, group, grid, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_reduce(const ReduceParams& p, int head_dim, uint32_t grid, hipStream_t stream) {
  if (head_dim == 64) {
    hipLaunchKernelGGL(reduce_kernel<64>, dim3(grid), dim3(64), 0, stream, p);
  } else if (head_dim == 128) {
    hipLaunchKernelGGL(reduce_kernel<128>, dim3(grid), dim3(128), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pdattn
