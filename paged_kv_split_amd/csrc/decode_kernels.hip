// gfx950 kernels for paged split-KV GQA decode attention.
//
// decode_kernel: a persistent grid sized to the GPU's resident capacity. The
// KV work of one step is the list of (sequence b, kv head) pairs, each cut
// into 16-token tiles; the pairs are laid end to end (b major, kv head minor)
// and every wave of the grid takes an equal contiguous range of that tile
// list. A wave therefore streams one long run of tiles, crossing pair
// boundaries, and no workgroup waits for the dispatcher: flash-decoding's
// split of the KV range (FlashQuant wiki "CUDA Kernels", paged_decode.cu:
// Grid, Partial Output) with the split points placed by equal work rather
// than by a fixed count per sequence (Atlas "CUDA Kernel Engineering",
// kernel inventory: adaptive split count; OASR "Kernel Layer", Fused
// attention: splits derived from shape and machine only).
//
// For each pair it visits, a wave computes all G query heads of the kv head,
// so a K/V row is read once per step rather than once per query head (AstrAI
// "CUDA Kernels", GQA head packing; FlashQuant wiki, GQA Support), keeping an
// online-softmax state (FlashQuant wiki, flash_attention.cu, Online Softmax)
// in base 2 with the scale pre-multiplied by log2(e) (same page, utils.cuh,
// the exp2/log2(e) trick). A pair the wave covers whole is finished and
// written to out; a pair cut by a wave boundary leaves an (m, l, acc) record
// per piece, and the wave holding the pair's last tile leaves a descriptor
// that the merge kernel follows.
//
// Per tile and wave:
//   * page gather (page = block_table[pos >> log2 P], slot = pos & (P - 1);
//     FlashQuant wiki, paged_decode.cu, Page Table Addressing): the wave's
//     block-table entries are staged in LDS; each tile's K rows, V rows and
//     fp8 scales travel by 16-byte (4-byte) direct-to-LDS loads into a
//     per-wave ring of kStages tiles, non-temporal, waited with explicit
//     vmcnt counts.
//   * S = K_tile (16 tokens x d) . Q^T (d x 16, the G heads zero-padded) on
//     v_mfma_f32_16x16x32_bf16: a 16-token x d x G contraction. The K tile
//     lands in LDS already in A-operand lane order; the head_dim order inside
//     a fragment is the same for Q and K, so the contraction is exact.
//   * softmax on the MFMA result layout (lane: one head, four tokens):
//     tile max by a 4-way local max and two cross-row exchanges, exp2.
//   * p . V on the VALU with fp32 accumulators: lane (row r, chunk c) owns
//     d-chunk c for tokens r, r+4, r+8, r+12 of each tile; their
//     probabilities for head g sit in lane g of the same 16-lane row and
//     arrive with a DPP row broadcast.
//
// fp8 pools: e4m3fn bytes are widened in registers (hardware convert; exact
// in bf16 for the K operand, fp32 for V); the per-(token, kv head) scales are
// folded into the score (k) and the probability (v) instead of being
// multiplied into the elements (OASR "Kernel Layer", FP8 KV variants: one
// fp32 scale per token and kv head).
//
// merge_kernel: one wave per descriptor: M = max m_s, out = sum 2^(m_s - M)
// acc_s / sum 2^(m_s - M) l_s, lse = ln 2 (M + log2 sum 2^(m_s - M) l_s)
// (FlashQuant wiki, split_k_reduce.cu, Algorithm and Numerical Stability,
// on un-normalised accumulators).

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


// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ long long wave_incl_scan(long long v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Range [t0, t1) of the tile list owned by worker w of nw, T tiles in all.
__device__ __forceinline__ void worker_range(long long w, long long nw, long long T, long long& t0, long long& t1) {
  t0 = w * T / nw;
  t1 = (w + 1) * T / nw;
}

template <int D, int G, bool FP8>
__global__ __launch_bounds__(kWaves * 64) void decode_kernel(DecodeParams p) {
  constexpr int ESZ = FP8 ? 1 : 2;             // bytes per stored element
  constexpr int ROW_BYTES = D * ESZ;           // one (token, kv head) row
  constexpr int KSTEPS = D / 32;               // MFMA k-steps over head_dim
  constexpr int K_LD = ROW_BYTES / 64;         // 16-byte loads per lane per tile, K
  constexpr int V_LD = ROW_BYTES / 64;         // and V (a tile is 16 rows)
  constexpr int C = K_LD + V_LD + (FP8 ? 1 : 0);  // direct-to-LDS loads per tile
  constexpr int VE = D / 16;                   // V elements per lane per row
  constexpr int VB = VE * ESZ;                 // V bytes per lane per row
  constexpr int NT = kWaves * 64;
  constexpr int S = kStages;
  // one ring stage: K tile in MFMA-operand lane order, V tile row-major,
  // then (fp8) 64 scale slots: k scales 0..15, v scales 16..31
  constexpr int K_TILE = kTileTokens * ROW_BYTES;
  constexpr int V_TILE = kTileTokens * ROW_BYTES;
  constexpr int STAGE = K_TILE + V_TILE + (FP8 ? 256 : 0);
  constexpr int RF = (int)record_floats(D, G);
  using VVec = typename VChunk<VB>::type;
  static_assert(K_LD >= 1 && (D == 64 || D == 128), "head_dim");
  static_assert(G >= 1 && G <= 16, "group size");
  static_assert(C * (S - 1) < 64, "vmcnt range");

  // LDS: per-wave load rings and block-table buffers; the length-scan scratch.
  __shared__ __attribute__((aligned(16))) unsigned char s_ring[kWaves][S * STAGE];
  __shared__ int s_pages[kWaves][kPagesPerWave];
  __shared__ long long s_wsum[kWaves];
  __shared__ int s_loc[kWaves][4];  // first pair of each wave: b, kv head, tile, valid

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;   // MFMA column / V chunk index
  const int row = lane >> 4;   // 16-lane row

  const int B = p.batch;
  const int Hq = p.num_q_heads;
  const int Hkv = p.num_kv_heads;
  const int lp = p.page_log2;
  const int P = 1 << lp;
  const long long cap = (long long)p.max_pages_per_seq << lp;
  const long long NW = p.num_workers;
  auto tiles_of = [&](int L) -> long long { return (L > 0 && (long long)L <= cap) ? (L + kTileTokens - 1) / kTileTokens : 0; };

  // ---- 1. tile counts of the sequences, prefix-summed across the workgroup
  const int CH = (B + NT - 1) / NT;
  const int b_lo = min(B, tid * CH);
  const int b_hi = min(B, b_lo + CH);
  long long mine = 0;
  for (int b = b_lo; b < b_hi; ++b) mine += tiles_of(p.context_lens[b]);
  const long long incl = wave_incl_scan(mine, lane);
  if (lane == 63) s_wsum[wave] = incl;
  if (tid < kWaves) s_loc[tid][3] = 0;
  __syncthreads();
  long long before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const long long x = s_wsum[w];
    before += w < wave ? x : 0;
    total += x;
  }
  const long long T = total * Hkv;             // tiles of all (b, kv head) pairs
  const long long pre = before + incl - mine;  // tiles per kv head before b_lo

  // ---- 2. place the waves of this workgroup; empty or over-long sequences
  // get their outputs here (out = 0, lse = -inf; NaN when the length does
  // not fit the block table)
  for (int lw = 0; lw < kWaves; ++lw) {
    const long long gw = (long long)blockIdx.x * kWaves + lw;
    if (gw >= NW) break;
    long long ts, te;
    worker_range(gw, NW, T, ts, te);
    if (ts >= te) continue;
    long long run = pre;
    for (int b = b_lo; b < b_hi; ++b) {
      const long long nt = tiles_of(p.context_lens[b]);
      if (nt > 0 && Hkv * run <= ts && ts < Hkv * (run + nt)) {
        const long long r = ts - Hkv * run;
        s_loc[lw][0] = b;
        s_loc[lw][1] = (int)(r / nt);
        s_loc[lw][2] = (int)(r % nt);
        s_loc[lw][3] = 1;
      }
      run += nt;
    }
  }
  if (blockIdx.x == 0) {
    for (int b = b_lo; b < b_hi; ++b) {
      const int L = p.context_lens[b];
      if (tiles_of(L) > 0) continue;
      const bool bad = L != 0;
      const float fo = bad ? __builtin_nanf("") : 0.0f;
      for (int i = 0; i < Hq * D; ++i) p.out[(long long)b * Hq * D + i] = fo;
      if (p.lse != nullptr)
        for (int h = 0; h < Hq; ++h) p.lse[(long long)b * Hq + h] = bad ? __builtin_nanf("") : -__builtin_inff();
    }
  }
  __syncthreads();

  // ---- 3. this wave's run of tiles
  const long long gw = (long long)blockIdx.x * kWaves + wave;
  if (gw >= NW) return;
  long long t0, t1;
  worker_range(gw, NW, T, t0, t1);
  int dsc[kDescWords] = {0, 0, 0, 0, 0, 0, 0, 0};

  unsigned char* ring = &s_ring[wave][0];
  int* pages = &s_pages[wave][0];
  if (t0 >= t1) {
    // no tiles: an empty record (m = -inf, l = acc = 0) in slot 0, read by
    // the merge of the pair this worker falls inside
    float* r = p.rec + gw * 2 * RF;
    for (int i = lane; i < RF; i += 64) r[i] = i < G ? -__builtin_inff() : 0.0f;
  }

  if (t0 < t1 && s_loc[wave][3]) {
    int b = __builtin_amdgcn_readfirstlane(s_loc[wave][0]);
    int kvh = __builtin_amdgcn_readfirstlane(s_loc[wave][1]);
    int j = __builtin_amdgcn_readfirstlane(s_loc[wave][2]);
    long long remaining = t1 - t0;
    bool first = true;
    while (remaining > 0) {
      const int L = __builtin_amdgcn_readfirstlane(p.context_lens[b]);
      const int nt = (L + kTileTokens - 1) / kTileTokens;
      const int seg = (int)min((long long)(nt - j), remaining);
      const bool cut_start = j > 0;
      const bool reaches_end = j + seg == nt;
      const int h0 = kvh * G;
      const int s0 = j * kTileTokens;
      const int s1 = min(L, (j + seg) * kTileTokens);

      // Q as the MFMA B operand: lane (row, col) holds head col (zero for
      // col >= G) at 8 head_dim positions per k-step; dpos() is the order
      // shared with the K fragments.
      auto dpos = [&](int kk) -> int {
        if constexpr (FP8) return (kk >> 1) * 64 + row * 16 + (kk & 1) * 8;
        else return kk * 32 + row * 8;
      };
      bf16x8 qop[KSTEPS];
      {
        const uint16_t* qrow = p.q + ((long long)b * Hq + h0 + min(col, G - 1)) * D;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          u32x4 raw = *reinterpret_cast<const u32x4*>(qrow + dpos(kk));
          if (col >= G) raw = u32x4{0u, 0u, 0u, 0u};
          qop[kk] = __builtin_bit_cast(bf16x8, raw);
        }
      }

      float m_run = -__builtin_inff();
      float l_run = 0.0f;
      float acc[G][VE];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[g][e] = 0.0f;
      int bad = 0;

      // sub-runs of at most kPagesPerWave pages (tile-aligned)
      for (int c0 = s0; c0 < s1;) {
        const int pg0 = c0 >> lp;
        const int c1 = (int)min((long long)s1, (long long)(pg0 + kPagesPerWave) << lp);
        const int npg = ((c1 - 1) >> lp) - pg0 + 1;
        {
          const int32_t* bt = p.block_table + (long long)b * p.max_pages_per_seq + pg0;
          for (int i = lane; i < npg; i += 64) {
            int pg = bt[i];
            if ((unsigned)pg >= (unsigned)p.num_pages) {
              bad = 1;
              pg = 0;
            }
            pages[i] = pg;
          }
        }
        // (token, kv head) row index of sequence position pos
        auto row_of = [&](int pos) -> long long {
          return ((((long long)pages[(pos >> lp) - pg0]) << lp) + (pos & (P - 1))) * Hkv + kvh;
        };
        const int nk = (c1 - c0 + kTileTokens - 1) / kTileTokens;

        // Issue the C direct-to-LDS loads of tile k of this sub-run into stage
        // k % S. Rows past the pair's last token are clamped onto that token
        // (finite data, masked in the softmax).
        auto issue = [&](int k) {
          unsigned char* st = ring + (k % S) * STAGE;
          const int tb = c0 + k * kTileTokens;
          {
            // K: lane (row, col) fetches bytes [j*64 + row*16, +16) of token
            // tile_token(col); it lands at j*1024 + lane*16, the lane's own
            // A-operand fragment for k-steps 2j, 2j+1 (fp8) or j (bf16).
            const int pos = min(tb + tile_token(col), s1 - 1);
            const unsigned char* src = p.k + row_of(pos) * ROW_BYTES + row * 16;
#pragma unroll
            for (int jj = 0; jj < K_LD; ++jj) dma16(src + jj * 64, st + jj * 1024 + lane * 16);
          }
#pragma unroll
          for (int jj = 0; jj < V_LD; ++jj) {
            // V: row-major tile, 64 lanes x 16 bytes per load
            const int byte = jj * 1024 + lane * 16;
            const int pos = min(tb + byte / ROW_BYTES, s1 - 1);
            dma16(p.v + row_of(pos) * ROW_BYTES + (byte % ROW_BYTES), st + K_TILE + jj * 1024 + lane * 16);
          }
          if constexpr (FP8) {
            // scale slot m < 16 holds k_scale of token tile_token(m); slot
            // 16 + m holds its v_scale; lanes 32..63 repeat lanes 0..31
            const int m = lane & 15;
            const int pos = min(tb + tile_token(m), s1 - 1);
            const float* src = ((lane & 16) ? p.v_scale : p.k_scale) + row_of(pos);
            dma4(src, st + K_TILE + V_TILE + lane * 4);
          }
        };

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
          read_stage<D, FP8>(st + lane * 16, st + K_TILE + row * ROW_BYTES + col * VB,
                             st + K_TILE + V_TILE + row * 16, kf, vf_raw, ks, vs);
          // the stage's reads have returned (read_stage waits for them): refill it
          if (k + S < nk) issue(k + S);

          const int tb = c0 + k * kTileTokens;
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
          for (int jj = 0; jj < 4; ++jj) {
            float vf[VE];
            if constexpr (FP8) {
#pragma unroll
              for (int w = 0; w < VB / 4; ++w) {
                const uint32_t x = dword(vf_raw[jj], w);
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
                const uint32_t x = dword(vf_raw[jj], w);
                vf[2 * w + 0] = bf16_lo(x);
                vf[2 * w + 1] = bf16_hi(x);
              }
            }
            const float pj = pr[jj];
            static_for<0, G>([&](auto gc) {
              constexpr int g = decltype(gc)::value;
              const float pg = row_bcast<g>(pj);
#pragma unroll
              for (int e = 0; e < VE; ++e) acc[g][e] = fmaf(pg, vf[e], acc[g][e]);
            });
          }
        }
        c0 = c1;
      }

      // ---- finish the piece: sum l and acc over the four rows (disjoint
      // tokens); every row then holds the totals
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
      const bool poisoned = __any(bad);
      const float nan = __builtin_nanf("");
      if (!cut_start && reaches_end) {
        // the whole pair: out = acc / l, lse = ln 2 (m + log2 l); row r
        // writes the heads g with g mod 4 == r
        static_for<0, G>([&](auto gc) {
          constexpr int g = decltype(gc)::value;
          const float lg = row_bcast<g>(l_run);
          if (row == (g & 3)) {
            float* o = p.out + ((long long)b * Hq + h0 + g) * D + col * VE;
#pragma unroll
            for (int e = 0; e < VE; ++e) o[e] = poisoned ? nan : acc[g][e] / lg;
          }
        });
        if (p.lse != nullptr && row == 0 && col < G)
          p.lse[(long long)b * Hq + h0 + col] = poisoned ? nan : (m_run + log2f(l_run)) * kLn2;
      } else {
        // a piece of a cut pair: record (m, l, acc); slot 0 for the wave's
        // first piece, 1 for its last
        float* r = p.rec + (gw * 2 + (first ? 0 : 1)) * RF;
        static_for<0, G>([&](auto gc) {
          constexpr int g = decltype(gc)::value;
          if (row == (g & 3)) {
            float* o = r + 2 * G + g * D + col * VE;
#pragma unroll
            for (int e = 0; e < VE; ++e) o[e] = poisoned ? nan : acc[g][e];
          }
        });
        if (row == 0 && col < G) {
          r[col] = poisoned ? 0.0f : m_run;
          r[G + col] = poisoned ? nan : l_run;
        }
        if (cut_start && reaches_end) {
          // this wave holds the pair's last tile (only possible for its first
          // piece): describe the pieces for the merge
          const long long pair_start = t0 - j;
          // first worker whose range reaches pair_start
          const long long wf = ((pair_start + 1) * NW + T - 1) / T - 1;
          long long wf0, wf1;
          worker_range(wf, NW, T, wf0, wf1);
          dsc[0] = 1;
          dsc[1] = b;
          dsc[2] = kvh;
          dsc[3] = (int)wf;
          dsc[4] = wf0 == pair_start ? 0 : 1;
          dsc[5] = (int)(T & 0xffffffffll);
          dsc[6] = (int)(T >> 32);
        }
      }

      remaining -= seg;
      first = false;
      // next pair with tiles
      j = 0;
      if (++kvh == Hkv) {
        kvh = 0;
        do {
          ++b;
        } while (remaining > 0 && b < B && tiles_of(__builtin_amdgcn_readfirstlane(p.context_lens[b])) == 0);
        if (b >= B) break;
      }
    }
  }
  if (lane < kDescWords) p.desc[gw * kDescWords + lane] = dsc[lane];
}

// One workgroup per worker descriptor; only the descriptors of cut pairs
// are valid. Every worker wf .. w holds a record for the pair (a worker
// with an empty tile range holds the empty record m = -inf, l = acc = 0).
// Pass 1 takes M[g] = max m over the pieces; in pass 2 the four waves take
// every fourth piece and each lane accumulates its own slice of one head's
// accumulator with vector loads, so the piece loop keeps many loads in
// flight; the waves' sums meet in LDS.
template <int D, int G>
__global__ __launch_bounds__(kWaves * 64) void merge_kernel(MergeParams p) {
  constexpr int RF = (int)record_floats(D, G);
  constexpr int NT = kWaves * 64;
  constexpr int EPL = G * D / 64;      // accumulator elements per lane
  constexpr int LPH = D / EPL;         // lanes per head
  static_assert(EPL >= 1 && D % EPL == 0, "lane slice");
  __shared__ float s_red[kWaves][G];
  __shared__ float s_M[G];
  __shared__ __attribute__((aligned(16))) float s_acc[kWaves][G * D];
  __shared__ float s_l[kWaves][G];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const long long w = blockIdx.x;
  if (w >= p.num_workers) return;
  const int* dsc = p.desc + w * kDescWords;
  if (dsc[0] != 1) return;
  const int b = dsc[1];
  const int kvh = dsc[2];
  const long long wf = dsc[3];
  const int slot_first = dsc[4];
  const long long n = w - wf + 1;  // pieces: workers wf .. w
  auto piece = [&](long long i) -> const float* {
    return p.rec + ((wf + i) * 2 + (i == 0 ? slot_first : 0)) * RF;
  };

  // pass 1
  float mloc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) mloc[g] = -__builtin_inff();
  for (long long i = tid; i < n; i += NT) {
    const float* r = piece(i);
#pragma unroll
    for (int g = 0; g < G; ++g) mloc[g] = fmaxf(mloc[g], r[g]);
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float x = mloc[g];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    if (lane == 0) s_red[wave][g] = x;
  }
  __syncthreads();
  if (tid < G) {
    float x = s_red[0][tid];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) x = fmaxf(x, s_red[k][tid]);
    s_M[tid] = x;
  }
  __syncthreads();

  // pass 2
  const int g = lane / LPH;             // this lane's head
  const int e0 = lane * EPL;            // first element of its slice (g * D + ...)
  const float Mg = s_M[g];
  float A[EPL];
#pragma unroll
  for (int k = 0; k < EPL; ++k) A[k] = 0.0f;
  float lsum = 0.0f;
#pragma unroll 4
  for (long long i = wave; i < n; i += kWaves) {
    const float* r = piece(i);
    const float wgt = __builtin_amdgcn_exp2f(r[g] - Mg);
    lsum = fmaf(wgt, r[G + g], lsum);
    const float* a = r + 2 * G + e0;
#pragma unroll
    for (int k = 0; k < EPL; ++k) A[k] = fmaf(wgt, a[k], A[k]);
  }
#pragma unroll
  for (int k = 0; k < EPL; ++k) s_acc[wave][e0 + k] = A[k];
  if (lane % LPH == 0) s_l[wave][g] = lsum;
  __syncthreads();
  for (int e = tid; e < G * D; e += NT) {
    const int gg = e / D;
    float Av = 0.0f, Ls = 0.0f;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) {
      Av += s_acc[q][e];
      Ls += s_l[q][gg];
    }
    const long long bh = (long long)b * p.num_q_heads + kvh * G + gg;
    p.out[bh * D + (e % D)] = Av / Ls;
    if (e % D == 0 && p.lse != nullptr) p.lse[bh] = (s_M[gg] + log2f(Ls)) * kLn2;
  }
}

template <int D, int G, bool FP8>
hipError_t launch_one(const DecodeParams& p, uint32_t grid, hipStream_t stream) {
  hipLaunchKernelGGL((decode_kernel<D, G, FP8>), dim3(grid), dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D, int G, bool FP8>
int occupancy_one() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<D, G, FP8>, kWaves * 64, 0) != hipSuccess)
    return 0;
  return n;
}

template <int D, bool FP8>
int occupancy_group(int group) {
  switch (group) {
    case 1: return occupancy_one<D, 1, FP8>();
    case 2: return occupancy_one<D, 2, FP8>();
    case 4: return occupancy_one<D, 4, FP8>();
    case 8: return occupancy_one<D, 8, FP8>();
    case 16: return occupancy_one<D, 16, FP8>();
    default: return 0;
  }
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

template <int D>
hipError_t launch_merge_d(const MergeParams& p, int group, uint32_t grid, hipStream_t stream) {
  // one workgroup per worker descriptor
  switch (group) {
    case 1: hipLaunchKernelGGL((merge_kernel<D, 1>), dim3(grid), dim3(kWaves * 64), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((merge_kernel<D, 2>), dim3(grid), dim3(kWaves * 64), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((merge_kernel<D, 4>), dim3(grid), dim3(kWaves * 64), 0, stream, p); break;
    case 8: hipLaunchKernelGGL((merge_kernel<D, 8>), dim3(grid), dim3(kWaves * 64), 0, stream, p); break;
    case 16: hipLaunchKernelGGL((merge_kernel<D, 16>), dim3(grid), dim3(kWaves * 64), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int decode_wgs_per_cu(int head_dim, int group, bool fp8) {
  if (head_dim == 64) return fp8 ? occupancy_group<64, true>(group) : occupancy_group<64, false>(group);
  if (head_dim == 128) return fp8 ? occupancy_group<128, true>(group) : occupancy_group<128, false>(group);
  return 0;
}

hipError_t launch_decode(const DecodeParams& p, int head_dim, int group, bool fp8, uint32_t grid,
                         hipStream_t stream) {
  if (head_dim == 64) return fp8 ? launch_group<64, true>(p, group, grid, stream)
                                 : launch_group<64, false>(p, group, grid, stream);
  if (head_dim == 128) return fp8 ? launch_group<128, true>(p, group, grid, stream)
                                  : launch_group<128, false>(p, group, grid, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const MergeParams& p, int head_dim, int group, uint32_t grid, hipStream_t stream) {
  if (head_dim == 64) return launch_merge_d<64>(p, group, grid, stream);
  if (head_dim == 128) return launch_merge_d<128>(p, group, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace pdattn
