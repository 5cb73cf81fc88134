// gfx950 kernels of the TQ4 compressed KV cache (FlashQuant wiki "CUDA
// Kernels": compress.cu, decompress.cu, fused_tq_attention.cu,
// paged_decode.cu, split_k_reduce.cu).
//
// Cache row of one (token, kv head), d + 8 bytes (paged_decode.cu, KV Cache
// Byte Layout): K codes (d/2 bytes) | K norm (fp32) | V codes (d/2 bytes) |
// V norm (fp32). Pages are head-major: row (page * Hkv + kvh) * P + slot, so
// the 16 rows of one 16-token tile are one contiguous block of 16 (d + 8)
// bytes (two blocks of 8 rows for P = 8).
//
// Codes (compress.cu, Algorithm): x_hat = x / (||x|| + 1e-10), y = R x_hat,
// code_i = #{boundaries b : b <= y_i}; byte j = code_2j << 4 | code_2j+1. A
// byte expands (decompress.cu, Sequential Layout) to element j (high
// nibble) and element d/2 + j (low nibble) of the row in the "sequential"
// rotated space, i.e. the rotation whose row j is R[2j] and whose row
// d/2 + j is R[2j + 1]. Attention runs in that space (fused_tq_attention.cu,
// Input/Output: q pre-rotated, output rotated back).
//
// tq4_append_kernel: 16 row vectors (the K and V rows of 8 (token, kv head)
//   pairs) per workgroup: norms by wave reductions and x_hat in LDS; thread
//   t forms rotated coordinate t mod D of several vectors (each rotation row
//   read once per 16 vectors) and counts the boundaries; then the packed
//   bytes and the norms are stored.
// tq4_rotate_q_kernel: q into the sequential rotated space, rounded to fp16
//   (the pages' rotated queries are 16-bit; fp16 keeps 11 significant bits).
// tq4_decode_kernel: a persistent grid; a work item is a run of 16-token
//   tiles of one (sequence, kv head) pair (paged_decode.cu, split-K over the
//   KV range, Partial Output), all G query heads at once. Per tile and wave:
//     * the tile block arrives by 16-byte non-temporal loads into registers,
//       two tiles ahead, and is written to the wave's LDS buffer;
//     * every code byte is looked up in a 256-entry LDS table whose entry is
//       the 16-bit pair (centroid[high nibble], centroid[low nibble]) — the
//       bytes' two elements in one 4-byte read (decompress.cu, Centroids in
//       shared memory); the table is held in 16 copies, entry v of copy c at
//       word 16 v + c, lane l reading copy l mod 16;
//     * S = K . Q^T on v_mfma_f32_16x16x32_f16 (K centroids and q in fp16,
//       whose 2^-11 rounding keeps the scores close; the norm is applied in
//       fp32): lane (token m, group r) builds its A operand from 4 code
//       bytes per 32-wide k-block (each lookup fills two k slots); Q's B
//       operand takes the same elements;
//     * the norms scale the scores (k) and the probabilities (v) instead of
//       the elements (fused_tq_attention.cu, the decompress * norm step);
//       online softmax in base 2 (flash_attention.cu, Online Softmax) with
//       a lazily moved running max;
//     * O^T += V^T . P on v_mfma_f32_16x16x32_bf16 (V centroids and the
//       norm-weighted probabilities in bf16, for the norms' range; two tiles
//       per product, the k slots of the second tile zero for a lone one): the
//       probabilities are already in B-operand order; lane (d row m, group
//       r) looks up the code bytes m * d/32 .. of tokens 4 r .. 4 r + 3,
//       and each lookup feeds the A operands of two d blocks (the high
//       nibble's element j, the low nibble's d/2 + j).
//   Each work item leaves (m, l, acc) per head in the workspace.
// tq4_merge_out_kernel: 8 (sequence, q head) rows per workgroup: one wave
//   per row merges the pair's work items by log-sum-exp (split_k_reduce.cu,
//   Algorithm) into LDS, then the rows are rotated back to model space.

#include "tq4.h"

#include "tile_ops.h"

namespace pdattn {
namespace {

using namespace dev;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kNormEps = 1e-10f;
constexpr int kTableCopies = 16;

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), f16x2));
}

// Max over the four 16-lane groups (lanes c, c + 16, c + 32, c + 48) by the
// gfx950 lane swaps (permlane16 swaps the middle groups' halves, permlane32
// the two halves: with both operands x, a lane's two results are its own
// value and its partner's): plain VALU, no LDS round trip.
__device__ __forceinline__ float max_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Number of the 15 sorted boundaries b with b <= y.
__device__ __forceinline__ uint32_t code_of(float y, const float* bnd) {
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 15; ++i) c += y >= bnd[i] ? 1u : 0u;
  return c;
}

// ---- compress and scatter --------------------------------------------------

constexpr int kAppendVecs = 16;  // row vectors per append workgroup

// Vector v of the append is (token v / (2 Hkv), kv head (v / 2) mod Hkv,
// K if v is even else V). A workgroup compresses kAppendVecs of them:
// wave w normalises vectors w, w + 4, ... into LDS (norm by a wave
// reduction); thread t then owns rotated coordinate i = t mod D of vectors
// t / D, t / D + 256 / D, ..., reading rotation row R[i] once for them, and
// leaves the codes in LDS; last, the packed bytes and norms are stored.
template <int D>
__global__ __launch_bounds__(256) void tq4_append_kernel(const Tq4AppendParams p) {
  constexpr int H = D / 2;
  constexpr int RB = D + 8;
  constexpr int EPL = D / 64;
  constexpr int TPC = 256 / D;                 // threads per coordinate
  constexpr int VPT = kAppendVecs / TPC;       // vectors per thread
  __shared__ __attribute__((aligned(16))) float s_x[kAppendVecs][D];
  __shared__ float s_norm[kAppendVecs];
  __shared__ uint8_t s_code[kAppendVecs][D];
  __shared__ long long s_row[kAppendVecs];     // destination byte offset, or -1
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int P = 1 << p.page_log2;
  const long long nvec = (long long)p.num_tokens * p.num_kv_heads * 2;
  for (long long v0 = (long long)blockIdx.x * kAppendVecs; v0 < nvec; v0 += (long long)gridDim.x * kAppendVecs) {
    // 1. norms and x_hat
    for (int lv = wave; lv < kAppendVecs; lv += 4) {
      const long long v = v0 + lv;
      long long dst = -1;
      float x[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[e] = 0.0f;
      if (v < nvec) {
        const int kind = (int)(v & 1);
        const long long th = v >> 1;           // token * Hkv + kv head
        const int t = (int)(th / p.num_kv_heads);
        const int kvh = (int)(th % p.num_kv_heads);
        const int s = p.token_seq[t];
        const int pos = p.token_pos[t];
        if (s >= 0 && s < p.batch && pos >= 0 && (pos >> p.page_log2) < p.max_pages_per_seq) {
          const int page = p.block_table[(long long)s * p.max_pages_per_seq + (pos >> p.page_log2)];
          if (page >= 0 && page < p.num_pages)
            dst = (((long long)page * p.num_kv_heads + kvh) * P + (pos & (P - 1))) * RB + (kind ? H + 4 : 0);
        }
        const uint16_t* src = (kind ? p.v_new : p.k_new) + th * D;
#pragma unroll
        for (int e = 0; e < EPL; ++e) x[e] = __uint_as_float((uint32_t)src[lane + 64 * e] << 16);
      }
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) ss += x[e] * x[e];
      const float norm = sqrtf(wave_sum(ss));
      const float den = norm + kNormEps;
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_x[lv][lane + 64 * e] = x[e] / den;
      if (lane == 0) {
        s_norm[lv] = norm;
        s_row[lv] = dst;
      }
    }
    __syncthreads();
    // 2. y_i = R[i] . x_hat and its code, for this thread's vectors
    {
      const int i = tid % D;
      const int vs = tid / D;
      const float* rrow = p.rotation + (long long)i * D;
      float y[VPT];
#pragma unroll
      for (int u = 0; u < VPT; ++u) y[u] = 0.0f;
#pragma unroll 1
      for (int k0 = 0; k0 < D; k0 += 32) {
        f32x4 a[8];
#pragma unroll
        for (int w = 0; w < 8; ++w) a[w] = *reinterpret_cast<const f32x4*>(rrow + k0 + 4 * w);
#pragma unroll
        for (int w = 0; w < 8; ++w)
#pragma unroll
          for (int u = 0; u < VPT; ++u) {
            const f32x4 xv = *reinterpret_cast<const f32x4*>(&s_x[vs + u * TPC][k0 + 4 * w]);
            y[u] = fmaf(a[w][0], xv[0], y[u]);
            y[u] = fmaf(a[w][1], xv[1], y[u]);
            y[u] = fmaf(a[w][2], xv[2], y[u]);
            y[u] = fmaf(a[w][3], xv[3], y[u]);
          }
      }
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const int lv = vs + u * TPC;
        // vectors alternate K, V: lv's kind is the parity of v0 + lv (v0 is even)
        s_code[lv][i] = (uint8_t)code_of(y[u], (lv & 1) ? p.v_bounds : p.k_bounds);
      }
    }
    __syncthreads();
    // 3. packed bytes and norms
    for (int e = tid; e < kAppendVecs * H; e += 256) {
      const int lv = e / H, j = e % H;
      const long long dst = s_row[lv];
      if (dst >= 0) p.cache[dst + j] = (uint8_t)((s_code[lv][2 * j] << 4) | s_code[lv][2 * j + 1]);
    }
    if (tid < kAppendVecs && s_row[tid] >= 0) *reinterpret_cast<float*>(p.cache + s_row[tid] + H) = s_norm[tid];
    __syncthreads();  // the LDS is rewritten by the next batch
  }
}

// ---- q into the sequential rotated space ------------------------------------

constexpr int kRotRows = 8;  // q rows per rotation workgroup

// y_seq[i] = sum_k R_seq[i][k] q[k] for kRotRows rows per workgroup: the
// rows sit in LDS; KP adjacent threads share output column i, each taking a
// D / KP slice of rotation row R_seq[i] for all the rows, so a thread's part
// of the row is one round trip of independent 16-byte loads (four for d 256);
// the KP partial sums meet by lane exchanges.
// (fewer workgroups than compute units: occupancy does not matter, and the
// loads are scheduled all ahead)
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void tq4_rotate_q_kernel(
    const Tq4DecodeParams p) {
  constexpr int H = D / 2;
  constexpr int KP = 256 / D;             // threads per output column (4, 2 or 1)
  constexpr int KL = D / KP;              // k per thread (16, 64 or 256)
  constexpr int KB = KL > 64 ? 64 : KL;   // k per round trip
  __shared__ __attribute__((aligned(16))) float s_q[kRotRows][D];
  const int tid = threadIdx.x;
  const long long rows = (long long)p.batch * p.num_q_heads;
  const long long r0 = (long long)blockIdx.x * kRotRows;
  for (int e = tid; e < kRotRows * D; e += 256) {
    const long long r = r0 + e / D;
    s_q[e / D][e % D] = r < rows ? __uint_as_float((uint32_t)p.q[r * D + e % D] << 16) : 0.0f;
  }
  __syncthreads();
  const int i = tid / KP;
  const int kp = tid % KP;
  const float* rrow = p.rotation + (long long)(i < H ? 2 * i : 2 * (i - H) + 1) * D + kp * KL;
  float y[kRotRows];
#pragma unroll
  for (int u = 0; u < kRotRows; ++u) y[u] = 0.0f;
#pragma unroll 1
  for (int kb = 0; kb < KL; kb += KB) {
    f32x4 a[KB / 4];
#pragma unroll
    for (int v = 0; v < KB / 4; ++v) a[v] = *reinterpret_cast<const f32x4*>(rrow + kb + 4 * v);
#pragma unroll
    for (int v = 0; v < KB / 4; ++v)
#pragma unroll
      for (int u = 0; u < kRotRows; ++u) {
        const f32x4 xv = *reinterpret_cast<const f32x4*>(&s_q[u][kp * KL + kb + 4 * v]);
        y[u] = fmaf(a[v][0], xv[0], y[u]);
        y[u] = fmaf(a[v][1], xv[1], y[u]);
        y[u] = fmaf(a[v][2], xv[2], y[u]);
        y[u] = fmaf(a[v][3], xv[3], y[u]);
      }
  }
#pragma unroll
  for (int o = 1; o < KP; o <<= 1)
#pragma unroll
    for (int u = 0; u < kRotRows; ++u) y[u] += __shfl_xor(y[u], o);
  // every thread of the column holds the sums: thread kp writes rows kp, kp + KP, ...
#pragma unroll
  for (int u = 0; u < kRotRows; ++u) {
    const long long r = r0 + u;
    if (u % KP == kp && r < rows) p.q_seq[r * D + i] = (uint16_t)(pack_f16(y[u], 0.0f) & 0xffffu);
  }
}

// ---- decode -----------------------------------------------------------------

// Tiles of a pair and its work items: the same formulas in the decode and the
// reduce kernels.
__device__ __forceinline__ int pair_tiles(int L, long long cap) {
  return (L > 0 && (long long)L <= cap) ? (L - 1) / kTileTokens + 1 : 0;
}
__device__ __forceinline__ int pair_chunks(int nt, int chunk_tiles, int max_chunks) {
  const int n = (nt + chunk_tiles - 1) / chunk_tiles;
  return n < max_chunks ? n : max_chunks;
}

template <int D>
struct Tq4Cfg {
  static constexpr int H = D / 2;
  static constexpr int RB = D + 8;                  // row bytes
  static constexpr int KB = D / 32;                 // 32-wide k blocks = code bytes / 16 lanes / 4
  static constexpr int NC = RB;                     // 16-byte chunks of a 16-row tile
  static constexpr int NI = (NC + 63) / 64;         // loads per lane per tile
  static constexpr int BUF = NI * 1024;             // LDS bytes of a wave's tile buffer
  static constexpr int LDS = 2 * 4 * 256 * kTableCopies + kTq4Waves * 2 * BUF;
};

template <int D>
__global__ __launch_bounds__(kTq4Waves * 64) __attribute__((amdgpu_waves_per_eu(D == 256 ? 2 : 4)))
void tq4_decode_kernel(const Tq4DecodeParams p) {
  using C = Tq4Cfg<D>;
  constexpr int H = C::H, RB = C::RB, KB = C::KB, NI = C::NI;
  __shared__ __attribute__((aligned(16))) uint32_t s_ktab[256 * kTableCopies];
  __shared__ __attribute__((aligned(16))) uint32_t s_vtab[256 * kTableCopies];
  __shared__ __attribute__((aligned(16))) unsigned char s_buf[kTq4Waves][2][C::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;   // MFMA column n / A row m
  const int grp = lane >> 4;   // 16-lane group r

  // centroid pair tables: entry v = (c[v >> 4], c[v & 15]), fp16 for K and
  // bf16 for V
  for (int e = tid; e < 256 * kTableCopies; e += kTq4Waves * 64) {
    const int v = e / kTableCopies;
    s_ktab[e] = pack_f16(p.k_cent[v >> 4], p.k_cent[v & 15]);
    s_vtab[e] = pack_bf16(p.v_cent[v >> 4], p.v_cent[v & 15]);
  }
  __syncthreads();
  const uint32_t* ktab = s_ktab + col;  // copy col of each entry
  const uint32_t* vtab = s_vtab + col;
  auto look = [](const uint32_t* tab, uint32_t byte) -> uint32_t { return tab[byte * kTableCopies]; };
  unsigned char* buf = s_buf[wave][0];
  unsigned char* buf1 = s_buf[wave][1];

  const int G = p.heads_per_kv;
  const int Hkv = p.num_kv_heads;
  const int pairs = p.batch * Hkv;
  const int P = 1 << p.page_log2;
  const long long cap = (long long)p.max_pages_per_seq << p.page_log2;
  const long long W = (long long)p.max_chunks * pairs;
  const float nan = __builtin_nanf("");

  for (long long w = (long long)blockIdx.x * kTq4Waves + wave; w < W; w += p.num_waves) {
    const int c = (int)(w / pairs);
    const int pair = (int)(w % pairs);
    const int b = pair / Hkv;
    const int kvh = pair % Hkv;
    const int L = p.context_lens[b];
    const int nt = pair_tiles(L, cap);
    const int nch = pair_chunks(nt, p.chunk_tiles, p.max_chunks);
    if (c >= nch) continue;
    const int t0 = (int)((long long)c * nt / nch);
    const int t1 = (int)((long long)(c + 1) * nt / nch);

    // Q operands: lane (column n, group r), k block kb, slots 2i / 2i + 1 =
    // elements 4 (r KB + kb) + i and d/2 + 4 (r KB + kb) + i
    f16x8 qop[KB];
    if (p.q_rotated) {
      // natural order: those two slots are elements 2 e and 2 e + 1 of y,
      // so the 8 slots of a k block are 8 consecutive fp16 values
      const bool live = col < G;
      const uint16_t* qr = p.q + ((long long)b * p.num_q_heads + kvh * G + (live ? col : 0)) * D;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        u32x4 v = *reinterpret_cast<const u32x4*>(qr + 8 * (grp * KB + kb));
        if (!live) v = u32x4{0u, 0u, 0u, 0u};
        qop[kb] = __builtin_bit_cast(f16x8, v);
      }
    } else {
      const bool live = col < G;
      const uint16_t* qr = p.q_seq + ((long long)b * p.num_q_heads + kvh * G + (live ? col : 0)) * D;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int e0 = 4 * (grp * KB + kb);
        u32x2 a = *reinterpret_cast<const u32x2*>(qr + e0);
        u32x2 h = *reinterpret_cast<const u32x2*>(qr + H + e0);
        if (!live) a = h = u32x2{0u, 0u};
        const u32x4 v = {__builtin_amdgcn_perm(h[0], a[0], 0x05040100u), __builtin_amdgcn_perm(h[0], a[0], 0x07060302u),
                         __builtin_amdgcn_perm(h[1], a[1], 0x05040100u), __builtin_amdgcn_perm(h[1], a[1], 0x07060302u)};
        qop[kb] = __builtin_bit_cast(f16x8, v);
      }
    }

    typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
    const const_i32_ptr bt = (const_i32_ptr)(p.block_table + (long long)b * p.max_pages_per_seq);
    bool bad_page = false;
    // Tile t = rows 16 t .. 16 t + 15 of the pair: one block of 16 rows when
    // a page holds 16 or more, else two 8-row blocks (P = 8; the second
    // block repeats the first when it lies wholly past the length). Lane l
    // loads 16-byte chunks l, 64 + l, ... (the last chunk repeated past the
    // block's end).
    // block-table entries of tile t (read one tile before they are used,
    // so that the scalar loads' latency hides behind a tile of compute)
    auto pages = [&](int t, int& e0, int& e1) {
      const int pos0 = t * kTileTokens;
      e0 = bt[pos0 >> p.page_log2];
      e1 = (P < kTileTokens && pos0 + 8 < L) ? bt[(pos0 + 8) >> p.page_log2] : e0;
    };
    auto load_tile = [&](int t, u32x4 (&r)[NI], int e0, int e1) {
      const int pos0 = t * kTileTokens;
      const bool ok0 = e0 >= 0 && e0 < p.num_pages, ok1 = e1 >= 0 && e1 < p.num_pages;
      bad_page |= !(ok0 && ok1);
      e0 = ok0 ? e0 : 0;
      e1 = ok1 ? e1 : 0;
      const uint8_t* base0 = p.cache + (((long long)e0 * Hkv + kvh) * P + (pos0 & (P - 1))) * RB;
      const uint8_t* base1 = p.cache + ((long long)e1 * Hkv + kvh) * P * RB;
      constexpr int CPR = 8 * RB / 16;  // chunks of 8 rows
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int ch = min(64 * i + lane, C::NC - 1);
        const uint8_t* src = (P >= kTileTokens || ch < CPR) ? base0 + ch * 16 : base1 + (ch - CPR) * 16;
        r[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
      }
    };

    float m_run = -__builtin_inff();
    float l_part = 0.0f;
    f32x4 acc[2 * KB];
#pragma unroll
    for (int e = 0; e < 2 * KB; ++e) acc[e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](int t, const u32x4 (&r)[NI]) {
      // the tile block into the wave's buffer
#pragma unroll
      for (int i = 0; i < NI; ++i) *reinterpret_cast<u32x4*>(buf + (64 * i + lane) * 16) = r[i];
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");

      // V codes first (independent of the scores): lane (d row m = col,
      // group r), tokens 4 r + jj,
      // code bytes m KB .. m KB + KB - 1 of each
      constexpr int VW = KB >= 4 ? KB / 4 : 1;  // code dwords per lane and token
      uint32_t vw[4][VW];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const unsigned char* vr = buf + (4 * grp + jj) * RB + H + 4 + col * KB;
        if constexpr (KB == 2) {
          vw[jj][0] = *reinterpret_cast<const uint16_t*>(vr);
        } else {
#pragma unroll
          for (int q = 0; q < VW; ++q) vw[jj][q] = *reinterpret_cast<const uint32_t*>(vr + 4 * q);
        }
      }
      // S = K . Q^T: lane (token m = col, group r)
      f32x4 S = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const uint32_t wd = *reinterpret_cast<const uint32_t*>(buf + col * RB + 4 * (grp * KB + kb));
          const u32x4 kop = {look(ktab, wd & 0xffu), look(ktab, (wd >> 8) & 0xffu), look(ktab, (wd >> 16) & 0xffu),
                             look(ktab, wd >> 24)};
          S = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, kop), qop[kb], S, 0, 0, 0);
        }
      }
      // scores of tokens 4 r + j for column n = col, in base 2
      const int tok0 = t * kTileTokens + 4 * grp;
      float x[4], vn[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // rows past the length hold any bytes: their loads are in bounds
        // and their values are selected away
        const unsigned char* row = buf + (4 * grp + j) * RB;
        const float kn = *reinterpret_cast<const float*>(row + H);
        vn[j] = *reinterpret_cast<const float*>(row + D + 4);
        const float xs = S[j] * kn * p.qk_scale_log2;
        x[j] = tok0 + j < L ? xs : -__builtin_inff();
      }
      const float mx = max_groups(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
      // the running max moves only when a tile's max exceeds it by more
      // than 8 (log2 units), so every weight stays below 2^8 and the
      // accumulators are rescaled rarely; numerator and denominator share
      // the reference, so the result does not depend on it
      const bool up = mx - m_run > 8.0f;
      const float m_new = up ? mx : m_run;
      const float m_ref = m_new == -__builtin_inff() ? 0.0f : m_new;
      if (__any(up)) {
        // a real branch (the marker keeps the compiler from executing the
        // rescale on every tile with a select)
        asm volatile("; tq4 rescale" ::: "memory");
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
        l_part *= alpha;
#pragma unroll
        for (int e = 0; e < 2 * KB; ++e) acc[e] *= alpha;
      }
      m_run = m_new;
      float pw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e = __builtin_amdgcn_exp2f(x[j] - m_ref);
        l_part += e;
        pw[j] = tok0 + j < L ? e * vn[j] : 0.0f;
      }
      // the same 16x16x32 shape as the two-tile step (k slots 8 r + 4 ..
      // 8 r + 7 zero in both operands), so that every product on an
      // accumulator has one shape
      const bf16x8 pop = __builtin_bit_cast(bf16x8, u32x4{pack_bf16(pw[0], pw[1]), pack_bf16(pw[2], pw[3]), 0u, 0u});

      // O^T += V^T . P
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        uint32_t lk[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) lk[jj] = look(vtab, (vw[jj][i / 4] >> (8 * (i % 4))) & 0xffu);
        const u32x4 hi = {__builtin_amdgcn_perm(lk[1], lk[0], 0x05040100u), __builtin_amdgcn_perm(lk[3], lk[2], 0x05040100u),
                          0u, 0u};
        const u32x4 lo = {__builtin_amdgcn_perm(lk[1], lk[0], 0x07060302u), __builtin_amdgcn_perm(lk[3], lk[2], 0x07060302u),
                          0u, 0u};
        acc[2 * i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, hi), pop, acc[2 * i], 0, 0, 0);
        acc[2 * i + 1] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, lo), pop, acc[2 * i + 1], 0, 0, 0);
      }
      __builtin_amdgcn_wave_barrier();  // the buffer is rewritten by the next tile
    };

    // Two tiles as one 32-token step: tile t in buf, tile t + 1 in buf1
    // (written by stage2, so that their registers take the next loads while
    // the step computes). One max exchange and one rescale test per step;
    // p.V on the 16x16x32 MFMA, whose k slot 8 r + j is token 4 r + j of
    // tile t for j < 4 and token 4 r + j - 4 of tile t + 1 after: the lane's
    // own probabilities and V lookups of the two tiles, side by side.
    auto stage2 = [&](const u32x4 (&r0)[NI], const u32x4 (&r1)[NI]) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        *reinterpret_cast<u32x4*>(buf + (64 * i + lane) * 16) = r0[i];
        *reinterpret_cast<u32x4*>(buf1 + (64 * i + lane) * 16) = r1[i];
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    };
    auto math2 = [&](int t) {
      constexpr int VW = KB >= 4 ? KB / 4 : 1;
      unsigned char* const bufs[2] = {buf, buf1};
      uint32_t vw[2][4][VW];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const unsigned char* vr = bufs[h] + (4 * grp + jj) * RB + H + 4 + col * KB;
          if constexpr (KB == 2) {
            vw[h][jj][0] = *reinterpret_cast<const uint16_t*>(vr);
          } else {
#pragma unroll
            for (int q = 0; q < VW; ++q) vw[h][jj][q] = *reinterpret_cast<const uint32_t*>(vr + 4 * q);
          }
        }
      f32x4 S[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        S[h] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const uint32_t wd = *reinterpret_cast<const uint32_t*>(bufs[h] + col * RB + 4 * (grp * KB + kb));
          const u32x4 kop = {look(ktab, wd & 0xffu), look(ktab, (wd >> 8) & 0xffu), look(ktab, (wd >> 16) & 0xffu),
                             look(ktab, wd >> 24)};
          S[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, kop), qop[kb], S[h], 0, 0, 0);
        }
      }
      float x[2][4], vn[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int tok0 = (t + h) * kTileTokens + 4 * grp;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const unsigned char* row = bufs[h] + (4 * grp + j) * RB;
          const float kn = *reinterpret_cast<const float*>(row + H);
          vn[h][j] = *reinterpret_cast<const float*>(row + D + 4);
          const float xs = S[h][j] * kn * p.qk_scale_log2;
          x[h][j] = tok0 + j < L ? xs : -__builtin_inff();
        }
      }
      const float mx = max_groups(fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                                        fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3]))));
      const bool up = mx - m_run > 8.0f;
      const float m_new = up ? mx : m_run;
      const float m_ref = m_new == -__builtin_inff() ? 0.0f : m_new;
      if (__any(up)) {
        asm volatile("; tq4 rescale" ::: "memory");
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
        l_part *= alpha;
#pragma unroll
        for (int e = 0; e < 2 * KB; ++e) acc[e] *= alpha;
      }
      m_run = m_new;
      float pw[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int tok0 = (t + h) * kTileTokens + 4 * grp;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float e = __builtin_amdgcn_exp2f(x[h][j] - m_ref);
          l_part += e;
          pw[h][j] = tok0 + j < L ? e * vn[h][j] : 0.0f;
        }
      }
      const bf16x8 pop = __builtin_bit_cast(
          bf16x8, u32x4{pack_bf16(pw[0][0], pw[0][1]), pack_bf16(pw[0][2], pw[0][3]), pack_bf16(pw[1][0], pw[1][1]),
                        pack_bf16(pw[1][2], pw[1][3])});
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        uint32_t lk[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) lk[h][jj] = look(vtab, (vw[h][jj][i / 4] >> (8 * (i % 4))) & 0xffu);
        const u32x4 hi = {__builtin_amdgcn_perm(lk[0][1], lk[0][0], 0x05040100u),
                          __builtin_amdgcn_perm(lk[0][3], lk[0][2], 0x05040100u),
                          __builtin_amdgcn_perm(lk[1][1], lk[1][0], 0x05040100u),
                          __builtin_amdgcn_perm(lk[1][3], lk[1][2], 0x05040100u)};
        const u32x4 lo = {__builtin_amdgcn_perm(lk[0][1], lk[0][0], 0x07060302u),
                          __builtin_amdgcn_perm(lk[0][3], lk[0][2], 0x07060302u),
                          __builtin_amdgcn_perm(lk[1][1], lk[1][0], 0x07060302u),
                          __builtin_amdgcn_perm(lk[1][3], lk[1][2], 0x07060302u)};
        acc[2 * i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, hi), pop, acc[2 * i], 0, 0, 0);
        acc[2 * i + 1] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, lo), pop, acc[2 * i + 1], 0, 0, 0);
      }
      __builtin_amdgcn_wave_barrier();  // the buffers are rewritten by the next step
    };

    // Two tiles in flight: A holds tile t, B tile t + 1. A step writes both
    // to LDS, loads tiles t + 2 and t + 3 into the freed registers (their
    // block-table entries were read a step earlier) and computes t, t + 1;
    // an odd last tile takes the one-tile step.
    u32x4 ra[NI], rb[NI];
    int e0, e1;
    int a0 = 0, a1 = 0, b0 = 0, b1 = 0;  // entries of tiles t + 2 and t + 3
    pages(t0, e0, e1);
    load_tile(t0, ra, e0, e1);
    if (t0 + 1 < t1) {
      pages(t0 + 1, e0, e1);
      load_tile(t0 + 1, rb, e0, e1);
    }
    if (t0 + 2 < t1) pages(t0 + 2, a0, a1);
    if (t0 + 3 < t1) pages(t0 + 3, b0, b1);
    int t = t0;
    for (; t + 1 < t1; t += 2) {
      stage2(ra, rb);
      if (t + 2 < t1) load_tile(t + 2, ra, a0, a1);
      if (t + 3 < t1) load_tile(t + 3, rb, b0, b1);
      if (t + 4 < t1) pages(t + 4, a0, a1);
      if (t + 5 < t1) pages(t + 5, b0, b1);
      math2(t);
    }
    if (t < t1) compute(t, ra);

    // The record (tq4_record_floats(G, D) floats, 16-byte aligned): m[G],
    // l[G], padding to a multiple of 4, then head n's accumulator as the
    // MFMA left it: block e = 2 i + half, group r, element j at
    // n D + 16 e + 4 r + j, which holds d = half d/2 + (4 r + j) KB + i.
    float l_tot = l_part;
    l_tot += __shfl_xor(l_tot, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (bad_page) l_tot = nan;
    if (col < G) {
      float* rec = p.rec + ((long long)c * pairs + pair) * tq4_record_floats(G, D);
      if (grp == 0) {
        rec[col] = m_run;
        rec[G + col] = l_tot;
      }
      f32x4* ra_ = reinterpret_cast<f32x4*>(rec + tq4_record_header(G) + col * D) + grp;
#pragma unroll
      for (int e = 0; e < 2 * KB; ++e) ra_[4 * e] = acc[e];
    }
  }
}

// Position of element d of a head's accumulator in its record (the decode
// kernel's MFMA output order).
template <int D>
__device__ __forceinline__ int acc_index(int d) {
  constexpr int H = D / 2, KB = D / 32;
  const int half = d >= H ? 1 : 0;
  const int dm = d - half * H;
  const int i = dm % KB, m = dm / KB;
  return 16 * (2 * i + half) + 4 * (m / 4) + (m % 4);
}

// The log-sum-exp merge of one (sequence, q head) row's work items
// (split_k_reduce.cu, Algorithm) by one wave, into `os` (D floats, the
// rotated space), and its lse.
template <int D>
__device__ __forceinline__ void merge_row(const Tq4DecodeParams& p, long long row, int lane, float* os) {
  constexpr int EPL = D / 64;
  const int G = p.heads_per_kv;
  const int b = (int)(row / p.num_q_heads);
  const int h = (int)(row % p.num_q_heads);
  const int n = h % G;
  const int pairs = p.batch * p.num_kv_heads;
  const long long pair = (long long)b * p.num_kv_heads + h / G;
  const long long cap = (long long)p.max_pages_per_seq << p.page_log2;
  const int L = p.context_lens[b];
  if (L <= 0 || (long long)L > cap) {
    const float v = L <= 0 ? 0.0f : __builtin_nanf("");
#pragma unroll
    for (int e = 0; e < EPL; ++e) os[lane + 64 * e] = v;
    if (p.lse != nullptr && lane == 0) p.lse[row] = L <= 0 ? -__builtin_inff() : __builtin_nanf("");
    return;
  }
  const int nch = pair_chunks(pair_tiles(L, cap), p.chunk_tiles, p.max_chunks);
  const long long stride = (long long)pairs * tq4_record_floats(G, D);
  const float* rec0 = p.rec + pair * tq4_record_floats(G, D);
  int aoff[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) aoff[e] = tq4_record_header(G) + n * D + acc_index<D>(lane + 64 * e);
  // the accumulators of the first kPre items: their loads go out with the m
  // loads below (one round trip for both; the sums keep the item order)
  constexpr int kPre = 16;
  float v0[kPre][EPL];
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const int c = u < nch ? u : nch - 1;
#pragma unroll
    for (int e = 0; e < EPL; ++e) v0[u][e] = rec0[c * stride + aoff[e]];
  }
  // the items' m and l, 64 items per pass, one per lane
  float M = -__builtin_inff();
  for (int c0 = 0; c0 < nch; c0 += 64)
    M = fmaxf(M, c0 + lane < nch ? rec0[(c0 + lane) * stride + n] : -__builtin_inff());
#pragma unroll
  for (int o_ = 32; o_ >= 1; o_ >>= 1) M = fmaxf(M, __shfl_xor(M, o_));
  float lsum = 0.0f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.0f;
  for (int c0 = 0; c0 < nch; c0 += 64) {
    const int cl = c0 + lane;
    const float wl = cl < nch ? __builtin_amdgcn_exp2f(rec0[cl * stride + n] - M) : 0.0f;
    lsum += cl < nch ? wl * rec0[cl * stride + G + n] : 0.0f;
    const int cn = nch - c0 < 64 ? nch - c0 : 64;
    int c = 0;
    if (c0 == 0) {
      // the prefetched items
      const int np = cn < kPre ? cn : kPre;
#pragma unroll
      for (int u = 0; u < kPre; ++u) {
        if (u < np) {
          const float wgt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), u));
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[e] = fmaf(wgt, v0[u][e], o[e]);
        }
      }
      c = np;
    }
    // the rest: eight items' loads in flight at a time
    for (; c + 8 <= cn; c += 8) {
      float v[8][EPL];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < EPL; ++e) v[u][e] = rec0[(c0 + c + u) * stride + aoff[e]];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wgt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), c + u));
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] = fmaf(wgt, v[u][e], o[e]);
      }
    }
    for (; c < cn; ++c) {
      const float wgt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), c));
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = fmaf(wgt, rec0[(c0 + c) * stride + aoff[e]], o[e]);
    }
  }
#pragma unroll
  for (int o_ = 32; o_ >= 1; o_ >>= 1) lsum += __shfl_xor(lsum, o_);
  const float inv = 1.0f / lsum;
#pragma unroll
  for (int e = 0; e < EPL; ++e) os[lane + 64 * e] = o[e] * inv;
  if (p.lse != nullptr && lane == 0) p.lse[row] = (M + __builtin_log2f(lsum)) * kLn2;
}

// tq4_merge_out_kernel: 8 rows (sequence, q head) per workgroup of 8
// waves: wave w merges row w into LDS; then thread t owns column e = t mod D
// and the d slice t / D of the back rotation out[r][e] = sum_d R_seq[d][e]
// o[r][d] for all the rows (its column's entries of R_seq read coalesced
// across the threads, one round trip of independent loads per 64 d); the
// slices' partial sums meet in LDS.
template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(1, 2))) void tq4_merge_out_kernel(
    const Tq4DecodeParams p) {
  constexpr int H = D / 2;
  constexpr int DQ = 512 / D;             // d slices (8, 4 or 2)
  constexpr int DL = D / DQ;              // d per thread (8, 32 or 128)
  constexpr int DB = DL > 64 ? 64 : DL;   // d per round trip
  static_assert(kRotRows == 8, "rows per workgroup");
  __shared__ __attribute__((aligned(16))) float s_o[kRotRows][D];
  __shared__ float s_part[DQ][kRotRows][D];
  const int tid = threadIdx.x;
  const long long rows = (long long)p.batch * p.num_q_heads;
  const long long r0 = (long long)blockIdx.x * kRotRows;
  {
    const int w = tid >> 6;
    if (r0 + w < rows) merge_row<D>(p, r0 + w, tid & 63, s_o[w]);
  }
  __syncthreads();
  const int e = tid % D;
  const int dq = tid / D;
  float y[kRotRows];
#pragma unroll
  for (int u = 0; u < kRotRows; ++u) y[u] = 0.0f;
#pragma unroll 1
  for (int db = 0; db < DL; db += DB) {
    float r[DB];
#pragma unroll
    for (int v = 0; v < DB; ++v) {
      const int dd = dq * DL + db + v;
      r[v] = p.rotation[(long long)(dd < H ? 2 * dd : 2 * (dd - H) + 1) * D + e];
    }
#pragma unroll
    for (int v = 0; v < DB; ++v)
#pragma unroll
      for (int u = 0; u < kRotRows; ++u) y[u] = fmaf(r[v], s_o[u][dq * DL + db + v], y[u]);
  }
#pragma unroll
  for (int u = 0; u < kRotRows; ++u) s_part[dq][u][e] = y[u];
  __syncthreads();
  // thread t: column e of rows dq, dq + DQ, ...
  for (int u = dq; u < kRotRows; u += DQ) {
    float v = 0.0f;
#pragma unroll
    for (int q = 0; q < DQ; ++q) v += s_part[q][u][e];
    const long long r = r0 + u;
    if (r < rows) p.out[r * D + e] = v;
  }
}

// tq4_merge_rot_kernel: the merge at the fused attention's own boundary
// (q pre-rotated, output left in the rotated space): one row (sequence, q
// head) per one-wave workgroup, so that the rows spread over every compute
// unit; the wave merges its row into LDS in the sequential order and writes
// it in the rotation's natural order (element 2 j = sequential j, element
// 2 j + 1 = sequential d/2 + j), one float2 per lane and step.
template <int D>
__global__ __launch_bounds__(64) void tq4_merge_rot_kernel(const Tq4DecodeParams p) {
  constexpr int H = D / 2;
  __shared__ __attribute__((aligned(16))) float s_o[D];
  const int lane = threadIdx.x;
  const long long row = blockIdx.x;
  merge_row<D>(p, row, lane, s_o);
  __syncthreads();
  float* o = p.out + row * D;
#pragma unroll
  for (int j = lane; j < H; j += 64) *reinterpret_cast<float2*>(o + 2 * j) = make_float2(s_o[j], s_o[H + j]);
}

template <int D>
hipError_t launch_all(const Tq4DecodeParams& p, uint32_t decode_grid, hipStream_t stream) {
  const long long rows = (long long)p.batch * p.num_q_heads;
  if (rows == 0) return hipSuccess;
  if (rows > 0x7fffffffll) return hipErrorInvalidValue;  // one merge workgroup per row in the rotated form
  hipError_t e = hipSuccess;
  if (!p.q_rotated) {
    hipLaunchKernelGGL(tq4_rotate_q_kernel<D>, dim3((uint32_t)((rows + kRotRows - 1) / kRotRows)), dim3(256), 0,
                       stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (decode_grid > 0) {
    hipLaunchKernelGGL(tq4_decode_kernel<D>, dim3(decode_grid), dim3(kTq4Waves * 64), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 merge_grid((uint32_t)((rows + kRotRows - 1) / kRotRows));
  if (p.q_rotated) hipLaunchKernelGGL(tq4_merge_rot_kernel<D>, dim3((uint32_t)rows), dim3(64), 0, stream, p);
  else hipLaunchKernelGGL(tq4_merge_out_kernel<D>, merge_grid, dim3(512), 0, stream, p);
  return hipGetLastError();
}

template <int D>
int occupancy() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, tq4_decode_kernel<D>, kTq4Waves * 64, 0) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

}  // namespace

int tq4_decode_wgs_per_cu(int head_dim) {
  if (head_dim == 64) return occupancy<64>();
  if (head_dim == 128) return occupancy<128>();
  if (head_dim == 256) return occupancy<256>();
  return 0;
}

hipError_t launch_tq4_append(const Tq4AppendParams& p, int head_dim, uint32_t grid, hipStream_t stream) {
  if (grid == 0) return hipSuccess;
  if (head_dim == 64) hipLaunchKernelGGL(tq4_append_kernel<64>, dim3(grid), dim3(256), 0, stream, p);
  else if (head_dim == 128) hipLaunchKernelGGL(tq4_append_kernel<128>, dim3(grid), dim3(256), 0, stream, p);
  else if (head_dim == 256) hipLaunchKernelGGL(tq4_append_kernel<256>, dim3(grid), dim3(256), 0, stream, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_tq4_decode(const Tq4DecodeParams& p, int head_dim, uint32_t decode_grid, hipStream_t stream) {
  if (head_dim == 64) return launch_all<64>(p, decode_grid, stream);
  if (head_dim == 128) return launch_all<128>(p, decode_grid, stream);
  if (head_dim == 256) return launch_all<256>(p, decode_grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace pdattn
