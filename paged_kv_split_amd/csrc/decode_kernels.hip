// gfx950 kernels for paged split-KV GQA decode attention.
//
// decode_kernel: the general decode kernel (every pool type and page size;
// decode_stream.hip holds the default one for the common pools). A
// persistent grid sized to the GPU's resident capacity. The
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
// per piece, and workgroup 0 leaves the tile prefix of the sequences, from
// which the merge kernel finds every cut pair's pieces.
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
//   * p . V on the matrix cores (tile_ops.h: the weights as two bf16
//     terms, fp32 accumulation).
//
// fp8 pools: e4m3fn bytes are widened in registers (hardware convert, exact
// in bf16 for both operands); the per-(token, kv head) scales are
// folded into the score (k) and the probability (v) instead of being
// multiplied into the elements (OASR "Kernel Layer", FP8 KV variants: one
// fp32 scale per token and kv head).
//
// merge_kernel: per cut pair, M = max m_s, out = sum 2^(m_s - M)
// acc_s / sum 2^(m_s - M) l_s, lse = ln 2 (M + log2 sum 2^(m_s - M) l_s)
// (FlashQuant wiki, split_k_reduce.cu, Algorithm and Numerical Stability,
// on un-normalised accumulators).

#include <algorithm>

#include "merge_ops.h"
#include "tile_ops.h"

namespace pdattn {
namespace {

using namespace dev;

// Range [t0, t1) of the tile list owned by worker w of nw, T tiles in all
// (the plan gives this kernel equal weights).
__device__ __forceinline__ void worker_range(long long w, long long nw, long long T, long long& t0, long long& t1) {
  t0 = worker_start(w, T, nw, 1, 1);
  t1 = worker_start(w + 1, T, nw, 1, 1);
}

// fp8 d128 with up to 4 columns: the LDS holds four workgroups per CU; the
// register budget is held to the 128 VGPRs that let four waves share a SIMD
template <int D, int G, bool FP8, int INL = 0>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(FP8 && D == 128 && G <= 4 ? 4 : 1)))
void decode_kernel(DecodeParams p) {
  using TL = Tile<D, G, FP8, INL>;
  constexpr int C = TL::C;
  constexpr int NT = kWaves * 64;
  constexpr int S = kStages;
  constexpr int STAGE = TL::STAGE;
  constexpr int RF = TL::RF;
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
  auto tiles_of = [&](int L) -> long long { return (L > 0 && (long long)L <= cap) ? (L - 1) / kTileTokens + 1 : 0; };

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
  if (blockIdx.x == 0) {
    // the prefix for the split reduce
    long long run = pre;
    for (int b = b_lo; b < b_hi; ++b) {
      p.pre[b] = run;
      run += tiles_of(p.context_lens[b]);
    }
    if (tid == 0) p.pre[B] = total;
  }

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
    // every query row of such a sequence (q_len rows of Hq heads)
    const int rows = p.q_len * Hq;
    for (int b = b_lo; b < b_hi; ++b) {
      const int L = p.context_lens[b];
      if (tiles_of(L) > 0) continue;
      const bool bad = L != 0;
      const float fo = bad ? __builtin_nanf("") : 0.0f;
      for (int i = 0; i < rows * D; ++i) p.out[(long long)b * rows * D + i] = fo;
      if (p.lse != nullptr)
        for (int h = 0; h < rows; ++h) p.lse[(long long)b * rows + h] = bad ? __builtin_nanf("") : -__builtin_inff();
    }
  }
  __syncthreads();

  // ---- 3. this wave's run of tiles
  const long long gw = (long long)blockIdx.x * kWaves + wave;
  if (gw >= NW) return;
  long long t0, t1;
  worker_range(gw, NW, T, t0, t1);
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
      const int nt = (L - 1) / kTileTokens + 1;  // L >= 1 here
      const int seg = (int)min((long long)(nt - j), remaining);
      const bool cut_start = j > 0;
      const bool reaches_end = j + seg == nt;
      const int s0 = j * kTileTokens;
      const int s1 = min(L, (j + seg) * kTileTokens);
      // Column c < num_cols = q_len * Gh (the rest of the G columns pad) is
      // query row c / Gh of head kvh * Gh + c % Gh; its rows of q, out and
      // lse sit (c / Gh) * Hq + c % Gh rows past base_row. Query row i sees
      // the positions before L - (q_len - 1 - i).
      const int Gh = p.heads_per_kv;
      auto col_row = [&](int c) { return (c / Gh) * Hq + c % Gh; };
      const long long base_row = (long long)b * p.q_len * Hq + (long long)kvh * Gh;
      const int cl = min(col, p.num_cols - 1);
      const int lim = min(s1, L - (p.q_len - 1 - cl / Gh));

      bf16x8 qop[TL::KSTEPS];
      TL::load_q(qop, p.q + (base_row + col_row(cl)) * D, row, col, p.num_cols);
      typename TL::State st;
      TL::reset(st);
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
        const long long page_rows = (long long)P * Hkv;
        const int kvh_off = kvh * p.head_stride;
        auto row_of = [&](int pos) -> long long {
          return (long long)pages[(pos >> lp) - pg0] * page_rows + (pos & (P - 1)) * p.slot_stride + kvh_off;
        };
        const int nk = (c1 - c0 + kTileTokens - 1) / kTileTokens;
        auto issue = [&](int k) {
          const int tb = c0 + k * kTileTokens;
          unsigned char* stg = ring + (k % S) * STAGE;
          if constexpr (INL == 0) {
            // pages of 16 tokens or more: a whole tile's rows share one page,
            // so one scalar base addresses it
            if (lp >= 4 && tb + kTileTokens <= s1) {
              const long long row0 = (long long)uniform(pages[(tb >> lp) - pg0]) * page_rows +
                                     (long long)((tb & (P - 1)) * p.slot_stride) + kvh_off;
              TL::issue_rows(stg, p.k, p.v, p.k_scale, p.v_scale, row0, p.slot_stride, lane, row, col);
              return;
            }
          }
          TL::issue(stg, p.k, p.v, p.k_scale, p.v_scale, row_of, tb, s1 - 1, lane, row, col);
        };

#pragma unroll
        for (int k = 0; k < S; ++k)
          if (k < nk) issue(k);

        for (int k = 0; k < nk; ++k) {
          // tiles k+1 .. min(k+S-1, nk-1) may stay in flight
          wait_tiles<C, S>(min(S - 1, nk - 1 - k));
          typename TL::Frag f;
          TL::read(f, ring + (k % S) * STAGE, lane, row, col, s1 - (c0 + k * kTileTokens));
          // the stage's reads have returned (read_stage waits for them): refill it
          if (k + S < nk) issue(k + S);
          TL::compute(st, f, qop, c0 + k * kTileTokens, lim, p.qk_scale_log2, row);
        }
        c0 = c1;
      }

      // ---- finish the piece
      TL::reduce_rows(st);
      const bool poisoned = __any(bad);
      if (!cut_start && reaches_end) {
        TL::store_out(st, p.out + base_row * D, p.lse ? p.lse + base_row : nullptr, col_row, p.num_cols,
                      poisoned, row, col);
      } else {
        // a piece of a cut pair: record (m, l, acc); slot 0 for the wave's
        // first piece, 1 for its last
        TL::store_record(st, p.rec + (gw * 2 + (first ? 0 : 1)) * RF, poisoned, row, col);
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
}

// Pieces one merge wave loads per step: fewer when a lane's slice is long
// (loads beyond a pair's pieces are wasted, so this stays small).
template <int D, int G>
constexpr int merge_unroll() {
  return G * D / 64 >= 64 ? 1 : (G * D / 64 >= 16 ? 2 : 4);
}
// A merge workgroup of W waves meets in LDS: W * G * D floats, held to 64 KB.
template <int D, int G, int W>
constexpr bool merge_fits() {
  return W * G * D * 4 <= 65536;
}
// Workgroup size (waves) of the one-pair-per-wave merge.
constexpr int kMergePairWaves = 4;

// The split reduce over the (sequence b, kv head) pairs: pair (b, kvh) has
// its tiles at ps = Hkv * pre[b] + kvh * nt (nt = pre[b + 1] - pre[b]) of the
// tile list; piece_span (merge_ops.h) finds the workers that hold them.
struct CutPair {
  PieceSpan s;
  int b, kvh;
};

__device__ __forceinline__ CutPair cut_pair(const MergeParams& p, int pair) {
  CutPair c;
  const int Hkv = p.num_kv_heads;
  c.b = pair / Hkv;
  c.kvh = pair - c.b * Hkv;
  const long long T = p.pre[p.batch] * Hkv;
  const long long pb = p.pre[c.b];
  const long long nt = p.pre[c.b + 1] - pb;
  // an empty or invalid sequence (nt = 0) was written by the decode
  c.s = piece_span(Hkv * pb + c.kvh * nt, nt, T, p.num_workers, p.split_wa, p.split_wb);
  return c;
}

// Pieces i0, i0 + S, i0 + 2 S, ... of a cut pair folded into one lane's
// running (M, L, A slice) with the online rule (a running maximum M, l and
// acc rescaled by 2^(M_old - M_new)); U pieces per step, their loads issued
// first so they overlap. Lane: head lane / (D / EPL), elements lane * EPL ..
template <int D, int G>
__device__ __forceinline__ void fold_pieces(const MergeParams& p, const CutPair& c, long long i0, long long S,
                                            int lane, float& M, float& L, float (&A)[G * D / 64]) {
  constexpr int RF = (int)record_floats(D, G);
  constexpr int EPL = G * D / 64;
  constexpr int LPH = D / EPL;
  constexpr int U = merge_unroll<D, G>();
  static_assert(EPL >= 1 && D % EPL == 0, "lane slice");
  const int g = lane / LPH;
  const int e0 = lane * EPL;
  for (long long i = i0; i < c.s.n; i += (long long)U * S) {
    float mu[U], lu[U], au[U][EPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long iu0 = i + (long long)u * S;
      const long long iu = iu0 < c.s.n ? iu0 : i;
      const float* r = p.rec + piece_record(c.s, iu) * RF;
      mu[u] = r[g];
      lu[u] = r[G + g];
#pragma unroll
      for (int k = 0; k < EPL; ++k) au[u][k] = r[2 * G + e0 + k];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i + (long long)u * S < c.s.n) fold_piece<EPL>(M, L, A, mu[u], lu[u], au[u]);
  }
}

// Output row of column c < num_cols of pair (b, kvh).
__device__ __forceinline__ long long merge_row(const MergeParams& p, int b, int kvh, int c) {
  return pair_out_row(b, kvh, c, p.q_len, p.num_q_heads, p.heads_per_kv);
}

// Short pairs: one pair per wave, kMergePairWaves pairs per workgroup; the
// grid strides over the pairs.
template <int D, int G>
__global__ __launch_bounds__(kMergePairWaves * 64) void merge_wave_kernel(MergeParams p) {
  constexpr int EPL = G * D / 64;
  constexpr int LPH = D / EPL;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane / LPH;
  const int e0 = lane * EPL;
  for (int pair = blockIdx.x * kMergePairWaves + wave; pair < p.batch * p.num_kv_heads;
       pair += gridDim.x * kMergePairWaves) {
    const CutPair c = cut_pair(p, pair);
    if (c.s.n == 0) continue;
    float M = -__builtin_inff(), L = 0.0f, A[EPL];
#pragma unroll
    for (int k = 0; k < EPL; ++k) A[k] = 0.0f;
    fold_pieces<D, G>(p, c, 0, 1, lane, M, L, A);
    if (g >= p.num_cols) continue;  // padding columns are not written
    write_merged<EPL>(p.out + merge_row(p, c.b, c.kvh, g) * D + (e0 % D),
                      p.lse != nullptr && lane % LPH == 0 ? p.lse + merge_row(p, c.b, c.kvh, g) : nullptr, M, L, A);
  }
}

// Longer pairs: one pair per workgroup of W waves, each wave taking every
// W-th piece; the waves' states meet in LDS under the same rule. The grid
// strides over the pairs.
template <int D, int G, int W>
__global__ __launch_bounds__(W * 64) void merge_kernel(MergeParams p) {
  constexpr int EPL = G * D / 64;
  constexpr int LPH = D / EPL;
  __shared__ float s_m[W][G];
  __shared__ float s_l[W][G];
  __shared__ __attribute__((aligned(16))) float s_acc[W][G * D];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane / LPH;
  const int e0 = lane * EPL;
  for (int pair = blockIdx.x; pair < p.batch * p.num_kv_heads; pair += gridDim.x) {
    const CutPair c = cut_pair(p, pair);
    if (c.s.n == 0) continue;  // uniform over the workgroup
    float M = -__builtin_inff(), L = 0.0f, A[EPL];
#pragma unroll
    for (int k = 0; k < EPL; ++k) A[k] = 0.0f;
    fold_pieces<D, G>(p, c, wave, W, lane, M, L, A);
#pragma unroll
    for (int k = 0; k < EPL; ++k) s_acc[wave][e0 + k] = A[k];
    if (lane % LPH == 0) {
      s_m[wave][g] = M;
      s_l[wave][g] = L;
    }
    __syncthreads();
    for (int e = tid; e < G * D; e += W * 64) {
      const int gg = e / D;
      if (gg >= p.num_cols) continue;
      float Mx = s_m[0][gg];
#pragma unroll
      for (int q = 1; q < W; ++q) Mx = fmaxf(Mx, s_m[q][gg]);
      float Av = 0.0f, Ls = 0.0f;
#pragma unroll
      for (int q = 0; q < W; ++q) {
        const float mq = s_m[q][gg];
        // a wave without pieces holds M = -inf, l = acc = 0: weight 0
        const float wq = mq == Mx ? 1.0f : __builtin_amdgcn_exp2f(mq - Mx);
        Av += wq * s_acc[q][e];
        Ls += wq * s_l[q][gg];
      }
      const long long bh = merge_row(p, c.b, c.kvh, gg);
      p.out[bh * D + (e % D)] = Ls != 0.0f ? Av / Ls : 0.0f;
      if (e % D == 0 && p.lse != nullptr) p.lse[bh] = Ls != 0.0f ? (Mx + log2f(Ls)) * kLn2 : -__builtin_inff();
    }
    __syncthreads();  // the LDS is reused by the next pair
  }
}

template <int D, int G, bool FP8, int INL>
hipError_t launch_one(const DecodeParams& p, uint32_t grid, hipStream_t stream) {
  hipLaunchKernelGGL((decode_kernel<D, G, FP8, INL>), dim3(grid), dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D, int G, bool FP8, int INL>
int occupancy_one() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<D, G, FP8, INL>, kWaves * 64, 0) != hipSuccess)
    return 0;
  return n;
}

template <int D, bool FP8, int INL>
int occupancy_group(int group) {
  switch (group) {
    case 1: return occupancy_one<D, 1, FP8, INL>();
    case 2: return occupancy_one<D, 2, FP8, INL>();
    case 4: return occupancy_one<D, 4, FP8, INL>();
    case 8: return occupancy_one<D, 8, FP8, INL>();
    case 16: return occupancy_one<D, 16, FP8, INL>();
    default: return 0;
  }
}

template <int D, bool FP8, int INL>
hipError_t launch_group(const DecodeParams& p, int group, uint32_t grid, hipStream_t stream) {
  switch (group) {
    case 1: return launch_one<D, 1, FP8, INL>(p, grid, stream);
    case 2: return launch_one<D, 2, FP8, INL>(p, grid, stream);
    case 4: return launch_one<D, 4, FP8, INL>(p, grid, stream);
    case 8: return launch_one<D, 8, FP8, INL>(p, grid, stream);
    case 16: return launch_one<D, 16, FP8, INL>(p, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

// kinds: see kernels.h (bf16; fp8 separate scales; fp8 inline scales by
// 4-byte loads; fp8 inline scales by raw-row blocks, head-major pools)
template <int D>
int occupancy_kind(int group, int kind) {
  switch (kind) {
    case kKindBf16: return occupancy_group<D, false, 0>(group);
    case kKindFp8: return occupancy_group<D, true, 0>(group);
    case kKindFp8Inline: return occupancy_group<D, true, 1>(group);
    case kKindFp8InlineRows: return occupancy_group<D, true, 2>(group);
    default: return 0;
  }
}

template <int D>
hipError_t launch_kind(const DecodeParams& p, int group, int kind, uint32_t grid, hipStream_t stream) {
  switch (kind) {
    case kKindBf16: return launch_group<D, false, 0>(p, group, grid, stream);
    case kKindFp8: return launch_group<D, true, 0>(p, group, grid, stream);
    case kKindFp8Inline: return launch_group<D, true, 1>(p, group, grid, stream);
    case kKindFp8InlineRows: return launch_group<D, true, 2>(p, group, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int G, int W>
hipError_t launch_merge_w(const MergeParams& p, uint32_t max_grid, hipStream_t stream) {
  const int64_t pairs = (int64_t)p.batch * p.num_kv_heads;
  if constexpr (W == 1) {
    const uint32_t grid = (uint32_t)std::min<int64_t>((pairs + kMergePairWaves - 1) / kMergePairWaves, max_grid);
    hipLaunchKernelGGL((merge_wave_kernel<D, G>), dim3(grid), dim3(kMergePairWaves * 64), 0, stream, p);
    return hipGetLastError();
  } else if constexpr (merge_fits<D, G, W>()) {
    const uint32_t grid = (uint32_t)std::min<int64_t>(pairs, max_grid);
    hipLaunchKernelGGL((merge_kernel<D, G, W>), dim3(grid), dim3(W * 64), 0, stream, p);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <int D, int G>
hipError_t launch_merge_g(const MergeParams& p, int waves, uint32_t max_grid, hipStream_t stream) {
  switch (waves) {
    case 1: return launch_merge_w<D, G, 1>(p, max_grid, stream);
    case 4: return launch_merge_w<D, G, 4>(p, max_grid, stream);
    case 8: return launch_merge_w<D, G, 8>(p, max_grid, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_merge_d(const MergeParams& p, int group, int waves, uint32_t max_grid, hipStream_t stream) {
  switch (group) {
    case 1: return launch_merge_g<D, 1>(p, waves, max_grid, stream);
    case 2: return launch_merge_g<D, 2>(p, waves, max_grid, stream);
    case 4: return launch_merge_g<D, 4>(p, waves, max_grid, stream);
    case 8: return launch_merge_g<D, 8>(p, waves, max_grid, stream);
    case 16: return launch_merge_g<D, 16>(p, waves, max_grid, stream);
    default: return hipErrorInvalidValue;
  }
}

// One pair per wave when one step of a wave covers the longest pair; four
// waves per pair up to four steps' worth; eight beyond (as LDS allows).
// Measured on MI355X: wider workgroups, or more pieces in flight per wave
// than a pair has, only lengthen the reduce.
template <int D, int G>
int merge_waves_g(int64_t max_pieces) {
  constexpr int U = merge_unroll<D, G>();
  if (max_pieces <= U) return 1;
  if (max_pieces <= 4 * U || !merge_fits<D, G, 8>()) return 4;
  return 8;
}

template <int D>
int merge_waves_d(int group, int64_t max_pieces) {
  switch (group) {
    case 1: return merge_waves_g<D, 1>(max_pieces);
    case 2: return merge_waves_g<D, 2>(max_pieces);
    case 4: return merge_waves_g<D, 4>(max_pieces);
    case 8: return merge_waves_g<D, 8>(max_pieces);
    case 16: return merge_waves_g<D, 16>(max_pieces);
    default: return 1;
  }
}

}  // namespace

int decode_wgs_per_cu(int head_dim, int group, int kind) {
  if (head_dim == 64) return occupancy_kind<64>(group, kind);
  if (head_dim == 128) return occupancy_kind<128>(group, kind);
  if (head_dim == 256) return occupancy_kind<256>(group, kind);
  return 0;
}

hipError_t launch_decode(const DecodeParams& p, int head_dim, int group, int kind, uint32_t grid,
                         hipStream_t stream) {
  if (kind < kKindBf16 || kind > kKindFp8InlineRows) return hipErrorInvalidValue;
  if (head_dim == 64) return launch_kind<64>(p, group, kind, grid, stream);
  if (head_dim == 128) return launch_kind<128>(p, group, kind, grid, stream);
  if (head_dim == 256) return launch_kind<256>(p, group, kind, grid, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const MergeParams& p, int head_dim, int group, int waves, uint32_t max_grid,
                        hipStream_t stream) {
  if (head_dim == 64) return launch_merge_d<64>(p, group, waves, max_grid, stream);
  if (head_dim == 128) return launch_merge_d<128>(p, group, waves, max_grid, stream);
  if (head_dim == 256) return launch_merge_d<256>(p, group, waves, max_grid, stream);
  return hipErrorInvalidValue;
}

int merge_waves(int head_dim, int group, int64_t max_pieces) {
  if (head_dim == 64) return merge_waves_d<64>(group, max_pieces);
  if (head_dim == 128) return merge_waves_d<128>(group, max_pieces);
  if (head_dim == 256) return merge_waves_d<256>(group, max_pieces);
  return 1;
}

}  // namespace pdattn
