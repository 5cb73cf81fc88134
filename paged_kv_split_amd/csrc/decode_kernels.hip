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
//   * p . V on the matrix cores (tile_ops.h: the weights as three bf16
//     terms, fp32 accumulation).
//
// fp8 pools: e4m3fn bytes are widened in registers (hardware convert, exact
// in bf16 for both operands); the per-(token, kv head) scales are
// folded into the score (k) and the probability (v) instead of being
// multiplied into the elements (OASR "Kernel Layer", FP8 KV variants: one
// fp32 scale per token and kv head).
//
// merge_kernel: one wave per descriptor: M = max m_s, out = sum 2^(m_s - M)
// acc_s / sum 2^(m_s - M) l_s, lse = ln 2 (M + log2 sum 2^(m_s - M) l_s)
// (FlashQuant wiki, split_k_reduce.cu, Algorithm and Numerical Stability,
// on un-normalised accumulators).

#include "tile_ops.h"

namespace pdattn {
namespace {

using namespace dev;

// Range [t0, t1) of the tile list owned by worker w of nw, T tiles in all.
__device__ __forceinline__ void worker_range(long long w, long long nw, long long T, long long& t0, long long& t1) {
  t0 = w * T / nw;
  t1 = (w + 1) * T / nw;
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
  // lane i writes word i (selected, not indexed: an indexed register array
  // would live in scratch memory)
  int dword_i = 0;
#pragma unroll
  for (int i = 0; i < kDescWords; ++i) dword_i = lane == i ? dsc[i] : dword_i;
  if (lane < kDescWords) p.desc[gw * kDescWords + lane] = dword_i;
}

// Waves of a merge workgroup, and the pieces one merge wave loads per step.
constexpr int kMergeWaves = kWaves;
constexpr int kMergeUnroll = 4;

// One workgroup per worker descriptor; only the descriptors of cut pairs
// are valid. Every worker wf .. w holds a record for the pair (a worker
// with an empty tile range holds the empty record m = -inf, l = acc = 0).
// One pass: each of the kMergeWaves waves merges every kMergeWaves-th piece
// with the online rule (a
// running maximum M, l and acc rescaled by 2^(M_old - M_new)), loading
// kMergeUnroll pieces per step so their loads overlap; each lane keeps its
// own slice of one head's accumulator. The four waves' (M, l, acc) meet in LDS and are
// merged by the same rule.
template <int D, int G>
__global__ __launch_bounds__(kMergeWaves * 64) void merge_kernel(MergeParams p) {
  constexpr int RF = (int)record_floats(D, G);
  constexpr int NT = kMergeWaves * 64;
  constexpr int EPL = G * D / 64;      // accumulator elements per lane
  constexpr int LPH = D / EPL;         // lanes per head
  static_assert(EPL >= 1 && D % EPL == 0, "lane slice");
  __shared__ float s_m[kMergeWaves][G];
  __shared__ float s_l[kMergeWaves][G];
  __shared__ __attribute__((aligned(16))) float s_acc[kMergeWaves][G * D];
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

  const int g = lane / LPH;   // this lane's head
  const int e0 = lane * EPL;  // first element of its slice (g * D + ...)
  float M = -__builtin_inff(), L = 0.0f, A[EPL];
#pragma unroll
  for (int k = 0; k < EPL; ++k) A[k] = 0.0f;
  // fold one piece (m, l, acc slice) into the running state
  auto fold = [&](float mi, float li, const float (&ai)[EPL]) {
    const float Mn = fmaxf(M, mi);
    // equal maxima (including both -inf: an empty record) scale by 1
    const float so = M == Mn ? 1.0f : __builtin_amdgcn_exp2f(M - Mn);
    const float si = mi == Mn ? 1.0f : __builtin_amdgcn_exp2f(mi - Mn);
    L = L * so + li * si;
#pragma unroll
    for (int k = 0; k < EPL; ++k) A[k] = A[k] * so + ai[k] * si;
    M = Mn;
  };
  // pieces in flight per step: fewer when a lane's slice is long
  constexpr int U = EPL >= 64 ? 1 : (EPL >= 16 ? 2 : kMergeUnroll);
  for (long long i = wave; i < n; i += U * kMergeWaves) {
    // U pieces per step (every fourth piece from i), all loads issued first
    float mu[U], lu[U], au[U][EPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long iu = i + (long long)u * kMergeWaves;
      const float* r = piece(iu < n ? iu : i);
      mu[u] = r[g];
      lu[u] = r[G + g];
#pragma unroll
      for (int k = 0; k < EPL; ++k) au[u][k] = r[2 * G + e0 + k];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i + (long long)u * kMergeWaves < n) fold(mu[u], lu[u], au[u]);
  }
#pragma unroll
  for (int k = 0; k < EPL; ++k) s_acc[wave][e0 + k] = A[k];
  if (lane % LPH == 0) {
    s_m[wave][g] = M;
    s_l[wave][g] = L;
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += NT) {
    const int gg = e / D;
    float Mx = s_m[0][gg];
#pragma unroll
    for (int q = 1; q < kMergeWaves; ++q) Mx = fmaxf(Mx, s_m[q][gg]);
    float Av = 0.0f, Ls = 0.0f;
#pragma unroll
    for (int q = 0; q < kMergeWaves; ++q) {
      const float mq = s_m[q][gg];
      // a wave without pieces holds M = -inf, l = acc = 0: weight 0
      const float wq = mq == Mx ? 1.0f : __builtin_amdgcn_exp2f(mq - Mx);
      Av += wq * s_acc[q][e];
      Ls += wq * s_l[q][gg];
    }
    // column gg < num_cols: query row gg / Gh of head kvh * Gh + gg % Gh
    // (padding columns are not written); a column that saw no token
    // (Ls = 0) gets 0 and -inf
    if (gg >= p.num_cols) continue;
    const int Gh = p.heads_per_kv;
    const long long bh = (long long)b * p.q_len * p.num_q_heads + (long long)kvh * Gh +
                         (long long)(gg / Gh) * p.num_q_heads + gg % Gh;
    // (a NaN sum, from a poisoned piece, stays NaN)
    p.out[bh * D + (e % D)] = Ls != 0.0f ? Av / Ls : 0.0f;
    if (e % D == 0 && p.lse != nullptr) p.lse[bh] = Ls != 0.0f ? (Mx + log2f(Ls)) * kLn2 : -__builtin_inff();
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

template <int D>
hipError_t launch_merge_d(const MergeParams& p, int group, uint32_t grid, hipStream_t stream) {
  // one workgroup per worker descriptor
  switch (group) {
    case 1: hipLaunchKernelGGL((merge_kernel<D, 1>), dim3(grid), dim3(kMergeWaves * 64), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((merge_kernel<D, 2>), dim3(grid), dim3(kMergeWaves * 64), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((merge_kernel<D, 4>), dim3(grid), dim3(kMergeWaves * 64), 0, stream, p); break;
    case 8: hipLaunchKernelGGL((merge_kernel<D, 8>), dim3(grid), dim3(kMergeWaves * 64), 0, stream, p); break;
    case 16: hipLaunchKernelGGL((merge_kernel<D, 16>), dim3(grid), dim3(kMergeWaves * 64), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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

hipError_t launch_merge(const MergeParams& p, int head_dim, int group, uint32_t grid, hipStream_t stream) {
  if (head_dim == 64) return launch_merge_d<64>(p, group, grid, stream);
  if (head_dim == 128) return launch_merge_d<128>(p, group, grid, stream);
  if (head_dim == 256) return launch_merge_d<256>(p, group, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace pdattn
