// gfx950 streaming decode kernel: the default decode path for pools whose
// pages hold at least one whole tile (page_size >= 16) and keep the scales,
// if any, in separate arrays, at batch <= kStreamMaxBatch.
//
// The work split is the one of decode_kernel (decode_kernels.hip): all
// (sequence b, kv head) pairs laid end to end, b major, cut into 16-token
// tiles, and every wave of a persistent grid takes a contiguous range of
// that tile list (flash-decoding's split of the KV range, FlashQuant wiki
// "CUDA Kernels", paged_decode.cu: Grid, Partial Output, with the split
// points placed by work: Atlas "CUDA Kernel Engineering", kernel inventory,
// adaptive split count), sized by the plan's worker weights (merge_ops.h:
// equal, or heavier for the first half of the grid, whose workgroups a CU
// serves first). What differs is how a wave walks its range:
//   * one table per 64 tiles, one tile per lane: the lane finds its tile's
//     sequence by a binary search of the workgroup's tile prefix sums, then
//     the kv head and the tile inside the pair; the tile's block-table entry
//     (FlashQuant wiki, paged_decode.cu, Page Table Addressing) and its
//     sequence's length arrive by 4-byte direct-to-LDS loads, 64 at once;
//   * the issue side runs through the whole range without stopping at pair
//     boundaries: a tile that starts a pair (or the range) also fetches that
//     pair's query rows into the stage's query slot, ahead of its K/V, so the
//     ring of 16-byte direct-to-LDS loads never drains inside a range;
//   * a tile's K and V rows are addressed from one wave-uniform base (its
//     page's row index) plus per-lane offsets that never change.
// The per-tile step (q.K on MFMA, online softmax in base 2, p.V) and the
// finish of a pair (out, or an (m, l, acc) record of a cut pair; workgroup 0
// leaves the tile prefix the merge walks) are those of decode_kernel, from
// tile_ops.h.

#include "merge_ops.h"
#include "tile_ops.h"

namespace pdattn {
namespace {

using namespace dev;

// Word 3 of a raw buffer resource on gfx9-family devices.
constexpr int kBufferWord3 = 0x00020000;
// Tiles of one table (one per lane).
constexpr int kTbl = 64;
// Bits of a table entry's j word: the tile's index inside its pair, and flags.
constexpr int kJMask = (1 << 27) - 1;
constexpr int kPairEnd = 1 << 27;    // the pair's last tile
constexpr int kPieceStart = 1 << 28; // first tile of the pair in this range
constexpr int kPieceEnd = 1 << 29;   // last tile of the pair in this range

template <int D, int G, bool FP8>
__global__ __launch_bounds__(kStreamWaves * 64) __attribute__((amdgpu_waves_per_eu(1)))
void decode_stream_kernel(DecodeParams p) {
  using TL = Tile<D, G, FP8, 0>;
  constexpr int C = TL::C;  // direct-to-LDS loads of one tile's K, V (and fp8 scales)
  constexpr int NT = kStreamWaves * 64;
  constexpr int S = kStages;
  constexpr int STAGE = TL::STAGE;
  constexpr int RF = TL::RF;
  constexpr int QSLOT = TL::QSLOT;
  static_assert(C * (S - 1) < 64, "vmcnt range");
  static_assert(2 * NT >= kStreamMaxBatch, "two sequences per thread");

  __shared__ __attribute__((aligned(16))) unsigned char s_ring[kStreamWaves][S * STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char s_q[kStreamWaves][S * QSLOT];
  __shared__ int s_bt[kStreamWaves][2][kTbl];   // block-table entry of each tile of a table
  __shared__ int s_len[kStreamWaves][2][kTbl];  // length of each tile's sequence
  __shared__ int s_pre[kStreamMaxBatch + 1];  // tiles per kv head before sequence b
  __shared__ int s_wsum[kStreamWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;
  const int row = lane >> 4;

  const int B = p.batch;
  const int Hq = p.num_q_heads;
  const int Hkv = p.num_kv_heads;
  const int lp = p.page_log2;
  const int P = 1 << lp;
  const long long cap = (long long)p.max_pages_per_seq << lp;
  const long long NW = p.num_workers;
  auto tiles_of = [&](int L) -> int { return (L > 0 && (long long)L <= cap) ? (L - 1) / kTileTokens + 1 : 0; };

  // ---- 1. tiles per kv head of each sequence, exclusive prefix in s_pre
  // (thread t: sequences 2t and 2t + 1)
  const int L0 = 2 * tid < B ? p.context_lens[2 * tid] : 0;
  const int L1 = 2 * tid + 1 < B ? p.context_lens[2 * tid + 1] : 0;
  const int n0 = tiles_of(L0), n1 = tiles_of(L1);
  int incl = n0 + n1;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kStreamWaves; ++w) {
    const int x = s_wsum[w];
    before += w < wave ? x : 0;
    total += x;
  }
  const int pre = before + incl - n0 - n1;
  // entries 0 .. B - 1 here, entry B (the total) by thread 0: at B =
  // kStreamMaxBatch no thread's pair of sequences reaches it
  if (2 * tid < B) s_pre[2 * tid] = pre;
  if (2 * tid + 1 < B) s_pre[2 * tid + 1] = pre + n0;
  if (tid == 0) s_pre[B] = total;
  if (blockIdx.x == 0) {
    // the prefix for the split reduce
    if (2 * tid < B) p.pre[2 * tid] = pre;
    if (2 * tid + 1 < B) p.pre[2 * tid + 1] = pre + n0;
    if (tid == 0) p.pre[B] = total;
  }
  // empty or over-long sequences get their outputs here (out = 0,
  // lse = -inf; NaN when the length does not fit the block table)
  if (blockIdx.x == 0) {
    const int rows = p.q_len * Hq;
    for (int h = 0; h < 2; ++h) {
      const int b = 2 * tid + h;
      const int L = h ? L1 : L0;
      if (b >= B || tiles_of(L) > 0) continue;
      const bool bad = L != 0;
      const float fo = bad ? __builtin_nanf("") : 0.0f;
      for (int i = 0; i < rows * D; ++i) p.out[(long long)b * rows * D + i] = fo;
      if (p.lse != nullptr)
        for (int r = 0; r < rows; ++r) p.lse[(long long)b * rows + r] = bad ? __builtin_nanf("") : -__builtin_inff();
    }
  }
  __syncthreads();

  // ---- 2. this wave's range [t0, t1) of the T tiles (T < 2^31: the plan
  // selects this kernel only then), by the plan's worker weights.
  const long long gw = (long long)blockIdx.x * kStreamWaves + wave;
  if (gw >= NW) return;
  const int T = total * Hkv;
  auto range_start = [&](long long w) -> int { return (int)worker_start(w, T, NW, p.split_wa, p.split_wb); };
  const int t0 = range_start(gw), t1 = range_start(gw + 1);
  const int n = t1 - t0;
  unsigned char* ring = &s_ring[wave][0];
  unsigned char* qs = &s_q[wave][0];

  if (n <= 0) {
    // no tiles: an empty record (m = -inf, l = acc = 0) in slot 0, read by
    // the merge of the pair this worker falls inside
    float* r = p.rec + gw * 2 * RF;
    for (int i = lane; i < RF; i += 64) r[i] = i < G ? -__builtin_inff() : 0.0f;
  } else {
    // ---- 3. tables: lane i of table c describes tile t0 + 64 c + i
    int tb_b0 = 0, tb_kvh0 = 0, tb_j0 = 0, tb_b1 = 0, tb_kvh1 = 0, tb_j1 = 0;
    auto build = [&](int c) {
      const int buf = c & 1;
      const int i = kTbl * c + lane;
      const int g = t0 + min(i, n - 1);
      // the tile's sequence: the last b with Hkv * pre[b] <= g
      int lo = 0, hi = B;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (Hkv * s_pre[mid] <= g) lo = mid;
        else hi = mid;
      }
      const int b = lo;
      const int nt = s_pre[b + 1] - s_pre[b];
      const int r = g - Hkv * s_pre[b];
      const int kvh = r / nt;
      const int j = r - kvh * nt;
      dma4_cached(p.block_table + (long long)b * p.max_pages_per_seq + ((j * kTileTokens) >> lp), &s_bt[wave][buf][0]);
      dma4_cached(p.context_lens + b, &s_len[wave][buf][0]);
      const int fl = (j == nt - 1 ? kPairEnd : 0) | (j == 0 || g == t0 ? kPieceStart : 0) |
                     (j == nt - 1 || g == t1 - 1 ? kPieceEnd : 0);
      if (buf) {
        tb_b1 = b; tb_kvh1 = kvh; tb_j1 = j | fl;
      } else {
        tb_b0 = b; tb_kvh0 = kvh; tb_j0 = j | fl;
      }
    };
    auto entry = [&](int k, int& b, int& kvh, int& jf) {
      const int i = k & (kTbl - 1);
      const bool b1 = (k / kTbl) & 1;
      b = __builtin_amdgcn_readlane(b1 ? tb_b1 : tb_b0, i);
      kvh = __builtin_amdgcn_readlane(b1 ? tb_kvh1 : tb_kvh0, i);
      jf = __builtin_amdgcn_readlane(b1 ? tb_j1 : tb_j0, i);
    };
    build(0);
    if (n > kTbl) build(1);
    wait_vmcnt<0>();

    const int Gh = p.heads_per_kv;
    auto col_row = [&](int c) { return (c / Gh) * Hq + c % Gh; };
    const long long page_rows = (long long)P * Hkv;
    unsigned long long badbits = 0;  // tiles in flight whose block-table entry is out of range

    // Issue tile k: its query rows first when it starts a piece, then its K
    // and V rows (and fp8 scales). Returns the loads issued before the C
    // K/V loads.
    auto issue = [&](int k) -> int {
      int b, kvh, jf;
      entry(k, b, kvh, jf);
      const int i = k & (kTbl - 1);
      const int buf = (k / kTbl) & 1;
      unsigned char* stg = ring + (k % S) * STAGE;
      int extra = 0;
      if (jf & kPieceStart) {
        const long long base_row = (long long)b * p.q_len * Hq + (long long)kvh * Gh;
        TL::q_issue(qs + (k % S) * QSLOT, p.q, [&](int c) { return base_row + col_row(c); }, p.num_cols, lane);
        extra = TL::CQ;
      }
      int pg = lds_uniform_i32(&s_bt[wave][buf][i]);
      if ((unsigned)pg >= (unsigned)p.num_pages) {
        badbits |= 1ull << (k & 63);
        pg = 0;
      }
      const int tb = (jf & kJMask) * kTileTokens;
      const long long row0 = (long long)pg * page_rows + (long long)((tb & (P - 1)) * p.slot_stride) +
                             (long long)kvh * p.head_stride;
      if (jf & kPairEnd) {
        const int last = lds_uniform_i32(&s_len[wave][buf][i]) - 1 - tb;
        if (last < kTileTokens - 1) {
          TL::issue_rows_clamped(stg, p.k, p.v, p.k_scale, p.v_scale, row0, p.slot_stride, last, lane, row, col);
          return extra;
        }
      }
      TL::issue_rows(stg, p.k, p.v, p.k_scale, p.v_scale, row0, p.slot_stride, lane, row, col);
      return extra;
    };

    // vmcnt bookkeeping. A wave's vector-memory operations complete in issue
    // order, so waiting for tile t means waiting until no more are
    // outstanding than were issued after t's K/V loads: the K/V loads of
    // the later tiles in flight, the query and table loads issued ahead of
    // them, and the finished pieces' stores. dx[i] (st[i]) counts the query
    // and table loads (stores) issued i + 1 steps ago.
    int dx[S], st[S];
#pragma unroll
    for (int i = 0; i < S; ++i) dx[i] = st[i] = 0;
    auto shift = [&](int dx_now, int st_now) {
#pragma unroll
      for (int i = S - 1; i > 0; --i) {
        dx[i] = dx[i - 1];
        st[i] = st[i - 1];
      }
      dx[0] = dx_now;
      st[0] = st_now;
    };

    // the first S tiles; query loads of tile t >= 1 sit after tile t - 1's
    // K/V loads (the bookkeeping's steps -S + t - 1)
    int pre_extra = 0;
#pragma unroll
    for (int k = 0; k < S; ++k)
      if (k < n) {
        const int x = issue(k);
        if (k > 0) pre_extra += x;
        if (k > 0) dx[S - 1 - k] = x;
      }

    // The compute side runs one tile behind the reads: the fragments of tile
    // k + 1 are taken out of the ring (and its stage refilled) before tile
    // k's arithmetic, so the ring refills as soon as a tile lands. A tile's
    // table entry, and for a piece start its query operand and length, are
    // taken along with its fragments.
    typename TL::Frag fa, fb;
    bf16x8 qn[TL::KSTEPS];
    int nb = 0, nkvh = 0, njf = 0, nL = 0;
    // returns the table and query loads issued
    auto read_ahead = [&](int k, typename TL::Frag& f) -> int {
      entry(k, nb, nkvh, njf);
      if (njf & kPieceStart) {
        nL = lds_uniform_i32(&s_len[wave][(k / kTbl) & 1][k & (kTbl - 1)]);
        TL::q_read(qn, qs + (k % S) * QSLOT, row, col, p.num_cols);
      }
      TL::read(f, ring + (k % S) * STAGE, lane, row, col);
      int x = 0;
      // entering table c >= 1: table c - 1 is done with (its last entry was
      // taken along above), so table c + 1 takes its place; its loads land
      // before the issue side reaches it
      if ((k & (kTbl - 1)) == 0 && k > 0 && k + kTbl < n) {
        build(k / kTbl + 1);
        x = 2;
      }
      if (k + S < n) x += issue(k + S);
      return x;
    };

    const __amdgpu_buffer_rsrc_t out_rs =
        __builtin_amdgcn_make_buffer_rsrc(p.out, 0, (int)((long long)B * p.q_len * Hq * D * 4), kBufferWord3);
    const __amdgpu_buffer_rsrc_t lse_rs = __builtin_amdgcn_make_buffer_rsrc(
        p.lse != nullptr ? p.lse : p.out, 0, p.lse != nullptr ? (int)((long long)B * p.q_len * Hq * 4) : 0,
        kBufferWord3);
    const __amdgpu_buffer_rsrc_t rec_rs =
        __builtin_amdgcn_make_buffer_rsrc(p.rec, 0, (int)(NW * 2 * RF * 4), kBufferWord3);

    bf16x8 qop[TL::KSTEPS];
    typename TL::State sta;
    TL::reset(sta);
    bool poisoned = false, first_piece = true, cut_start = false;
    int lim = 0;
    long long base_row = 0;
    // tile k's arithmetic, f holding its fragments; g receives tile k + 1's
    auto step = [&](int k, typename TL::Frag& f, typename TL::Frag& g) {
      const int jf = njf;
      const int j = jf & kJMask;
      if (jf & kPieceStart) {
        base_row = (long long)nb * p.q_len * Hq + (long long)nkvh * Gh;
        const int cl = min(col, p.num_cols - 1);
        lim = nL - (p.q_len - 1 - cl / Gh);
#pragma unroll
        for (int kk = 0; kk < TL::KSTEPS; ++kk) qop[kk] = qn[kk];
        TL::reset(sta);
        poisoned = false;
        cut_start = j > 0;
      }
      poisoned |= ((badbits >> (k & 63)) & 1ull) != 0;
      badbits &= ~(1ull << (k & 63));
      int dx_now = 0, st_now = 0;
      if (k + 1 < n) {
        // tile k + 1: the K/V loads of tiles k+2 .. min(k+S, n-1) may stay
        // in flight, and the query / table loads and stores issued after it
        int allow = C * min(S - 1, n - 2 - k);
#pragma unroll
        for (int i = 0; i < S; ++i) allow += (i < S - 1 ? dx[i] : 0) + st[i];
        wait_vmcnt_le(allow);
        dx_now = read_ahead(k + 1, g);
      }
      TL::compute(sta, f, qop, j * kTileTokens, lim, p.qk_scale_log2, row);

      if (jf & kPieceEnd) {
        TL::reduce_rows(sta);
        const bool reaches_end = (jf & kPairEnd) != 0;
        if (!cut_start && reaches_end) {
          TL::store_out_counted(sta, out_rs, lse_rs, [&](int c) { return base_row + col_row(c); }, p.num_cols,
                                poisoned, row, col);
          st_now = TL::N_OUT_STORES;
        } else {
          // a piece of a cut pair: slot 0 for the wave's first piece, 1 for
          // its last
          TL::store_record_counted(sta, rec_rs, (uint32_t)((gw * 2 + (first_piece ? 0 : 1)) * RF), poisoned, row,
                                   col);
          st_now = TL::N_REC_STORES;
        }
        first_piece = false;
      }
      shift(dx_now, st_now);
    };

    {
      // tile 0: tiles 1 .. min(S, n) - 1 and their query loads may stay in
      // flight
      wait_vmcnt_le(C * (min(S, n) - 1) + pre_extra);
      shift(read_ahead(0, fa), 0);
    }
    for (int k = 0; k < n; k += 2) {
      step(k, fa, fb);
      if (k + 1 < n) step(k + 1, fb, fa);
    }
  }
}

// LDS of one workgroup; instantiations beyond the 160 KB of a CU are not
// built (the general kernel serves them).
template <int D, int G, bool FP8>
constexpr bool stream_fits() {
  using TL = Tile<D, G, FP8, 0>;
  return kStreamWaves * (kStages * (TL::STAGE + TL::QSLOT) + 4 * 2 * kTbl * 4) + 4 * (kStreamMaxBatch + 1 + kStreamWaves) <=
         160 * 1024;
}

template <int D, int G, bool FP8>
hipError_t launch_one(const DecodeParams& p, uint32_t grid, hipStream_t stream) {
  if constexpr (!stream_fits<D, G, FP8>()) {
    return hipErrorInvalidValue;
  } else {
    hipLaunchKernelGGL((decode_stream_kernel<D, G, FP8>), dim3(grid), dim3(kStreamWaves * 64), 0, stream, p);
    return hipGetLastError();
  }
}

template <int D, int G, bool FP8>
int occupancy_one() {
  if constexpr (!stream_fits<D, G, FP8>()) {
    return 0;
  } else {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_stream_kernel<D, G, FP8>, kStreamWaves * 64, 0) != hipSuccess)
      return 0;
    return n;
  }
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

template <int D, bool FP8>
bool fits_group(int group) {
  switch (group) {
    case 1: return stream_fits<D, 1, FP8>();
    case 2: return stream_fits<D, 2, FP8>();
    case 4: return stream_fits<D, 4, FP8>();
    case 8: return stream_fits<D, 8, FP8>();
    case 16: return stream_fits<D, 16, FP8>();
    default: return false;
  }
}

}  // namespace

bool stream_built(int head_dim, int group, bool fp8) {
  if (head_dim == 64) return fp8 ? fits_group<64, true>(group) : fits_group<64, false>(group);
  if (head_dim == 128) return fp8 ? fits_group<128, true>(group) : fits_group<128, false>(group);
  if (head_dim == 256) return fp8 ? fits_group<256, true>(group) : fits_group<256, false>(group);
  return false;
}

int stream_wgs_per_cu(int head_dim, int group, bool fp8) {
  if (head_dim == 64) return fp8 ? occupancy_group<64, true>(group) : occupancy_group<64, false>(group);
  if (head_dim == 128) return fp8 ? occupancy_group<128, true>(group) : occupancy_group<128, false>(group);
  if (head_dim == 256) return fp8 ? occupancy_group<256, true>(group) : occupancy_group<256, false>(group);
  return 0;
}

hipError_t launch_decode_stream(const DecodeParams& p, int head_dim, int group, bool fp8, uint32_t grid,
                                hipStream_t stream) {
  if (head_dim == 64) return fp8 ? launch_group<64, true>(p, group, grid, stream) : launch_group<64, false>(p, group, grid, stream);
  if (head_dim == 128) return fp8 ? launch_group<128, true>(p, group, grid, stream) : launch_group<128, false>(p, group, grid, stream);
  if (head_dim == 256) return fp8 ? launch_group<256, true>(p, group, grid, stream) : launch_group<256, false>(p, group, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace pdattn
