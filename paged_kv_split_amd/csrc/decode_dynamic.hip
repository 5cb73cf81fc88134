// gfx950 decode kernel with on-device work balancing: flash-decoding's split
// of the KV range (FlashQuant wiki "CUDA Kernels", paged_decode.cu: Grid,
// Partial Output) where the split points are decided while the kernel runs,
// by how fast each wave actually streams, instead of by a fixed count per
// sequence (Atlas "CUDA Kernel Engineering", kernel inventory: adaptive split
// count). The split merge (split_k_reduce.cu, Algorithm and Numerical
// Stability) runs inside the same kernel, on the wave that completes a unit.
//
// Work: every (sequence b, kv head) pair is cut into units of at most
// kUnitTiles 16-token tiles; units are laid end to end (b major, kv head,
// then position), T tiles in all. A persistent grid of NW waves:
//   * wave w's home range is [w T / NW, (w+1) T / NW); it is a home member
//     of every unit that range meets, and it is also a helper member of the
//     unit holding position (t0 + T/2) mod T and of the one holding
//     (t0 + T/4) mod T. Membership is a pure function of the lengths, so
//     every wave can count the members of any unit.
//   * a unit's first half is split evenly over its home members (each
//     streams its share without any synchronisation, from the first cycle);
//     the second half is handed out kClaimTiles at a time by an atomic
//     counter to whichever member asks first. A wave visits its units in
//     order (home units, then the two helper units) and leaves a unit when
//     a claim finds it exhausted, so fast waves end up doing more.
//   * a wave keeps one online-softmax state per unit visit. A wave that did
//     all of a unit's tiles writes the result directly; otherwise it leaves
//     an (m, l, acc) record in the unit's slots and adds its tile count to
//     the unit's done counter; the wave whose addition completes the count
//     merges the records (log-sum-exp rule). Pairs longer than one unit
//     merge their unit results once more the same way.
// Counters live in the caller's workspace, zeroed once by
// pdattn_workspace_init; each call leaves them zero again: the last claim on
// a unit (every member makes exactly one claim that finds it exhausted, so
// the last claim's number is known) resets the claim counter, and each
// merging wave resets the counters it consumed.
//
// Per wave, tiles stream through a 2-stage direct-to-LDS ring (as in the
// static kernel); block-table windows are staged in LDS by direct loads one
// segment ahead, and the q operand of the next pair is loaded in registers
// one segment ahead, so moving between units costs no extra round trip.

#include "tile_ops.h"

namespace pdattn {
namespace {

using namespace dev;

#ifndef PDATTN_CLAIM_TILES
#define PDATTN_CLAIM_TILES 2
#endif
#ifndef PDATTN_STATIC_NUM
#define PDATTN_STATIC_NUM 1
#endif
#ifndef PDATTN_STATIC_DEN
#define PDATTN_STATIC_DEN 2
#endif
constexpr int kClaimTiles = PDATTN_CLAIM_TILES;  // tiles per claim of a unit's shared part
constexpr int kStaticNum = PDATTN_STATIC_NUM;    // fraction of a unit split statically
constexpr int kStaticDen = PDATTN_STATIC_DEN;    //   over its home members

// One unit (b, kv head, seg) with its sequence's running prefixes. Tile
// positions fit in 31 bits (the planner refuses larger problems).
struct Unit {
  int b, kvh, seg;
  int L;     // context length of sequence b
  int nt;    // tiles of each pair of b
  int ns;    // units of each pair of b
  int tpre;  // tiles of all pairs of the sequences before b
  int upre;  // units of all pairs of the sequences before b
};

// Launch-wide uniform quantities.
struct Glob {
  int T;     // tiles of all pairs
  int NW;    // active worker waves (min(num_workers, T))
  int off1;  // helper position offsets
  int off2;
  int Hkv;
  int seg_max;
};

// What the compute side and the merges need to know about a unit; one LDS
// slot per piece.
struct alignas(16) UnitRef {
  int b, kvh, seg, L;
  int n;     // tiles of the unit
  int ns;    // units of the pair
  int uid;   // counter index: (b * Hkv + kvh) * seg_max + seg
  int base;  // first record slot
  int cap;   // record slots
  int pad[3];
};

// Membership and claim parameters of a unit (identical on every wave).
struct Geo {
  UnitRef r;
  int U0, U1;   // the unit in the tile list
  int members;  // home + helper memberships
  int D0;       // first shared tile (unit-relative)
  int Ns;       // claims that find tiles
};

// The membership counts need thirteen values of wf(x) = ceil(x * NW / T),
// the number of workers whose home range starts before tile x; lane i
// computes the i-th with one vector division. cnt(y, off), the number of
// workers whose helper position (t0 + off) mod T lies below y, is
// wf(clamp(y - off)) + [y > 0] (wf(min(T, y + T - off)) - wf(T - off)).
__device__ __forceinline__ Geo geo_of(const Unit& u, const Glob& gl, int lane) {
  Geo g;
  g.r.b = u.b;
  g.r.kvh = u.kvh;
  g.r.seg = u.seg;
  g.r.L = u.L;
  g.r.ns = u.ns;
  g.r.n = min(kUnitTiles, u.nt - u.seg * kUnitTiles);
  const int U0 = u.tpre + u.kvh * u.nt + u.seg * kUnitTiles;
  g.U0 = U0;
  g.U1 = U0 + g.r.n;
  const int T = gl.T;
  auto clampT = [&](int a) -> int { return a < 0 ? 0 : (a > T ? T : a); };
  int x = 0;
  x = lane == 0 ? U0 : x;
  x = lane == 1 ? U0 + 1 : x;
  x = lane == 2 ? g.U1 : x;
  x = lane == 3 ? clampT(U0 - gl.off1) : x;
  x = lane == 4 ? min(T, U0 + T - gl.off1) : x;
  x = lane == 5 ? T - gl.off1 : x;
  x = lane == 6 ? clampT(g.U1 - gl.off1) : x;
  x = lane == 7 ? min(T, g.U1 + T - gl.off1) : x;
  x = lane == 8 ? clampT(U0 - gl.off2) : x;
  x = lane == 9 ? min(T, U0 + T - gl.off2) : x;
  x = lane == 10 ? T - gl.off2 : x;
  x = lane == 11 ? clampT(g.U1 - gl.off2) : x;
  x = lane == 12 ? min(T, g.U1 + T - gl.off2) : x;
  const int q = (int)(((long long)x * gl.NW + T - 1) / T);
  auto at = [&](int i) -> int { return __builtin_amdgcn_readlane(q, i); };
  const int w0 = at(0), w0p = at(1), w1 = at(2);
  const int c10 = at(3) + (U0 > 0 ? at(4) - at(5) : 0);
  const int c11 = at(6) + at(7) - at(5);
  const int c20 = at(8) + (U0 > 0 ? at(9) - at(10) : 0);
  const int c21 = at(11) + at(12) - at(10);
  const int k0 = w1 - w0p + 1;
  g.members = k0 + (c11 - c10) + (c21 - c20);
  g.r.cap = 1 + (w1 - w0) + (c11 - c10) + (c21 - c20);
  const int ord = u.upre + u.kvh * u.ns + u.seg;
  g.r.base = ord + w0 + c10 + c20;
  g.D0 = (g.r.n * kStaticNum) / kStaticDen;
  g.Ns = (g.r.n - g.D0 + kClaimTiles - 1) / kClaimTiles;
  g.r.uid = (u.b * gl.Hkv + u.kvh) * gl.seg_max + u.seg;
  return g;
}

// The segment producer's state, kept in LDS between runs so that the tile
// loop carries only its own state.
struct alignas(16) Cold {
  Unit pu;                          // unit of the current visit
  int level, phase, st_lo, st_hi;   // membership level; 0 entering, 1 static pieces, 2 claiming
  int c_uid, c_D0, c_n, c_last;     // claim parameters (c_last: value of the unit's last claim)
  int c_base, c_cap, c_U1, c_piece; // record layout; end of the unit; its piece (-1 before its first segment)
  int next_piece, pad0, pad1, pad2;
};

// Records cross waves on different XCDs inside one kernel. They are written
// and read with device-scope atomic accesses (single stores and loads
// coherent at device level: no write-back or invalidation of a whole L2),
// and a writer waits for its stores to complete before the counter update
// that publishes them.
__device__ __forceinline__ void st_coherent(float* a, float v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* a) {
  return __hip_atomic_load(const_cast<float*>(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Merge n records (m[G], l[G], acc[G][D], stride RF floats) in slot order
// with the log-sum-exp rule; lane holds head g = lane * EPL / D and
// accumulator elements [lane * EPL, +EPL).
template <int D, int G>
__device__ __forceinline__ void merge_records(const float* r0, int n, int lane, float& M, float& Lsum,
                                              float (&A)[G * D / 64]) {
  constexpr int EPL = G * D / 64;
  constexpr int RF = (int)record_floats(D, G);
  const int g = lane * EPL / D;
  M = -__builtin_inff();
  Lsum = 0.0f;
#pragma unroll
  for (int k = 0; k < EPL; ++k) A[k] = 0.0f;
#pragma unroll 2
  for (int i = 0; i < n; ++i) {
    const float* r = r0 + (long long)i * RF;
    const float mi = ld_coherent(r + g);
    const float li = ld_coherent(r + G + g);
    float a[EPL];
#pragma unroll
    for (int k = 0; k < EPL; ++k) a[k] = ld_coherent(r + 2 * G + lane * EPL + k);
    const float Mn = fmaxf(M, mi);
    // equal maxima (including both -inf: an empty record) scale by 1
    const float so = M == Mn ? 1.0f : __builtin_amdgcn_exp2f(M - Mn);
    const float si = mi == Mn ? 1.0f : __builtin_amdgcn_exp2f(mi - Mn);
    Lsum = Lsum * so + li * si;
#pragma unroll
    for (int k = 0; k < EPL; ++k) A[k] = A[k] * so + a[k] * si;
    M = Mn;
  }
}

__device__ __forceinline__ uint32_t atomic_add_lane0(uint32_t* a, uint32_t v, int lane) {
  uint32_t r = 0;
  if (lane == 0) r = __hip_atomic_fetch_add(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return __builtin_amdgcn_readfirstlane(r);
}

// A struct held in LDS, read by the whole wave as uniform values.
template <typename T>
__device__ __forceinline__ T load_uniform(const T& src) {
  static_assert(sizeof(T) % 4 == 0, "int-sized fields");
  T out;
  const int* s = reinterpret_cast<const int*>(&src);
  int* d = reinterpret_cast<int*>(&out);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) d[i] = __builtin_amdgcn_readfirstlane(s[i]);
  return out;
}

// Two waves per SIMD (the LDS allows two workgroups per CU): the register
// budget is 256 per lane; group size 16 needs more and runs one wave per SIMD.
template <int D, int G, bool FP8>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(G >= 16 ? 1 : 2)))
void decode_dynamic_kernel(DynParams p) {
  using TL = Tile<D, G, FP8>;
  constexpr int C = TL::C;
  constexpr int NT = kWaves * 64;
  constexpr int S = kStages;
  constexpr int STAGE = TL::STAGE;
  constexpr int RF = TL::RF;
  constexpr int EPL = TL::EPL;
  constexpr int W = kPagesPerWave;
  static_assert(C * (S - 1) < 64, "vmcnt range");

  __shared__ __attribute__((aligned(16))) unsigned char s_ring[kWaves][S * STAGE];
  __shared__ int s_pages[kWaves][kPagesPerWave];
  __shared__ Cold s_cold[kWaves];
  __shared__ long long s_wsum[kWaves][2];
  __shared__ int s_loc[kWaves][3][6];  // per wave and membership level: b, kvh, seg, L, tile and unit prefix of b

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
  auto tiles_of = [&](int L) -> int { return (L > 0 && (long long)L <= cap) ? (L - 1) / kTileTokens + 1 : 0; };
  auto units_of = [&](int nt) -> int { return (nt + kUnitTiles - 1) / kUnitTiles; };

  uint32_t* const ctr = p.ctl;                                 // claims handed out, per unit
  uint32_t* const nrec = p.ctl + p.units_max;                  // records written, per unit
  uint32_t* const done = p.ctl + 2 * (long long)p.units_max;   // tiles finished, per unit
  uint32_t* const done2 = p.ctl + 3 * (long long)p.units_max;  // units finished, per pair

  // A workspace that pdattn_workspace_init has not prepared for this counter
  // layout: every output NaN.
  if (p.ws_magic[0] != kWorkspaceMagic || p.ws_magic[1] != (uint32_t)p.units_max ||
      p.ws_magic[2] != (uint32_t)(B * Hkv)) {
    if (blockIdx.x == 0) {
      for (long long i = tid; i < (long long)B * Hq * D; i += NT) p.out[i] = __builtin_nanf("");
      if (p.lse != nullptr)
        for (long long i = tid; i < (long long)B * Hq; i += NT) p.lse[i] = __builtin_nanf("");
    }
    return;
  }

  // ---- 1. tile and unit counts of the sequences, prefix-summed
  const int CH = (B + NT - 1) / NT;
  const int b_lo = min(B, tid * CH);
  const int b_hi = min(B, b_lo + CH);
  long long my_t = 0, my_u = 0;
  for (int b = b_lo; b < b_hi; ++b) {
    const int nt = tiles_of(p.context_lens[b]);
    my_t += nt;
    my_u += units_of(nt);
  }
  const long long inc_t = wave_incl_scan(my_t, lane);
  const long long inc_u = wave_incl_scan(my_u, lane);
  if (lane == 63) {
    s_wsum[wave][0] = inc_t;
    s_wsum[wave][1] = inc_u;
  }
  __syncthreads();
  long long bef_t = 0, tot_t = 0, bef_u = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    bef_t += w < wave ? s_wsum[w][0] : 0;
    bef_u += w < wave ? s_wsum[w][1] : 0;
    tot_t += s_wsum[w][0];
  }
  Glob gl;
  gl.T = (int)(tot_t * Hkv);
  gl.NW = min(p.num_workers, gl.T);
  gl.off1 = gl.T / 2;
  gl.off2 = gl.T / 4;
  gl.Hkv = Hkv;
  gl.seg_max = p.seg_max;
  const int pre_t = (int)(bef_t + inc_t - my_t);  // tiles per kv head before b_lo
  const int pre_u = (int)(bef_u + inc_u - my_u);

  // ---- 2. locate each wave's home start and helper positions; empty or
  // over-long sequences get their outputs here (out = 0, lse = -inf; NaN
  // when the length does not fit the block table)
  if (gl.T > 0) {
    for (int lw = 0; lw < kWaves; ++lw) {
      const int gw = blockIdx.x * kWaves + lw;
      if (gw >= gl.NW) break;
      const int t0 = (int)((long long)gw * gl.T / gl.NW);
      for (int lvl = 0; lvl < 3; ++lvl) {
        const int x = lvl == 0 ? t0 : (int)(((long long)t0 + (lvl == 1 ? gl.off1 : gl.off2)) % gl.T);
        int rt = pre_t, ru = pre_u;
        for (int b = b_lo; b < b_hi; ++b) {
          const int L = p.context_lens[b];
          const int nt = tiles_of(L);
          if (nt > 0 && Hkv * rt <= x && x < Hkv * (rt + nt)) {
            const int r = x - Hkv * rt;
            s_loc[lw][lvl][0] = b;
            s_loc[lw][lvl][1] = r / nt;
            s_loc[lw][lvl][2] = (r % nt) / kUnitTiles;
            s_loc[lw][lvl][3] = L;
            s_loc[lw][lvl][4] = Hkv * rt;
            s_loc[lw][lvl][5] = Hkv * ru;
          }
          rt += nt;
          ru += units_of(nt);
        }
      }
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

  const int w = blockIdx.x * kWaves + wave;
  if (w >= gl.NW) return;
  const int t1 = (int)((long long)(w + 1) * gl.T / gl.NW);

  auto unit_from_lds = [&](int lvl) -> Unit {
    Unit u;
    u.b = uniform(s_loc[wave][lvl][0]);
    u.kvh = uniform(s_loc[wave][lvl][1]);
    u.seg = uniform(s_loc[wave][lvl][2]);
    u.L = uniform(s_loc[wave][lvl][3]);
    u.nt = tiles_of(u.L);
    u.ns = units_of(u.nt);
    u.tpre = uniform(s_loc[wave][lvl][4]);
    u.upre = uniform(s_loc[wave][lvl][5]);
    return u;
  };
  auto cold_store = [&](const Cold& c) {
    if (lane == 0) s_cold[wave] = c;
  };
  {
    Cold c;
    c.pu = unit_from_lds(0);
    c.level = 0;
    c.phase = 0;
    c.st_lo = c.st_hi = 0;
    c.c_uid = c.c_D0 = c.c_n = c.c_last = 0;
    c.c_base = c.c_cap = c.c_U1 = 0;
    c.c_piece = -1;
    c.next_piece = 0;
    c.pad0 = c.pad1 = c.pad2 = 0;
    cold_store(c);
  }

  // ---- 3. the segment producer: home units in order, then the helper units.
  // The next claim on a unit goes out when a segment of it is handed over
  // and is read back when that segment has been streamed (the wave has no
  // loads in flight then), so its round trip overlaps the segment.
  const int t0 = (int)((long long)w * gl.T / gl.NW);
  uint32_t claim_reg = 0;  // lane 0: result of the pending claim
  auto issue_claim = [&](int uid) {
    if (lane == 0)
      claim_reg = __hip_atomic_fetch_add(ctr + uid, (uint32_t)kClaimTiles, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto take_claim = [&]() -> uint32_t { return __builtin_amdgcn_readfirstlane(claim_reg); };
  // longest run the staged block-table entries cover from any starting token
  const int max_seg = ((W - 1) << lp) / kTileTokens;

  auto next_unit_in_order = [&](Unit u) -> Unit {
    if (u.seg + 1 < u.ns) {
      ++u.seg;
    } else if (u.kvh + 1 < Hkv) {
      ++u.kvh;
      u.seg = 0;
    } else {
      u.tpre += Hkv * u.nt;
      u.upre += Hkv * u.ns;
      u.kvh = 0;
      u.seg = 0;
      u.nt = 0;
      while (u.nt == 0 && u.b + 1 < B) {
        ++u.b;
        u.L = uniform(p.context_lens[u.b]);
        u.nt = tiles_of(u.L);
      }
      u.ns = units_of(u.nt);
    }
    return u;
  };
  // Next segment [lo, hi) of piece `piece` (the unit of c's current visit).
  // 1: produced; -1: nothing left.
  auto produce = [&](Cold& c, int& piece, int& lo, int& hi) -> int {
    for (;;) {
      if (c.level >= 3) return -1;
      if (c.phase == 0) {
        if (c.pu.nt <= 0) {  // inconsistent lengths: nothing more to visit
          c.level = 3;
          continue;
        }
        const Geo g = geo_of(c.pu, gl, lane);
        c.c_uid = g.r.uid;
        c.c_D0 = g.D0;
        c.c_n = g.r.n;
        c.c_last = (g.Ns + g.members - 1) * kClaimTiles;
        c.c_base = g.r.base;
        c.c_cap = g.r.cap;
        c.c_U1 = g.U1;
        c.c_piece = -1;
        c.phase = 2;
        if (c.level == 0) {
          // the static part [0, D0) of the unit is split over its home
          // members in proportion to their home ranges' overlaps with it
          const int a = max(t0, g.U0) - g.U0, e = min(t1, g.U1) - g.U0;
          c.st_lo = (a * kStaticNum) / kStaticDen;
          c.st_hi = (e * kStaticNum) / kStaticDen;
          if (c.st_hi > c.st_lo) c.phase = 1;
        }
        issue_claim(c.c_uid);  // the visit's first claim
      }
      bool got = false;
      if (c.phase == 1) {
        lo = c.st_lo;
        hi = min(c.st_hi, lo + max_seg);
        c.st_lo = hi;
        if (c.st_lo >= c.st_hi) c.phase = 2;
        got = true;
      } else {
        const uint32_t old = take_claim();
        if ((int)old == c.c_last && lane == 0)  // the unit's last claim
          __hip_atomic_store(ctr + c.c_uid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const long long l = (long long)c.c_D0 + old;
        if (l < c.c_n) {
          lo = (int)l;
          hi = min(c.c_n, lo + kClaimTiles);
          issue_claim(c.c_uid);  // the next one, read back after this segment
          got = true;
        }
      }
      if (got) {
        if (c.c_piece < 0) c.c_piece = c.next_piece++;  // first segment of this visit: a new piece
        piece = c.c_piece;
        return 1;
      }
      // the unit is exhausted: next membership
      c.phase = 0;
      if (c.level == 0 && c.c_U1 < t1) {
        c.pu = next_unit_in_order(c.pu);
      } else if (c.level < 2) {
        ++c.level;
        c.pu = unit_from_lds(c.level);
      } else {
        c.level = 3;
      }
    }
  };

  // ---- 4. runs: each segment the producer yields is streamed through the
  // wave's ring; consecutive segments of one unit share one online-softmax
  // state (a piece); a piece ends when the next segment belongs to another
  // unit, or when the producer is done.
  unsigned char* ring = &s_ring[wave][0];
  int* pages = &s_pages[wave][0];
  int winb = -1, winpg = 0, winn = 0, winbad = 0;  // staged block-table entries: sequence, first page, count,
                                                   // an out-of-range entry among them

  int piece_c = -1;  // piece being computed
  UnitRef cu;        // its unit
  cu.b = cu.kvh = cu.seg = cu.L = cu.n = cu.ns = cu.uid = cu.base = cu.cap = 0;
  bf16x8 qop[TL::KSTEPS];
  typename TL::State st;
  TL::reset(st);
  int my_tiles = 0;
  int bad_piece = 0;

  // Emit a unit result: out / lse for a single-unit pair, else a unit record
  // and the pair-level merge when it completes the pair. `store_rec` writes
  // the unit's (m, l, acc) record at the given address, `store_final` the
  // normalised output.
  auto emit_unit = [&](const UnitRef& r, auto&& store_rec, auto&& store_final) {
    if (r.ns == 1) {
      store_final(p.out + ((long long)r.b * Hq + r.kvh * G) * D, p.lse ? p.lse + (long long)r.b * Hq + r.kvh * G : nullptr);
      return;
    }
    const int pair = r.b * Hkv + r.kvh;
    float* r2 = p.rec2 + (long long)pair * p.seg_max * RF;
    store_rec(r2 + (long long)r.seg * RF);
    wait_stores_done();
    const uint32_t old = atomic_add_lane0(done2 + pair, 1u, lane);
    if (old + 1 != (uint32_t)r.ns) return;
    if (lane == 0) __hip_atomic_store(done2 + pair, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    float M, Ls, A[EPL];
    merge_records<D, G>(r2, r.ns, lane, M, Ls, A);
    const int g = lane * EPL / D;
    const long long bh = (long long)r.b * Hq + r.kvh * G + g;
    float* o = p.out + bh * D + (lane * EPL) % D;
#pragma unroll
    for (int k = 0; k < EPL; ++k) o[k] = A[k] / Ls;
    if (p.lse != nullptr && (lane * EPL) % D == 0) p.lse[bh] = (M + log2f(Ls)) * kLn2;
  };

  auto finish_piece = [&]() {
    TL::reduce_rows(st);
    const bool poisoned = __any(bad_piece);
    const UnitRef r = cu;
    auto rec_from_state = [&](float* dst) { TL::template store_record<true>(st, dst, poisoned, row, col); };
    auto out_from_state = [&](float* o, float* lo) {
      TL::store_out(st, o, lo, [](int c) { return c; }, G, poisoned, row, col);
    };
    if (my_tiles == r.n) {  // this wave did the whole unit
      emit_unit(r, rec_from_state, out_from_state);
      return;
    }
    uint32_t idx = atomic_add_lane0(nrec + r.uid, 1u, lane);
    if (idx >= (uint32_t)r.cap) idx = r.cap - 1;  // unreachable with a consistent workspace
    float* const recs = p.rec + (long long)r.base * RF;
    TL::template store_record<true>(st, recs + (long long)idx * RF, poisoned, row, col);
    wait_stores_done();
    const uint32_t old = atomic_add_lane0(done + r.uid, (uint32_t)my_tiles, lane);
    if (old + (uint32_t)my_tiles != (uint32_t)r.n) return;
    // this wave completed the unit: merge its records
    const int n = min((int)__builtin_amdgcn_readfirstlane(
                          __hip_atomic_load(nrec + r.uid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)),
                      r.cap);
    if (lane == 0) {
      __hip_atomic_store(nrec + r.uid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(done + r.uid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    float M, Ls, A[EPL];
    merge_records<D, G>(recs, n, lane, M, Ls, A);
    const int g = lane * EPL / D;
    auto rec_from_merge = [&](float* dst) {
#pragma unroll
      for (int k = 0; k < EPL; ++k) st_coherent(dst + 2 * G + lane * EPL + k, A[k]);
      if ((lane * EPL) % D == 0) {
        st_coherent(dst + g, M);
        st_coherent(dst + G + g, Ls);
      }
    };
    auto out_from_merge = [&](float* o, float* lo) {
#pragma unroll
      for (int k = 0; k < EPL; ++k) o[lane * EPL + k] = A[k] / Ls;
      if (lo != nullptr && (lane * EPL) % D == 0) lo[g] = (M + log2f(Ls)) * kLn2;
    };
    emit_unit(r, rec_from_merge, out_from_merge);
  };

  for (;;) {
    int piece = 0, lo = 0, hi = 0;
    UnitRef r;
    {
      Cold c = load_uniform(s_cold[wave]);
      const int got = produce(c, piece, lo, hi);
      cold_store(c);
      if (got < 0) break;
      r.b = c.pu.b;
      r.kvh = c.pu.kvh;
      r.seg = c.pu.seg;
      r.L = c.pu.L;
      r.n = c.c_n;
      r.ns = c.pu.ns;
      r.uid = c.c_uid;
      r.base = c.c_base;
      r.cap = c.c_cap;
    }
    if (piece != piece_c) {
      if (piece_c >= 0) finish_piece();
      cu = r;
      TL::load_q(qop, p.q + ((long long)cu.b * Hq + cu.kvh * G + min(col, G - 1)) * D, row, col, G);
#pragma unroll
      for (int kk = 0; kk < TL::KSTEPS; ++kk) asm volatile("" : "+v"(qop[kk]));  // q in registers before the run
      TL::reset(st);
      my_tiles = 0;
      bad_piece = 0;
      piece_c = piece;
    }
    // block-table entries of the run, staged in LDS unless already there
    const int s0 = (cu.seg * kUnitTiles + lo) * kTileTokens;  // first token
    const int s1 = min(cu.L, (cu.seg * kUnitTiles + hi) * kTileTokens);
    const int pg_lo = s0 >> lp, pg_hi = (s1 - 1) >> lp;
    if (cu.b != winb || pg_lo < winpg || pg_hi >= winpg + winn) {
      // entries from the run's first page to the sequence's last, at most W
      const int npg = min(W, ((cu.L - 1) >> lp) - pg_lo + 1);
      const int32_t* bt = p.block_table + (long long)cu.b * p.max_pages_per_seq + pg_lo;
      int bad = 0;
      for (int i = lane; i < npg; i += 64) {
        int pg = bt[i];
        if ((unsigned)pg >= (unsigned)p.num_pages) {
          bad = 1;
          pg = 0;
        }
        pages[i] = pg;
      }
      winb = cu.b;
      winpg = pg_lo;
      winn = npg;
      winbad = __any(bad);
    }
    // an out-of-range entry among the staged pages (all of them belong to
    // this sequence, whose every pair reads every page) poisons the piece
    bad_piece |= winbad;
    const long long page_rows = (long long)P * Hkv;
    const int kvh_off = cu.kvh * p.head_stride;
    auto row_of = [&](int pos) -> long long {
      return (long long)pages[(pos >> lp) - winpg] * page_rows + (pos & (P - 1)) * p.slot_stride + kvh_off;
    };
    const int nk = hi - lo;
    auto issue = [&](int k) {
      TL::issue(ring + (k % S) * STAGE, p.k, p.v, p.k_scale, p.v_scale, row_of, s0 + k * kTileTokens, cu.L - 1,
                lane, row, col);
    };
#pragma unroll
    for (int k = 0; k < S; ++k)
      if (k < nk) issue(k);
    for (int k = 0; k < nk; ++k) {
      // tiles k+1 .. min(k+S-1, nk-1) may stay in flight
      wait_tiles<C, S>(min(S - 1, nk - 1 - k));
      typename TL::Frag f;
      TL::read(f, ring + (k % S) * STAGE, lane, row, col);
      if (k + S < nk) issue(k + S);
      TL::compute(st, f, qop, s0 + k * kTileTokens, cu.L, p.qk_scale_log2, row);
    }
    my_tiles += nk;
  }
  if (piece_c >= 0) finish_piece();
}

template <int D, int G, bool FP8>
int occupancy_one() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_dynamic_kernel<D, G, FP8>, kWaves * 64, 0) !=
      hipSuccess)
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

template <int D, int G, bool FP8>
hipError_t launch_one(const DynParams& p, uint32_t grid, hipStream_t stream) {
  hipLaunchKernelGGL((decode_dynamic_kernel<D, G, FP8>), dim3(grid), dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool FP8>
hipError_t launch_group(const DynParams& p, int group, uint32_t grid, hipStream_t stream) {
  switch (group) {
    case 1: return launch_one<D, 1, FP8>(p, grid, stream);
    case 2: return launch_one<D, 2, FP8>(p, grid, stream);
    case 4: return launch_one<D, 4, FP8>(p, grid, stream);
    case 8: return launch_one<D, 8, FP8>(p, grid, stream);
    case 16: return launch_one<D, 16, FP8>(p, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

// Zero the counter words and stamp the header: the magic word and the
// counter layout (units_max, batch * num_kv_heads) it was prepared for.
__global__ __launch_bounds__(256) void workspace_init_kernel(uint32_t* ctl, uint64_t words, uint32_t* header,
                                                             uint32_t units_max, uint32_t pairs) {
  for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (uint64_t)gridDim.x * 256) ctl[i] = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    header[0] = kWorkspaceMagic;
    header[1] = units_max;
    header[2] = pairs;
  }
}

}  // namespace

int dynamic_wgs_per_cu(int head_dim, int group, bool fp8) {
  if (head_dim == 64) return fp8 ? occupancy_group<64, true>(group) : occupancy_group<64, false>(group);
  if (head_dim == 128) return fp8 ? occupancy_group<128, true>(group) : occupancy_group<128, false>(group);
  return 0;
}

hipError_t launch_dynamic(const DynParams& p, int head_dim, int group, bool fp8, uint32_t grid,
                          hipStream_t stream) {
  if (head_dim == 64) return fp8 ? launch_group<64, true>(p, group, grid, stream)
                                 : launch_group<64, false>(p, group, grid, stream);
  if (head_dim == 128) return fp8 ? launch_group<128, true>(p, group, grid, stream)
                                  : launch_group<128, false>(p, group, grid, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_workspace_init(uint32_t* ctl, uint64_t words, uint32_t* header, uint32_t units_max,
                                 uint32_t pairs, hipStream_t stream) {
  uint64_t blocks = (words + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(workspace_init_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, ctl, words, header,
                     units_max, pairs);
  return hipGetLastError();
}

}  // namespace pdattn
