// Device helpers of the static split and its reduce: the worker ranges the
// decode kernels (decode_stream.hip, decode_kernels.hip) stream, and how
// the merge kernels find a cut pair's pieces in them and fold them.
//
// The rule (FlashQuant wiki "CUDA Kernels", split_k_reduce.cu, Algorithm and
// Numerical Stability, on un-normalised accumulators): for the pieces s of a
// pair, M = max m_s, out = sum 2^(m_s - M) acc_s / sum 2^(m_s - M) l_s, taken
// here in one pass, piece by piece in tile order, with a running maximum.
#pragma once

#include <hip/hip_runtime.h>

namespace pdattn {
namespace dev {

// floor(x / d) for 0 <= x, 0 < d: below 2^53 the fp64 quotient, corrected by
// one step (its error is below one); the integer division beyond.
__device__ __forceinline__ long long floor_div(long long x, long long d) {
  if (x >= (1ll << 53)) return x / d;
  long long q = (long long)((double)x / (double)d);
  if (q * d > x) --q;
  else if ((q + 1) * d <= x) ++q;
  return q;
}

// The static split of the T-tile list over NW workers, by weight: workers
// 0 .. NW/2 - 1 weigh wa, the others wb (wa = wb: equal shares). With
// W(w) = the weight of workers 0 .. w - 1, worker w holds
// [floor(T W(w) / W(NW)), floor(T W(w + 1) / W(NW))).
__device__ __forceinline__ long long weight_before(long long w, long long NW, long long wa, long long wb) {
  const long long h = NW / 2;
  return w <= h ? wa * w : wa * h + wb * (w - h);
}
// (Equal weights take the short forms floor(w T / NW) and
// ceil((g + 1) NW / T) - 1: the same values, fewer divisions.)
__device__ __forceinline__ long long worker_start(long long w, long long T, long long NW, long long wa, long long wb) {
  if (wa == wb) return floor_div(w * T, NW);
  return floor_div(T * weight_before(w, NW, wa, wb), weight_before(NW, NW, wa, wb));
}
// The worker holding tile g < T, the last w whose start is <= g: with
// c = ceil((g + 1) W(NW) / T) - 1, the last w with W(w) <= c.
__device__ __forceinline__ long long worker_of(long long g, long long T, long long NW, long long wa, long long wb) {
  if (wa == wb) return floor_div((g + 1) * NW + T - 1, T) - 1;
  const long long c = floor_div((g + 1) * weight_before(NW, NW, wa, wb) + T - 1, T) - 1;
  const long long h = NW / 2;
  // c < 2^24 here (at most 16 times 2^20 workers): 32-bit quotients
  const long long w = c < wa * h ? (long long)((uint32_t)c / (uint32_t)wa)
                                 : h + (long long)((uint32_t)(c - wa * h) / (uint32_t)wb);
  return w < NW - 1 ? w : NW - 1;
}

// Where the pieces of a pair sit. The pair's tiles are [ps, ps + nt) of the
// tile list; the workers holding its first and last tiles are
// wf = worker_of(ps) and wl = worker_of(ps + nt - 1); with wf == wl one
// worker finished the pair (n = 0 here). Otherwise workers wf .. wl each
// left one record of it: wf in slot 0 when its range starts at ps, else in
// slot 1 (its last piece); every later worker in slot 0 (its first piece;
// a worker with an empty range holds the empty record m = -inf,
// l = acc = 0).
struct PieceSpan {
  long long wf;  // first worker
  long long n;   // pieces (workers wf .. wf + n - 1); 0: nothing to merge
  int slot_first;
};

__device__ __forceinline__ PieceSpan piece_span(long long ps, long long nt, long long T, long long NW, long long wa,
                                                long long wb) {
  PieceSpan s;
  s.wf = 0;
  s.n = 0;
  s.slot_first = 0;
  if (nt <= 0) return s;
  const long long wf = worker_of(ps, T, NW, wa, wb);
  const long long wl = worker_of(ps + nt - 1, T, NW, wa, wb);
  if (wf == wl) return s;
  s.wf = wf;
  s.n = wl - wf + 1;
  s.slot_first = worker_start(wf, T, NW, wa, wb) == ps ? 0 : 1;
  return s;
}

// Record index (in records of record_floats floats) of piece i of a span.
__device__ __forceinline__ long long piece_record(const PieceSpan& s, long long i) {
  return (s.wf + i) * 2 + (i == 0 ? s.slot_first : 0);
}

// One piece (mu, lu, au) folded into a running (M, L, A): the larger maximum
// is kept and the side below it is scaled by 2^(its max - the new max);
// equal maxima (both -inf included: an empty record) scale by exactly 1.
template <int N>
__device__ __forceinline__ void fold_piece(float& M, float& L, float (&A)[N], float mu, float lu,
                                           const float (&au)[N]) {
  const float Mn = fmaxf(M, mu);
  const float so = M == Mn ? 1.0f : __builtin_amdgcn_exp2f(M - Mn);
  const float si = mu == Mn ? 1.0f : __builtin_amdgcn_exp2f(mu - Mn);
  L = fmaf(L, so, lu * si);
#pragma unroll
  for (int k = 0; k < N; ++k) A[k] = fmaf(A[k], so, au[k] * si);
  M = Mn;
}

// Output row of column c of pair (b, kvh): query row c / Gh of head
// kvh * Gh + c % Gh (n query rows per sequence, Hq heads).
__device__ __forceinline__ long long pair_out_row(int b, int kvh, int c, int n, int Hq, int Gh) {
  return (long long)b * n * Hq + (long long)kvh * Gh + (long long)(c / Gh) * Hq + c % Gh;
}

// A lane's N consecutive output floats at dst (aligned to N floats when N
// is 2 or a multiple of 4: out is 16-byte aligned and slices start at
// multiples of N), in the widest stores that alignment allows.
template <int N>
__device__ __forceinline__ void store_slice(float* dst, const float (&v)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int k = 0; k < N; k += 4)
      *reinterpret_cast<float4*>(dst + k) = make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
  } else if constexpr (N == 2) {
    *reinterpret_cast<float2*>(dst) = make_float2(v[0], v[1]);
  } else {
#pragma unroll
    for (int k = 0; k < N; ++k) dst[k] = v[k];
  }
}

// A merged slice: out = A / L and, where lse_dst is given, lse =
// ln 2 (M + log2 L). A column that saw no token (L = 0) gets 0 and -inf; a
// NaN sum, from a poisoned piece, stays NaN.
template <int N>
__device__ __forceinline__ void write_merged(float* out_dst, float* lse_dst, float M, float L, const float (&A)[N]) {
  float o[N];
#pragma unroll
  for (int k = 0; k < N; ++k) o[k] = L != 0.0f ? A[k] / L : 0.0f;
  store_slice<N>(out_dst, o);
  if (lse_dst != nullptr) *lse_dst = L != 0.0f ? (M + log2f(L)) * 0.69314718055994530942f : -__builtin_inff();
}

}  // namespace dev
}  // namespace pdattn
