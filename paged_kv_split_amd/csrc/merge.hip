// Merge of exported partial attention states: pieces s of a row, each a
// normalised output o_s and a natural-log log-sum-exp lse_s over disjoint
// key sets, combine into the row's attention over the union (FlashQuant wiki
// "CUDA Kernels", split_k_reduce.cu Algorithm and Numerical Stability: the
// global maximum, weights rescaled by the exponential of each piece's
// maximum minus it, the weighted sum over the summed weights):
//
//   M = max_s lse_s,  w_s = exp(lse_s - M),
//   out = sum_s w_s o_s / sum_s w_s,  lse = M + ln sum_s w_s.
//
// The pass is online over s (a running maximum with the partial sums
// rescaled when it grows), so a piece is read once. A piece with
// lse = -inf weighs nothing; a row with every piece empty gets out = 0 and
// lse = -inf; a NaN or +inf lse makes the row NaN.
//
// Layout: 16-byte lanes, 256 / D rows per wave (D / 4 lanes per row), four
// pieces' loads in flight per step.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "merge.h"

namespace pdattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMergeUnroll = 4;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

template <int D>
__global__ __launch_bounds__(256) void merge_states_kernel(MergeStatesParams p) {
  constexpr int kLanesPerRow = D / 4;
  constexpr int kRowsPerWave = 64 / kLanesPerRow;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t r = wave * kRowsPerWave + lane / kLanesPerRow;
  if (r >= p.num_rows) return;
  const int col = (lane % kLanesPerRow) * 4;
  const int64_t piece_stride = p.num_rows * D;

  float m = -INFINITY, l = 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  bool bad = false;
  for (int s0 = 0; s0 < p.num_partials; s0 += kMergeUnroll) {
    float ls[kMergeUnroll];
    f32x4 os[kMergeUnroll];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int s = min(s0 + u, p.num_partials - 1);  // in bounds; repeats are skipped below
      ls[u] = p.partial_lse[(int64_t)s * p.num_rows + r];
      os[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p.partial_out + s * piece_stride + r * D + col));
    }
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      if (s0 + u >= p.num_partials) break;
      const float li = ls[u];
      if (isnan(li) || li == INFINITY) bad = true;
      if (!(li > -INFINITY) || bad) continue;  // empty piece (or the row is already NaN)
      const float mn = fmaxf(m, li);
      const float a = m == mn ? 1.0f : exp2f((m - mn) * kLog2e);
      const float b = li == mn ? 1.0f : exp2f((li - mn) * kLog2e);
      l = l * a + b;
      acc = acc * a + os[u] * b;
      m = mn;
    }
  }
  f32x4 o;
  float lse;
  if (bad) {
    o = f32x4{NAN, NAN, NAN, NAN};
    lse = NAN;
  } else if (m == -INFINITY) {
    o = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    lse = -INFINITY;
  } else {
    const float inv = 1.0f / l;
    o = acc * inv;
    lse = m + log2f(l) * kLn2;
  }
  *reinterpret_cast<f32x4*>(p.out + r * D + col) = o;
  if (p.lse && col == 0) p.lse[r] = lse;
}

template <int D>
hipError_t launch_d(const MergeStatesParams& p, hipStream_t stream) {
  constexpr int kRowsPerWg = 4 * (256 / D);
  const int64_t grid = (p.num_rows + kRowsPerWg - 1) / kRowsPerWg;
  hipLaunchKernelGGL((merge_states_kernel<D>), dim3((uint32_t)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge_states(const MergeStatesParams& p, int head_dim, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_d<64>(p, stream);
    case 128: return launch_d<128>(p, stream);
    case 256: return launch_d<256>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pdattn
