// Streaming-read bandwidth reference (a measurement aid, not part of the
// decode path): the same 16-byte non-temporal loads the decode kernel
// streams K/V with, over a plain buffer.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace pdattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Bandwidth reference: each wave reads 4 KB chunks of a buffer (grid-stride,
// 16-byte non-temporal loads, 4 in flight per lane) and folds them into one
// word per thread, so the result cannot be optimised away.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, uint64_t nchunks,
                                                          uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const uint64_t wave = (uint64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const uint64_t nw = (uint64_t)gridDim.x * 4;
  uint32_t acc = 0;
  for (uint64_t c = wave; c < nchunks; c += nw) {
    const u32x4* p = src + c * 256 + lane;
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(p + u * 64);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  sink[(uint64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, uint32_t grid, hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const u32x4*>(buf),
                     bytes / 4096, sink);
  return hipGetLastError();
}

}  // namespace pdattn
