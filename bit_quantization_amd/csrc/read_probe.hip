// A plain streaming read, the reference rate the decode kernels are compared with:
// how fast this GPU reads n bytes once from HBM when nothing else is done with them.
// Not part of the method.
#include "kivi_internal.h"

namespace kivi {
namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;

// Thread i XORs the 16-byte words i, i + stride, ... (stride = all threads of the grid)
// and writes the result to sink[i], so that no load can be dropped.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4* __restrict__ p,
                                                                   size_t n16, unsigned* sink) {
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
  unsigned acc = 0;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(size_t)blockIdx.x * kReadThreads + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, unsigned* sink, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamReadBlocks), dim3(kReadThreads), 0, s,
                     static_cast<const uint4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace kivi
