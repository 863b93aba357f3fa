// A plain streaming read: the reference rate the decode kernels are compared with,
// i.e. how fast this GPU reads n bytes once from HBM when nothing else is done with
// them.  Not part of the method and not part of libkivi.so: it is built into a library
// of its own that only the benchmark loads.
//
// Persistent layout: `workgroups` workgroups (one per CU by default), workgroup w reads
// the contiguous w-th share of the buffer, every lane keeping U 16-byte loads in
// flight per iteration (the workgroup's U loads per lane cover U * threads * 16
// contiguous bytes).  Each thread XORs what it read into one word of `sink`, so that
// no load can be dropped.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

template <int U>
__global__ __launch_bounds__(1024) void stream_read_kernel(const uint4* __restrict__ p, size_t n16,
                                                           size_t share16, unsigned* sink) {
  const size_t lo = (size_t)blockIdx.x * share16;
  const size_t hi = lo + share16 < n16 ? lo + share16 : n16;
  const size_t step = blockDim.x;
  size_t i = lo + threadIdx.x;
  unsigned acc = 0;
  for (; i + (U - 1) * step < hi; i += U * step) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = p[i + u * step];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += step) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) at `buf` (device, 16-byte aligned) with `workgroups`
// workgroups of `threads` threads (a multiple of 64, at most 1024), `unroll` in {1, 2,
// 4, 8, 16} loads per lane in flight; `sink` (device) must hold workgroups * threads
// words.  With start_event and stop_event (hipEvent_t, both or neither) the launch
// records them at the kernel's own start and end (hipExtLaunchKernel).  Returns 0 when
// the launch was enqueued on `stream`, 1 for a bad argument, 2 for a launch error.
int kivi_probe_stream_read(const void* buf, size_t bytes, int workgroups, int threads, int unroll,
                           void* sink, size_t sink_bytes, void* stream, void* start_event,
                           void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr)) return 1;
  if (!buf || !sink || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15u) != 0)
    return 1;
  if (workgroups < 1 || workgroups > 65536 || threads < 64 || threads > 1024 || threads % 64 != 0)
    return 1;
  if (sink_bytes < (size_t)workgroups * threads * sizeof(unsigned)) return 1;
  if (bytes == 0) return 0;
  const size_t n16 = bytes / 16;
  const size_t share16 = (n16 + workgroups - 1) / workgroups;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const uint4* p = static_cast<const uint4*>(buf);
  unsigned* k = static_cast<unsigned*>(sink);
  const dim3 g(workgroups), b(threads);
  const hipEvent_t e0 = static_cast<hipEvent_t>(start_event);
  const hipEvent_t e1 = static_cast<hipEvent_t>(stop_event);
  auto launch = [&](auto kernel) {
    if (e0)
      hipExtLaunchKernelGGL(kernel, g, b, 0, s, e0, e1, 0, p, n16, share16, k);
    else
      hipLaunchKernelGGL(kernel, g, b, 0, s, p, n16, share16, k);
  };
  switch (unroll) {
    case 1: launch(stream_read_kernel<1>); break;
    case 2: launch(stream_read_kernel<2>); break;
    case 4: launch(stream_read_kernel<4>); break;
    case 8: launch(stream_read_kernel<8>); break;
    case 16: launch(stream_read_kernel<16>); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
