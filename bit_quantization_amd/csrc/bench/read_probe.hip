// Reference reads the decode kernels are compared with.  Not part of the method and not
// part of libkivi.so: they are built into a library of its own that only the benchmark
// loads.
//
// 1. A plain streaming read: how fast this GPU reads n bytes once from HBM when nothing
// else is done with them.
//
// Persistent layout: `workgroups` workgroups (one per CU by default), workgroup w reads
// the contiguous w-th share of the buffer, every lane keeping U 16-byte loads in
// flight per iteration (the workgroup's U loads per lane cover U * threads * 16
// contiguous bytes).  Each thread XORs what it read into one word of `sink`, so that
// no load can be dropped.
//
// 2. The 2-bit decode's access pattern without its arithmetic (G = 32, d = 128): per
// 64-token block of a (sequence, KV head) pair 2048 B of Key codes, 512 + 512 B of Key
// scales and zeros, 2048 B of Value codes and 128 + 128 B of Value scales and zeros,
// 5376 B in all.  A pair's blocks lie in six arrays as in the cache (codes by token,
// Key scales by group, Value codes by 16-token run) and are read with the decode
// kernel's lane offsets and load widths; or, for comparison, each block's 5376 B lie
// contiguously.  `nw` consecutive workgroups of 8 waves share a pair's blocks in
// contiguous shares, the waves of a workgroup take the share's blocks round-robin, and
// each wave keeps `ahead` blocks in flight while it folds one (a ring of register sets,
// no copies between them).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

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

constexpr int kPatWaves = 8, kPatThreads = 64 * kPatWaves;
constexpr int64_t kPatBlockBytes = 5376;

struct PatRegs {
  u32x2 k[4];
  u32x4 v[2], ks[2], kz[2];
  unsigned sv[2], zv[2];
};
struct PatBufs {
  __amdgpu_buffer_rsrc_t kc, vc, ks, kz, vs, vz, fused;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t pat_rsrc(const uint8_t* p, int64_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, (int)n, 0x00020000);
}

template <bool FUSED>
__device__ __forceinline__ void pat_load(PatRegs& R, const PatBufs& pb, int blk, int lane) {
  const int lo = lane & 15, j = lane >> 4;
  if constexpr (FUSED) {
    const int b0 = (int)(blk * kPatBlockBytes);
    R.v[0] = __builtin_amdgcn_raw_buffer_load_b128(pb.fused, lane * 16, b0, 0);
    R.v[1] = __builtin_amdgcn_raw_buffer_load_b128(pb.fused, lane * 16, b0 + 1024, 0);
    R.ks[0] = __builtin_amdgcn_raw_buffer_load_b128(pb.fused, lane * 16, b0 + 2048, 0);
    R.ks[1] = __builtin_amdgcn_raw_buffer_load_b128(pb.fused, lane * 16, b0 + 3072, 0);
    R.kz[0] = __builtin_amdgcn_raw_buffer_load_b128(pb.fused, lane * 16, b0 + 4096, 0);
    R.kz[1] = lane < 16 ? __builtin_amdgcn_raw_buffer_load_b128(pb.fused, lane * 16, b0 + 5120, 0)
                        : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) R.k[i] = u32x2{0u, 0u};
    R.sv[0] = R.sv[1] = R.zv[0] = R.zv[1] = 0u;
    return;
  }
  const int tb = blk * 64;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {   // token 2lo + (nt & 1) + 32 (nt >> 1), bytes 8j .. 8j+7
    const int tok = 2 * lo + (nt & 1) + 32 * (nt >> 1);
    R.k[nt] = __builtin_amdgcn_raw_buffer_load_b64(pb.kc, tok * 32 + 8 * j, tb * 32, 0);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q)        // run j of the block, channels 8lo .. 8lo+7
    R.v[q] = __builtin_amdgcn_raw_buffer_load_b128(pb.vc, j * 512 + lo * 32 + 16 * q, tb * 32, 0);
#pragma unroll
  for (int g = 0; g < 2; ++g) {      // the block's two Key groups, channels 8lo .. 8lo+7
    R.ks[g] = __builtin_amdgcn_raw_buffer_load_b128(pb.ks, 16 * lo + 256 * g, (tb / 32) * 256, 0);
    R.kz[g] = __builtin_amdgcn_raw_buffer_load_b128(pb.kz, 16 * lo + 256 * g, (tb / 32) * 256, 0);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {      // Value scale/zero of tokens 32k + 2lo, 32k + 2lo + 1
    R.sv[k] = __builtin_amdgcn_raw_buffer_load_b32(pb.vs, 4 * lo + 64 * k, tb * 2, 0);
    R.zv[k] = __builtin_amdgcn_raw_buffer_load_b32(pb.vz, 4 * lo + 64 * k, tb * 2, 0);
  }
}

__device__ __forceinline__ unsigned pat_fold(const PatRegs& R) {
  unsigned x = R.sv[0] ^ R.sv[1] ^ R.zv[0] ^ R.zv[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) x ^= R.k[i][0] ^ R.k[i][1];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int w = 0; w < 4; ++w) x ^= R.v[i][w] ^ R.ks[i][w] ^ R.kz[i][w];
  return x;
}

template <int AHEAD, bool FUSED>
__global__ __launch_bounds__(kPatThreads, 1) void pattern_read_kernel(const uint8_t* __restrict__ data,
                                                                      int blocks, int nw,
                                                                      unsigned* sink) {
  constexpr int RING = AHEAD + 1;
  const int pair = blockIdx.x / nw, s = blockIdx.x % nw;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t pb_bytes = (int64_t)blocks * kPatBlockBytes;
  const uint8_t* base = data + pair * pb_bytes;
  const int64_t codes = (int64_t)blocks * 2048, kscale = (int64_t)blocks * 512,
                vscale = (int64_t)blocks * 128;
  PatBufs pb;
  pb.kc = pat_rsrc(base, codes);
  pb.vc = pat_rsrc(base + codes, codes);
  pb.ks = pat_rsrc(base + 2 * codes, kscale);
  pb.kz = pat_rsrc(base + 2 * codes + kscale, kscale);
  pb.vs = pat_rsrc(base + 2 * codes + 2 * kscale, vscale);
  pb.vz = pat_rsrc(base + 2 * codes + 2 * kscale + vscale, vscale);
  pb.fused = pat_rsrc(base, pb_bytes);
  const int b_lo = (int)((int64_t)blocks * s / nw), b_hi = (int)((int64_t)blocks * (s + 1) / nw);
  unsigned acc = 0;
  PatRegs r[RING];
#pragma unroll
  for (int d = 0; d < RING; ++d) {
    const int bb = b_lo + wave + d * kPatWaves;
    if (bb < b_hi) pat_load<FUSED>(r[d], pb, bb, lane);
  }
  for (int b = b_lo + wave; b < b_hi; b += kPatWaves * RING) {
#pragma unroll
    for (int d = 0; d < RING; ++d) {
      const int bc = b + d * kPatWaves;
      if (bc < b_hi) {
        acc ^= pat_fold(r[d]);
        const int bn = bc + RING * kPatWaves;
        if (bn < b_hi) pat_load<FUSED>(r[d], pb, bn, lane);
      }
    }
  }
  sink[(size_t)blockIdx.x * kPatThreads + threadIdx.x] = acc;
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

// The decode's access pattern (see the top of this file) over `pairs` pairs of `blocks`
// 64-token blocks each, pair p's 5376 * blocks bytes at buf + p * 5376 * blocks (device,
// 16-byte aligned; `bytes` must cover all pairs), read by pairs * nw workgroups of 512
// threads with `ahead` in {1, 2, 3} blocks in flight per wave; fused != 0 reads each
// block's bytes contiguously instead of from the six arrays.  `sink` (device) must hold
// pairs * nw * 512 words.  Events, stream and return codes as kivi_probe_stream_read.
int kivi_probe_pattern_read(const void* buf, size_t bytes, int pairs, int blocks, int nw,
                            int ahead, int fused, void* sink, size_t sink_bytes, void* stream,
                            void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr)) return 1;
  if (!buf || !sink || (reinterpret_cast<uintptr_t>(buf) & 15u) != 0) return 1;
  if (pairs < 1 || blocks < 1 || nw < 1 || nw > blocks) return 1;
  if ((int64_t)blocks * kPatBlockBytes >= ((int64_t)1 << 31)) return 1;
  if ((int64_t)pairs * nw > 65536) return 1;
  if (bytes < (size_t)pairs * (size_t)blocks * (size_t)kPatBlockBytes) return 1;
  if (sink_bytes < (size_t)pairs * nw * kPatThreads * sizeof(unsigned)) return 1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* p = static_cast<const uint8_t*>(buf);
  unsigned* k = static_cast<unsigned*>(sink);
  const dim3 g(pairs * nw), b(kPatThreads);
  const hipEvent_t e0 = static_cast<hipEvent_t>(start_event);
  const hipEvent_t e1 = static_cast<hipEvent_t>(stop_event);
  auto launch = [&](auto kernel) {
    if (e0)
      hipExtLaunchKernelGGL(kernel, g, b, 0, s, e0, e1, 0, p, blocks, nw, k);
    else
      hipLaunchKernelGGL(kernel, g, b, 0, s, p, blocks, nw, k);
  };
  switch (ahead * 2 + (fused ? 1 : 0)) {
    case 2: launch(pattern_read_kernel<1, false>); break;
    case 3: launch(pattern_read_kernel<1, true>); break;
    case 4: launch(pattern_read_kernel<2, false>); break;
    case 5: launch(pattern_read_kernel<2, true>); break;
    case 6: launch(pattern_read_kernel<3, false>); break;
    case 7: launch(pattern_read_kernel<3, true>); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
