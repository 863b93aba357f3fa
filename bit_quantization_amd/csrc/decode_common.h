// Device pieces shared by the decode kernels: wave reductions, buffer descriptors,
// the workgroup's LDS work queue, and the exchange of per-workgroup partial results
// (m, l, acc per query head) with the merge of the last workgroup of a pair.
#pragma once

#include "kivi_internal.h"

namespace kivi {
namespace {

constexpr int D = kHeadDim;
constexpr int PSTRIDE = D + 4;       // partial per head: acc[D], m, l, 2 unused (16-byte rows)
// Each pair's arrival counter sits in a 256-byte slot of its own: atomics on one
// cache line serialize.
constexpr int kCounterStride = 64;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// ---- small device helpers ---------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF,
                                                            0xF, true));
}
// Reductions over the 16 lanes of a DPP row (rotations stay inside the row).
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<0x128>(x));
  x = fmaxf(x, dpp<0x124>(x));
  x = fmaxf(x, dpp<0x122>(x));
  x = fmaxf(x, dpp<0x121>(x));
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0x128>(x);
  x += dpp<0x124>(x);
  x += dpp<0x122>(x);
  x += dpp<0x121>(x);
  return x;
}
// Lane ^ 16 inside each 32-lane half (ds_swizzle bit-mask mode: and 0x1F, xor 0x10),
// then reductions over 32 lanes and over the wave without lane-index registers.
__device__ __forceinline__ float swizzle_xor16(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}
__device__ __forceinline__ float half_max32(float x) {
  x = row_max16(x);
  return fmaxf(x, swizzle_xor16(x));
}
__device__ __forceinline__ float half_sum32(float x) {
  x = row_sum16(x);
  return x + swizzle_xor16(x);
}
__device__ __forceinline__ float wave_max(float x) {
  x = half_max32(x);
  const int b = __builtin_bit_cast(int, x);
  return fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)),
               __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)));
}
// ---- timeline stamps (measurement build only) -----------------------------------------
// With KIVI_TIMELINE defined (the benchmark's libkivi_timeline.so, never libkivi.so) the
// decode kernel records, per launch slot and workgroup, the 100 MHz real-time counter
// and the shader clock counter at: 0 start, 1 its blocks done (all waves), 2 its arrival
// counted, and in the last arriver only 3 the merge done, 4 its own partial stores
// complete (the merge begins) and 5 the first round of partial loads complete.
// Otherwise the stamps compile to nothing.
constexpr int kTlSlots = 64, kTlWgs = 1024, kTlMarks = 6;
#ifdef KIVI_TIMELINE
__device__ unsigned long long g_timeline[(size_t)kTlSlots * kTlWgs * kTlMarks * 2];
__device__ __forceinline__ void tl_stamp(int slot, int mark) {
  if (slot >= 0 && threadIdx.x == 0 && blockIdx.x < (unsigned)kTlWgs) {
    const unsigned long long rt = __builtin_amdgcn_s_memrealtime();
    const unsigned long long ck = __builtin_amdgcn_s_memtime();
    const size_t o = (((size_t)slot * kTlWgs + blockIdx.x) * kTlMarks + mark) * 2;
    if (mark == 0)                                 // the slot's older marks are cleared
      for (int m = 1; m < kTlMarks; ++m) g_timeline[o + 2 * m] = g_timeline[o + 2 * m + 1] = 0;
    g_timeline[o] = rt;
    g_timeline[o + 1] = ck;
  }
}
#else
__device__ __forceinline__ void tl_stamp(int, int) {}
#endif

// LDS hand-off between lanes of one wave: LDS operations of a wave execute in order,
// so only the compiler must be kept from moving LDS accesses across this point; the
// wait covers LDS (lgkm) only and leaves prefetched global loads in flight.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}
// Partials pass between workgroups through the workspace with write-through stores and
// L2-bypassing loads (the sc1 cache policy, device coherence across the XCDs' L2
// caches).  A stored float carries its lowest mantissa bit set as a "written" mark
// (at most one ulp of change; the reader clears it, which keeps 0 and -inf exact).
// Each workgroup zeroes its own slot when it starts and waits for that before it
// stores its partial (by then a free wait), so a reader that has seen the owner
// arrive finds in each word either this call's value, marked, or zero: it knows a
// word is current from the word alone, with no ordering between the partial's stores.
constexpr int kCoherent = 16;        // sc1
__device__ __forceinline__ uint32_t marked(float v) { return __float_as_uint(v) | 1u; }
__device__ __forceinline__ float unmarked(uint32_t w) { return __uint_as_float(w & ~1u); }
// Wait until this thread's global stores have completed.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes < 0x7FFFFFFF ? (int)bytes : 0x7FFFFFFF;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// ---- work queue of one workgroup ---------------------------------------------------

// Items of a workgroup's queue: the first n_res are 32-row chunks of the float16
// window (first workgroup of a pair only), the rest its share of 64-token blocks.
// Waves take items in order from an LDS counter; lane 0 does the LDS atomic.
__device__ __forceinline__ int grab_item(int* counter) {
  int v = 0;
  if ((threadIdx.x & 63) == 0) v = atomicAdd(counter, 1);
  return __builtin_amdgcn_readfirstlane(v);
}

// Combine N [GQA][PSTRIDE] records (a workgroup's per-wave results) in a fixed order;
// src(i) returns the i-th record.  Thread (head hd, channels 4k .. 4k+3) calls
// sink(hd, k, acc4, l), and the thread with k == 0 also sink_ml(hd, m, l).  Every LDS
// read is independent of the others (no branches on loaded values), so they all go
// out together.  NTH threads take part.
template <int GQA, int NTH, int N, typename Src, typename Sink, typename SinkMl>
__device__ __forceinline__ void combine(Src src, Sink sink, SinkMl sink_ml) {
  for (int idx = threadIdx.x; idx < GQA * (D / 4); idx += NTH) {
    const int hd = idx / (D / 4), k = idx % (D / 4);
    float2 mli[N];
    float4 vi[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float* rec = src(i) + hd * PSTRIDE;
      mli[i] = *reinterpret_cast<const float2*>(rec + D);
      vi[i] = *reinterpret_cast<const float4*>(rec + 4 * k);
    }
    float mstar = -INFINITY;
#pragma unroll
    for (int i = 0; i < N; ++i) mstar = fmaxf(mstar, mli[i].y > 0.f ? mli[i].x : -INFINITY);
    const float mref = mstar > -INFINITY ? mstar : 0.f;
    float l = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float w = mli[i].y > 0.f ? __builtin_amdgcn_exp2f(mli[i].x - mref) : 0.f;
      l = fmaf(mli[i].y, w, l);
      o.x = fmaf(vi[i].x, w, o.x);
      o.y = fmaf(vi[i].y, w, o.y);
      o.z = fmaf(vi[i].z, w, o.z);
      o.w = fmaf(vi[i].w, w, o.w);
    }
    sink(hd, k, o, l);
    if (k == 0) sink_ml(hd, mstar, l);
  }
}

// Final merge by the last workgroup of a pair to arrive, MC partials per round (the
// round size is picked from the partial count, at most 32 / items per thread).  A
// round's words count only when all carry the "written" mark; otherwise the round is
// read again (a bounded wait: every other workgroup of the pair issued its stores
// before it arrived, and this one waited for its own, so they become visible; were the
// bound ever reached the output would be NaN).  A wave's items are the D / 2 channel
// pairs of one head: lane (c / 2) loads the accumulators (c, c+1) of every partial of
// the round, all in flight together, and lane u < MC also that partial's (m, l).  The
// partial weights w_u = 2^(m_u - m*) are then found in registers (a wave maximum, one
// exp2 per lane, a wave sum for l) and read lane by lane into the multiply-adds, with
// no LDS tables.  Indices past the last partial are clamped and weighted 0, empty
// partials (l == 0) weigh 0, and rounds fold in split order with an online rescale.
constexpr int kMaxPolls = 1 << 20;
template <int GQA, int NTH, int MC>
__device__ __forceinline__ void merge_pair(__amdgpu_buffer_rsrc_t parts, int n_parts,
                                           float* __restrict__ out, int* vote, int tl_slot) {
  constexpr int ITEMS = GQA * (D / 2);
  constexpr int IPT = (ITEMS + NTH - 1) / NTH;     // (head, channel pair) items per thread
  static_assert(D / 2 == 64 && NTH % 64 == 0, "a wave's items are one head's channel pairs");
  static_assert(MC <= 32 && MC * IPT <= 32, "loads in flight per thread");
  const int lane = threadIdx.x & 63, c = 2 * lane;
  float m_run[IPT], l[IPT], o0[IPT], o1[IPT];
#pragma unroll
  for (int it = 0; it < IPT; ++it) {
    m_run[it] = -INFINITY;
    l[it] = o0[it] = o1[it] = 0.f;
  }
  if (threadIdx.x < 3) vote[threadIdx.x] = 0;
  __syncthreads();
  tl_stamp(tl_slot, 4);
  bool failed = false;
  int poll = 0;
  for (int i0 = 0; i0 < n_parts; i0 += MC) {
    const int nc = n_parts - i0 < MC ? n_parts - i0 : MC;
    float2 ov[IPT][MC];
    float2 ml[IPT];
    for (;; ++poll) {
      // vote[poll % 3] collects this pass; vote[(poll + 1) % 3], last read two passes
      // ago, is cleared for the next one
      if (threadIdx.x == 0) vote[(poll + 1) % 3] = 0;
      bool stale = false;
#pragma unroll
      for (int it = 0; it < IPT; ++it) {
        const int idx = threadIdx.x + it * NTH;
        const int hd = idx / (D / 2);
        ml[it] = make_float2(-INFINITY, 0.f);
        if (idx < ITEMS) {                           // the whole wave, or none of it
#pragma unroll
          for (int u = 0; u < MC; ++u) {
            const int i = min(i0 + u, n_parts - 1);
            const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(
                parts, ((i * GQA + hd) * PSTRIDE + c) * 4, 0, kCoherent);
            ov[it][u] = make_float2(unmarked(w.x), unmarked(w.y));
            stale |= (w.x & w.y & 1u) == 0u;
          }
          if (lane < MC) {
            const int i = min(i0 + lane, n_parts - 1);
            const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(
                parts, ((i * GQA + hd) * PSTRIDE + D) * 4, 0, kCoherent);
            stale |= (w.x & w.y & 1u) == 0u;
            if (lane < nc) ml[it] = make_float2(unmarked(w.x), unmarked(w.y));
          }
        }
      }
      if (stale) vote[poll % 3] = 1;
      __syncthreads();
      const int any = vote[poll % 3];
      if (!any) break;
      if (poll == kMaxPolls) {
        failed = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    ++poll;
    if (i0 == 0) tl_stamp(tl_slot, 5);
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      if (threadIdx.x + it * NTH >= ITEMS) continue;
      const float mc = fmaxf(m_run[it], wave_max(ml[it].y > 0.f ? ml[it].x : -INFINITY));
      const float mref = mc > -INFINITY ? mc : 0.f;
      const float w = ml[it].y > 0.f ? __builtin_amdgcn_exp2f(ml[it].x - mref) : 0.f;
      const int wb = __builtin_bit_cast(int, w);
      // sum of l_u w_u over lanes 0 .. 31 (lanes from MC on hold 0)
      const float lw = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, half_sum32(ml[it].y * w)), 0));
      const float al = __builtin_amdgcn_exp2f(m_run[it] - mref);
      m_run[it] = mc;
      float a0 = o0[it] * al, a1 = o1[it] * al;
#pragma unroll
      for (int u = 0; u < MC; ++u) {
        const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(wb, u));
        a0 = fmaf(ov[it][u].x, wu, a0);
        a1 = fmaf(ov[it][u].y, wu, a1);
      }
      l[it] = fmaf(l[it], al, lw);
      o0[it] = a0;
      o1[it] = a1;
    }
  }
#pragma unroll
  for (int it = 0; it < IPT; ++it) {
    const int idx = threadIdx.x + it * NTH;
    if (idx >= ITEMS) continue;
    const int hd = idx / (D / 2);
    const float inv = failed ? __builtin_nanf("") : 1.f / l[it];
    *reinterpret_cast<float2*>(out + (int64_t)hd * D + c) = make_float2(o0[it] * inv, o1[it] * inv);
  }
}

// The end of a pair's work in one workgroup.  n_parts == 1: the combined record is the
// output.  Otherwise the record goes to slot `my` of `parts` (marked, write-through,
// nobody waits for it) and the workgroup counts its arrival on *counter; the last to
// arrive waits for its own stores, merges every slot into `out` and resets the
// counter.  `lds` holds the merge's poll votes (3 words).
template <int GQA, int NTH, int N, typename Src>
__device__ __forceinline__ void finish_pair(Src rec, __amdgpu_buffer_rsrc_t parts, int my,
                                            int n_parts, unsigned* counter, float* out,
                                            float* lds, int tl_slot = -1) {
  __shared__ unsigned arrival;
  if (n_parts == 1) {
    combine<GQA, NTH, N>(
        rec,
        [&](int hd, int k, float4 v, float l) {
          const float inv = 1.f / l;
          *reinterpret_cast<float4*>(out + hd * D + 4 * k) =
              make_float4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
        },
        [](int, float, float) {});
    return;
  }
  // Partial -> workspace, marked, after the slot's clear has completed.
  wait_stores();
  combine<GQA, NTH, N>(
      rec,
      [&](int hd, int k, float4 v, float) {
        const u32x4 w = {marked(v.x), marked(v.y), marked(v.z), marked(v.w)};
        __builtin_amdgcn_raw_buffer_store_b128(w, parts, my + (hd * PSTRIDE + 4 * k) * 4, 0,
                                               kCoherent);
      },
      [&](int hd, float mv, float lv) {
        const u32x2 w = {marked(mv), marked(lv)};
        __builtin_amdgcn_raw_buffer_store_b64(w, parts, my + (hd * PSTRIDE + D) * 4, 0, kCoherent);
      });
  __syncthreads();
  if (threadIdx.x == 0)
    arrival = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  tl_stamp(tl_slot, 2);
  if (arrival != (unsigned)(n_parts - 1)) return;
  // Last to arrive: other threads read this workgroup's own words back, so its stores
  // (issued an atomic round trip ago) must be complete first.
  wait_stores();
  __syncthreads();
  constexpr int MCMAX = 32 / ((GQA * (D / 2) + NTH - 1) / NTH);
  int* vote = reinterpret_cast<int*>(lds);
  if (n_parts <= 8)
    merge_pair<GQA, NTH, (MCMAX < 8 ? MCMAX : 8)>(parts, n_parts, out, vote, tl_slot);
  else if (n_parts <= 16)
    merge_pair<GQA, NTH, (MCMAX < 16 ? MCMAX : 16)>(parts, n_parts, out, vote, tl_slot);
  else
    merge_pair<GQA, NTH, MCMAX>(parts, n_parts, out, vote, tl_slot);
  tl_stamp(tl_slot, 3);
  if (threadIdx.x == 0)
    __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Zero a workgroup's partial slot at `my`, each thread the words it stores in
// finish_pair (same thread, same address: the later store lands last).
template <int GQA, int NTH>
__device__ __forceinline__ void clear_partial(__amdgpu_buffer_rsrc_t parts, int my) {
  for (int idx = threadIdx.x; idx < GQA * (D / 4); idx += NTH) {
    const int hd = idx / (D / 4), k = idx % (D / 4);
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, parts,
                                           my + (hd * PSTRIDE + 4 * k) * 4, 0, kCoherent);
    if (k == 0)
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, parts, my + (hd * PSTRIDE + D) * 4, 0,
                                            kCoherent);
  }
}

}  // namespace
}  // namespace kivi
