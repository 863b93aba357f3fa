// Prefill quantization of Keys and Values, and the streaming append/flush.
//
// Keys are quantized per channel over groups of G consecutive tokens and Values per
// token over groups of G_v consecutive channels ("4.4 KV Cache quantization" §3.1;
// "KV Cache Quantization (KIVI & FP4)" §3).  Inside a group the mapping is the
// asymmetric min/max quantizer with float16 scale and zero ("09 — KV Cache
// Quantization", "KIVI — the reference paper"; step = range / (2^b - 1) as in "KV
// Cache INT4 Quantization for 1M+ Token Context Windows" §2).  The flush of the
// residual window reuses the same device functions, so prefill and streaming write
// identical bytes ("KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache",
// "The streaming complication").
//
// The arithmetic must match the definition bit for bit: float32 subtraction and
// correctly rounded division, round-half-to-even (rintf), float32->float16 by
// round-to-nearest-even, -0 canonicalized to +0, no contraction into FMAs.
#include <type_traits>

#include "kivi_internal.h"

#pragma clang fp contract(off)

namespace kivi {
namespace {

constexpr int D = kHeadDim;

struct GroupParams {
  float mn;      // group minimum (float32, exact float16 value)
  float s;       // float32 value of the stored float16 scale
  __half scale;
  __half zero;
};

__device__ __forceinline__ GroupParams group_params(float mn, float mx, int bits) {
  GroupParams p;
  const float qmax = (float)((1 << bits) - 1);
  const float rng = mx - mn;
  const float s32 = rng / qmax;          // IEEE division (correctly rounded)
  p.scale = __float2half_rn(s32);
  p.zero = __float2half_rn(mn);          // exact: mn is a float16 value
  p.mn = mn;
  p.s = __half2float(p.scale);
  return p;
}

// Largest value over the wave, then raised into *p (scale maxima: non-negative floats
// order like their bit patterns, so an unsigned atomic max is a float max).
__device__ __forceinline__ void raise_scale_max(float* p, float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  if (threadIdx.x == 0)
    __hip_atomic_fetch_max(reinterpret_cast<unsigned*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

template <int BITS>
__device__ __forceinline__ uint32_t quant_code(float x, const GroupParams& p) {
  constexpr float qmax = (float)((1 << BITS) - 1);
  if (p.s == 0.0f) return 0u;
  float q = rintf((x - p.mn) / p.s);     // ties to even
  q = fminf(fmaxf(q, 0.0f), qmax);
  return (uint32_t)q;
}

// One wave quantizes one Key group: G tokens x D channels, rows of D float16 at
// `src`.  Lane l owns channels 2l and 2l+1.  Writes G packed rows at `codes`
// (row stride D*BITS/8 bytes) and D scales/zeros.  `lds` holds G*D bytes.
template <int BITS, int G>
__device__ __forceinline__ void quantize_k_group(const __half* __restrict__ src,
                                                 uint8_t* __restrict__ codes,
                                                 __half* __restrict__ scale,
                                                 __half* __restrict__ zero, uint8_t* lds,
                                                 float* smax) {
  const int lane = threadIdx.x;
  const __half2* s2 = reinterpret_cast<const __half2*>(src);
  float x0[G], x1[G];
  float mn0 = INFINITY, mx0 = -INFINITY, mn1 = INFINITY, mx1 = -INFINITY;
#pragma unroll
  for (int t = 0; t < G; ++t) {
    const __half2 v = s2[t * (D / 2) + lane];
    x0[t] = __low2float(v) + 0.0f;       // -0 -> +0
    x1[t] = __high2float(v) + 0.0f;
    mn0 = fminf(mn0, x0[t]);
    mx0 = fmaxf(mx0, x0[t]);
    mn1 = fminf(mn1, x1[t]);
    mx1 = fmaxf(mx1, x1[t]);
  }
  const GroupParams p0 = group_params(mn0, mx0, BITS);
  const GroupParams p1 = group_params(mn1, mx1, BITS);
  reinterpret_cast<__half2*>(scale)[lane] = __halves2half2(p0.scale, p1.scale);
  reinterpret_cast<__half2*>(zero)[lane] = __halves2half2(p0.zero, p1.zero);
  raise_scale_max(smax, fmaxf(p0.s, p1.s));
#pragma unroll
  for (int t = 0; t < G; ++t) {
    const uint32_t c0 = quant_code<BITS>(x0[t], p0);
    const uint32_t c1 = quant_code<BITS>(x1[t], p1);
    reinterpret_cast<uint16_t*>(lds + t * D)[lane] = (uint16_t)(c0 | (c1 << 8));
  }
  __syncthreads();
  // Pack each token row along channels: 32/BITS codes per 32-bit word, code k of a
  // word in byte k % 4 at bit offset BITS * (k / 4).
  constexpr int CPW = 32 / BITS;
  constexpr int WPR = D / CPW;           // words per token row
  for (int w = lane; w < G * WPR; w += 64) {
    const int t = w / WPR, j = w % WPR;
    const uint8_t* c = lds + t * D + j * CPW;
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < CPW; ++k) word |= (uint32_t)c[k] << (8 * (k % 4) + BITS * (k / 4));
    reinterpret_cast<uint32_t*>(codes + (int64_t)t * (D * BITS / 8))[j] = word;
  }
}

// One wave quantizes one run of 16 Value tokens (each token in groups of GV
// channels).  Lane l owns token l/4 and channels 32*(l%4) .. +31.  Writes the run's
// packed codes ([D][16*BITS/8] bytes at `codes`) and 16*(D/GV) scales/zeros.
template <int BITS, int GV>
__device__ __forceinline__ void quantize_v_run(const __half* __restrict__ src,
                                               uint8_t* __restrict__ codes,
                                               __half* __restrict__ scale,
                                               __half* __restrict__ zero, uint8_t* lds,
                                               float* smax) {
  const int lane = threadIdx.x;
  const int tau = lane >> 2, part = lane & 3;
  const uint4* row = reinterpret_cast<const uint4*>(src + tau * D + part * 32);
  float x[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 u = row[i];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const __half2 h2 = *reinterpret_cast<const __half2*>(&w[k]);
      x[8 * i + 2 * k] = __low2float(h2) + 0.0f;
      x[8 * i + 2 * k + 1] = __high2float(h2) + 0.0f;
    }
  }
  constexpr int SUB = GV < 32 ? GV : 32;   // channels of one group inside this lane
  constexpr int NSUB = 32 / SUB;
  float mn[NSUB], mx[NSUB];
#pragma unroll
  for (int k = 0; k < NSUB; ++k) {
    mn[k] = INFINITY;
    mx[k] = -INFINITY;
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
      mn[k] = fminf(mn[k], x[k * SUB + i]);
      mx[k] = fmaxf(mx[k], x[k * SUB + i]);
    }
  }
  if constexpr (GV > 32) {                 // groups span GV/32 neighbouring lanes
#pragma unroll
    for (int off = 1; off < GV / 32; off <<= 1) {
      mn[0] = fminf(mn[0], __shfl_xor(mn[0], off, 64));
      mx[0] = fmaxf(mx[0], __shfl_xor(mx[0], off, 64));
    }
  }
  GroupParams p[NSUB];
  float smx = 0.f;
#pragma unroll
  for (int k = 0; k < NSUB; ++k) {
    p[k] = group_params(mn[k], mx[k], BITS);
    smx = fmaxf(smx, p[k].s);
  }
  raise_scale_max(smax, smx);
  constexpr int NG = D / GV;               // groups per token
  if constexpr (GV >= 32) {
    if ((part % (GV / 32)) == 0) {
      const int j = part * 32 / GV;
      scale[tau * NG + j] = p[0].scale;
      zero[tau * NG + j] = p[0].zero;
    }
  } else {
#pragma unroll
    for (int k = 0; k < NSUB; ++k) {
      const int j = (part * 32 + k * SUB) / GV;
      scale[tau * NG + j] = p[k].scale;
      zero[tau * NG + j] = p[k].zero;
    }
  }
  uint8_t* myrow = lds + tau * D + part * 32;
#pragma unroll
  for (int i = 0; i < 32; ++i) myrow[i] = (uint8_t)quant_code<BITS>(x[i], p[i / SUB]);
  __syncthreads();
  // Pack each channel's 16 tokens along tokens, in the same word order as the Keys.
  for (int c = lane; c < D; c += 64) {
    if constexpr (BITS == 2) {
      uint32_t word = 0;
#pragma unroll
      for (int t = 0; t < 16; ++t) word |= (uint32_t)lds[t * D + c] << (8 * (t % 4) + 2 * (t / 4));
      reinterpret_cast<uint32_t*>(codes)[c] = word;
    } else {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        lo |= (uint32_t)lds[t * D + c] << (8 * (t % 4) + 4 * (t / 4));
        hi |= (uint32_t)lds[(t + 8) * D + c] << (8 * (t % 4) + 4 * (t / 4));
      }
      reinterpret_cast<uint2*>(codes)[c] = make_uint2(lo, hi);
    }
  }
}

// Copy `rows` rows of D float16 from src to dst with one wave (16-byte moves).
__device__ __forceinline__ void copy_rows(const __half* __restrict__ src, __half* __restrict__ dst,
                                          int64_t rows) {
  const uint4* s = reinterpret_cast<const uint4*>(src);
  uint4* d = reinterpret_cast<uint4*>(dst);
  const int64_t n = rows * (D / 8);
  for (int64_t i = threadIdx.x; i < n; i += 64) d[i] = s[i];
}

// ---- kernels ----------------------------------------------------------------------

// grid = (Tq/G + 1, B*H): blocks [0, Tq/G) quantize one Key group each; the last
// block copies the tail [Tq, T) into the residual rows.
template <int BITS, int G>
__global__ __launch_bounds__(64) void prefill_k_kernel(LayerView L, const __half* __restrict__ src,
                                                       int64_t ld, int64_t Tq, int64_t T) {
  __shared__ uint8_t lds[G * D];
  const int64_t pair = blockIdx.y;
  const __half* s = src + pair * ld * D;
  const int64_t ngroups = Tq / G;
  const int64_t g = blockIdx.x;
  if (g < ngroups) {
    quantize_k_group<BITS, G>(s + g * G * D,
                              L.k_codes + pair * L.kc_pair() + g * G * (D * BITS / 8),
                              L.k_scale + pair * L.ks_pair() + g * D,
                              L.k_zero + pair * L.ks_pair() + g * D, lds, L.scale_max + 2 * pair);
  } else {
    copy_rows(s + Tq * D, L.k_resid + pair * L.rs_pair(), T - Tq);
  }
}

// grid = (Tq/16 + 1, B*H): blocks [0, Tq/16) quantize one 16-token Value run each;
// the last block copies the tail into the residual rows.
template <int BITS, int GV>
__global__ __launch_bounds__(64) void prefill_v_kernel(LayerView L, const __half* __restrict__ src,
                                                       int64_t ld, int64_t Tq, int64_t T) {
  __shared__ uint8_t lds[kVRun * D];
  const int64_t pair = blockIdx.y;
  const __half* s = src + pair * ld * D;
  const int64_t nruns = Tq / kVRun;
  const int64_t j = blockIdx.x;
  if (j < nruns) {
    quantize_v_run<BITS, GV>(s + j * kVRun * D,
                             L.v_codes + pair * L.vc_pair() + j * (D * kVRun * BITS / 8),
                             L.v_scale + pair * L.vs_pair() + j * kVRun * (D / GV),
                             L.v_zero + pair * L.vs_pair() + j * kVRun * (D / GV), lds,
                             L.scale_max + 2 * pair + 1);
  } else {
    copy_rows(s + Tq * D, L.v_resid + pair * L.rs_pair(), T - Tq);
  }
}

// Append one token per (b, h).  flush == 0: grid (1, B*H), the new row goes to row
// `slot`.  flush == 1: grid (R/G + R/16, B*H); blocks [0, R/G) quantize the Key
// groups of the window and blocks [R/G, R/G + R/16) its Value runs, into the history
// at token t0 = T_before - R.  The blocks that read window row 0 (Key group 0 and
// Value run 0) then store the new row in row 0 after their reads.
template <int BITS, int G, int GV>
__global__ __launch_bounds__(64) void append_kernel(LayerView L, int64_t t0, int slot, int flush,
                                                    const __half* __restrict__ k_new,
                                                    const __half* __restrict__ v_new) {
  constexpr int LROWS = G > kVRun ? G : kVRun;
  __shared__ uint8_t lds[LROWS * D];
  const int64_t pair = blockIdx.y;
  __half* kr = L.k_resid + pair * L.rs_pair();
  __half* vr = L.v_resid + pair * L.rs_pair();
  const __half* kn = k_new + pair * D;
  const __half* vn = v_new + pair * D;
  if (!flush) {
    copy_rows(kn, kr + (int64_t)slot * D, 1);
    copy_rows(vn, vr + (int64_t)slot * D, 1);
    return;
  }
  const int nk = L.R / G;
  const int blk = blockIdx.x;
  if (blk < nk) {
    quantize_k_group<BITS, G>(kr + (int64_t)blk * G * D,
                              L.k_codes + pair * L.kc_pair() + (t0 + blk * G) * (D * BITS / 8),
                              L.k_scale + pair * L.ks_pair() + (t0 / G + blk) * D,
                              L.k_zero + pair * L.ks_pair() + (t0 / G + blk) * D, lds,
                              L.scale_max + 2 * pair);
    if (blk == 0) {
      __syncthreads();
      copy_rows(kn, kr, 1);
    }
  } else {
    const int j = blk - nk;
    quantize_v_run<BITS, GV>(vr + (int64_t)j * kVRun * D,
                             L.v_codes + pair * L.vc_pair() +
                                 (t0 / kVRun + j) * (D * kVRun * BITS / 8),
                             L.v_scale + pair * L.vs_pair() + (t0 + j * kVRun) * (D / GV),
                             L.v_zero + pair * L.vs_pair() + (t0 + j * kVRun) * (D / GV), lds,
                             L.scale_max + 2 * pair + 1);
    if (j == 0) {
      __syncthreads();
      copy_rows(vn, vr, 1);
    }
  }
}

// Entry `which` (0: Keys, 1: Values) of every (b, h) of the layer's scale_max := 0.
__global__ __launch_bounds__(256) void reset_scale_max_kernel(float* sm, int which, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) sm[2 * i + which] = 0.f;
}

template <typename F>
bool dispatch_bits_g(int bits, int G, F&& f) {
  if (bits == 2 && G == 16) return f(std::integral_constant<int, 2>{}, std::integral_constant<int, 16>{});
  if (bits == 2 && G == 32) return f(std::integral_constant<int, 2>{}, std::integral_constant<int, 32>{});
  if (bits == 2 && G == 64) return f(std::integral_constant<int, 2>{}, std::integral_constant<int, 64>{});
  if (bits == 4 && G == 16) return f(std::integral_constant<int, 4>{}, std::integral_constant<int, 16>{});
  if (bits == 4 && G == 32) return f(std::integral_constant<int, 4>{}, std::integral_constant<int, 32>{});
  if (bits == 4 && G == 64) return f(std::integral_constant<int, 4>{}, std::integral_constant<int, 64>{});
  return false;
}

template <typename F>
bool dispatch_gv(int Gv, F&& f) {
  if (Gv == 16) return f(std::integral_constant<int, 16>{});
  if (Gv == 32) return f(std::integral_constant<int, 32>{});
  if (Gv == 64) return f(std::integral_constant<int, 64>{});
  if (Gv == 128) return f(std::integral_constant<int, 128>{});
  return false;
}

}  // namespace

hipError_t launch_quantize_k(const LayerView& L, const __half* src, int64_t ld, int64_t T,
                             hipStream_t s) {
  const int64_t Tq = quantized_len(T, L.R);
  const int pairs = L.B * L.H;
  hipLaunchKernelGGL(reset_scale_max_kernel, dim3((pairs + 255) / 256), dim3(256), 0, s,
                     L.scale_max, 0, pairs);
  const dim3 grid((unsigned)(Tq / L.G + 1), (unsigned)(L.B * L.H));
  bool ok = dispatch_bits_g(L.bits, L.G, [&](auto b, auto g) {
    hipLaunchKernelGGL((prefill_k_kernel<decltype(b)::value, decltype(g)::value>), grid, dim3(64),
                       0, s, L, src, ld, Tq, T);
    return true;
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_quantize_v(const LayerView& L, const __half* src, int64_t ld, int64_t T,
                             hipStream_t s) {
  const int64_t Tq = quantized_len(T, L.R);
  const int pairs = L.B * L.H;
  hipLaunchKernelGGL(reset_scale_max_kernel, dim3((pairs + 255) / 256), dim3(256), 0, s,
                     L.scale_max, 1, pairs);
  const dim3 grid((unsigned)(Tq / kVRun + 1), (unsigned)(L.B * L.H));
  bool ok = dispatch_gv(L.Gv, [&](auto gv) {
    if (L.bits == 2)
      hipLaunchKernelGGL((prefill_v_kernel<2, decltype(gv)::value>), grid, dim3(64), 0, s, L, src,
                         ld, Tq, T);
    else
      hipLaunchKernelGGL((prefill_v_kernel<4, decltype(gv)::value>), grid, dim3(64), 0, s, L, src,
                         ld, Tq, T);
    return true;
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_append_flush(const LayerView& L, int64_t T_before, const __half* k_new,
                               const __half* v_new, hipStream_t s) {
  const int64_t r = residual_len(T_before, L.R);
  const int flush = (r == L.R) ? 1 : 0;
  const int slot = flush ? 0 : (int)r;
  const int64_t t0 = T_before - L.R;
  const dim3 grid(flush ? (unsigned)(L.R / L.G + L.R / kVRun) : 1u, (unsigned)(L.B * L.H));
  bool ok = dispatch_bits_g(L.bits, L.G, [&](auto b, auto g) {
    return dispatch_gv(L.Gv, [&](auto gv) {
      hipLaunchKernelGGL(
          (append_kernel<decltype(b)::value, decltype(g)::value, decltype(gv)::value>), grid,
          dim3(64), 0, s, L, t0, slot, flush, k_new, v_new);
      return true;
    });
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kivi
