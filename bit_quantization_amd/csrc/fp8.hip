// FP8 KV codec: coding float16 Keys and Values as E4M3 or E5M2 with a float32 scale per
// KV head, and decode attention over the FP8 cache.
//
// "09 — KV Cache Quantization", "The lazy default: FP8 KV": the cache is stored as FP8
// (E4M3 or E5M2), half of float16.  "4.4 KV Cache quantization" §4.2: values are
// divided by a scale, one per tensor or per attention head (1.0 when uncalibrated),
// to land in FP8's range; §4.5: the stored precision is not the compute precision.
//
// Coding: code = the FP8 value nearest to float32(x) / s, ties to even, saturating at
// the largest finite value (E4M3 448, E5M2 57344), sign kept; float32 division.
//
// Decode.  Every FP8 value is a float16 value, so the codes are widened exactly
// (v_cvt_scalef32_pk_f16_fp8 / _bf8 with scale 1) and both products run on the
// float16 matrix cores (v_mfma_f32_16x16x32_f16), the per-head scales applied in
// float32 outside them:
//   S^T = K q^T: rows = 16 tokens, columns = the query heads of the pair (padded to 16),
//        the contraction over channels; a lane holds 32 contiguous channels of a token.
//   O^T = V^T P^T: rows = 16 channels, columns = heads, the contraction over the 32
//        tokens of a run.  Lane (head, j) of S^T's two 16-token tiles holds tokens
//        4j .. 4j+3 and 16+4j .. 16+4j+3 — exactly the tokens lane (head, j) must supply
//        to P^T — so the probabilities never leave the registers, and each channel's
//        32 Value bytes are stored in that token order, so that a lane reads its 8
//        Value bytes with one load.
// P is fed as two float16 halves (p = hi + lo, 22 bits), so P.V loses nothing that
// matters next to float32 accumulation.
#include <type_traits>

#include "decode_common.h"

namespace kivi {
namespace {

// Position of token t of a 32-token run in its channel's Value bytes (inverse of the
// order 0-3, 16-19, 4-7, 20-23, ..., 12-15, 28-31).
__host__ __device__ __forceinline__ int run_pos(int t) {
  return 8 * ((t & 15) >> 2) + 4 * (t >> 4) + (t & 3);
}

// FP8 code of a finite float32 y: round to nearest, ties to even, saturating.  With
// e the exponent of |y| clamped below at the format's smallest normal exponent, the
// code is ((e + bias) << M) + rint(|y| * 2^(M - e)) - 2^M: the scaling is exact, rint
// rounds half to even, a mantissa that rounds up to 2^(M+1) carries into the exponent
// field, and below the normal range the same formula gives the subnormal codes.
template <int FMT>
__device__ __forceinline__ uint32_t fp8_code(float y) {
  constexpr int M = FMT ? 2 : 3;
  constexpr int BIAS = FMT ? 15 : 7;
  constexpr int EMIN = 1 - BIAS;
  constexpr float MAXV = FMT ? 57344.f : 448.f;
  constexpr uint32_t MAXC = FMT ? 0x7Bu : 0x7Eu;
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;
  e = e < EMIN ? EMIN : e;
  const int r = (int)rintf(ldexpf(a, M - e));
  const uint32_t code = (uint32_t)(((e + BIAS) << M) + r - (1 << M));
  return sign | (a >= MAXV ? MAXC : code);
}

// ---- coding ---------------------------------------------------------------------------

// grid = (ceil(T / 32), B*H), 256 threads: one 32-token run of one (sequence, KV head).
// Thread (token tt, channels cc .. cc+15) codes its Key and Value elements; the Key
// bytes go straight to their row, the Value bytes to the run's LDS image, written out
// whole (positions of tokens >= T are 0).
template <int FMT>
__global__ __launch_bounds__(256) void fp8_quantize_kernel(Fp8View L, const __half* __restrict__ k,
                                                           const __half* __restrict__ v,
                                                           int64_t ld, int64_t T) {
  __shared__ alignas(16) uint8_t vrun[D * kFp8Run];
  const int64_t pair = blockIdx.y;
  const int h = (int)(pair % L.H);
  const int64_t run = blockIdx.x;
  const int tt = threadIdx.x >> 3, cc = (threadIdx.x & 7) * 16;
  const int64_t t = run * kFp8Run + tt;
  reinterpret_cast<uint4*>(vrun)[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  if (t < T) {
    const float sk = L.k_scale[h], sv = L.v_scale[h];
    const uint4* kr = reinterpret_cast<const uint4*>(k + (pair * ld + t) * D + cc);
    const uint4* vr = reinterpret_cast<const uint4*>(v + (pair * ld + t) * D + cc);
    const uint4 kw[2] = {kr[0], kr[1]}, vw[2] = {vr[0], vr[1]};
    uint32_t kc[4] = {0u, 0u, 0u, 0u};
    const int p = run_pos(tt);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t kword = (&kw[i / 8].x)[(i % 8) / 2], vword = (&vw[i / 8].x)[(i % 8) / 2];
      const unsigned short kb = (unsigned short)(kword >> (16 * (i & 1)));
      const unsigned short vb = (unsigned short)(vword >> (16 * (i & 1)));
      kc[i / 4] |= fp8_code<FMT>(__half2float(__ushort_as_half(kb)) / sk) << (8 * (i % 4));
      vrun[(cc + i) * kFp8Run + p] = (uint8_t)fp8_code<FMT>(__half2float(__ushort_as_half(vb)) / sv);
    }
    *reinterpret_cast<uint4*>(L.k + pair * L.pair_bytes() + t * D + cc) =
        make_uint4(kc[0], kc[1], kc[2], kc[3]);
  }
  __syncthreads();
  reinterpret_cast<uint4*>(L.v + pair * L.pair_bytes() + run * D * kFp8Run)[threadIdx.x] =
      reinterpret_cast<const uint4*>(vrun)[threadIdx.x];
}

// grid = B*H, 64 threads: token t of each (sequence, KV head); lane l codes channels
// 2l, 2l+1.
template <int FMT>
__global__ __launch_bounds__(64) void fp8_append_kernel(Fp8View L, const __half* __restrict__ kn,
                                                        const __half* __restrict__ vn, int64_t t) {
  const int64_t pair = blockIdx.x;
  const int h = (int)(pair % L.H);
  const int lane = threadIdx.x;
  const float sk = L.k_scale[h], sv = L.v_scale[h];
  const __half2 k2 = reinterpret_cast<const __half2*>(kn + pair * D)[lane];
  const __half2 v2 = reinterpret_cast<const __half2*>(vn + pair * D)[lane];
  const uint32_t k0 = fp8_code<FMT>(__low2float(k2) / sk), k1 = fp8_code<FMT>(__high2float(k2) / sk);
  reinterpret_cast<uint16_t*>(L.k + pair * L.pair_bytes() + t * D)[lane] = (uint16_t)(k0 | (k1 << 8));
  uint8_t* vrun = L.v + pair * L.pair_bytes() + (t / kFp8Run) * D * kFp8Run + run_pos((int)(t % kFp8Run));
  vrun[(2 * lane) * kFp8Run] = (uint8_t)fp8_code<FMT>(__low2float(v2) / sv);
  vrun[(2 * lane + 1) * kFp8Run] = (uint8_t)fp8_code<FMT>(__high2float(v2) / sv);
}

// ---- decode ---------------------------------------------------------------------------

struct Fp8DecodeArgs {
  Fp8View L;
  const __half* q;
  float* out;
  float* part;          // [P][nw][GQA][PSTRIDE]
  unsigned* counters;   // [P][kCounterStride]
  int64_t T;
  int64_t nblk;         // 32-token blocks per pair
  int nw;               // workgroups per pair
  float qscale;         // sm_scale * log2(e)
};

constexpr int kFp8WavesPerSimd = 4;   // 127 VGPRs or fewer: four waves per SIMD

// Eight FP8 bytes (two words) -> eight float16 (exact).
template <int FMT>
__device__ __forceinline__ f16x8 widen8(uint32_t w0, uint32_t w1) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 a, b, c, d;
  if constexpr (FMT == 0) {
    a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
    b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
    c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
    d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  } else {
    a = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w0, 1.0f, false);
    b = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w0, 1.0f, true);
    c = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w1, 1.0f, false);
    d = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w1, 1.0f, true);
  }
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Token of the run that k-slot e (0..7) of lane group j supplies to P.V.
__device__ __forceinline__ int slot_token(int j, int e) { return 4 * j + (e & 3) + 16 * (e >> 2); }

// One workgroup per CU; workgroup s of a pair takes 32-token blocks [nblk*s/nw,
// nblk*(s+1)/nw), its waves take them from an LDS counter.  Each wave keeps an online
// softmax per head (lane group j of lane (head, j) sees a quarter of the tokens; the
// block maximum is reduced over the four groups, the sum l at the end).
template <int FMT, int GQA>
__global__ __launch_bounds__(256 * kFp8WavesPerSimd, 1) void fp8_decode_kernel(Fp8DecodeArgs a) {
  constexpr int WAVES = 4 * kFp8WavesPerSimd;
  constexpr int NTH = 64 * WAVES;
  __shared__ alignas(16) float comb[WAVES][GQA * PSTRIDE];
  __shared__ int counter;

  const Fp8View& L = a.L;
  const int64_t P = (int64_t)L.B * L.H;
  const int64_t pair = blockIdx.x % P;
  const int s = (int)(blockIdx.x / P);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, lo = lane & 15, j = lane >> 4;
  const int64_t b = pair / L.H;
  const int h = (int)(pair % L.H);
  const int64_t b_lo = a.nblk * s / a.nw, b_hi = a.nblk * (s + 1) / a.nw;

  if (threadIdx.x == 0) counter = 0;
  const int n_parts = a.nw;
  const int64_t pair_floats = (int64_t)n_parts * GQA * PSTRIDE;
  const __amdgpu_buffer_rsrc_t parts = make_rsrc(a.part + pair * pair_floats, pair_floats * 4);
  const int my = s * GQA * PSTRIDE * 4;
  if (n_parts > 1) clear_partial<GQA, NTH>(parts, my);
  __syncthreads();

  // q^T operand: lane (head lo, j) holds channels 32j + 8ks .. +7 for K-step ks
  f16x8 bq[4];
  const __half* qp = a.q + ((b * L.H + h) * GQA) * D;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    f16x8 v = {};
    if (lo < GQA) v = *reinterpret_cast<const f16x8*>(qp + lo * D + 32 * j + 8 * ks);
    bq[ks] = v;
  }
  const float zscale = a.qscale * L.k_scale[h];
  const float vscale = L.v_scale[h];
  const __amdgpu_buffer_rsrc_t kres = make_rsrc(L.k + pair * L.pair_bytes(), L.pair_bytes());
  const __amdgpu_buffer_rsrc_t vres = make_rsrc(L.v + pair * L.pair_bytes(), L.pair_bytes());

  float m = -INFINITY, l = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int item = grab_item(&counter); b_lo + item < b_hi; item = grab_item(&counter)) {
    const int64_t blk = b_lo + item;
    const int64_t t0 = blk * kFp8Run;
    // Key bytes: tile nt, token t0 + 16nt + lo, channels 32j .. 32j+31
    u32x4 kw[2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        kw[nt][hf] = __builtin_amdgcn_raw_buffer_load_b128(
            kres, (int)((t0 + 16 * nt + lo) * D + 32 * j + 16 * hf), 0, 0);
    // Value bytes: channel 16mt + lo, run positions 8j .. 8j+7
    u32x2 vw[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
      vw[mt] = __builtin_amdgcn_raw_buffer_load_b64(
          vres, (int)(blk * D * kFp8Run + (16 * mt + lo) * kFp8Run + 8 * j), 0, 0);

    // S^T = K q^T for the two 16-token tiles
    f32x4 d[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      d[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 w = kw[nt][ks / 2];
        const f16x8 kf = widen8<FMT>(ks & 1 ? w[2] : w[0], ks & 1 ? w[3] : w[1]);
        d[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, bq[ks], d[nt], 0, 0, 0);
      }
    }
    // logits of head lo, tokens slot_token(j, e), base 2
    const bool partial = t0 + kFp8Run > a.T;
    float z[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      z[e] = d[e >> 2][e & 3] * zscale;
      if (partial && t0 + slot_token(j, e) >= a.T) z[e] = -INFINITY;
    }
    float mx = z[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, z[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    f16x8 ph, pl;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __builtin_amdgcn_exp2f(z[e] - m_new);
      psum += p;
      const _Float16 hi = (_Float16)p;
      ph[e] = hi;
      pl[e] = (_Float16)(p - (float)hi);
    }
    l = l * alpha + psum;
    // O^T += V^T P^T for the eight 16-channel tiles
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      f16x8 vf = widen8<FMT>(vw[mt][0], vw[mt][1]);
      if (partial) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (t0 + slot_token(j, e) >= a.T) vf[e] = (_Float16)0.f;
      }
      acc[mt] = acc[mt] * alpha;
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, ph, acc[mt], 0, 0, 0);
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pl, acc[mt], 0, 0, 0);
    }
  }

  // the wave's record: acc of head lo, channels 16mt + 4j + i; l summed over the groups
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (lo < GQA) {
    float* rec = comb[wave] + lo * PSTRIDE;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) rec[16 * mt + 4 * j + i] = acc[mt][i] * vscale;
    if (j == 0) {
      rec[D] = m;
      rec[D + 1] = l;
    }
  }
  __syncthreads();
  float* o = a.out + (b * L.H + h) * GQA * D;
  finish_pair<GQA, NTH, WAVES>([&](int i) { return (const float*)comb[i]; }, parts, my, n_parts,
                               a.counters + kCounterStride * pair, o, &comb[0][0]);
}

template <typename F>
bool dispatch_fmt(int fmt, F&& f) {
  if (fmt == 0) return f(std::integral_constant<int, 0>{});
  if (fmt == 1) return f(std::integral_constant<int, 1>{});
  return false;
}

}  // namespace

hipError_t launch_fp8_quantize(const Fp8View& L, const __half* k, const __half* v, int64_t ld,
                               int64_t T, hipStream_t s) {
  const dim3 grid((unsigned)((T + kFp8Run - 1) / kFp8Run), (unsigned)(L.B * L.H));
  if (!dispatch_fmt(L.fmt, [&](auto f) {
        hipLaunchKernelGGL((fp8_quantize_kernel<decltype(f)::value>), grid, dim3(256), 0, s, L, k, v,
                           ld, T);
        return true;
      }))
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_fp8_append(const Fp8View& L, const __half* k_new, const __half* v_new, int64_t t,
                             hipStream_t s) {
  if (!dispatch_fmt(L.fmt, [&](auto f) {
        hipLaunchKernelGGL((fp8_append_kernel<decltype(f)::value>), dim3((unsigned)(L.B * L.H)),
                           dim3(64), 0, s, L, k_new, v_new, t);
        return true;
      }))
    return hipErrorInvalidValue;
  return hipGetLastError();
}

Fp8Plan plan_fp8_decode(int B, int H, int q_heads, int64_t T, int n_split_req) {
  Fp8Plan p{};
  const int gqa = q_heads / H;
  const int64_t nblk = (T + kFp8Run - 1) / kFp8Run;
  const int64_t pairs = (int64_t)B * H;
  int64_t nw = n_split_req > 0 ? n_split_req : device_cus() / pairs;
  if (n_split_req <= 0) {
    // by default no more workgroups than keep every wave busy with a 32-token run:
    // beyond that they only add partials to merge (the count still grows with T, so a
    // workspace sized for T serves every smaller T)
    const int64_t waves = 4 * kFp8WavesPerSimd;
    const int64_t busy = (nblk + waves - 1) / waves;
    if (nw > busy) nw = busy;
  }
  if (nw > nblk) nw = nblk;
  if (nw < 1) nw = 1;
  p.n_split = (int)nw;
  p.ws_counters = (size_t)pairs * kCounterStride * sizeof(uint32_t);
  p.ws_partials = nw > 1 ? (size_t)pairs * nw * gqa * PSTRIDE * sizeof(float) : 0;
  p.ws_total = p.ws_counters + p.ws_partials;
  return p;
}

hipError_t launch_fp8_decode(const Fp8View& L, int q_heads, int64_t T, const __half* q,
                             float sm_scale, float* out, void* ws, const Fp8Plan& plan,
                             hipStream_t s) {
  Fp8DecodeArgs a;
  a.L = L;
  a.q = q;
  a.out = out;
  a.counters = reinterpret_cast<unsigned*>(ws);
  a.part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + plan.ws_counters);
  a.T = T;
  a.nblk = (T + kFp8Run - 1) / kFp8Run;
  a.nw = plan.n_split;
  a.qscale = sm_scale * 1.4426950408889634f;
  const int gqa = q_heads / L.H;
  const dim3 grid((unsigned)((int64_t)L.B * L.H * plan.n_split));
  const dim3 block(256 * kFp8WavesPerSimd);
  bool ok = dispatch_fmt(L.fmt, [&](auto f) {
    constexpr int F = decltype(f)::value;
    switch (gqa) {
      case 1: launch_decode_kernel(fp8_decode_kernel<F, 1>, grid, block, s, a); return true;
      case 2: launch_decode_kernel(fp8_decode_kernel<F, 2>, grid, block, s, a); return true;
      case 4: launch_decode_kernel(fp8_decode_kernel<F, 4>, grid, block, s, a); return true;
      case 8: launch_decode_kernel(fp8_decode_kernel<F, 8>, grid, block, s, a); return true;
      default: return false;
    }
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kivi
