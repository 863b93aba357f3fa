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
#include <algorithm>
#include <type_traits>

#include "kivi_internal.h"
#include "quantizer.h"

#pragma clang fp contract(off)

namespace kivi {
namespace {

constexpr int D = kHeadDim;
constexpr int V_LDS = 4 * (32 * 16 + 16);    // bytes of LDS one Value run needs
constexpr int QW = 4;                        // waves (groups or runs) per workgroup

// LDS hand-off between the lanes of one wave: LDS operations of a wave execute in
// order, so only the compiler must be kept from moving LDS accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Lane-wise min / max of float16 pairs (exact: no rounding).  Issued directly: the
// generic minnum lowering first canonicalizes each operand (one more instruction per
// loaded pair) to quiet signalling NaNs, and inputs here are finite.
__device__ __forceinline__ __half2 hmin2(__half2 a, __half2 b) {
  uint32_t r;
  asm("v_pk_min_f16 %0, %1, %2" : "=v"(r) : "v"(__builtin_bit_cast(uint32_t, a)),
      "v"(__builtin_bit_cast(uint32_t, b)));
  return __builtin_bit_cast(__half2, r);
}
__device__ __forceinline__ __half2 hmax2(__half2 a, __half2 b) {
  uint32_t r;
  asm("v_pk_max_f16 %0, %1, %2" : "=v"(r) : "v"(__builtin_bit_cast(uint32_t, a)),
      "v"(__builtin_bit_cast(uint32_t, b)));
  return __builtin_bit_cast(__half2, r);
}


// Largest value over the NW waves of the workgroup, raised into *p by one atomic
// (scale maxima: non-negative floats order like their bit patterns, so an unsigned
// atomic max is a float max).  Every thread of the workgroup must call it.  One
// atomic per workgroup matters: the entries of neighbouring (b, h) share a cache
// line, and atomics on one line serialize.
template <int NW>
__device__ __forceinline__ void raise_scale_max(float* p, float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  if constexpr (NW > 1) {
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) v = fmaxf(v, red[w]);
  }
  if (threadIdx.x == 0)
    __hip_atomic_fetch_max(reinterpret_cast<unsigned*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}


// One wave quantizes one Key group: G tokens x D channels, rows of D float16 at
// `src`.  Lane l owns channels 2l and 2l+1.  Writes G packed rows at `codes`
// (row stride D*BITS/8 bytes) and D scales/zeros, and returns the lane's larger
// scale.  `lds` holds G*D bytes private to the wave.  A -0 input acts as +0: only
// the minimum and maximum can carry the sign into a result (zero, scale), and both
// are canonicalized.
template <int BITS, int G>
__device__ __forceinline__ float quantize_k_group(const __half* __restrict__ src,
                                                  uint8_t* __restrict__ codes,
                                                  __half* __restrict__ scale,
                                                  __half* __restrict__ zero, uint8_t* lds) {
  const int lane = threadIdx.x & 63;
  const __half2* s2 = reinterpret_cast<const __half2*>(src);
  __half2 x[G];
#pragma unroll
  for (int t = 0; t < G; ++t) x[t] = s2[t * (D / 2) + lane];
  __half2 mn = x[0], mx = x[0];              // float16 min/max are exact
#pragma unroll
  for (int t = 1; t < G; ++t) {
    mn = hmin2(mn, x[t]);
    mx = hmax2(mx, x[t]);
  }
  const GroupParams p0 = group_params(__low2float(mn) + 0.0f, __low2float(mx) + 0.0f, BITS);
  const GroupParams p1 = group_params(__high2float(mn) + 0.0f, __high2float(mx) + 0.0f, BITS);
  reinterpret_cast<__half2*>(scale)[lane] = __halves2half2(p0.scale, p1.scale);
  reinterpret_cast<__half2*>(zero)[lane] = __halves2half2(p0.zero, p1.zero);
  // codes into LDS as bytes, [token][channel]
#pragma unroll
  for (int t = 0; t < G; ++t) {
    const uint32_t c0 = quant_bits<BITS>(__low2half(x[t]), p0);
    const uint32_t c1 = quant_bits<BITS>(__high2half(x[t]), p1);
    // low bytes of c0 and c1 side by side
    reinterpret_cast<uint16_t*>(lds + t * D)[lane] =
        (uint16_t)__builtin_amdgcn_perm(c1, c0, 0x0c0c0400u);
  }
  wave_lds_sync();
  // Pack each token row along channels.  A 16-byte chunk holds the codes of 16
  // consecutive channels; its dword k holds channels 4k .. 4k+3, and shifting dword
  // k by BITS*k puts each code at bit BITS*k of its byte: 2-bit, one word per chunk
  // (code e of the word in byte e % 4 at bit 2(e / 4)); 4-bit, two words.
  constexpr int CHUNKS = G * (D / 16);
  for (int i = lane; i < CHUNKS; i += 64) {
    const int t = i / (D / 16), ch = i % (D / 16);
    const uint4 d = *reinterpret_cast<const uint4*>(lds + t * D + 16 * ch);
    if constexpr (BITS == 2) {
      const uint32_t word = d.x | (d.y << 2) | (d.z << 4) | (d.w << 6);
      reinterpret_cast<uint32_t*>(codes + (int64_t)t * (D * BITS / 8))[ch] = word;
    } else {
      reinterpret_cast<uint2*>(codes + (int64_t)t * (D * BITS / 8))[ch] =
          make_uint2(d.x | (d.y << 4), d.z | (d.w << 4));
    }
  }
  return fmaxf(p0.s, p1.s);
}

// One wave quantizes one run of 16 Value tokens (each token in groups of GV
// channels).  Lane l owns token l/4 and channels 32*(l%4) .. +31.  Writes the run's
// packed codes ([D][16*BITS/8] bytes at `codes`) and 16*(D/GV) scales/zeros, and
// returns the largest scale among the lane's groups.  `lds` holds V_LDS bytes private
// to the wave.  -0 is handled as in quantize_k_group.
// With n_valid < 16 (the last run of a Value history that ends inside a run, per-token
// Value window only) tokens n_valid .. 15 get code 0 and no scale or zero: the bytes the
// definition gives a run whose later tokens are not yet quantized.
template <int BITS, int GV>
__device__ __forceinline__ float quantize_v_run(const __half* __restrict__ src,
                                                uint8_t* __restrict__ codes,
                                                __half* __restrict__ scale,
                                                __half* __restrict__ zero, uint8_t* lds,
                                                int n_valid = kVRun) {
  const int lane = threadIdx.x & 63;
  const int tau = lane >> 2, part = lane & 3;
  const bool valid = tau < n_valid;
  const uint4* row = reinterpret_cast<const uint4*>(src + tau * D + part * 32);
  __half2 x2[16];                          // channels 2i, 2i+1 of the lane's 32
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 u = row[i];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) x2[4 * i + k] = *reinterpret_cast<const __half2*>(&w[k]);
  }
  auto xh = [&](int i) { return (i & 1) ? __high2half(x2[i >> 1]) : __low2half(x2[i >> 1]); };
  constexpr int SUB = GV < 32 ? GV : 32;   // channels of one group inside this lane
  constexpr int NSUB = 32 / SUB;
  float mn[NSUB], mx[NSUB];
#pragma unroll
  for (int k = 0; k < NSUB; ++k) {        // float16 min/max over pairs, then the halves
    __half2 m2 = x2[k * SUB / 2], M2 = x2[k * SUB / 2];
#pragma unroll
    for (int i = 1; i < SUB / 2; ++i) {
      m2 = hmin2(m2, x2[k * SUB / 2 + i]);
      M2 = hmax2(M2, x2[k * SUB / 2 + i]);
    }
    mn[k] = fminf(__low2float(m2), __high2float(m2));
    mx[k] = fmaxf(__low2float(M2), __high2float(M2));
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
    p[k] = group_params(mn[k] + 0.0f, mx[k] + 0.0f, BITS);   // -0 -> +0
    if (valid) smx = fmaxf(smx, p[k].s);
  }
  constexpr int NG = D / GV;               // groups per token
  if (!valid) {
  } else if constexpr (GV >= 32) {
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
  // codes into LDS transposed, [channel][token] (16 bytes per channel, plus 16 bytes
  // after every 32 channels so that the four lane groups' byte writes use different
  // banks)
  uint8_t* col = lds + part * (32 * 16 + 16) + tau;
#pragma unroll
  for (int i = 0; i < 32; ++i)
    col[16 * i] = valid ? (uint8_t)quant_bits<BITS>(xh(i), p[i / SUB]) : (uint8_t)0;
  wave_lds_sync();
  // Pack each channel's 16 tokens: dword k of the channel's 16 bytes holds tokens
  // 4k .. 4k+3, shifted by BITS*k into the word order of the Keys.
  for (int c = lane; c < D; c += 64) {
    const uint4 d = *reinterpret_cast<const uint4*>(lds + (c >> 5) * (32 * 16 + 16) + (c & 31) * 16);
    if constexpr (BITS == 2) {
      reinterpret_cast<uint32_t*>(codes)[c] = d.x | (d.y << 2) | (d.z << 4) | (d.w << 6);
    } else {
      reinterpret_cast<uint2*>(codes)[c] = make_uint2(d.x | (d.y << 4), d.z | (d.w << 4));
    }
  }
  return smx;
}

// One wave quantizes one Value token (D float16 at `src`, groups of GV channels) into
// position e of its 16-token run (`run`: [D][16*BITS/8] bytes), leaving the other
// tokens' codes as they are: lane l owns channels 2l and 2l+1, and rewrites the bits of
// its code in each channel's word(s) (code e of a run in byte e mod 4 at bit b*(e/4) of
// its 32-bit word, the word order of quantize_v_run).  Writes the token's D/GV scales
// and zeros and returns the lane's scale.  "4.4 KV Cache quantization" §3.2: the Value
// that leaves the float16 window is quantized on its own.
template <int BITS, int GV>
__device__ __forceinline__ float quantize_v_token(const __half* __restrict__ src,
                                                  uint8_t* __restrict__ run, int e,
                                                  __half* __restrict__ scale,
                                                  __half* __restrict__ zero) {
  const int lane = threadIdx.x & 63;
  const __half2 x = reinterpret_cast<const __half2*>(src)[lane];
  // group min / max over the GV / 2 lanes of the group (float16 values, exact)
  float mn = fminf(__low2float(x), __high2float(x));
  float mx = fmaxf(__low2float(x), __high2float(x));
#pragma unroll
  for (int off = 1; off < GV / 2; off <<= 1) {
    mn = fminf(mn, __shfl_xor(mn, off, 64));
    mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  }
  const GroupParams p = group_params(mn + 0.0f, mx + 0.0f, BITS);   // -0 -> +0
  if ((lane % (GV / 2)) == 0) {
    scale[2 * lane / GV] = p.scale;
    zero[2 * lane / GV] = p.zero;
  }
  const uint32_t c0 = quant_bits<BITS>(__low2half(x), p) & 0xFFu;
  const uint32_t c1 = quant_bits<BITS>(__high2half(x), p) & 0xFFu;
  constexpr uint32_t mask = (1u << BITS) - 1u;
  if constexpr (BITS == 2) {
    uint32_t* w = reinterpret_cast<uint32_t*>(run) + 2 * lane;   // one word per channel
    const int pos = 8 * (e & 3) + 2 * (e >> 2);
    w[0] = (w[0] & ~(mask << pos)) | (c0 << pos);
    w[1] = (w[1] & ~(mask << pos)) | (c1 << pos);
  } else {
    uint32_t* w = reinterpret_cast<uint32_t*>(run) + 4 * lane + (e >> 3);   // two per channel
    const int pos = 8 * (e & 3) + 4 * ((e & 7) >> 2);
    w[0] = (w[0] & ~(mask << pos)) | (c0 << pos);
    w[2] = (w[2] & ~(mask << pos)) | (c1 << pos);
  }
  return p.s;
}

// Copy `rows` rows of D float16 from src to dst with one wave (16-byte moves).
__device__ __forceinline__ void copy_rows(const __half* __restrict__ src, __half* __restrict__ dst,
                                          int64_t rows) {
  const uint4* s = reinterpret_cast<const uint4*>(src);
  uint4* d = reinterpret_cast<uint4*>(dst);
  const int64_t n = rows * (D / 8);
  for (int64_t i = threadIdx.x & 63; i < n; i += 64) d[i] = s[i];
}

// The float16 rows of one (b, h) after a prefill: the ns sink tokens (the first rows
// of the sequence s0) to residual rows [0, ns), and the r window tokens (w, the
// tokens after the quantized history) to their ring rows S + ring .. wrapping after
// row S + R - 1.
__device__ __forceinline__ void store_fp16_rows(const LayerView& L, const __half* s0,
                                                const __half* w, __half* resid, int64_t ns,
                                                int64_t r, int ring) {
  copy_rows(s0, resid, ns);
  const int64_t n1 = r < L.R - ring ? r : L.R - ring;
  copy_rows(w, resid + (int64_t)(L.S + ring) * D, n1);
  copy_rows(w + n1 * D, resid + (int64_t)L.S * D, r - n1);
}

// ---- kernels ----------------------------------------------------------------------

// LayerView's history geometry with PAGED (a page table is set) known at compile time,
// so that the contiguous kernels carry no page-table branches: the section of a pair,
// its rows, and where history token t of sequence b sits in it.
template <bool PAGED>
struct Hist {
  int64_t sec, rows;
  __device__ Hist(const LayerView& L, int64_t pair)
      : sec(PAGED ? pair % L.H : pair), rows(PAGED ? L.pages << L.page_log2 : L.Tmax) {}
  __device__ int64_t token(const LayerView& L, int64_t b, int64_t t) const {
    return PAGED ? L.hist_token(b, t) : t;
  }
};

// Items of one (b, h): the Tq/G Key groups (or Tq/16 Value runs) of the tokens after
// the sink, then one item that copies the sink tokens and the r window tokens into
// their residual rows.  grid = (ceil(items /
// (QW*npw)), B*H) for the items of T tokens; workgroup x takes items QW*npw*x ..
// +QW*npw - 1, its waves interleaved (wave w takes item QW*npw*x + QW*i + w for
// i < npw).  A ragged batch gives sequence b lens.get(b, 0) <= T tokens, so its pairs
// have no more items than the grid covers.
template <int BITS, int G, bool PAGED>
__global__ __launch_bounds__(64 * QW) void prefill_k_kernel(LayerView L, const __half* __restrict__ src,
                                                            int64_t ld, int64_t T, Lens lens,
                                                            int npw) {
  __shared__ alignas(16) uint8_t lds[QW][G * D];
  __shared__ float red[QW];
  const int64_t pair = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const TokenSplit ts = split_tokens(L, lens.p ? lens.get(pair / L.H, 0) : T);
  const int64_t Tq = ts.Tq;
  const __half* s0 = src + pair * ld * D;
  const __half* s = s0 + (int64_t)L.S * D;        // the tokens after the sink
  const int64_t ngroups = Tq / G;
  float smx = 0.f;
  for (int i = 0; i < npw; ++i) {
    const int64_t g = ((int64_t)blockIdx.x * npw + i) * QW + wave;
    if (g < ngroups) {
      const Hist<PAGED> hs(L, pair);
      const int64_t ht = hs.token(L, pair / L.H, g * G);
      const int64_t kc = hs.sec * hs.rows * (D * BITS / 8), ks = hs.sec * (hs.rows / G) * D;
      smx = fmaxf(smx, quantize_k_group<BITS, G>(
                           s + g * G * D, L.k_codes + kc + ht * (D * BITS / 8),
                           L.k_scale + ks + (ht / G) * D, L.k_zero + ks + (ht / G) * D, lds[wave]));
    } else if (g == ngroups) {
      store_fp16_rows(L, s0, s + Tq * D, L.k_resid + pair * L.rs_pair(), ts.ns, ts.r, ts.ring);
    }
  }
  raise_scale_max<QW>(L.scale_max + 2 * pair, smx, red);
}

// As prefill_k_kernel, over the Value runs.
template <int BITS, int GV, bool PAGED>
__global__ __launch_bounds__(64 * QW) void prefill_v_kernel(LayerView L, const __half* __restrict__ src,
                                                            int64_t ld, int64_t T, Lens lens,
                                                            int npw) {
  __shared__ alignas(16) uint8_t lds[QW][V_LDS];
  __shared__ float red[QW];
  const int64_t pair = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const TokenSplit ts = split_tokens(L, lens.p ? lens.get(pair / L.H, 0) : T);
  const int64_t Tqv = ts.Tqv;                     // Tq unless the per-token Value window
  const __half* s0 = src + pair * ld * D;
  const __half* s = s0 + (int64_t)L.S * D;        // the tokens after the sink
  const int64_t nruns = (Tqv + kVRun - 1) / kVRun;
  float smx = 0.f;
  for (int i = 0; i < npw; ++i) {
    const int64_t j = ((int64_t)blockIdx.x * npw + i) * QW + wave;
    if (j < nruns) {
      const Hist<PAGED> hs(L, pair);
      const int64_t ht = hs.token(L, pair / L.H, j * kVRun);
      const int64_t vc = hs.sec * hs.rows * (D * BITS / 8), vs = hs.sec * hs.rows * (D / GV);
      const int n_valid = Tqv - j * kVRun < kVRun ? (int)(Tqv - j * kVRun) : kVRun;
      smx = fmaxf(smx, quantize_v_run<BITS, GV>(
                           s + j * kVRun * D,
                           L.v_codes + vc + (ht / kVRun) * (D * kVRun * BITS / 8),
                           L.v_scale + vs + ht * (D / GV), L.v_zero + vs + ht * (D / GV),
                           lds[wave], n_valid));
    } else if (j == nruns) {
      store_fp16_rows(L, s0, s + Tqv * D, L.v_resid + pair * L.rs_pair(), ts.ns, ts.rv,
                      ts.ring_v);
    }
  }
  raise_scale_max<QW>(L.scale_max + 2 * pair + 1, smx, red);
}

// Items per wave so that all (b, h) together launch about kPrefillBlocks workgroups.
constexpr int64_t kPrefillBlocks = 2048;
int items_per_wave(int64_t items, int pairs) {
  const int64_t blocks_per_pair = std::max<int64_t>(1, kPrefillBlocks / pairs);
  return (int)std::max<int64_t>(1, (items + QW * blocks_per_pair - 1) / (QW * blocks_per_pair));
}

// Append one token per (b, h).  n == 0: grid (1, B*H), the new row goes to residual
// row `slot`.  n > 0 (the window is full): grid (n/G + n/16, B*H); blocks [0, n/G)
// quantize the Key groups of the n oldest window tokens (residual rows [first,
// first + n)) and blocks [n/G, n/G + n/16) their Value runs, into the history at token
// t0.  The blocks that read row `first` (Key group 0 and Value run 0) then store the
// new row there (slot == first) after their reads.  A ragged batch (lens.p set) plans
// each sequence on the device: the grid has the blocks of the largest flush, blocks a
// sequence does not need return at once, and with flush_only a sequence that does
// not flush leaves its new row to the decode launch that follows.
// With the per-token Value window (L.vwin; uniform batches only) Keys flush as above
// over blocks [0, n/G) and block n/G (the only block when nothing flushes) quantizes
// the Value leaving the window, if any (vtok: history token vt, read from row `slot`),
// then stores the new Value row there (and the new Key row when no Key flush does).
template <int BITS, int G, int GV>
__global__ __launch_bounds__(64) void append_kernel(LayerView L, int64_t t0, int slot, int n,
                                                    const __half* __restrict__ k_new,
                                                    const __half* __restrict__ v_new, Lens lens,
                                                    int flush_only, int vtok, int64_t vt) {
  constexpr int LBYTES = G * D > V_LDS ? G * D : V_LDS;
  __shared__ alignas(16) uint8_t lds[LBYTES];
  const int64_t pair = blockIdx.y;
  if (lens.p) {
    const AppendPlan ap = plan_append(L, lens.get(pair / L.H, 0));
    n = ap.flush ? ap.n : 0;
    slot = ap.slot;
    t0 = ap.t0;
    if (n == 0 ? (flush_only || blockIdx.x > 0) : (int)blockIdx.x >= n / G + n / kVRun) return;
  }
  const __half* kn = k_new + pair * D;
  const __half* vn = v_new + pair * D;
  __half* kr = L.k_resid + pair * L.rs_pair() + (int64_t)slot * D;
  __half* vr = L.v_resid + pair * L.rs_pair() + (int64_t)slot * D;
  const int nk = n / G;
  const int blk = blockIdx.x;
  const int64_t sec = L.section(pair);
  if (L.vwin) {
    // per-token Value window: blocks [0, nk) flush Key groups (block 0 then stores the
    // new Key row over the oldest), block nk the Value side
    if (blk < nk) {
      const int64_t ht = t0 + (int64_t)blk * G;
      const float smx = quantize_k_group<BITS, G>(
          kr + (int64_t)blk * G * D, L.k_codes + sec * L.kc_pair() + ht * (D * BITS / 8),
          L.k_scale + sec * L.ks_pair() + (ht / G) * D, L.k_zero + sec * L.ks_pair() + (ht / G) * D,
          lds);
      raise_scale_max<1>(L.scale_max + 2 * pair, smx, nullptr);
      if (blk == 0) {
        __syncthreads();
        copy_rows(kn, kr, 1);
      }
      return;
    }
    if (vtok) {
      // the oldest Value leaves the full window: quantized on its own into history
      // token vt (its row is the new token's slot), then the new Value takes the row
      const float smx = quantize_v_token<BITS, GV>(
          vr, L.v_codes + sec * L.vc_pair() + (vt / kVRun) * (D * kVRun * BITS / 8),
          (int)(vt % kVRun), L.v_scale + sec * L.vs_pair() + vt * (D / GV),
          L.v_zero + sec * L.vs_pair() + vt * (D / GV));
      raise_scale_max<1>(L.scale_max + 2 * pair + 1, smx, nullptr);
      __syncthreads();
    }
    copy_rows(vn, vr, 1);
    if (nk == 0) copy_rows(kn, kr, 1);
    return;
  }
  if (n == 0) {
    copy_rows(kn, kr, 1);
    copy_rows(vn, vr, 1);
    return;
  }
  if (blk < nk) {
    const int64_t ht = L.hist_token(pair / L.H, t0 + (int64_t)blk * G);
    const float smx = quantize_k_group<BITS, G>(
        kr + (int64_t)blk * G * D, L.k_codes + sec * L.kc_pair() + ht * (D * BITS / 8),
        L.k_scale + sec * L.ks_pair() + (ht / G) * D, L.k_zero + sec * L.ks_pair() + (ht / G) * D,
        lds);
    raise_scale_max<1>(L.scale_max + 2 * pair, smx, nullptr);
    if (blk == 0) {
      __syncthreads();
      copy_rows(kn, kr, 1);
    }
  } else {
    const int j = blk - nk;
    const int64_t ht = L.hist_token(pair / L.H, t0 + (int64_t)j * kVRun);
    const float smx = quantize_v_run<BITS, GV>(
        vr + (int64_t)j * kVRun * D,
        L.v_codes + sec * L.vc_pair() + (ht / kVRun) * (D * kVRun * BITS / 8),
        L.v_scale + sec * L.vs_pair() + ht * (D / GV), L.v_zero + sec * L.vs_pair() + ht * (D / GV),
        lds);
    raise_scale_max<1>(L.scale_max + 2 * pair + 1, smx, nullptr);
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
                             Lens lens, hipStream_t s) {
  const TokenSplit ts = split_tokens(L, T);
  const int64_t Tq = ts.Tq;
  const int pairs = L.B * L.H;
  hipLaunchKernelGGL(reset_scale_max_kernel, dim3((pairs + 255) / 256), dim3(256), 0, s,
                     L.scale_max, 0, pairs);
  const int64_t items = Tq / L.G + 1;
  const int npw = items_per_wave(items, pairs);
  const dim3 grid((unsigned)((items + QW * npw - 1) / (QW * npw)), (unsigned)pairs);
  bool ok = dispatch_bits_g(L.bits, L.G, [&](auto b, auto g) {
    if (L.table)
      hipLaunchKernelGGL((prefill_k_kernel<decltype(b)::value, decltype(g)::value, true>), grid,
                         dim3(64 * QW), 0, s, L, src, ld, T, lens, npw);
    else
      hipLaunchKernelGGL((prefill_k_kernel<decltype(b)::value, decltype(g)::value, false>), grid,
                         dim3(64 * QW), 0, s, L, src, ld, T, lens, npw);
    return true;
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_quantize_v(const LayerView& L, const __half* src, int64_t ld, int64_t T,
                             Lens lens, hipStream_t s) {
  const TokenSplit ts = split_tokens(L, T);
  const int pairs = L.B * L.H;
  hipLaunchKernelGGL(reset_scale_max_kernel, dim3((pairs + 255) / 256), dim3(256), 0, s,
                     L.scale_max, 1, pairs);
  const int64_t items = (ts.Tqv + kVRun - 1) / kVRun + 1;
  const int npw = items_per_wave(items, pairs);
  const dim3 grid((unsigned)((items + QW * npw - 1) / (QW * npw)), (unsigned)pairs);
  bool ok = dispatch_gv(L.Gv, [&](auto gv) {
    constexpr int GV = decltype(gv)::value;
    const bool paged = L.table != nullptr;
    if (L.bits == 2 && !paged)
      hipLaunchKernelGGL((prefill_v_kernel<2, GV, false>), grid, dim3(64 * QW), 0, s, L, src, ld,
                         T, lens, npw);
    else if (L.bits == 2)
      hipLaunchKernelGGL((prefill_v_kernel<2, GV, true>), grid, dim3(64 * QW), 0, s, L, src, ld,
                         T, lens, npw);
    else if (!paged)
      hipLaunchKernelGGL((prefill_v_kernel<4, GV, false>), grid, dim3(64 * QW), 0, s, L, src, ld,
                         T, lens, npw);
    else
      hipLaunchKernelGGL((prefill_v_kernel<4, GV, true>), grid, dim3(64 * QW), 0, s, L, src, ld,
                         T, lens, npw);
    return true;
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_append_flush(const LayerView& L, int64_t T_before, const __half* k_new,
                               const __half* v_new, Lens lens, bool flush_only,
                               hipStream_t s) {
  const AppendPlan ap = plan_append(L, T_before);
  int n = ap.flush ? ap.n : 0;
  const int slot = ap.slot;
  const int64_t t0 = ap.t0;
  if (lens.p) n = L.aging ? L.G : L.R;           // room for any sequence's flush
  const unsigned blocks = L.vwin ? (unsigned)(n / L.G + 1)
                                 : n ? (unsigned)(n / L.G + n / kVRun) : 1u;
  const dim3 grid(blocks, (unsigned)(L.B * L.H));
  bool ok = dispatch_bits_g(L.bits, L.G, [&](auto b, auto g) {
    return dispatch_gv(L.Gv, [&](auto gv) {
      hipLaunchKernelGGL(
          (append_kernel<decltype(b)::value, decltype(g)::value, decltype(gv)::value>), grid,
          dim3(64), 0, s, L, t0, slot, n, k_new, v_new, lens, flush_only ? 1 : 0, ap.vtok,
          ap.vt);
      return true;
    });
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kivi
