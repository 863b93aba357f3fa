// Decode attention over the packed cache, dequantizing inside the kernel.
//
// "09 — KV Cache Quantization", "Per-channel vs per-token in the actual attention
// kernel": the Key tile is read together with its per-channel scales and the Value
// tile with its per-row scales, and dequantization happens inside the attention tile
// loop — never into a full fp16 buffer.  The logits are the scaled dot products of
// "4.4 KV Cache quantization" §2 and "KV Cache Quantization (KIVI & FP4)" §2.
//
// Split-K: every (sequence, KV head) pair's tokens are cut into n_split ranges of
// whole Key groups; each workgroup keeps an online softmax (running max m, sum l,
// accumulator acc) for the g = H_q/H_kv query heads of its KV head and writes one
// partial.  The merge kernel combines the partials of a pair in split order:
//   m* = max_s m_s,  l* = sum_s l_s 2^(m_s - m*),  o = sum_s acc_s 2^(m_s - m*) / l*.
//
// The per-channel Key scale s_c and zero z_c of a group are folded into the query:
//   q . k_hat_t = sum_c (q_c s_c) code_tc + sum_c q_c z_c,
// and the per-token Value scale and zero into the probabilities:
//   sum_t p_t v_hat_tc = sum_t (p_t s_t) code_tc + sum_t p_t z_t.
// Logits are kept in base 2 (the query is pre-multiplied by sm_scale*log2(e)).
#include <type_traits>

#include "kivi_internal.h"

namespace kivi {
namespace {

constexpr int D = kHeadDim;
constexpr int TB = 32;            // tokens per block step
constexpr int NT = 256;           // threads per workgroup

// Partial layout per (pair, split, head): acc[D], m, l.
constexpr int PSTRIDE = D + 2;

template <int BITS, int GQA>
__global__ __launch_bounds__(NT) void decode_split_kernel(LayerView L, const __half* __restrict__ q,
                                                          float* __restrict__ part,
                                                          int64_t n_groups, int r, int n_split,
                                                          float qscale) {
  constexpr int KB = D * BITS / 8;                 // Key code bytes per token
  constexpr int RB = kVRun * BITS / 8;             // Value code bytes per (run, channel)
  constexpr int NACC = (GQA + 1) / 2;              // heads per PV thread
  __shared__ float qf[GQA][D];                     // q * sm_scale * log2(e)
  __shared__ float qs[GQA][D];                     // folded with the group's Key scale
  __shared__ float pt[GQA][TB];                    // p_t * s_t of the current block
  __shared__ float qz_part[GQA][2];
  __shared__ float alpha_s[GQA];
  __shared__ float pz_s[GQA];

  const int split = blockIdx.x;
  const int64_t pair = blockIdx.y;
  const int64_t b = pair / L.H, h = pair % L.H;
  const int tid = threadIdx.x;
  const int Hq = L.H * GQA;

  const __half* qp = q + (b * Hq + h * GQA) * D;
  for (int i = tid; i < GQA * D; i += NT) qf[i / D][i % D] = __half2float(qp[i]) * qscale;

  const int G = L.G;
  const int64_t g0 = n_groups * split / n_split;
  const int64_t g1 = n_groups * (split + 1) / n_split;
  const bool has_resid = (split == n_split - 1) && r > 0;

  const uint8_t* kc = L.k_codes + pair * L.kc_pair();
  const __half* ksc = L.k_scale + pair * L.ks_pair();
  const __half* kze = L.k_zero + pair * L.ks_pair();
  const uint8_t* vc = L.v_codes + pair * L.vc_pair();
  const __half* vsc = L.v_scale + pair * L.vs_pair();
  const __half* vze = L.v_zero + pair * L.vs_pair();
  const __half* kr = L.k_resid + pair * L.rs_pair();
  const __half* vr = L.v_resid + pair * L.rs_pair();

  // Logit role: token t of the block for head hh.
  const int lt = tid & (TB - 1);
  const int lh = tid / TB;
  float m_run = -INFINITY, l_run = 0.f, pz_run = 0.f;
  // PV role: channel c for heads ph, ph + 2, ...
  const int pc = tid & (D - 1);
  const int ph = tid / D;
  float acc[NACC];
#pragma unroll
  for (int k = 0; k < NACC; ++k) acc[k] = 0.f;

  const int64_t tq0 = g0 * G, tq1 = g1 * G;        // quantized token range
  const int64_t n_blocks_q = (tq1 - tq0) / TB;
  const int n_blocks_r = has_resid ? (r + TB - 1) / TB : 0;
  int64_t cur_group = -1;
  __syncthreads();

  for (int64_t blk = 0; blk < n_blocks_q + n_blocks_r; ++blk) {
    const bool resid = blk >= n_blocks_q;
    const int64_t t_base = resid ? (blk - n_blocks_q) * TB : tq0 + blk * TB;
    const int n_valid = resid ? (int)((r - t_base) < TB ? (r - t_base) : TB) : TB;

    // (1) fold the Key group's scale/zero into the query.
    if (!resid) {
      const int64_t grp = t_base / G;
      if (grp != cur_group) {
        cur_group = grp;
        const float sk = __half2float(ksc[grp * D + pc]);
        const float zk = __half2float(kze[grp * D + pc]);
        for (int hh = ph; hh < GQA; hh += 2) {
          qs[hh][pc] = qf[hh][pc] * sk;
          float z = qf[hh][pc] * zk;
#pragma unroll
          for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off, 64);
          if ((tid & 63) == 0) qz_part[hh][(tid >> 6) & 1] = z;
        }
        __syncthreads();
      }
    }

    // (2) logits and online softmax for (token lt, head lh).
    if (lh < GQA) {
      float z = -INFINITY;
      if (lt < n_valid) {
        float dot = 0.f;
        if (!resid) {
          const uint4* row = reinterpret_cast<const uint4*>(kc + (t_base + lt) * KB);
#pragma unroll
          for (int i = 0; i < KB / 16; ++i) {
            const uint4 u = row[i];
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              constexpr int CPW = 32 / BITS;
              const int c0 = (4 * i + k) * CPW;
#pragma unroll
              for (int j = 0; j < CPW; ++j) {
                const float code = (float)((w[k] >> (BITS * j)) & ((1u << BITS) - 1));
                dot += qs[lh][c0 + j] * code;
              }
            }
          }
          dot += qz_part[lh][0] + qz_part[lh][1];
        } else {
          const __half2* row = reinterpret_cast<const __half2*>(kr + (t_base + lt) * D);
#pragma unroll 8
          for (int c2 = 0; c2 < D / 2; ++c2) {
            const __half2 v = row[c2];
            dot += qf[lh][2 * c2] * __low2float(v);
            dot += qf[lh][2 * c2 + 1] * __high2float(v);
          }
        }
        z = dot;
      }
      float bm = z;
#pragma unroll
      for (int off = TB / 2; off >= 1; off >>= 1) bm = fmaxf(bm, __shfl_xor(bm, off, TB));
      const float m_new = fmaxf(m_run, bm);
      const float alpha = exp2f(m_run - m_new);
      const float p = (lt < n_valid) ? exp2f(z - m_new) : 0.f;
      float ps = p, pzv = 0.f;
      if (!resid && lt < n_valid) {
        ps = p * __half2float(vsc[t_base + lt]);
        pzv = p * __half2float(vze[t_base + lt]);
      }
      float sp = p;
#pragma unroll
      for (int off = TB / 2; off >= 1; off >>= 1) {
        sp += __shfl_xor(sp, off, TB);
        pzv += __shfl_xor(pzv, off, TB);
      }
      l_run = l_run * alpha + sp;
      pz_run = pz_run * alpha + pzv;
      m_run = m_new;
      pt[lh][lt] = ps;
      if (lt == 0) alpha_s[lh] = alpha;
    }
    __syncthreads();

    // (3) acc = acc * alpha + sum_t pt_t * v_t for channel pc.
    if (!resid) {
      uint32_t wv[2][RB / 4];
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const uint8_t* src = vc + ((t_base / kVRun) + rr) * (D * RB) + pc * RB;
        if constexpr (BITS == 2) {
          wv[rr][0] = *reinterpret_cast<const uint32_t*>(src);
        } else {
          const uint2 u = *reinterpret_cast<const uint2*>(src);
          wv[rr][0] = u.x;
          wv[rr][1] = u.y;
        }
      }
#pragma unroll
      for (int k = 0; k < NACC; ++k) {
        const int hh = ph + 2 * k;
        if (hh < GQA) {
          float a = acc[k] * alpha_s[hh];
#pragma unroll
          for (int t = 0; t < TB; ++t) {
            const int rr = t / kVRun, tau = t % kVRun;
            const uint32_t word = wv[rr][(tau * BITS) / 32];
            const float code = (float)((word >> ((tau * BITS) % 32)) & ((1u << BITS) - 1));
            a += pt[hh][t] * code;
          }
          acc[k] = a;
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < NACC; ++k) {
        const int hh = ph + 2 * k;
        if (hh < GQA) {
          float a = acc[k] * alpha_s[hh];
          for (int t = 0; t < n_valid; ++t)
            a += pt[hh][t] * __half2float(vr[(t_base + t) * D + pc]);
          acc[k] = a;
        }
      }
    }
    __syncthreads();
  }

  // (4) write the partial: acc + pz (the Value zero term is shared by all channels).
  if (lh < GQA && lt == 0) pz_s[lh] = pz_run;
  float* out = part + ((pair * n_split + split) * GQA) * PSTRIDE;
  if (lh < GQA && lt == 0) {
    out[lh * PSTRIDE + D] = m_run;
    out[lh * PSTRIDE + D + 1] = l_run;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NACC; ++k) {
    const int hh = ph + 2 * k;
    if (hh < GQA) out[hh * PSTRIDE + pc] = acc[k] + pz_s[hh];
  }
}

// One workgroup of D threads per (sequence, query head): fixed-order merge.
__global__ __launch_bounds__(D) void merge_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                  int H, int gqa, int n_split) {
  const int64_t bq = blockIdx.x;                 // b * Hq + hq
  const int Hq = H * gqa;
  const int64_t b = bq / Hq;
  const int hq = (int)(bq % Hq);
  const int64_t pair = b * H + hq / gqa;
  const int hl = hq % gqa;
  const int c = threadIdx.x;
  const float* p0 = part + (pair * n_split * gqa + hl) * PSTRIDE;
  const int64_t sstride = (int64_t)gqa * PSTRIDE;
  float mstar = -INFINITY;
  for (int s = 0; s < n_split; ++s) mstar = fmaxf(mstar, p0[s * sstride + D]);
  float l = 0.f, o = 0.f;
  for (int s = 0; s < n_split; ++s) {
    const float* ps = p0 + s * sstride;
    const float ls = ps[D + 1];
    if (ls > 0.f) {
      const float w = exp2f(ps[D] - mstar);
      l += ls * w;
      o += ps[c] * w;
    }
  }
  out[bq * D + c] = o / l;
}

template <typename F>
bool dispatch_decode(int bits, int gqa, F&& f) {
#define KIVI_CASE(B, Q) \
  if (bits == B && gqa == Q) return f(std::integral_constant<int, B>{}, std::integral_constant<int, Q>{});
  KIVI_CASE(2, 1) KIVI_CASE(2, 2) KIVI_CASE(2, 4) KIVI_CASE(2, 8)
  KIVI_CASE(4, 1) KIVI_CASE(4, 2) KIVI_CASE(4, 4) KIVI_CASE(4, 8)
#undef KIVI_CASE
  return false;
}

}  // namespace

DecodePlan plan_decode(const LayerView& L, int q_heads, int64_t T, int n_split_req) {
  DecodePlan p{};
  const int gqa = q_heads / L.H;
  const int64_t Tq = quantized_len(T, L.R);
  p.r = (int)(T - Tq);
  p.n_groups = Tq / L.G;
  const int64_t pairs = (int64_t)L.B * L.H;
  int64_t ns = n_split_req;
  if (ns <= 0) {
    const int64_t target = 1024;                 // workgroups to spread over 256 CUs
    ns = (target + pairs - 1) / pairs;
  }
  if (ns > p.n_groups) ns = p.n_groups;
  if (ns < 1) ns = 1;
  p.n_split = (int)ns;
  p.ws_partials = (size_t)pairs * ns * gqa * PSTRIDE * sizeof(float);
  p.ws_partials = (p.ws_partials + 255) / 256 * 256;
  p.ws_counters = ((size_t)pairs * sizeof(uint32_t) + 255) / 256 * 256;
  p.ws_total = p.ws_partials + p.ws_counters;
  return p;
}

hipError_t launch_decode(const LayerView& L, int q_heads, int64_t T, const __half* q,
                         float sm_scale, float* out, void* ws, const DecodePlan& plan,
                         hipStream_t s) {
  const int gqa = q_heads / L.H;
  float* part = reinterpret_cast<float*>(ws);
  const float qscale = sm_scale * 1.4426950408889634f;
  const dim3 grid((unsigned)plan.n_split, (unsigned)(L.B * L.H));
  bool ok = dispatch_decode(L.bits, gqa, [&](auto b, auto g) {
    hipLaunchKernelGGL((decode_split_kernel<decltype(b)::value, decltype(g)::value>), grid,
                       dim3(NT), 0, s, L, q, part, plan.n_groups, plan.r, plan.n_split, qscale);
    return true;
  });
  if (!ok) return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)(L.B * q_heads)), dim3(D), 0, s, part, out,
                     L.H, gqa, plan.n_split);
  return hipGetLastError();
}

}  // namespace kivi
