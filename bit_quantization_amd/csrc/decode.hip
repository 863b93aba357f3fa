// Decode attention over the packed cache, dequantizing inside the kernel.
//
// "09 — KV Cache Quantization", "Per-channel vs per-token in the actual attention
// kernel": the Key tile is read with its per-channel scales and the Value tile with
// its per-row scales, and dequantization happens inside the attention tile loop —
// never into a full fp16 buffer.  The logits are the scaled dot products of "4.4 KV
// Cache quantization" §2 and "KV Cache Quantization (KIVI & FP4)" §2; "KV Cache
// Quantization (KIVI & FP4)" §4 and "KV Cache INT4 Quantization for 1M+ Token Context
// Windows" §2 motivate reading the packed codes directly.
//
// Algebra.  The per-channel Key scale s_c and zero z_c of a group fold into the
// query, the per-token Value scale and zero into the probabilities:
//   q . k_hat_t      = sum_c (q_c s_c) code_tc + sum_c q_c z_c
//   sum_t p_t v_hat_t = sum_t (p_t s_t) code_tc + sum_t p_t z_t
// Both remaining products are integer-code matrices times real vectors.  They run on
// the int8 matrix cores (v_mfma_i32_16x16x64_i8): the codes are already small
// integers (one shift and mask per four codes), and the real side is written in
// 32-bit fixed point as four balanced int8 limbs, one MFMA row per limb:
//   x = round_toward_zero(v * 2^E),  x = l0 + 2^8 l1 + 2^16 l2 + 2^24 l3,  l_i in [-128, 127]
// E is chosen per wave from the largest |q| s (resp. s_t) of the wave's token range
// so that |x| <= 2^30.  Integer products are exact; the limb sums are recombined in
// float32.
//
// Work split.  Each (sequence, KV head) pair's quantized tokens are cut into 64-token
// blocks; the 4 waves of each of n_split workgroups take contiguous runs of blocks,
// each wave with its own online softmax (running max m, sum l).
// One extra workgroup per pair attends over the float16 residual rows.  The 4 waves
// of a workgroup combine in LDS; the workgroups of a pair write partials, and the
// last one to arrive (an integer arrival counter, reset by that workgroup) merges
// them in split order:  m* = max m_s,  l* = sum l_s 2^(m_s - m*),  o = sum acc_s
// 2^(m_s - m*) / l*.  No floating-point atomics; the result is deterministic.
//
// Logits are kept in base 2 (the query is pre-multiplied by sm_scale * log2(e)).
#include <type_traits>

#include "kivi_internal.h"

namespace kivi {
namespace {

constexpr int D = kHeadDim;
constexpr int WAVES = 4;
constexpr int NT = 64 * WAVES;
constexpr int BLK = 64;              // tokens per block step of a wave
constexpr int PSTRIDE = D + 2;       // partial per head: acc[D], m, l

typedef int i32x4 __attribute__((ext_vector_type(4)));

struct DecodeArgs {
  LayerView L;
  const __half* q;
  float* out;
  float* part;          // [P][n_parts][GQA][PSTRIDE]
  unsigned* counters;   // [P], zero between calls
  int64_t Tq;           // quantized tokens
  int64_t nblk;         // 64-token blocks per pair (the last may hold 32 tokens)
  int r;                // residual tokens
  int n_split;          // quantized workgroups per pair
  float qscale;         // sm_scale * log2(e)
};

// ---- small device helpers ---------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
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
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}
__device__ __forceinline__ float h2f(unsigned short h) {
  return __half2float(__ushort_as_half(h));
}
// 32-bit fixed point -> four balanced int8 limbs packed in one word (byte i = limb i).
__device__ __forceinline__ uint32_t to_limbs(float v) {
  const int x = (int)v;                          // round toward zero, |x| <= 2^30
  return ((uint32_t)x + 0x00808080u) ^ 0x00808080u;
}
// exponent E with |v| * 2^E < 2^30 for every |v| <= vmax (0 if vmax == 0)
__device__ __forceinline__ int fixed_exponent(float vmax) {
  if (!(vmax > 0.f)) return 0;
  const int e = __builtin_amdgcn_frexp_expf(vmax);   // vmax < 2^e
  const int E = 30 - e;
  return E > 60 ? 60 : E;
}
__device__ __forceinline__ i32x4 mfma_i8(i32x4 a, i32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Code operand layouts (byte position p of a lane's 16-byte operand <-> element).
// Keys, one token, K-step ks, lane group j: the 16 channels 32j + 16ks + [0, 16).
//   2-bit: p = 4s + b  <-> channel 32j + 16ks + 4b + s
//   4-bit: p = 4(2dd + s) + b <-> channel 32j + 16ks + 8dd + 2b + s
// Values, one channel, one 16-token run: same formulas with "token of the run".
template <int BITS>
__device__ __forceinline__ void channel_to_pos(int c, int& ks, int& j, int& p) {
  j = c >> 5;
  ks = (c >> 4) & 1;
  if constexpr (BITS == 2) {
    const int b = (c & 15) >> 2, s = c & 3;
    p = 4 * s + b;
  } else {
    const int dd = (c >> 3) & 1, b = (c & 7) >> 1, s = c & 1;
    p = 4 * (2 * dd + s) + b;
  }
}
template <int BITS>
__device__ __forceinline__ int run_token_to_pos(int u) {
  if constexpr (BITS == 2) return 4 * (u & 3) + (u >> 2);
  else return 8 * (u >> 3) + 4 * (u & 1) + ((u & 7) >> 1);
}
// Unpack 16 codes of one K-step (2-bit: one word; 4-bit: two words) into int8 bytes.
template <int BITS>
__device__ __forceinline__ i32x4 unpack16(uint32_t w0, uint32_t w1) {
  i32x4 u;
  if constexpr (BITS == 2) {
    u[0] = (int)(w0 & 0x03030303u);
    u[1] = (int)((w0 >> 2) & 0x03030303u);
    u[2] = (int)((w0 >> 4) & 0x03030303u);
    u[3] = (int)((w0 >> 6) & 0x03030303u);
  } else {
    u[0] = (int)(w0 & 0x0F0F0F0Fu);
    u[1] = (int)((w0 >> 4) & 0x0F0F0F0Fu);
    u[2] = (int)(w1 & 0x0F0F0F0Fu);
    u[3] = (int)((w1 >> 4) & 0x0F0F0F0Fu);
  }
  return u;
}

// Per-wave LDS of the quantized path.
template <int NMT>
struct WaveLds {
  uint8_t qa[2][NMT][2][16][4][16];   // [group in block][M-tile][K-step][row][lane grp][pos]
  uint8_t pa[NMT][16][4][16];         // [M-tile][row][run][pos]
};

// ---- the quantized token range of one wave ----------------------------------------
// Writes comb[GQA][PSTRIDE] (acc with the Value-zero term folded in, m, l).
template <int BITS, int GQA>
__device__ void quantized_wave(const DecodeArgs& a, int64_t pair, int64_t blk0, int64_t blk1,
                               WaveLds<(GQA + 3) / 4>& lds, float* comb) {
  constexpr int NMT = (GQA + 3) / 4;              // M-tiles of 4 heads x 4 limbs
  constexpr int KB = D * BITS / 8;                // Key code bytes per token
  constexpr int RB = kVRun * BITS / 8;            // Value code bytes per (run, channel)
  const LayerView& L = a.L;
  const int G = L.G;
  const int lane = threadIdx.x & 63;
  const int lo = lane & 15, j = lane >> 4;
  const int64_t b = pair / L.H, h = pair % L.H;

  const uint8_t* kc = L.k_codes + pair * L.kc_pair();
  const __half* ksc = L.k_scale + pair * L.ks_pair();
  const __half* kze = L.k_zero + pair * L.ks_pair();
  const uint8_t* vc = L.v_codes + pair * L.vc_pair();
  const unsigned short* vsc = reinterpret_cast<const unsigned short*>(L.v_scale + pair * L.vs_pair());
  const unsigned short* vze = reinterpret_cast<const unsigned short*>(L.v_zero + pair * L.vs_pair());
  const int Hq = L.H * GQA;
  const __half* qp = a.q + (b * Hq + h * GQA) * D;

  const int64_t t_lo = blk0 * BLK;
  const int64_t t_hi = blk1 * BLK < a.Tq ? blk1 * BLK : a.Tq;

  // -- pre-pass: largest |q| (scaled), largest Key scale and Value scale in range --
  float qmax = 0.f;
  for (int i = lane; i < GQA * D; i += 64) qmax = fmaxf(qmax, fabsf(__half2float(qp[i])));
  qmax = wave_max(qmax) * fabsf(a.qscale);
  float skmax = 0.f, svmax = 0.f;
  if (t_hi > t_lo) {
    const int64_t g_lo = t_lo / G, g_hi = (t_hi + G - 1) / G;
    const uint4* ks4 = reinterpret_cast<const uint4*>(ksc + g_lo * D);
    const int64_t n4 = (g_hi - g_lo) * D / 8;
    uint32_t mk = 0;
    for (int64_t i = lane; i < n4; i += 64) {
      const uint4 u = ks4[i];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) mk = max(mk, max(w[k] & 0xFFFFu, w[k] >> 16));
    }
    uint32_t mv = 0;
    for (int64_t t = t_lo + lane; t < t_hi; t += 64) mv = max(mv, (uint32_t)vsc[t]);
    // non-negative float16 values order like their bit patterns
    skmax = wave_max(h2f((unsigned short)mk));
    svmax = wave_max(h2f((unsigned short)mv));
  }
  const int Ek = fixed_exponent(qmax * skmax);
  const int Ev = fixed_exponent(svmax);
  const float k_unscale = __builtin_amdgcn_ldexpf(1.f, -Ek);
  const float v_unscale = __builtin_amdgcn_ldexpf(1.f, -Ev);

  // Query values of this lane for the group preparation: heads 4mt + j, channels
  // 8lo .. 8lo+7, scaled by sm_scale*log2(e)*2^Ek.
  float qv[NMT][8];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int hd = 4 * mt + j;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      qv[mt][i] = hd < GQA ? __builtin_amdgcn_ldexpf(__half2float(qp[hd * D + 8 * lo + i]) * a.qscale, Ek)
                           : 0.f;
  }

  // Online-softmax state per M-tile: head 4mt + j for this lane's row.
  float m_run[NMT], l_run[NMT], pz_run[NMT];
  float acc_f[NMT][8];            // channels 8lo + n, in units of 2^Ev
  i32x4 acc_i[NMT][8];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    m_run[mt] = -INFINITY;
    l_run[mt] = 0.f;
    pz_run[mt] = 0.f;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      acc_f[mt][n] = 0.f;
      acc_i[mt][n] = i32x4{0, 0, 0, 0};
    }
  }

  for (int64_t blk = blk0; blk < blk1; ++blk) {
    const int64_t tb = blk * BLK;
    const int n_valid = (int)((a.Tq - tb) < BLK ? (a.Tq - tb) : BLK);    // 64 or 32
    const int n_groups_blk = (n_valid + G - 1) / G;                      // groups touched
    const int n_tiles = n_valid / 16;

    // (1) group preparation: query limbs into LDS, and sum_c q_c z_c per head.
    float qz[2][NMT];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) qz[gi][mt] = 0.f;
      if (gi < n_groups_blk) {
        const int64_t grp = tb / G + gi;
        const uint4 su = *reinterpret_cast<const uint4*>(ksc + grp * D + 8 * lo);
        const uint4 zu = *reinterpret_cast<const uint4*>(kze + grp * D + 8 * lo);
        const uint32_t sw[4] = {su.x, su.y, su.z, su.w};
        const uint32_t zw[4] = {zu.x, zu.y, zu.z, zu.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float s = h2f((unsigned short)(sw[i >> 1] >> (16 * (i & 1))));
          const float z = h2f((unsigned short)(zw[i >> 1] >> (16 * (i & 1))));
          const int c = 8 * lo + i;
          int ks, jg, p;
          channel_to_pos<BITS>(c, ks, jg, p);
#pragma unroll
          for (int mt = 0; mt < NMT; ++mt) {
            const uint32_t lw = to_limbs(qv[mt][i] * s);
            uint8_t* dst = &lds.qa[gi][mt][ks][4 * j][jg][p];
            dst[0] = (uint8_t)lw;
            dst[64] = (uint8_t)(lw >> 8);
            dst[128] = (uint8_t)(lw >> 16);
            dst[192] = (uint8_t)(lw >> 24);
            qz[gi][mt] += qv[mt][i] * z;
          }
        }
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) qz[gi][mt] = row_sum16(qz[gi][mt]) * k_unscale;
      }
      if (G == 64) break;     // one group spans the whole block
    }
    wave_lds_sync();

    // (2) Q.K^T on the matrix cores: C[mt][nt] rows (head, limb), columns tokens.
    i32x4 cqk[NMT][4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) cqk[mt][nt] = i32x4{0, 0, 0, 0};
      if (nt < n_tiles) {
        const int gi = (G == 64) ? 0 : (nt >> 1);
        const uint8_t* row = kc + (tb + 16 * nt + lo) * KB;
        uint32_t w[4];
        if constexpr (BITS == 2) {
          const uint2 u = *reinterpret_cast<const uint2*>(row + 8 * j);
          w[0] = u.x; w[1] = 0; w[2] = u.y; w[3] = 0;
        } else {
          const uint4 u = *reinterpret_cast<const uint4*>(row + 16 * j);
          w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const i32x4 bop = unpack16<BITS>(w[2 * ks], w[2 * ks + 1]);
#pragma unroll
          for (int mt = 0; mt < NMT; ++mt) {
            const i32x4 aop = *reinterpret_cast<const i32x4*>(&lds.qa[gi][mt][ks][lo][j][0]);
            cqk[mt][nt] = mfma_i8(aop, bop, cqk[mt][nt]);
          }
        }
      }
    }

    // (3) logits, online softmax, probability limbs into LDS.
    float sv[4], zv[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t t = tb + 16 * nt + lo;
      sv[nt] = nt < n_tiles ? h2f(vsc[t]) : 0.f;
      zv[nt] = nt < n_tiles ? h2f(vze[t]) : 0.f;
    }
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      float z[4];
      float bm = -INFINITY;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int gi = (G == 64) ? 0 : (nt >> 1);
        const i32x4 c = cqk[mt][nt];
        const float lo16 = (float)(c[0] + c[1] * 256);      // |c_i| < 2^18: exact int
        const float hi16 = (float)(c[2] + c[3] * 256);
        z[nt] = nt < n_tiles ? fmaf(hi16, 65536.f * k_unscale, fmaf(lo16, k_unscale, qz[gi][mt]))
                             : -INFINITY;
        bm = fmaxf(bm, z[nt]);
      }
      bm = row_max16(bm);
      const float m_new = fmaxf(m_run[mt], bm);
      if (m_new > m_run[mt]) {               // the running max rose: rescale what we have
        const float alpha = __builtin_amdgcn_exp2f(m_run[mt] - m_new);
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const i32x4 ci = acc_i[mt][n];
          float v = acc_f[mt][n] + (float)ci[0] + 256.f * (float)ci[1] + 65536.f * (float)ci[2] +
                    16777216.f * (float)ci[3];
          acc_f[mt][n] = v * alpha;
          acc_i[mt][n] = i32x4{0, 0, 0, 0};
        }
        l_run[mt] *= alpha;
        pz_run[mt] *= alpha;
        m_run[mt] = m_new;
      }
      const float m_shift = m_run[mt] - (float)Ev;     // p' = p * 2^Ev
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float p = nt < n_tiles ? __builtin_amdgcn_exp2f(z[nt] - m_shift) : 0.f;
        l_run[mt] += p;
        pz_run[mt] = fmaf(p, zv[nt], pz_run[mt]);
        const uint32_t lw = nt < n_tiles ? to_limbs(p * sv[nt]) : 0u;
        uint8_t* dst = &lds.pa[mt][4 * j][nt][run_token_to_pos<BITS>(lo)];
        dst[0] = (uint8_t)lw;
        dst[64] = (uint8_t)(lw >> 8);
        dst[128] = (uint8_t)(lw >> 16);
        dst[192] = (uint8_t)(lw >> 24);
      }
    }
    wave_lds_sync();

    // (4) P.V on the matrix cores: rows (head, limb), K = 64 tokens, columns channels
    // 8lo + n (n = 0..7) of the lane's Value run j.
    {
      const uint8_t* vrow = vc + (tb / kVRun + j) * (int64_t)(D * RB) + (8 * lo) * RB;
      uint32_t vw[8][2];
      const bool run_ok = j < n_tiles;
      if constexpr (BITS == 2) {
        const uint4 u0 = run_ok ? *reinterpret_cast<const uint4*>(vrow) : make_uint4(0, 0, 0, 0);
        const uint4 u1 = run_ok ? *reinterpret_cast<const uint4*>(vrow + 16) : make_uint4(0, 0, 0, 0);
        const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int n = 0; n < 8; ++n) { vw[n][0] = w[n]; vw[n][1] = 0; }
      } else {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const uint4 u = run_ok ? *reinterpret_cast<const uint4*>(vrow + 16 * q4) : make_uint4(0, 0, 0, 0);
          vw[2 * q4][0] = u.x; vw[2 * q4][1] = u.y;
          vw[2 * q4 + 1][0] = u.z; vw[2 * q4 + 1][1] = u.w;
        }
      }
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const i32x4 aop = *reinterpret_cast<const i32x4*>(&lds.pa[mt][lo][j][0]);
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const i32x4 bop = unpack16<BITS>(vw[n][0], vw[n][1]);
          acc_i[mt][n] = mfma_i8(aop, bop, acc_i[mt][n]);
        }
      }
    }
  }

  // Finish: fold the integer accumulators and the Value-zero term, undo 2^Ev.
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int hd = 4 * mt + j;
    const float lsum = row_sum16(l_run[mt]);
    const float pz = row_sum16(pz_run[mt]);
    if (hd < GQA) {
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const i32x4 ci = acc_i[mt][n];
        const float v = acc_f[mt][n] + (float)ci[0] + 256.f * (float)ci[1] + 65536.f * (float)ci[2] +
                        16777216.f * (float)ci[3];
        comb[hd * PSTRIDE + 8 * lo + n] = (v + pz) * v_unscale;
      }
      if (lo == 0) {
        comb[hd * PSTRIDE + D] = m_run[mt];
        comb[hd * PSTRIDE + D + 1] = lsum * v_unscale;
      }
    }
  }
}

// ---- float16 residual rows [t0, t1) of one wave (VALU) ------------------------------
template <int GQA>
__device__ void residual_wave(const DecodeArgs& a, int64_t pair, int t0, int t1, const float* qf,
                              float* pw, float* comb) {
  const LayerView& L = a.L;
  const int lane = threadIdx.x & 63;
  const int t_l = lane & 31, half = lane >> 5;
  const __half* kr = L.k_resid + pair * L.rs_pair();
  const __half* vr = L.v_resid + pair * L.rs_pair();
  constexpr int NH = (GQA + 1) / 2;              // heads per lane in the logit phase
  float m_run[GQA], l_run[GQA];
  float acc[GQA][2];                             // channels 2*lane, 2*lane+1
#pragma unroll
  for (int hd = 0; hd < GQA; ++hd) {
    m_run[hd] = -INFINITY;
    l_run[hd] = 0.f;
    acc[hd][0] = acc[hd][1] = 0.f;
  }
  float* palpha = pw + GQA * 32;
  for (int c0 = t0; c0 < t1; c0 += 32) {
    const int n_valid = (t1 - c0) < 32 ? (t1 - c0) : 32;
    const bool valid = t_l < n_valid;
    float z[NH];
#pragma unroll
    for (int k = 0; k < NH; ++k) z[k] = 0.f;
    if (valid) {
      const uint4* row = reinterpret_cast<const uint4*>(kr + (int64_t)(c0 + t_l) * D);
#pragma unroll 4
      for (int i = 0; i < D / 8; ++i) {
        const uint4 u = row[i];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = h2f((unsigned short)w[e]), x1 = h2f((unsigned short)(w[e] >> 16));
#pragma unroll
          for (int k = 0; k < NH; ++k) {
            const int hd = half + 2 * k;
            if (hd < GQA) z[k] += qf[hd * D + 8 * i + 2 * e] * x0 + qf[hd * D + 8 * i + 2 * e + 1] * x1;
          }
        }
      }
    }
#pragma unroll
    for (int k = 0; k < NH; ++k) {
      const int hd = half + 2 * k;
      if (hd >= GQA) continue;
      const float zz = valid ? z[k] : -INFINITY;
      float bm = zz;
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) bm = fmaxf(bm, __shfl_xor(bm, off, 32));
      const float m_new = fmaxf(m_run[hd], bm);
      const float alpha = __builtin_amdgcn_exp2f(m_run[hd] - m_new);
      const float p = valid ? __builtin_amdgcn_exp2f(zz - m_new) : 0.f;
      l_run[hd] = l_run[hd] * alpha + p;
      m_run[hd] = m_new;
      pw[hd * 32 + t_l] = p;
      if (t_l == 0) palpha[hd] = alpha;
    }
    wave_lds_sync();
    // every lane needs every head's running max for the final write
#pragma unroll
    for (int hd = 0; hd < GQA; ++hd) {
      const float al = palpha[hd];
      float s0 = acc[hd][0] * al, s1 = acc[hd][1] * al;
      for (int t = 0; t < n_valid; ++t) {
        const __half2 v = *reinterpret_cast<const __half2*>(vr + (int64_t)(c0 + t) * D + 2 * lane);
        const float p = pw[hd * 32 + t];
        s0 = fmaf(p, __low2float(v), s0);
        s1 = fmaf(p, __high2float(v), s1);
      }
      acc[hd][0] = s0;
      acc[hd][1] = s1;
    }
    wave_lds_sync();
  }
#pragma unroll
  for (int hd = 0; hd < GQA; ++hd) {
    comb[hd * PSTRIDE + 2 * lane] = acc[hd][0];
    comb[hd * PSTRIDE + 2 * lane + 1] = acc[hd][1];
    // m_run is uniform over the lanes of the half that owns the head
    float lsum = l_run[hd];
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off, 32);
    if (lane == (hd & 1) * 32) {
      comb[hd * PSTRIDE + D] = m_run[hd];
      comb[hd * PSTRIDE + D + 1] = lsum;
    }
  }
}

// Combine the 4 per-wave results of a workgroup (or the n_parts partials of a pair)
// in a fixed order.  src(i) returns the i-th [GQA][PSTRIDE] record.
template <int GQA, typename Src>
__device__ __forceinline__ void combine(int n, Src src, float* dst, int64_t dst_hstride,
                                        bool with_ml) {
  for (int idx = threadIdx.x; idx < GQA * D; idx += NT) {
    const int hd = idx / D, c = idx % D;
    float mstar = -INFINITY;
    for (int i = 0; i < n; ++i) mstar = fmaxf(mstar, src(i)[hd * PSTRIDE + D]);
    float l = 0.f, o = 0.f;
    if (mstar > -INFINITY) {
      for (int i = 0; i < n; ++i) {
        const float* rec = src(i) + hd * PSTRIDE;
        const float li = rec[D + 1];
        if (li > 0.f) {
          const float wgt = __builtin_amdgcn_exp2f(rec[D] - mstar);
          l += li * wgt;
          o += rec[c] * wgt;
        }
      }
    }
    if (with_ml) {
      dst[hd * dst_hstride + c] = o;
      if (c == 0) {
        dst[hd * dst_hstride + D] = mstar;
        dst[hd * dst_hstride + D + 1] = l;
      }
    } else {
      dst[hd * dst_hstride + c] = o / l;
    }
  }
}

template <int BITS, int GQA>
__global__ __launch_bounds__(NT, 2) void decode_kernel(DecodeArgs a) {
  constexpr int NMT = (GQA + 3) / 4;
  struct ResidLds {
    float qf[GQA * D];
    float pw[WAVES][GQA * 32 + GQA];
  };
  union Lds {
    WaveLds<NMT> wave[WAVES];
    ResidLds res;
  };
  __shared__ Lds lds;
  __shared__ float comb[WAVES][GQA * PSTRIDE];
  __shared__ int last_flag;

  const int64_t P = (int64_t)a.L.B * a.L.H;
  const int64_t pair = blockIdx.x % P;
  const int s = (int)(blockIdx.x / P);            // 0: residual rows, s >= 1: split s - 1
  const int wave = threadIdx.x >> 6;
  const int n_parts = a.n_split + 1;

  if (s == 0) {
    const int64_t b = pair / a.L.H, h = pair % a.L.H;
    const __half* qp = a.q + (b * a.L.H * GQA + h * GQA) * D;
    for (int i = threadIdx.x; i < GQA * D; i += NT) lds.res.qf[i] = __half2float(qp[i]) * a.qscale;
    __syncthreads();
    // wave w takes 32-row chunks w, w + 4, ...
    float* cw = comb[wave];
    for (int i = threadIdx.x & 63; i < GQA * PSTRIDE; i += 64) cw[i] = 0.f;
    for (int hd = 0; hd < GQA; ++hd) cw[hd * PSTRIDE + D] = -INFINITY;
    wave_lds_sync();
    // contiguous share of rows per wave, in 32-row chunks
    const int chunks = (a.r + 31) / 32;
    const int c_lo = chunks * wave / WAVES, c_hi = chunks * (wave + 1) / WAVES;
    const int t0 = 32 * c_lo, t1 = (32 * c_hi < a.r) ? 32 * c_hi : a.r;
    if (t1 > t0) residual_wave<GQA>(a, pair, t0, t1, lds.res.qf, lds.res.pw[wave], cw);
  } else {
    const int split = s - 1;
    const int64_t wb = (int64_t)a.n_split * WAVES;    // waves per pair
    const int64_t wi = (int64_t)split * WAVES + wave;
    const int64_t blk0 = a.nblk * wi / wb, blk1 = a.nblk * (wi + 1) / wb;
    float* cw = comb[wave];
    for (int i = threadIdx.x & 63; i < GQA * PSTRIDE; i += 64) cw[i] = 0.f;
    for (int hd = 0; hd < GQA; ++hd) cw[hd * PSTRIDE + D] = -INFINITY;
    wave_lds_sync();
    if (blk1 > blk0) quantized_wave<BITS, GQA>(a, pair, blk0, blk1, lds.wave[wave], cw);
  }
  __syncthreads();

  // Workgroup partial -> workspace.
  float* mine = a.part + ((pair * n_parts + s) * GQA) * PSTRIDE;
  combine<GQA>(WAVES, [&](int i) { return (const float*)comb[i]; }, mine, PSTRIDE, true);

  // Last workgroup of the pair merges all partials and resets the counter.
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(&a.counters[pair], 1u);
    last_flag = (prev == (unsigned)(n_parts - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  const float* base = a.part + (pair * n_parts * GQA) * PSTRIDE;
  const int64_t b = pair / a.L.H, h = pair % a.L.H;
  float* o = a.out + (b * a.L.H * GQA + h * GQA) * D;
  combine<GQA>(n_parts, [&](int i) { return base + (int64_t)i * GQA * PSTRIDE; }, o, D, false);
  if (threadIdx.x == 0) a.counters[pair] = 0u;
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
  const int64_t nblk = (Tq + BLK - 1) / BLK;
  const int64_t pairs = (int64_t)L.B * L.H;
  int64_t ns = n_split_req;
  if (ns <= 0) {
    // about two 4-wave workgroups per CU on 256 CUs, at least 4 blocks per wave
    const int64_t target_wgs = 512;
    ns = (target_wgs + pairs - 1) / pairs;
    const int64_t cap = (nblk + 4 * WAVES - 1) / (4 * WAVES);
    if (ns > cap) ns = cap;
  }
  if (ns > nblk) ns = nblk;
  if (nblk == 0) ns = 0;
  if (ns < 1 && nblk > 0) ns = 1;
  p.n_split = (int)ns;
  const int64_t n_parts = ns + 1;
  p.ws_counters = ((size_t)pairs * sizeof(uint32_t) + 255) / 256 * 256;
  p.ws_partials = (size_t)pairs * n_parts * gqa * PSTRIDE * sizeof(float);
  p.ws_partials = (p.ws_partials + 255) / 256 * 256;
  p.ws_total = p.ws_counters + p.ws_partials;
  return p;
}

hipError_t launch_decode(const LayerView& L, int q_heads, int64_t T, const __half* q,
                         float sm_scale, float* out, void* ws, const DecodePlan& plan,
                         hipStream_t s) {
  const int gqa = q_heads / L.H;
  DecodeArgs a;
  a.L = L;
  a.q = q;
  a.out = out;
  a.counters = reinterpret_cast<unsigned*>(ws);
  a.part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + plan.ws_counters);
  a.Tq = quantized_len(T, L.R);
  a.nblk = (a.Tq + BLK - 1) / BLK;
  a.r = plan.r;
  a.n_split = plan.n_split;
  a.qscale = sm_scale * 1.4426950408889634f;
  const int64_t P = (int64_t)L.B * L.H;
  const dim3 grid((unsigned)(P * (plan.n_split + 1)));
  bool ok = dispatch_decode(L.bits, gqa, [&](auto b, auto g) {
    hipLaunchKernelGGL((decode_kernel<decltype(b)::value, decltype(g)::value>), grid, dim3(NT), 0,
                       s, a);
    return true;
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kivi
