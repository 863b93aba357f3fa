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
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}
// LDS hand-off between lanes of one wave: LDS operations of a wave execute in order,
// so only the compiler must be kept from moving LDS accesses across this point; the
// wait covers LDS (lgkm) only and leaves prefetched global loads in flight.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}
// Partials are exchanged between workgroups with system-scope relaxed stores/loads,
// which write through / bypass the per-XCD L2, so no L2 write-back fence is needed.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
typedef __attribute__((address_space(1))) unsigned long long global_u64;
__device__ __forceinline__ float2 load_coherent2(const float* p) {
  const unsigned long long u = __hip_atomic_load((global_u64*)(p), __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_SYSTEM);
  return make_float2(__uint_as_float((uint32_t)u), __uint_as_float((uint32_t)(u >> 32)));
}
// Wait until this thread's global stores have completed.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
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

// Per-wave LDS of the quantized path.  The query-limb operand of one (group, M-tile,
// K-step) is 16 rows of 4 lane-group blocks of 16 bytes; rows are padded to 80 bytes
// and K-steps to 1344 bytes so that the 16-bit limb writes of the group preparation hit
// at most two lanes per bank and the 16-byte operand reads of 8 lanes are conflict-free.
constexpr int QA_ROW = 80;                 // bytes per operand row (64 used)
constexpr int QA_KS = 16 * QA_ROW + 64;    // bytes per K-step block
template <int NMT>
struct WaveLds {
  uint8_t qa[2][NMT][2][QA_KS];       // [group in block][M-tile][K-step][row*QA_ROW + jg*16 + pos]
  uint8_t pa[NMT][16][4][16];         // [M-tile][row][run][pos]
};

// ---- the quantized token range of one wave ----------------------------------------

// Global-memory inputs of one 64-token block for one lane (loaded a block ahead).
template <int BITS>
struct BlockRegs {
  static constexpr int KW = BITS == 2 ? 2 : 4;    // Key-code words per token per lane
  static constexpr int VW = BITS == 2 ? 8 : 16;   // Value-code words per lane
  uint32_t k[4][KW];        // N-tile nt: token tb + 16nt + lo, channels 32j .. 32j+31
  uint32_t v[VW];           // run j of the block, channels 8lo .. 8lo+7
  i32x4 ks[2], kz[2];       // Key scale/zero of the block's groups, channels 8lo .. 8lo+7
  unsigned short sv[4], zv[4];   // token tb + 16nt + lo: Value scale and zero
};

// Buffer descriptors of one (sequence, KV head) pair's slabs, and the lane offsets
// that stay fixed from block to block (the block base goes in the scalar offset).
struct PairBufs {
  __amdgpu_buffer_rsrc_t kc, ksc, kze, vc, vsc, vze;
  int off_k, off_v, off_ks, off_sv;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes < 0x7FFFFFFF ? (int)bytes : 0x7FFFFFFF;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// The loads of one block come in four sets, each refilled for the next block right
// after its last use in the current one.  FULL: all 64 tokens of the block are in the
// history (compile-time: no branches); otherwise n_valid (a multiple of 16) are.
template <int BITS, bool FULL>
__device__ __forceinline__ void load_kcodes(BlockRegs<BITS>& R, const PairBufs& pb, int64_t tb,
                                            int n_valid, int nt) {
  constexpr int KB = D * BITS / 8;
  const int sk = (int)(tb * KB);
  if (FULL || nt < n_valid / 16) {
    if constexpr (BITS == 2) {
      const auto u = __builtin_amdgcn_raw_buffer_load_b64(pb.kc, pb.off_k + 16 * KB * nt, sk, 0);
      R.k[nt][0] = (uint32_t)u[0];
      R.k[nt][1] = (uint32_t)u[1];
    } else {
      const auto u = __builtin_amdgcn_raw_buffer_load_b128(pb.kc, pb.off_k + 16 * KB * nt, sk, 0);
#pragma unroll
      for (int w = 0; w < 4; ++w) R.k[nt][w] = (uint32_t)u[w];
    }
  } else {
#pragma unroll
    for (int w = 0; w < BlockRegs<BITS>::KW; ++w) R.k[nt][w] = 0u;
  }
}
template <int BITS, bool FULL>
__device__ __forceinline__ void load_vscale(BlockRegs<BITS>& R, const PairBufs& pb, int64_t tb,
                                            int n_valid, int nt) {
  const int ssv = (int)(tb * 2);
  if (FULL || nt < n_valid / 16) {
    R.sv[nt] = __builtin_amdgcn_raw_buffer_load_b16(pb.vsc, pb.off_sv + 32 * nt, ssv, 0);
    R.zv[nt] = __builtin_amdgcn_raw_buffer_load_b16(pb.vze, pb.off_sv + 32 * nt, ssv, 0);
  } else {
    R.sv[nt] = 0;
    R.zv[nt] = 0;
  }
}
template <int BITS, int G, bool FULL>
__device__ __forceinline__ void load_kscale(BlockRegs<BITS>& R, const PairBufs& pb, int64_t tb,
                                            int n_valid, int gi) {
  const int sg = (int)((tb / G) * D * 2);
  if (FULL || gi < (n_valid + G - 1) / G) {
    R.ks[gi] = __builtin_amdgcn_raw_buffer_load_b128(pb.ksc, pb.off_ks + gi * D * 2, sg, 0);
    R.kz[gi] = __builtin_amdgcn_raw_buffer_load_b128(pb.kze, pb.off_ks + gi * D * 2, sg, 0);
  } else {
    R.ks[gi] = i32x4{0, 0, 0, 0};
    R.kz[gi] = i32x4{0, 0, 0, 0};
  }
}
template <int BITS, bool FULL>
__device__ __forceinline__ void load_vcodes(BlockRegs<BITS>& R, const PairBufs& pb, int64_t tb,
                                            int n_valid, int j) {
  constexpr int VRB = kVRun * BITS / 8;
  const int sv_off = (int)((tb / kVRun) * D * VRB);
  if (FULL || j < n_valid / 16) {
#pragma unroll
    for (int q4 = 0; q4 < BlockRegs<BITS>::VW / 4; ++q4) {
      const auto u = __builtin_amdgcn_raw_buffer_load_b128(pb.vc, pb.off_v + 16 * q4, sv_off, 0);
#pragma unroll
      for (int w = 0; w < 4; ++w) R.v[4 * q4 + w] = (uint32_t)u[w];
    }
  } else {
#pragma unroll
    for (int w = 0; w < BlockRegs<BITS>::VW; ++w) R.v[w] = 0u;
  }
}
template <int BITS, int G, bool FULL>
__device__ __forceinline__ void load_block(BlockRegs<BITS>& R, const PairBufs& pb, int64_t tb,
                                           int n_valid, int j) {
#pragma unroll
  for (int gi = 0; gi < BLK / G; ++gi) load_kscale<BITS, G, FULL>(R, pb, tb, n_valid, gi);
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    load_kcodes<BITS, FULL>(R, pb, tb, n_valid, nt);
    load_vscale<BITS, FULL>(R, pb, tb, n_valid, nt);
  }
  load_vcodes<BITS, FULL>(R, pb, tb, n_valid, j);
}
// Keeps the scheduler from moving a refill above the last use of the registers it
// overwrites.
__device__ __forceinline__ void refill_point() { __builtin_amdgcn_sched_barrier(0); }

// Online-softmax and accumulator state of one wave (head 4mt + j on this lane's row).
template <int NMT>
struct WaveState {
  float m_run[NMT], l_run[NMT], pz_run[NMT];
  float acc_f[NMT][8];            // channels 8lo + n, in units of 2^Ev
  i32x4 acc_i[NMT][8];
};

// One 64-token block: group preparation, Q.K^T, online softmax, P.V.
// REFILL: each register set is reloaded with the full block at token tb_next right
// after its last use here.
template <int BITS, int GQA, int G, bool FULL, bool REFILL>
__device__ __forceinline__ void process_block(BlockRegs<BITS>& R, int n_valid,
                                              const float (&qv)[(GQA + 3) / 4][8],
                                              float k_unscale, int Ev,
                                              WaveLds<(GQA + 3) / 4>& lds,
                                              WaveState<(GQA + 3) / 4>& st, int lo, int j,
                                              const PairBufs& pb, int64_t tb_next) {
  constexpr int NMT = (GQA + 3) / 4;
  constexpr int NG = BLK / G;
  const int n_groups_blk = FULL ? NG : (n_valid + G - 1) / G;
  const int n_tiles = FULL ? 4 : n_valid / 16;

  // (1) group preparation: query limbs into LDS, and sum_c q_c z_c per head.
  // Lane (lo, j) owns channels 8lo .. 8lo+7 of head 4mt + j; its limbs are transposed
  // in registers (v_perm) so that each write carries one limb of 2 (2-bit) or 4 (4-bit)
  // channels that are adjacent in the operand.
  float qz[NG][NMT];
  const int jg = lo >> 2, ksl = (lo >> 1) & 1;
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) qz[gi][mt] = 0.f;
    if (FULL || gi < n_groups_blk) {
      const uint32_t sw[4] = {(uint32_t)R.ks[gi][0], (uint32_t)R.ks[gi][1], (uint32_t)R.ks[gi][2],
                              (uint32_t)R.ks[gi][3]};
      const uint32_t zw[4] = {(uint32_t)R.kz[gi][0], (uint32_t)R.kz[gi][1], (uint32_t)R.kz[gi][2],
                              (uint32_t)R.kz[gi][3]};
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        uint32_t x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float sc = h2f((unsigned short)(sw[i >> 1] >> (16 * (i & 1))));
          const float ze = h2f((unsigned short)(zw[i >> 1] >> (16 * (i & 1))));
          x[i] = to_limbs(qv[mt][i] * sc);
          qz[gi][mt] = fmaf(qv[mt][i], ze, qz[gi][mt]);
        }
        uint8_t* blkp = &lds.qa[gi][mt][ksl][(4 * j) * QA_ROW + jg * 16];
        if constexpr (BITS == 2) {
          // channel 8lo + i sits at position 4(i%4) + 2(lo%2) + i/4 of its row block
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) {
            const uint32_t w01 = __builtin_amdgcn_perm(x[s4 + 4], x[s4], 0x05010400u);
            const uint32_t w23 = __builtin_amdgcn_perm(x[s4 + 4], x[s4], 0x07030602u);
            uint8_t* d = blkp + 4 * s4 + 2 * (lo & 1);
            *reinterpret_cast<uint16_t*>(d) = (uint16_t)w01;
            *reinterpret_cast<uint16_t*>(d + QA_ROW) = (uint16_t)(w01 >> 16);
            *reinterpret_cast<uint16_t*>(d + 2 * QA_ROW) = (uint16_t)w23;
            *reinterpret_cast<uint16_t*>(d + 3 * QA_ROW) = (uint16_t)(w23 >> 16);
          }
        } else {
          // channel 8lo + i sits at position 4(2(lo%2) + i%2) + i/2 of its row block
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const uint32_t a = x[s2], b = x[s2 + 2], c = x[s2 + 4], e = x[s2 + 6];
            const uint32_t t0 = __builtin_amdgcn_perm(b, a, 0x05010400u);   // a0 b0 a1 b1
            const uint32_t t1 = __builtin_amdgcn_perm(b, a, 0x07030602u);   // a2 b2 a3 b3
            const uint32_t t2 = __builtin_amdgcn_perm(e, c, 0x05010400u);   // c0 e0 c1 e1
            const uint32_t t3 = __builtin_amdgcn_perm(e, c, 0x07030602u);   // c2 e2 c3 e3
            uint8_t* d = blkp + 4 * (2 * (lo & 1) + s2);
            *reinterpret_cast<uint32_t*>(d) = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
            *reinterpret_cast<uint32_t*>(d + QA_ROW) = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
            *reinterpret_cast<uint32_t*>(d + 2 * QA_ROW) = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
            *reinterpret_cast<uint32_t*>(d + 3 * QA_ROW) = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
          }
        }
      }
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) qz[gi][mt] = row_sum16(qz[gi][mt]) * k_unscale;
    }
    if constexpr (REFILL) {
      refill_point();
      load_kscale<BITS, G, true>(R, pb, tb_next, BLK, gi);
    }
  }
  wave_lds_sync();

  // (2) Q.K^T on the matrix cores: C[mt][nt] rows (head, limb), columns tokens.
  i32x4 cqk[NMT][4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) cqk[mt][nt] = i32x4{0, 0, 0, 0};
    if (FULL || nt < n_tiles) {
      const int gi = nt * 16 / G;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const i32x4 bop = BITS == 2 ? unpack16<BITS>(R.k[nt][ks], 0u)
                                    : unpack16<BITS>(R.k[nt][2 * ks % BlockRegs<BITS>::KW],
                                                     R.k[nt][(2 * ks + 1) % BlockRegs<BITS>::KW]);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
          const i32x4 aop = *reinterpret_cast<const i32x4*>(&lds.qa[gi][mt][ks][lo * QA_ROW + j * 16]);
          cqk[mt][nt] = mfma_i8(aop, bop, cqk[mt][nt]);
        }
      }
    }
    if constexpr (REFILL) {
      refill_point();
      load_kcodes<BITS, true>(R, pb, tb_next, BLK, nt);
    }
  }

  // (3) logits, online softmax, probability limbs into LDS.
  float sv[4], zv[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    sv[nt] = h2f(R.sv[nt]);
    zv[nt] = h2f(R.zv[nt]);
  }
  if constexpr (REFILL) {
    refill_point();
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) load_vscale<BITS, true>(R, pb, tb_next, BLK, nt);
  }
  const float k_hi = 65536.f * k_unscale;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    float z[4];
    float bm = -INFINITY;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int gi = nt * 16 / G;
      const i32x4 c = cqk[mt][nt];
      const float lo16 = (float)(c[0] + c[1] * 256);      // |c_i| < 2^18: exact int
      const float hi16 = (float)(c[2] + c[3] * 256);
      z[nt] = fmaf(hi16, k_hi, fmaf(lo16, k_unscale, qz[gi][mt]));
      if (!FULL && nt >= n_tiles) z[nt] = -INFINITY;
      bm = fmaxf(bm, z[nt]);
    }
    bm = row_max16(bm);
    const float m_new = fmaxf(st.m_run[mt], bm);
    // The running max rose on some row: fold the integer accumulators of those rows
    // into float and rescale (a wave-uniform branch; alpha = 1 on the other rows).
    if (__builtin_amdgcn_read_exec() & __ballot(m_new > st.m_run[mt])) {
      const float alpha = __builtin_amdgcn_exp2f(st.m_run[mt] - m_new);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const i32x4 ci = st.acc_i[mt][n];
        const float v = st.acc_f[mt][n] + (float)ci[0] + 256.f * (float)ci[1] +
                        65536.f * (float)ci[2] + 16777216.f * (float)ci[3];
        st.acc_f[mt][n] = v * alpha;
        st.acc_i[mt][n] = i32x4{0, 0, 0, 0};
      }
      st.l_run[mt] *= alpha;
      st.pz_run[mt] *= alpha;
      st.m_run[mt] = m_new;
    }
    const float m_shift = st.m_run[mt] - (float)Ev;     // p' = p * 2^Ev
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      float p = __builtin_amdgcn_exp2f(z[nt] - m_shift);
      if (!FULL && nt >= n_tiles) p = 0.f;
      st.l_run[mt] += p;
      st.pz_run[mt] = fmaf(p, zv[nt], st.pz_run[mt]);
      const uint32_t lw = to_limbs(p * sv[nt]);
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
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const i32x4 aop = *reinterpret_cast<const i32x4*>(&lds.pa[mt][lo][j][0]);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const i32x4 bop = BITS == 2 ? unpack16<BITS>(R.v[n], 0u)
                                  : unpack16<BITS>(R.v[2 * n], R.v[2 * n + 1]);
      st.acc_i[mt][n] = mfma_i8(aop, bop, st.acc_i[mt][n]);
    }
  }
  if constexpr (REFILL) {
    refill_point();
    load_vcodes<BITS, true>(R, pb, tb_next, BLK, j);
  }
}

// Writes comb[GQA][PSTRIDE] (acc with the Value-zero term folded in, m, l).
template <int BITS, int GQA, int G>
__device__ void quantized_wave(const DecodeArgs& a, int64_t pair, int64_t blk0, int64_t blk1,
                               WaveLds<(GQA + 3) / 4>& lds, float* comb) {
  constexpr int NMT = (GQA + 3) / 4;              // M-tiles of 4 heads x 4 limbs
  const LayerView& L = a.L;
  const int lane = threadIdx.x & 63;
  const int lo = lane & 15, j = lane >> 4;
  const int64_t b = pair / L.H, h = pair % L.H;

  constexpr int KB = D * BITS / 8;
  constexpr int VRB = kVRun * BITS / 8;             // Value code bytes per (run, channel)
  const uint8_t* kc = L.k_codes + pair * L.kc_pair();
  const __half* ksc = L.k_scale + pair * L.ks_pair();
  const __half* kze = L.k_zero + pair * L.ks_pair();
  const uint8_t* vc = L.v_codes + pair * L.vc_pair();
  const unsigned short* vsc = reinterpret_cast<const unsigned short*>(L.v_scale + pair * L.vs_pair());
  const unsigned short* vze = reinterpret_cast<const unsigned short*>(L.v_zero + pair * L.vs_pair());
  PairBufs pb;
  pb.kc = make_rsrc(kc, L.kc_pair());
  pb.ksc = make_rsrc(ksc, L.ks_pair() * 2);
  pb.kze = make_rsrc(kze, L.ks_pair() * 2);
  pb.vc = make_rsrc(vc, L.vc_pair());
  pb.vsc = make_rsrc(vsc, L.vs_pair() * 2);
  pb.vze = make_rsrc(vze, L.vs_pair() * 2);
  pb.off_k = lo * KB + j * (KB / 4);
  pb.off_v = j * D * VRB + 8 * lo * VRB;
  pb.off_ks = 16 * lo;
  pb.off_sv = 2 * lo;
  const int Hq = L.H * GQA;
  const __half* qp = a.q + (b * Hq + h * GQA) * D;

  const int64_t t_lo = blk0 * BLK;
  const int64_t t_hi = blk1 * BLK < a.Tq ? blk1 * BLK : a.Tq;
  // Blocks [blk0, nfull) hold 64 tokens; a last half block (32 tokens) may follow.
  const int64_t nfull = (t_hi - t_lo) / BLK + blk0;
  const bool tail = nfull < blk1;

  // The first block's loads go out before the pre-pass so that both latencies overlap.
  BlockRegs<BITS> R;
  if (nfull > blk0) load_block<BITS, G, true>(R, pb, blk0 * BLK, BLK, j);

  // -- pre-pass: largest |q| (scaled), largest Key scale and Value scale in range --
  // Lane (lo, j) holds the query values it prepares later: head 4mt + j, channels
  // 8lo .. 8lo+7, i.e. the 16 bytes at offset 16*lane of M-tile mt's 4 heads.
  float qraw[NMT][8];
  float qmax = 0.f;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int hd = 4 * mt + j;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (hd < GQA) u = *reinterpret_cast<const uint4*>(qp + (int64_t)hd * D + 8 * lo);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qraw[mt][i] = h2f((unsigned short)(w[i >> 1] >> (16 * (i & 1))));
      qmax = fmaxf(qmax, fabsf(qraw[mt][i]));
    }
  }
  uint32_t mk = 0, mv = 0;
  {
    const int64_t g_lo = t_lo / G, g_hi = (t_hi + G - 1) / G;
    const uint4* ks4 = reinterpret_cast<const uint4*>(ksc + g_lo * D);
    const int64_t n4 = (g_hi - g_lo) * (D / 8);
    const uint4* vs4 = reinterpret_cast<const uint4*>(vsc + t_lo);
    const int64_t v4 = (t_hi - t_lo) / 8;
    auto fold = [](uint32_t m, const uint4& u) {
      // non-negative float16 values order like their bit patterns
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) m = max(m, max(w[k] & 0xFFFFu, w[k] >> 16));
      return m;
    };
    // Every load of a round is issued before any is folded: one round covers 16 blocks.
    constexpr int UK = 8, UV = 2;
    const int64_t rounds_k = (n4 + 64 * UK - 1) / (64 * UK), rounds_v = (v4 + 64 * UV - 1) / (64 * UV);
    const int64_t rounds = rounds_k > rounds_v ? rounds_k : rounds_v;
    for (int64_t r = 0; r < rounds; ++r) {
      uint4 uk[UK], uv[UV];
#pragma unroll
      for (int u = 0; u < UK; ++u) {
        const int64_t i = r * 64 * UK + 64 * u + lane;
        uk[u] = i < n4 ? ks4[i] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < UV; ++u) {
        const int64_t i = r * 64 * UV + 64 * u + lane;
        uv[u] = i < v4 ? vs4[i] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < UK; ++u) mk = fold(mk, uk[u]);
#pragma unroll
      for (int u = 0; u < UV; ++u) mv = fold(mv, uv[u]);
    }
  }
  qmax = wave_max(qmax) * fabsf(a.qscale);
  const float skmax = wave_max(h2f((unsigned short)mk));
  const float svmax = wave_max(h2f((unsigned short)mv));
  const int Ek = fixed_exponent(qmax * skmax);
  const int Ev = fixed_exponent(svmax);
  const float k_unscale = __builtin_amdgcn_ldexpf(1.f, -Ek);
  const float v_unscale = __builtin_amdgcn_ldexpf(1.f, -Ev);

  // Query values of this lane for the group preparation: heads 4mt + j, channels
  // 8lo .. 8lo+7, scaled by sm_scale*log2(e)*2^Ek.
  float qv[NMT][8];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[mt][i] = __builtin_amdgcn_ldexpf(qraw[mt][i] * a.qscale, Ek);

  WaveState<NMT> st;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    st.m_run[mt] = -INFINITY;
    st.l_run[mt] = 0.f;
    st.pz_run[mt] = 0.f;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      st.acc_f[mt][n] = 0.f;
      st.acc_i[mt][n] = i32x4{0, 0, 0, 0};
    }
  }

  // Full blocks: every register set is refilled with the next block right after its
  // last use, so each set's loads have a whole block of work to hide behind.  The
  // refills are unconditional (clamped to the last full block, whose repeated load hits
  // the cache and is not used) so that no branch surrounds a load.
  const int64_t last_full = nfull - 1;
  for (int64_t blk = blk0; blk < nfull; ++blk) {
    const int64_t nb = blk + 1 < last_full ? blk + 1 : last_full;
    process_block<BITS, GQA, G, true, true>(R, BLK, qv, k_unscale, Ev, lds, st, lo, j, pb, nb * BLK);
  }
  if (tail) {
    const int nv = (int)(t_hi - nfull * BLK);
    load_block<BITS, G, false>(R, pb, nfull * BLK, nv, j);
    process_block<BITS, GQA, G, false, false>(R, nv, qv, k_unscale, Ev, lds, st, lo, j, pb, 0);
  }

  // Finish: fold the integer accumulators and the Value-zero term, undo 2^Ev.
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int hd = 4 * mt + j;
    const float lsum = row_sum16(st.l_run[mt]);
    const float pz = row_sum16(st.pz_run[mt]);
    if (hd < GQA) {
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const i32x4 ci = st.acc_i[mt][n];
        const float v = st.acc_f[mt][n] + (float)ci[0] + 256.f * (float)ci[1] +
                        65536.f * (float)ci[2] + 16777216.f * (float)ci[3];
        comb[hd * PSTRIDE + 8 * lo + n] = (v + pz) * v_unscale;
      }
      if (lo == 0) {
        comb[hd * PSTRIDE + D] = st.m_run[mt];
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
    // All 32 rows' Value pairs of this lane are loaded before use (rows past the
    // chunk re-read its last row; their probabilities are 0).
    __half2 vv[32];
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const int row = t < n_valid ? t : n_valid - 1;
      vv[t] = *reinterpret_cast<const __half2*>(vr + (int64_t)(c0 + row) * D + 2 * lane);
    }
#pragma unroll
    for (int hd = 0; hd < GQA; ++hd) {
      const float al = palpha[hd];
      float s0 = acc[hd][0] * al, s1 = acc[hd][1] * al;
#pragma unroll
      for (int t = 0; t < 32; ++t) {
        const float p = pw[hd * 32 + t];
        s0 = fmaf(p, __low2float(vv[t]), s0);
        s1 = fmaf(p, __high2float(vv[t]), s1);
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
      store_coherent(&dst[hd * dst_hstride + c], o);
      if (c == 0) {
        store_coherent(&dst[hd * dst_hstride + D], mstar);
        store_coherent(&dst[hd * dst_hstride + D + 1], l);
      }
    } else {
      dst[hd * dst_hstride + c] = o / l;
    }
  }
}

// Final merge by the last workgroup of a pair, 32 partials per round.  Each (partial,
// head) pair's (m, l) is loaded once, by one thread, into LDS ([head][partial]); thread
// (head hd, channels c, c+1) loads the accumulators of every partial of the round, and
// both kinds of loads are in flight together.  The fold has no branches: indices past
// the last partial are clamped and weighted 0, and empty partials (l == 0) weigh 0.
// Partials are folded in a fixed order with an online rescale.
template <int GQA>
__device__ __forceinline__ void merge_pair(const float* __restrict__ base, int n_parts,
                                           float* __restrict__ out, float2* ml_lds) {
  constexpr int MERGE_CH = 32;
  constexpr int ITEMS = GQA * (D / 2);
  constexpr int IPT = (ITEMS + NT - 1) / NT;       // (head, channel pair) items per thread
  static_assert(MERGE_CH * GQA <= NT, "one (m, l) load per thread and round");
  float m[IPT], l[IPT], o0[IPT], o1[IPT];
#pragma unroll
  for (int it = 0; it < IPT; ++it) {
    m[it] = -INFINITY;
    l[it] = o0[it] = o1[it] = 0.f;
  }
  for (int i0 = 0; i0 < n_parts; i0 += MERGE_CH) {
    const int nc = n_parts - i0 < MERGE_CH ? n_parts - i0 : MERGE_CH;
    float2 ov[IPT][MERGE_CH];
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int idx = threadIdx.x + it * NT;
      const int hd = min(idx / (D / 2), GQA - 1), c = 2 * (idx % (D / 2));
#pragma unroll
      for (int u = 0; u < MERGE_CH; ++u) {
        const int i = min(i0 + u, n_parts - 1);
        ov[it][u] = load_coherent2(base + ((int64_t)i * GQA + hd) * PSTRIDE + c);
      }
    }
    if (threadIdx.x < MERGE_CH * GQA) {
      const int u = threadIdx.x / GQA, hd = threadIdx.x % GQA;
      const int i = min(i0 + u, n_parts - 1);
      const float2 ml = load_coherent2(base + ((int64_t)i * GQA + hd) * PSTRIDE + D);
      ml_lds[hd * MERGE_CH + u] = u < nc ? ml : make_float2(-INFINITY, 0.f);
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int idx = threadIdx.x + it * NT;
      const int hd = min(idx / (D / 2), GQA - 1);
      float2 ml[MERGE_CH];
#pragma unroll
      for (int u = 0; u < MERGE_CH; u += 2) {
        const float4 q = *reinterpret_cast<const float4*>(&ml_lds[hd * MERGE_CH + u]);
        ml[u] = make_float2(q.x, q.y);
        ml[u + 1] = make_float2(q.z, q.w);
      }
      float mc = m[it];
#pragma unroll
      for (int u = 0; u < MERGE_CH; ++u) mc = fmaxf(mc, ml[u].y > 0.f ? ml[u].x : -INFINITY);
      const float mref = mc > -INFINITY ? mc : 0.f;
      const float wa = __builtin_amdgcn_exp2f(m[it] - mref);
      float lt = l[it] * wa, a0 = o0[it] * wa, a1 = o1[it] * wa;
#pragma unroll
      for (int u = 0; u < MERGE_CH; ++u) {
        const float w = ml[u].y > 0.f ? __builtin_amdgcn_exp2f(ml[u].x - mref) : 0.f;
        lt = fmaf(ml[u].y, w, lt);
        a0 = fmaf(ov[it][u].x, w, a0);
        a1 = fmaf(ov[it][u].y, w, a1);
      }
      l[it] = lt;
      o0[it] = a0;
      o1[it] = a1;
      m[it] = mc;
    }
    __syncthreads();                                 // ml_lds is rewritten next round
  }
#pragma unroll
  for (int it = 0; it < IPT; ++it) {
    const int idx = threadIdx.x + it * NT;
    if (idx >= ITEMS) continue;
    const int hd = idx / (D / 2), c = 2 * (idx % (D / 2));
    const float inv = 1.f / l[it];
    *reinterpret_cast<float2*>(out + (int64_t)hd * D + c) = make_float2(o0[it] * inv, o1[it] * inv);
  }
}

// Workgroups per CU that the register budget of each variant allows (the build turns
// a missed occupancy target into an error, so this table stays true).
constexpr int wgs_per_cu(int bits, int gqa, int G) {
  return gqa > 4 ? 1 : (bits == 2 || G == 64) ? 3 : 2;
}

template <int BITS, int GQA, int G>
__global__ __launch_bounds__(NT, wgs_per_cu(BITS, GQA, G)) void decode_kernel(DecodeArgs a) {
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
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
    if (blk1 > blk0) quantized_wave<BITS, GQA, G>(a, pair, blk0, blk1, lds.wave[wave], cw);
  }
  __syncthreads();

  // Workgroup partial -> workspace.
  float* mine = a.part + ((pair * n_parts + s) * GQA) * PSTRIDE;
  combine<GQA>(WAVES, [&](int i) { return (const float*)comb[i]; }, mine, PSTRIDE, true);

  // Last workgroup of the pair merges all partials and resets the counter.  Every
  // thread's partial stores complete before the arrival is counted; the merging
  // workgroup reads the partials with coherent loads after it has seen all arrivals.
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(&a.counters[pair], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (prev == (unsigned)(n_parts - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!last_flag) return;
  const float* base = a.part + (pair * n_parts * GQA) * PSTRIDE;
  const int64_t b = pair / a.L.H, h = pair % a.L.H;
  float* o = a.out + (b * a.L.H * GQA + h * GQA) * D;
  merge_pair<GQA>(base, n_parts, o, reinterpret_cast<float2*>(&comb[0][0]));
  if (threadIdx.x == 0)
    __hip_atomic_store(&a.counters[pair], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename F>
bool dispatch_decode(int bits, int gqa, int G, F&& f) {
#define KIVI_CASE(B, Q, GG)                                                              \
  if (bits == B && gqa == Q && G == GG)                                                 \
    return f(std::integral_constant<int, B>{}, std::integral_constant<int, Q>{},         \
             std::integral_constant<int, GG>{});
  KIVI_CASE(2, 1, 32) KIVI_CASE(2, 2, 32) KIVI_CASE(2, 4, 32) KIVI_CASE(2, 8, 32)
  KIVI_CASE(4, 1, 32) KIVI_CASE(4, 2, 32) KIVI_CASE(4, 4, 32) KIVI_CASE(4, 8, 32)
  KIVI_CASE(2, 1, 64) KIVI_CASE(2, 2, 64) KIVI_CASE(2, 4, 64) KIVI_CASE(2, 8, 64)
  KIVI_CASE(4, 1, 64) KIVI_CASE(4, 2, 64) KIVI_CASE(4, 4, 64) KIVI_CASE(4, 8, 64)
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
    // one round of resident workgroups on 256 CUs, at least 4 blocks per wave
    const int per_cu = wgs_per_cu(L.bits, gqa, L.G);
    const int64_t target_wgs = 256 * per_cu;                    // incl. one residual wg/pair
    ns = target_wgs > 2 * pairs ? (target_wgs - pairs) / pairs : 1;
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
  bool ok = dispatch_decode(L.bits, gqa, L.G, [&](auto b, auto g, auto gg) {
    hipLaunchKernelGGL((decode_kernel<decltype(b)::value, decltype(g)::value, decltype(gg)::value>),
                       grid, dim3(NT), 0, s, a);
    return true;
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kivi
