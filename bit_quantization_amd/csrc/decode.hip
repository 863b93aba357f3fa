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
// E is chosen per (sequence, KV head) from its largest |q| s (resp. s_t), which the
// quantizer keeps in scale_max, so that |x| <= 2^30.  Integer products are exact; the
// limb sums are recombined in float32.
//
// Work split.  One workgroup per CU holds all the waves that fit there.  Each
// (sequence, KV head) pair's quantized tokens are cut into 64-token blocks, and
// n_split workgroups take contiguous shares of them; the first also takes the float16
// window rows in 32-row chunks.  Inside a workgroup the waves take chunks and blocks
// from an LDS counter, each wave with its own online softmax (running max m, sum l),
// so waves that run ahead take more blocks.  The waves combine in LDS in wave order.
// Each workgroup clears its partial slot when it starts and at the end writes its
// partial there, every float with its lowest bit set as a "written" mark; without
// waiting for those stores it counts its arrival on the pair's counter.  The last to
// arrive waits until every word it needs is marked and folds the partials in split
// order:
//   m* = max m_s,  l* = sum l_s 2^(m_s - m*),  o = sum acc_s 2^(m_s - m*) / l*.
// No floating-point atomics.  Which wave takes which block varies from run to run,
// and float sums in a different order round differently, so repeated runs agree to
// float32 rounding rather than bit for bit.
//
// Logits are kept in base 2 (the query is pre-multiplied by sm_scale * log2(e)).
#include <type_traits>

#include "decode_common.h"
#include "quantizer.h"

namespace kivi {
namespace {

constexpr int BLK = kDecodeBlockTokens;   // tokens per block step of a wave
// Work of one 32-row float16 window chunk in blocks (it moves three blocks' bytes with
// fewer loads in flight and takes about three blocks of wave time)
constexpr int RES_COST = 3;

typedef int i32x4 __attribute__((ext_vector_type(4)));

struct DecodeArgs {
  LayerView L;
  const __half* q;
  float* out;
  float* part;          // [P][n_parts][GQA][PSTRIDE]; slot s cleared by its owner first
  unsigned* counters;   // [P][kCounterStride]: arrival counter, zero between calls
  int64_t Tq;           // tokens of the 64-token blocks (with the per-token Value window,
                        // the blocks end at 64 * floor(Tqv / 64))
  int64_t nblk;         // 64-token blocks per pair (the last may hold 32 tokens)
  int64_t Tqk;          // quantized Key tokens (Tq unless the per-token Value window)
  int64_t Tqv;          // quantized Value tokens (likewise)
  int n_mix;            // 32-row chunks of [Tq, Tqk): quantized Keys, Values quantized
                        // below Tqv and float16 from Tqv on
  int r;                // float16 tokens: sink rows, then the window
  int ring;             // window ring start: window token i is in row S + (ring + i) mod R
  int nw;               // workgroups per pair
  float qscale;         // sm_scale * log2(e)
  const __half* k_new;  // [P][D]: window row new_slot comes from here (new_slot >= 0)
  const __half* v_new;
  int new_slot;         // -1: every window row is read from the cache
  int tl_slot;          // timeline slot of this launch (measurement build), else -1
  int64_t vt;           // per-token Value window, fused step: the history token whose
                        // Value leaves the window in this step (its row is new_slot);
                        // -1: none
  Lens lens;            // ragged batch: per-sequence counts (the fields above are for T)
};

// A ragged batch: the tokens sequence b attends over.
__device__ __forceinline__ int64_t ragged_tokens(const DecodeArgs& a, int64_t b) {
  return a.new_slot >= 0 ? a.lens.get(b, 0) + 1 : a.lens.get(b, 1);
}

// A ragged batch shares out the workgroups of each KV head's slice of the grid (B * nw
// of them) among the sequences in proportion to their token counts, at least one
// each, so that a long sequence gets more workgroups than a short one (the spare
// workgroups beyond one each are cut at the rounded cumulative token shares, so all
// of them are used).  Sets the workgroup's pair, its index s among the pair's nw
// workgroups and the pair's first partial slot; returns false if none is left for it.
struct RaggedSlot {
  int64_t pair, slot0;
  int s, nw;
};
__device__ __forceinline__ bool ragged_assign(const DecodeArgs& a, RaggedSlot& out) {
  const int B = a.L.B, H = a.L.H;
  const int64_t per_head = gridDim.x / H;
  const int64_t h = blockIdx.x / per_head, i = blockIdx.x % per_head;
  int64_t sum = 0;
  for (int b = 0; b < B; ++b) sum += ragged_tokens(a, b);
  const int64_t spare = per_head - B;
  int64_t acc = 0, cum = 0, cut = 0;
  for (int b = 0; b < B; ++b) {
    cum += ragged_tokens(a, b);
    const int64_t next_cut = spare * cum / sum;
    const int64_t w = 1 + next_cut - cut;
    cut = next_cut;
    if (i < acc + w) {
      out.pair = (int64_t)b * H + h;
      out.s = (int)(i - acc);
      out.nw = (int)w;
      out.slot0 = h * per_head + acc;
      return true;
    }
    acc += w;
  }
  return false;
}

// A ragged batch: the token split of sequence b (and its new row's slot), computed by
// each workgroup for its own pair.
__device__ __forceinline__ void ragged_split(DecodeArgs& a, int64_t b) {
  int64_t T;
  if (a.new_slot >= 0) {
    const int64_t T_before = a.lens.get(b, 0);
    a.new_slot = plan_append(a.L, T_before).slot;
    T = T_before + 1;
  } else {
    T = a.lens.get(b, 1);
  }
  const TokenSplit ts = split_tokens(a.L, T);
  a.Tq = a.Tqk = a.Tqv = ts.Tq;
  a.n_mix = 0;
  a.nblk = (ts.Tq + BLK - 1) / BLK;
  a.r = (int)ts.fp16_rows();
  a.ring = ts.ring;
}

// Waves per SIMD that the register budget of each variant allows; a workgroup holds
// 4 SIMDs' worth.  The build turns a kernel that misses this occupancy into an error
// (launch bounds of one workgroup per CU with a register limit derived from it).
constexpr int waves_per_simd(int bits, int gqa, int G) {
  return gqa > 2 ? 2 : (bits == 2 || G == 64) ? 3 : 2;
}

__device__ __forceinline__ float h2f(unsigned short h) {
  return __half2float(__ushort_as_half(h));
}
// 32-bit fixed point -> four balanced int8 limbs packed in one word (byte i = limb i,
// sum of limb_i * 256^i = x).  The caller passes vb = v + LIMB_BIAS computed in float
// (one fused multiply-add with the product that forms v); for |v| < 2^30 the float
// addition rounds by at most 64, far below the resolution of the operands, and then
// x = trunc(vb) - 0x808080 has the limbs trunc(vb) ^ 0x808080.
constexpr float LIMB_BIAS = 8421504.f;           // 0x808080
__device__ __forceinline__ uint32_t limbs_biased(float vb) {
  return (uint32_t)(int)vb ^ 0x00808080u;
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

// Code operands.  With the word-interleaved packing, shifting a packed word right by
// BITS*s and masking one field per byte yields codes 4s .. 4s+3 of the word in byte
// order, so a lane's 16-byte operand holds its codes in natural order (Keys: channels
// 32j + 16ks + [0, 16) of one token; Values: the 16 tokens of run j of one channel).
// 2-bit words skip the shift where a mask alone isolates the field: byte p of the
// operand then carries code * 2^code_shift(p), and the other operand of the product
// carries the matching 2^-code_shift(p).
template <int BITS>
__host__ __device__ constexpr int code_shift(int p) {
  return BITS == 2 ? 2 * (((p & 15) >> 2) < 2 ? ((p & 15) >> 2) : 2) : 0;
}
template <int BITS>
__device__ __forceinline__ i32x4 unpack16(uint32_t w0, uint32_t w1) {
  i32x4 u;
  if constexpr (BITS == 2) {
    u[0] = (int)(w0 & 0x03030303u);            // codes 0..3    (x1)
    u[1] = (int)(w0 & 0x0C0C0C0Cu);            // codes 4..7    (x4)
    u[2] = (int)(w0 & 0x30303030u);            // codes 8..11   (x16)
    u[3] = (int)((w0 >> 2) & 0x30303030u);     // codes 12..15  (x16)
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
// so that the 16-byte operand reads of 8 lanes are conflict-free.  The probability
// operand is 16 rows of 4 Value runs of 16 bytes.
constexpr int QA_ROW = 80;                 // bytes per operand row (64 used)
constexpr int QA_KS = 16 * QA_ROW + 64;    // bytes per K-step block
template <int NMT>
struct WaveLds {
  alignas(16) uint8_t qa[2][NMT][2][QA_KS];   // [group in block][M-tile][K-step][row*QA_ROW + jg*16 + pos]
  alignas(16) uint8_t pa[NMT][16][4][16];     // [M-tile][row][run][token in run]
};

// The items of one wave of a workgroup (window chunks first, then 64-token blocks).
// By default waves take them from the workgroup's LDS counter, so that waves that run
// ahead take more.  Deterministic decode (KIVI_FLAG_DETERMINISTIC): a fixed round-robin
// instead, chunk c to wave c mod W and block turns in wave order, each wave skipping
// RES_COST turns per chunk it holds, so that every wave's cost is within RES_COST of
// the others' and the blocks a wave accumulates, and their order, do not depend on the
// run.
struct WaveItems {
  int* counter;           // LDS counter (dynamic) or nullptr (round-robin)
  int w, W, n_res, nb, C, A, cnext, r;
  __device__ WaveItems(int* counter_, int w_, int W_, int n_res_, int nb_)
      : counter(counter_), w(w_), W(W_), n_res(n_res_), nb(nb_), C(n_res_ / W_), A(n_res_ % W_),
        cnext(w_), r(RES_COST * (n_res_ / W_ + (w_ < n_res_ % W_ ? 1 : 0))) {}
  __device__ int next() {
    if (counter) return grab_item(counter);
    if (cnext < n_res) {
      const int c = cnext;
      cnext += W;
      return c;
    }
    const int s0 = RES_COST * C;
    const int k = A * max(0, r - s0 - RES_COST) + (W - A) * max(0, r - s0) +
                  (r >= s0 + RES_COST ? min(w, A) : 0) + (r >= s0 ? max(0, w - A) : 0);
    ++r;
    return k < nb ? n_res + k : n_res + nb;
  }
};

// ---- the quantized token range of one wave ----------------------------------------

// Column lo of Q.K^T N-tile nt is token 2lo + (nt & 1) + 32 (nt >> 1) of the block:
// tiles 0-1 cover tokens 0..31 and tiles 2-3 tokens 32..63, so each tile lies in one
// Key group, and a lane's four tokens are two adjacent pairs of the Value runs lo/8
// and 2 + lo/8.
__device__ __forceinline__ int tile_token(int lo, int nt) { return 2 * lo + (nt & 1) + 32 * (nt >> 1); }

// Global-memory inputs of one 64-token block for one lane.
template <int BITS>
struct BlockRegs {
  static constexpr int KW = BITS == 2 ? 2 : 4;    // Key-code words per token per lane
  static constexpr int VW = BITS == 2 ? 8 : 16;   // Value-code words per lane
  uint32_t k[4][KW];        // N-tile nt: token tile_token(lo, nt), channels 32j .. 32j+31
  uint32_t v[VW];           // run j of the block, channels 8lo .. 8lo+7
  i32x4 ks[2], kz[2];       // Key scale/zero of the block's groups, channels 8lo .. 8lo+7
  uint32_t sv[2], zv[2];    // Value scale/zero of tokens 32k + 2lo, 32k + 2lo + 1
};

// Buffer descriptors of one (sequence, KV head) pair's slabs, and the lane offsets
// that stay fixed from block to block (the block base goes in the scalar offset).
struct PairBufs {
  __amdgpu_buffer_rsrc_t kc, ksc, kze, vc, vsc, vze;
  int off_k, off_v, off_ks, off_sv;
};

// The loads of one block come in four sets, each refilled for the next block right
// after its last use in the current one.  FULL: all 64 tokens of the block are in the
// history (compile-time: no branches); otherwise the first n_valid = 32 are.
template <int BITS, bool FULL>
__device__ __forceinline__ void load_kcodes(BlockRegs<BITS>& R, const PairBufs& pb, int64_t tb,
                                            int n_valid, int nt) {
  constexpr int KB = D * BITS / 8;
  const int sk = (int)(tb * KB);
  const int off = pb.off_k + ((nt & 1) + 32 * (nt >> 1)) * KB;
  if (FULL || 32 * (nt >> 1) < n_valid) {
    if constexpr (BITS == 2) {
      const auto u = __builtin_amdgcn_raw_buffer_load_b64(pb.kc, off, sk, 0);
      R.k[nt][0] = (uint32_t)u[0];
      R.k[nt][1] = (uint32_t)u[1];
    } else {
      const auto u = __builtin_amdgcn_raw_buffer_load_b128(pb.kc, off, sk, 0);
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
                                            int n_valid, int k) {
  const int ssv = (int)(tb * 2);
  if (FULL || 32 * k < n_valid) {
    R.sv[k] = __builtin_amdgcn_raw_buffer_load_b32(pb.vsc, pb.off_sv + 64 * k, ssv, 0);
    R.zv[k] = __builtin_amdgcn_raw_buffer_load_b32(pb.vze, pb.off_sv + 64 * k, ssv, 0);
  } else {
    R.sv[k] = 0u;
    R.zv[k] = 0u;
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
  for (int nt = 0; nt < 4; ++nt) load_kcodes<BITS, FULL>(R, pb, tb, n_valid, nt);
#pragma unroll
  for (int k = 0; k < 2; ++k) load_vscale<BITS, FULL>(R, pb, tb, n_valid, k);
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

// Fold the integer accumulators into the float ones (scale factor alpha).
template <int NMT>
__device__ __forceinline__ void fold_acc(WaveState<NMT>& st, int mt, float alpha) {
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const i32x4 ci = st.acc_i[mt][n];
    const float v = st.acc_f[mt][n] + (float)ci[0] + 256.f * (float)ci[1] +
                    65536.f * (float)ci[2] + 16777216.f * (float)ci[3];
    st.acc_f[mt][n] = v * alpha;
    st.acc_i[mt][n] = i32x4{0, 0, 0, 0};
  }
}

// Per-lane constants of the quantized path.
struct LaneConsts {
  float k_unscale;     // 2^-Ek
  float zk[2];         // 2^(code_shift - Ek) of the lane's channels 8lo+0..3 and 8lo+4..7
  int Ev;              // probability limbs carry p * 2^(Ev - vshift)
  int vshift;          // code_shift of the lane's token positions 2(lo%8), 2(lo%8)+1
};

// One 64-token block: group preparation, Q.K^T, online softmax, P.V.
// REFILL: each register set is reloaded with the full block at token tb_next right
// after its last use here.
template <int BITS, int GQA, int G, bool FULL, bool REFILL>
__device__ __forceinline__ void process_block(BlockRegs<BITS>& R, int n_valid,
                                              const float (&qk)[(GQA + 3) / 4][8],
                                              const LaneConsts& lc,
                                              WaveLds<(GQA + 3) / 4>& lds,
                                              WaveState<(GQA + 3) / 4>& st, int lo, int j,
                                              const PairBufs& pb, int64_t tb_next) {
  constexpr int NMT = (GQA + 3) / 4;
  constexpr int NG = BLK / G;
  const int n_groups_blk = FULL ? NG : (n_valid + G - 1) / G;

  // (1) group preparation: query limbs into LDS, and sum_c q_c z_c per head.
  // Lane (lo, j) owns channels 8lo .. 8lo+7 of head 4mt + j: operand row 4j + limb,
  // K-step (lo/2)%2, bytes 16(lo/4) + 8(lo%2) .. +7.  The four limbs of its 8 values
  // are transposed in registers (v_perm) and written as one 8-byte store per limb.
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
        float za = 0.f, zb = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float sc = h2f((unsigned short)(sw[i >> 1] >> (16 * (i & 1))));
          const float ze = h2f((unsigned short)(zw[i >> 1] >> (16 * (i & 1))));
          x[i] = limbs_biased(fmaf(qk[mt][i], sc, LIMB_BIAS));
          if (i < 4) za = fmaf(qk[mt][i], ze, za);
          else zb = fmaf(qk[mt][i], ze, zb);
        }
        qz[gi][mt] = fmaf(za, lc.zk[0], zb * lc.zk[1]);
        uint32_t t[2][4];                         // t[h][L]: limb L of values 4h .. 4h+3
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint32_t a01 = __builtin_amdgcn_perm(x[4 * hh + 1], x[4 * hh], 0x05010400u);
          const uint32_t b01 = __builtin_amdgcn_perm(x[4 * hh + 1], x[4 * hh], 0x07030602u);
          const uint32_t a23 = __builtin_amdgcn_perm(x[4 * hh + 3], x[4 * hh + 2], 0x05010400u);
          const uint32_t b23 = __builtin_amdgcn_perm(x[4 * hh + 3], x[4 * hh + 2], 0x07030602u);
          t[hh][0] = __builtin_amdgcn_perm(a23, a01, 0x05040100u);
          t[hh][1] = __builtin_amdgcn_perm(a23, a01, 0x07060302u);
          t[hh][2] = __builtin_amdgcn_perm(b23, b01, 0x05040100u);
          t[hh][3] = __builtin_amdgcn_perm(b23, b01, 0x07060302u);
        }
        uint8_t* rowp = &lds.qa[gi][mt][ksl][(4 * j) * QA_ROW + jg * 16 + 8 * (lo & 1)];
#pragma unroll
        for (int L = 0; L < 4; ++L)
          *reinterpret_cast<uint2*>(rowp + L * QA_ROW) = make_uint2(t[0][L], t[1][L]);
      }
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) qz[gi][mt] = row_sum16(qz[gi][mt]);
    }
    if constexpr (REFILL) {
      refill_point();
      load_kscale<BITS, G, true>(R, pb, tb_next, BLK, gi);
    }
  }
  wave_lds_sync();

  // (2) Q.K^T on the matrix cores: C[mt][nt] rows (head, limb), columns tokens.  The
  // query operands of a group are read once, at the group's first tile.
  i32x4 cqk[NMT][4];
  i32x4 aop[NMT][2];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) cqk[mt][nt] = i32x4{0, 0, 0, 0};
    if (FULL || 32 * (nt >> 1) < n_valid) {
      const int gi = nt * 16 / G;
      if ((nt * 16) % G == 0) {
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            aop[mt][ks] = *reinterpret_cast<const i32x4*>(&lds.qa[gi][mt][ks][lo * QA_ROW + j * 16]);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const i32x4 bop = BITS == 2 ? unpack16<BITS>(R.k[nt][ks], 0u)
                                    : unpack16<BITS>(R.k[nt][2 * ks % BlockRegs<BITS>::KW],
                                                     R.k[nt][(2 * ks + 1) % BlockRegs<BITS>::KW]);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) cqk[mt][nt] = mfma_i8(aop[mt][ks], bop, cqk[mt][nt]);
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
    sv[nt] = h2f((unsigned short)(R.sv[nt >> 1] >> (16 * (nt & 1))));
    zv[nt] = h2f((unsigned short)(R.zv[nt >> 1] >> (16 * (nt & 1))));
  }
  if constexpr (REFILL) {
    refill_point();
#pragma unroll
    for (int k = 0; k < 2; ++k) load_vscale<BITS, true>(R, pb, tb_next, BLK, k);
  }
  const float k_hi = 65536.f * lc.k_unscale;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    float z[4];
    float bm = -INFINITY;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int gi = nt * 16 / G;
      const i32x4 c = cqk[mt][nt];
      // |c_i| < 2^20, so c0 + 256 c1 fits in int32; rounding it to float stays far
      // below the resolution of the fixed-point operands
      const float lo16 = (float)(c[0] + c[1] * 256);
      const float hi16 = (float)(c[2] + c[3] * 256);
      z[nt] = fmaf(hi16, k_hi, fmaf(lo16, lc.k_unscale, qz[gi][mt]));
      if (!FULL && 32 * (nt >> 1) >= n_valid) z[nt] = -INFINITY;
      bm = fmaxf(bm, z[nt]);
    }
    bm = row_max16(bm);
    const float m_new = fmaxf(st.m_run[mt], bm);
    // The running max rose on some row: fold the integer accumulators of those rows
    // into float and rescale (a wave-uniform branch; alpha = 1 on the other rows).
    if (__builtin_amdgcn_read_exec() & __ballot(m_new > st.m_run[mt])) {
      const float alpha = __builtin_amdgcn_exp2f(st.m_run[mt] - m_new);
      fold_acc(st, mt, alpha);
      st.l_run[mt] *= alpha;
      st.pz_run[mt] *= alpha;
      st.m_run[mt] = m_new;
    }
    // p' = p * 2^(Ev - vshift): the Value operand bytes of this lane's token positions
    // carry 2^vshift.
    const float m_shift = st.m_run[mt] - (float)(lc.Ev - lc.vshift);
    uint32_t lw[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      float p = __builtin_amdgcn_exp2f(z[nt] - m_shift);
      if (!FULL && 32 * (nt >> 1) >= n_valid) p = 0.f;
      st.l_run[mt] += p;
      st.pz_run[mt] = fmaf(p, zv[nt], st.pz_run[mt]);
      lw[nt] = limbs_biased(fmaf(p, sv[nt], LIMB_BIAS));
    }
    // tokens 2lo, 2lo+1 sit at positions 2(lo%8), 2(lo%8)+1 of run lo/8; tokens
    // 32+2lo, 33+2lo at the same positions of run 2 + lo/8; row 4j + limb.
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint32_t l01 = __builtin_amdgcn_perm(lw[2 * hh + 1], lw[2 * hh], 0x05010400u);
      const uint32_t l23 = __builtin_amdgcn_perm(lw[2 * hh + 1], lw[2 * hh], 0x07030602u);
      uint8_t* dst = &lds.pa[mt][4 * j][2 * hh + (lo >> 3)][2 * (lo & 7)];
      *reinterpret_cast<uint16_t*>(dst) = (uint16_t)l01;
      *reinterpret_cast<uint16_t*>(dst + 64) = (uint16_t)(l01 >> 16);
      *reinterpret_cast<uint16_t*>(dst + 128) = (uint16_t)l23;
      *reinterpret_cast<uint16_t*>(dst + 192) = (uint16_t)(l23 >> 16);
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

// ---- the quantized blocks of one wave -----------------------------------------------

// Processes the block items handed out by the queue, starting with `item` (>= n_res),
// and writes comb[GQA][PSTRIDE] (acc with the Value-zero term folded in, m, l).  The
// fixed-point exponents come from the pair's largest Key/Value scale, so they hold for
// any block of the pair.  PAGED: the history is paged (a.L.table is set).  comb may
// overlay lds: it is written after the last block.
template <int BITS, int GQA, int G, bool PAGED>
__device__ __forceinline__ void quantized_items(const DecodeArgs& a, int64_t pair, int item, int n_res,
                                int n_items, int64_t b_lo, int64_t b_hi, WaveItems* counter,
                                WaveLds<(GQA + 3) / 4>& lds, float* comb) {
  constexpr int NMT = (GQA + 3) / 4;              // M-tiles of 4 heads x 4 limbs
  const LayerView& L = a.L;
  const int lane = threadIdx.x & 63;
  const int lo = lane & 15, j = lane >> 4;
  const int64_t b = pair / L.H, h = pair % L.H;

  constexpr int KB = D * BITS / 8;
  constexpr int VRB = kVRun * BITS / 8;             // Value code bytes per (run, channel)
  PairBufs pb;
  // the pair's history section; block loads address it with hist(t) (a paged cache
  // maps each 64-token block through the page table)
  // (the section geometry of LayerView, with PAGED known at compile time; decode has
  // G_v == d, so Value scales are one per token)
  const int64_t sec = PAGED ? pair % L.H : pair;
  const int64_t rows = PAGED ? L.pages << L.page_log2 : L.Tmax;
  const int64_t kc = rows * KB, ks = (rows / G) * D;
  pb.kc = make_rsrc(L.k_codes + sec * kc, kc);
  pb.ksc = make_rsrc(L.k_scale + sec * ks, ks * 2);
  pb.kze = make_rsrc(L.k_zero + sec * ks, ks * 2);
  pb.vc = make_rsrc(L.v_codes + sec * kc, kc);
  pb.vsc = make_rsrc(L.v_scale + sec * rows, rows * 2);
  pb.vze = make_rsrc(L.v_zero + sec * rows, rows * 2);
  // (the page entry is read once per wave and made wave-uniform: b and t are, and a
  // block base the compiler takes for a per-lane value turns every load of the loop,
  // whose offsets carry it from block to block, into a loop over distinct lane values)
  auto hist = [&](int64_t t) -> int64_t {
    if constexpr (!PAGED) {
      return t;
    } else {
      int64_t pg = __builtin_amdgcn_readfirstlane(L.table[b * L.pages_per_seq + (t >> L.page_log2)]);
      pg = pg < 0 ? 0 : pg >= L.pages ? L.pages - 1 : pg;
      return (pg << L.page_log2) + (t & ((int64_t(1) << L.page_log2) - 1));
    }
  };
  pb.off_k = 2 * lo * KB + j * (KB / 4);
  pb.off_v = j * D * VRB + 8 * lo * VRB;
  pb.off_ks = 16 * lo;
  pb.off_sv = 4 * lo;
  const __half* qp = a.q + (b * L.H * GQA + h * GQA) * D;

  // The last block of the history holds 32 tokens when T_q is not a multiple of 64.
  // In the share that contains it, it is the first block item, so the wave that takes
  // it handles it before any full block and the loop below sees full blocks only.
  const bool has_partial = (a.Tq % BLK) != 0 && b_hi == a.nblk && b_hi > b_lo;
  auto block_of = [&](int it) -> int64_t {
    if (!has_partial) return b_lo + (it - n_res);
    return it == n_res ? a.nblk - 1 : b_lo + (it - n_res - 1);
  };
  const int partial_item = has_partial ? n_res : -1;

  // The first block's loads go out before the exponent set-up so that both overlap.
  BlockRegs<BITS> R;
  if (item < n_items && item != partial_item)
    load_block<BITS, G, true>(R, pb, hist(block_of(item) * BLK), BLK, j);

  // Query values of this lane: head 4mt + j, channels 8lo .. 8lo+7.
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
  qmax = wave_max(qmax) * fabsf(a.qscale);
  const float kmax = L.scale_max[2 * pair], vmax = L.scale_max[2 * pair + 1];
  const int Ek = fixed_exponent(qmax * kmax);
  LaneConsts lc;
  lc.Ev = fixed_exponent(vmax);
  lc.k_unscale = __builtin_amdgcn_ldexpf(1.f, -Ek);
  const float v_unscale = __builtin_amdgcn_ldexpf(1.f, -lc.Ev);
  // this lane's channels 8lo + i sit at operand positions 8(lo%2) + i
  const int ksh0 = code_shift<BITS>(8 * (lo & 1)), ksh1 = code_shift<BITS>(8 * (lo & 1) + 4);
  lc.zk[0] = __builtin_amdgcn_ldexpf(1.f, ksh0 - Ek);
  lc.zk[1] = __builtin_amdgcn_ldexpf(1.f, ksh1 - Ek);
  lc.vshift = code_shift<BITS>(2 * (lo & 7));
  // scaled by sm_scale*log2(e)*2^(Ek - code_shift)
  float qk[NMT][8];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      qk[mt][i] = __builtin_amdgcn_ldexpf(qraw[mt][i] * a.qscale, Ek - (i < 4 ? ksh0 : ksh1));

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

  // Every register set is refilled with the wave's next block right after its last
  // use, so each set's loads have a whole block of work to hide behind; the item after
  // that is taken from the queue one block ahead.  Refills target the current block
  // again when there is no next full block (a cache hit whose data is not used).
  // Every 1024 blocks the integer accumulators are folded into float, which bounds
  // them by 1024 * 64 * 128 * 48 < 2^31.
  if (item == partial_item) {
    const int64_t blk = a.nblk - 1;
    const int nv = (int)(a.Tq - blk * BLK);
    load_block<BITS, G, false>(R, pb, hist(blk * BLK), nv, j);
    process_block<BITS, GQA, G, false, false>(R, nv, qk, lc, lds, st, lo, j, pb, 0);
    item = counter->next();
    if (item < n_items) load_block<BITS, G, true>(R, pb, hist(block_of(item) * BLK), BLK, j);
  }
  int nxt = item < n_items ? counter->next() : n_items;
  int done = 0;
  // Paged: the refill target of the next iteration is looked up one block ahead, with
  // a vector load issued before this block's refill loads and read after the block,
  // so that its latency hides behind the block (a scalar load would be waited for at
  // the block's first LDS wait).
  const __amdgpu_buffer_rsrc_t tbl =
      make_rsrc(PAGED ? L.table + b * L.pages_per_seq : nullptr, PAGED ? L.pages_per_seq * 4 : 0);
  int64_t tgt_next = 0;
  if constexpr (PAGED)
    if (item < n_items) tgt_next = hist((nxt < n_items ? block_of(nxt) : block_of(item)) * BLK);
  while (item < n_items) {
    const int after = nxt < n_items ? counter->next() : n_items;
    const int64_t blk = block_of(item);
    const int64_t nb = nxt < n_items ? block_of(nxt) : blk;
    int64_t tgt = nb * BLK, na = 0;
    int page_v = 0;
    if constexpr (PAGED) {
      tgt = tgt_next;
      na = (after < n_items ? block_of(after) : nb) * BLK;
      page_v = (int)__builtin_amdgcn_raw_buffer_load_b32(tbl, 0, (int)((na >> L.page_log2) * 4), 0);
    }
    process_block<BITS, GQA, G, true, true>(R, BLK, qk, lc, lds, st, lo, j, pb, tgt);
    if constexpr (PAGED) {
      int64_t pg = __builtin_amdgcn_readfirstlane(page_v);
      pg = pg < 0 ? 0 : pg >= L.pages ? L.pages - 1 : pg;
      tgt_next = (pg << L.page_log2) + (na & ((int64_t(1) << L.page_log2) - 1));
    }
    if ((++done & 1023) == 0) {
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) fold_acc(st, mt, 1.f);
    }
    item = nxt;
    nxt = after;
  }

  // Finish: fold the integer accumulators and the Value-zero term, undo 2^Ev (and the
  // lane's 2^-vshift on l and the zero term).  comb may overlay lds, which the blocks
  // read through other types: no store below may move above those reads.
  asm volatile("" ::: "memory");
  const float vsh = __builtin_amdgcn_ldexpf(1.f, lc.vshift);
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int hd = 4 * mt + j;
    const float lsum = row_sum16(st.l_run[mt] * vsh);
    const float pz = row_sum16(st.pz_run[mt] * vsh);
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

// ---- float16 window rows ------------------------------------------------------------

// Online-softmax state of one wave over window rows.  Q.K^T runs on the float16
// matrix cores (v_mfma_f32_16x16x32_f16: query heads as rows, window rows as
// columns), so lane group j = lane / 16 holds heads 4j .. 4j+3: m[i] and l[i] are those
// heads' running max and sum, equal over the 16 lanes of the group.  P.V runs on the
// VALU with every lane holding channels 2*lane, 2*lane+1 of acc for every head.
template <int GQA>
struct ResidState {
  float m[4], l[4];
  float acc[GQA][2];
};

// Query operand of the window product: lane (lo, j) holds head lo (zero past GQA),
// channels 32ks + 8j .. +7 for K-step ks.
template <int GQA>
__device__ __forceinline__ void load_q_f16(const __half* qp, f16x8 (&aq)[4]) {
  const int lane = threadIdx.x & 63, lo = lane & 15, j = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    f16x8 v = {};
    if (lo < GQA) v = *reinterpret_cast<const f16x8*>(qp + (int64_t)lo * D + 32 * ks + 8 * j);
    aq[ks] = v;
  }
}

// Residual row of float16 token i (i < a.r): the sink rows, then the window's ring.
__device__ __forceinline__ int fp16_row(const DecodeArgs& a, int i) {
  if (i < a.L.S) return i;
  const int p = i + a.ring;
  return p >= a.L.S + a.L.R ? p - a.L.R : p;
}

// Float16 tokens [c0, c0 + n_valid), n_valid <= 32.  Every Key and Value load of the
// chunk goes out before any is used (rows past the chunk re-read its last row; their
// probabilities are 0).  Row a.new_slot, when set, is read from the appended token.  Float16 products are exact in float32 (subnormal operands
// aside), accumulated in float32.
template <int GQA>
__device__ __forceinline__ void residual_rows(const DecodeArgs& a, int64_t pair, int c0,
                                              int n_valid, const f16x8 (&aq)[4], float* pw,
                                              ResidState<GQA>& rs) {
  const LayerView& L = a.L;
  const int lane = threadIdx.x & 63, lo = lane & 15, j = lane >> 4;
  const __half* kr = L.k_resid + pair * L.rs_pair();
  const __half* vr = L.v_resid + pair * L.rs_pair();
  float* palpha = pw + GQA * 32;
  // Key operands: column lo of tile nt is row 16nt + lo; lane group j holds channels
  // 32ks + 8j .. +7 of K-step ks.
  f16x8 bk[2][4];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int rr = 16 * nt + lo < n_valid ? 16 * nt + lo : n_valid - 1;
    const int pr = fp16_row(a, c0 + rr);
    const __half* row = pr == a.new_slot ? a.k_new + pair * D : kr + (int64_t)pr * D;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      bk[nt][ks] = *reinterpret_cast<const f16x8*>(row + 32 * ks + 8 * j);
  }
  // Value pairs, channels 2*lane, 2*lane+1 of the 32 rows (one descriptor: shared lane
  // offset, wave-uniform row offset in the scalar offset)
  const __amdgpu_buffer_rsrc_t vres = make_rsrc(vr, L.rs_pair() * 2);
  const __amdgpu_buffer_rsrc_t vnew = make_rsrc(a.v_new ? a.v_new + pair * D : vr, D * 2);
  __half2 vv[32];
#pragma unroll
  for (int t = 0; t < 32; ++t) {
    const int rr = t < n_valid ? t : n_valid - 1;
    const int pr = fp16_row(a, c0 + rr);
    const bool fresh = pr == a.new_slot;
    vv[t] = __builtin_bit_cast(__half2, __builtin_amdgcn_raw_buffer_load_b32(
                                            fresh ? vnew : vres, 4 * lane, fresh ? 0 : pr * D * 2, 0));
  }
  f32x4 d[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    d[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      d[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[ks], bk[nt][ks], d[nt], 0, 0, 0);
  }
  // logits of head 4j + i, rows lo and 16 + lo, in base 2
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hd = 4 * j + i;
    const float z0 = lo < n_valid ? d[0][i] * a.qscale : -INFINITY;
    const float z1 = 16 + lo < n_valid ? d[1][i] * a.qscale : -INFINITY;
    const float m_new = fmaxf(rs.m[i], row_max16(fmaxf(z0, z1)));
    const float alpha = __builtin_amdgcn_exp2f(rs.m[i] - m_new);
    const float p0 = __builtin_amdgcn_exp2f(z0 - m_new), p1 = __builtin_amdgcn_exp2f(z1 - m_new);
    rs.l[i] = rs.l[i] * alpha + row_sum16(p0 + p1);
    rs.m[i] = m_new;
    if (hd < GQA) {
      pw[hd * 32 + lo] = p0;
      pw[hd * 32 + 16 + lo] = p1;
      if (lo == 0) palpha[hd] = alpha;
    }
  }
  wave_lds_sync();
#pragma unroll
  for (int hd = 0; hd < GQA; ++hd) {
    const float al = palpha[hd];
    rs.acc[hd][0] *= al;
    rs.acc[hd][1] *= al;
  }
  // 4 rows at a time for every head, so that few probabilities are live at once
#pragma unroll
  for (int t4 = 0; t4 < 8; ++t4) {
    __builtin_amdgcn_sched_barrier(0);
    const float2 v[4] = {__half22float2(vv[4 * t4]), __half22float2(vv[4 * t4 + 1]),
                         __half22float2(vv[4 * t4 + 2]), __half22float2(vv[4 * t4 + 3])};
#pragma unroll
    for (int hd = 0; hd < GQA; ++hd) {
      const float4 p = reinterpret_cast<const float4*>(pw + hd * 32)[t4];
      const float pv[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rs.acc[hd][0] = fmaf(pv[e], v[e].x, rs.acc[hd][0]);
        rs.acc[hd][1] = fmaf(pv[e], v[e].y, rs.acc[hd][1]);
      }
      // The compiler would otherwise sink these multiply-adds below the whole loop
      // and keep every probability read live until then (4 registers per head and
      // 4 rows).
      asm volatile("" : "+v"(rs.acc[hd][0]), "+v"(rs.acc[hd][1]));
    }
  }
  wave_lds_sync();
}

template <int GQA>
__device__ __forceinline__ void residual_record(const ResidState<GQA>& rs, float* comb) {
  const int lane = threadIdx.x & 63, lo = lane & 15, j = lane >> 4;
#pragma unroll
  for (int hd = 0; hd < GQA; ++hd) {
    comb[hd * PSTRIDE + 2 * lane] = rs.acc[hd][0];
    comb[hd * PSTRIDE + 2 * lane + 1] = rs.acc[hd][1];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hd = 4 * j + i;
    if (hd < GQA && lo == 0) {
      comb[hd * PSTRIDE + D] = rs.m[i];
      comb[hd * PSTRIDE + D + 1] = rs.l[i];
    }
  }
}

// Rows [t0, t0 + 32) of the history with the per-token Value window, t0 >= a.Tq a
// multiple of 32, all below a.Tqk: Keys from their codes, Values from their codes below
// a.Tqv and from the float16 window (row S + (t mod R)) from a.Tqv on.  The dequantized
// Keys (float32, code * scale + zero with one rounding) are split into two float16
// terms hi + lo (after a 2^-4 prescale that keeps every value inside the float16
// range), so Q.K^T runs on the float16 matrix cores as in residual_rows with products
// exact in float32 and about 22 bits of each Key kept; P.V runs on the VALU.
template <int BITS, int GQA, int G>
__device__ __forceinline__ void mixed_rows(const DecodeArgs& a, int64_t pair, int64_t t0,
                                           const f16x8 (&aq)[4], float* pw,
                                           ResidState<GQA>& rs) {
  const LayerView& L = a.L;
  const int lane = threadIdx.x & 63, lo = lane & 15, j = lane >> 4;
  constexpr int KB = D * BITS / 8;                 // Key code bytes per token
  constexpr int VRB = kVRun * BITS / 8;            // Value code bytes per (run, channel)
  const uint8_t* kc = L.k_codes + pair * L.kc_pair();
  const __half* ksc = L.k_scale + pair * L.ks_pair() + (t0 / G) * D;
  const __half* kze = L.k_zero + pair * L.ks_pair() + (t0 / G) * D;
  const __half* vsc = L.v_scale + pair * L.vs_pair() + t0;   // G_v == d: one per token
  const __half* vze = L.v_zero + pair * L.vs_pair() + t0;
  const uint8_t* vc = L.v_codes + pair * L.vc_pair() + (t0 / kVRun) * (D * VRB);
  const __half* vr = L.v_resid + pair * L.rs_pair();
  float* palpha = pw + GQA * 32;
  const int nq = a.Tqv - t0 <= 0 ? 0 : a.Tqv - t0 >= 32 ? 32 : (int)(a.Tqv - t0);
  // Value inputs of the lane's channels 2*lane, 2*lane+1: the two 16-token runs' code
  // words, the 32 tokens' scales and zeros, and the float16 rows
  uint32_t vw[2][BITS == 2 ? 2 : 4];
#pragma unroll
  for (int run = 0; run < 2; ++run) {
    const uint8_t* base = vc + (int64_t)run * D * VRB + 2 * lane * VRB;
    if constexpr (BITS == 2) {
      const uint2 u = *reinterpret_cast<const uint2*>(base);
      vw[run][0] = u.x;
      vw[run][1] = u.y;
    } else {
      const uint4 u = *reinterpret_cast<const uint4*>(base);
      vw[run][0] = u.x;
      vw[run][1] = u.y;
      vw[run][2] = u.z;
      vw[run][3] = u.w;
    }
  }
  uint4 vs4[4], vz4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    vs4[i] = reinterpret_cast<const uint4*>(vsc)[i];
    vz4[i] = reinterpret_cast<const uint4*>(vze)[i];
  }
  __half2 vv[32];
#pragma unroll
  for (int t = 0; t < 32; ++t) {
    const int64_t row = L.S + (t0 + t) % L.R;
    vv[t] = reinterpret_cast<const __half2*>(vr + row * D)[lane];
  }
  // A fused step (a.vt >= 0): the Value leaving the window, token a.vt, is quantized by
  // the wave whose chunk holds it, from its float16 row (the appended token's row), with
  // the append kernel's quantizer ("4.4 KV Cache quantization" §3.2: the oldest Value
  // is quantized on its own).  Each lane rewrites its two channels' code bits in the
  // token's 16-token run; lane 0 writes the scale and zero and raises the scale maximum.
  // The wave attends with the new codes (vq) and then stores the appended token's rows
  // over that row.  No other wave of the launch reads these bytes: the run is in this
  // chunk, and the row holds no other token this launch reads.
  const int64_t tv = a.vt - t0;
  const bool leaving = a.vt >= 0 && tv >= 0 && tv < 32;
  float2 vq = make_float2(0.f, 0.f);
  if (leaving) {
    const __half2 x = reinterpret_cast<const __half2*>(vr + (int64_t)a.new_slot * D)[lane];
    float mn = fminf(__low2float(x), __high2float(x));
    float mx = fmaxf(__low2float(x), __high2float(x));
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {   // G_v == d: the group is the whole row
      mn = fminf(mn, __shfl_xor(mn, off, 64));
      mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    }
    const GroupParams gp = group_params(mn + 0.0f, mx + 0.0f, BITS);   // -0 -> +0
    const uint32_t c0 = quant_bits<BITS>(__low2half(x), gp) & 0xFFu;
    const uint32_t c1 = quant_bits<BITS>(__high2half(x), gp) & 0xFFu;
    const int e = (int)(a.vt % kVRun);
    uint32_t* w = reinterpret_cast<uint32_t*>(L.v_codes + pair * L.vc_pair() +
                                              (a.vt / kVRun) * (D * VRB));
    constexpr uint32_t mask = (1u << BITS) - 1u;
    if constexpr (BITS == 2) {
      w += 2 * lane;                                 // one word per channel
      const int pos = 8 * (e & 3) + 2 * (e >> 2);
      w[0] = (w[0] & ~(mask << pos)) | (c0 << pos);
      w[1] = (w[1] & ~(mask << pos)) | (c1 << pos);
    } else {
      w += 4 * lane + (e >> 3);                      // two words per channel
      const int pos = 8 * (e & 3) + 4 * ((e & 7) >> 2);
      w[0] = (w[0] & ~(mask << pos)) | (c0 << pos);
      w[2] = (w[2] & ~(mask << pos)) | (c1 << pos);
    }
    if (lane == 0) {
      L.v_scale[pair * L.vs_pair() + a.vt] = gp.scale;
      L.v_zero[pair * L.vs_pair() + a.vt] = gp.zero;
      __hip_atomic_fetch_max(reinterpret_cast<unsigned*>(L.scale_max + 2 * pair + 1),
                             __float_as_uint(gp.s), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the dequantized pair, as the code path below forms it (float16 scale and zero,
    // zero == mn exactly)
    vq = make_float2(fmaf((float)c0, gp.s, gp.mn), fmaf((float)c1, gp.s, gp.mn));
    // the row is read: it takes the appended token's Key and Value (the empty asm
    // orders the stores after the codes, which depend on the row's loaded values)
    asm volatile("" ::"v"(c0), "v"(c1) : "memory");
    if (lane < 2 * (D / 8)) {
      const int part = lane / (D / 8), k = lane % (D / 8);
      const __half* src = (part ? a.v_new : a.k_new) + pair * D;
      __half* dst = (part ? L.v_resid : L.k_resid) + pair * L.rs_pair() + (int64_t)a.new_slot * D;
      reinterpret_cast<uint4*>(dst)[k] = reinterpret_cast<const uint4*>(src)[k];
    }
  }
  // Q.K^T: column lo of tile nt is token t0 + 16nt + lo; lane group j holds channels
  // 32ks + 8j .. +7 of K-step ks
  f32x4 d[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const f16x8 sc = *reinterpret_cast<const f16x8*>(ksc + 32 * ks + 8 * j);
    const f16x8 ze = *reinterpret_cast<const f16x8*>(kze + 32 * ks + 8 * j);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const uint8_t* row = kc + (t0 + 16 * nt + lo) * KB;
      f16x8 hi, lw;
      if constexpr (BITS == 2) {
        // channels 32ks + 8j + m: word 2ks + j/2, code 8(j%2) + m at byte m%4, bit
        // 2((8(j%2) + m)/4)
        const uint32_t w = *reinterpret_cast<const uint32_t*>(row + 4 * (2 * ks + (j >> 1)));
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const uint32_t code = (w >> (8 * (m & 3) + 4 * (j & 1) + 2 * (m >> 2))) & 3u;
          const float x = fmaf((float)code, (float)sc[m], (float)ze[m]) * 0.0625f;
          const _Float16 h = (_Float16)x;
          hi[m] = h;
          lw[m] = (_Float16)(x - (float)h);
        }
      } else {
        // channels 32ks + 8j + m: word 4ks + j, code m at byte m%4, bit 4(m/4)
        const uint32_t w = *reinterpret_cast<const uint32_t*>(row + 4 * (4 * ks + j));
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const uint32_t code = (w >> (8 * (m & 3) + 4 * (m >> 2))) & 15u;
          const float x = fmaf((float)code, (float)sc[m], (float)ze[m]) * 0.0625f;
          const _Float16 h = (_Float16)x;
          hi[m] = h;
          lw[m] = (_Float16)(x - (float)h);
        }
      }
      d[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[ks], hi, d[nt], 0, 0, 0);
      d[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[ks], lw, d[nt], 0, 0, 0);
    }
  }
  // logits of head 4j + i, rows lo and 16 + lo, in base 2 (the 2^-4 prescale undone)
  const float zs = a.qscale * 16.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hd = 4 * j + i;
    const float z0 = d[0][i] * zs, z1 = d[1][i] * zs;
    const float m_new = fmaxf(rs.m[i], row_max16(fmaxf(z0, z1)));
    const float alpha = __builtin_amdgcn_exp2f(rs.m[i] - m_new);
    const float p0 = __builtin_amdgcn_exp2f(z0 - m_new), p1 = __builtin_amdgcn_exp2f(z1 - m_new);
    rs.l[i] = rs.l[i] * alpha + row_sum16(p0 + p1);
    rs.m[i] = m_new;
    if (hd < GQA) {
      pw[hd * 32 + lo] = p0;
      pw[hd * 32 + 16 + lo] = p1;
      if (lo == 0) palpha[hd] = alpha;
    }
  }
  wave_lds_sync();
#pragma unroll
  for (int hd = 0; hd < GQA; ++hd) {
    const float al = palpha[hd];
    rs.acc[hd][0] *= al;
    rs.acc[hd][1] *= al;
  }
  // P.V, 4 rows at a time
#pragma unroll
  for (int t4 = 0; t4 < 8; ++t4) {
    __builtin_amdgcn_sched_barrier(0);
    float2 v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 4 * t4 + e;
      if (t < nq) {
        const int run = t >> 4, q = t & 15;
        uint32_t c0, c1;
        if constexpr (BITS == 2) {
          const int pos = 8 * (q & 3) + 2 * (q >> 2);
          c0 = (vw[run][0] >> pos) & 3u;
          c1 = (vw[run][1] >> pos) & 3u;
        } else {
          const int pos = 8 * (q & 3) + 4 * ((q & 7) >> 2);
          c0 = (vw[run][q >> 3] >> pos) & 15u;
          c1 = (vw[run][2 + (q >> 3)] >> pos) & 15u;
        }
        const uint32_t sw = reinterpret_cast<const uint32_t*>(&vs4[t >> 3])[(t & 7) >> 1];
        const uint32_t zw = reinterpret_cast<const uint32_t*>(&vz4[t >> 3])[(t & 7) >> 1];
        const float sv = h2f((unsigned short)(sw >> (16 * (t & 1))));
        const float zv = h2f((unsigned short)(zw >> (16 * (t & 1))));
        v[e] = make_float2(fmaf((float)c0, sv, zv), fmaf((float)c1, sv, zv));
        if (leaving && t == tv) v[e] = vq;
      } else {
        v[e] = __half22float2(vv[t]);
      }
    }
#pragma unroll
    for (int hd = 0; hd < GQA; ++hd) {
      const float4 p = reinterpret_cast<const float4*>(pw + hd * 32)[t4];
      const float pv[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rs.acc[hd][0] = fmaf(pv[e], v[e].x, rs.acc[hd][0]);
        rs.acc[hd][1] = fmaf(pv[e], v[e].y, rs.acc[hd][1]);
      }
      asm volatile("" : "+v"(rs.acc[hd][0]), "+v"(rs.acc[hd][1]));
    }
  }
  wave_lds_sync();
}

// ---- the kernel ---------------------------------------------------------------------

// One workgroup per CU holding every wave the register budget allows there: WAVES =
// 4 SIMDs x waves_per_simd.  Workgroup 0 of a pair takes the float16 window, whose
// 32-row chunks count RES_COST blocks each (a chunk moves three blocks' bytes with fewer
// loads in flight and takes about three blocks of wave time), and the blocks that fill
// its fair share of the pair's work; workgroups 1 .. nw-1 split the remaining 64-token
// blocks evenly into contiguous shares.  Inside a workgroup, waves take window chunks,
// then blocks, from an LDS counter.  The last workgroup of the pair to arrive merges
// the partials.
__device__ __forceinline__ void block_share(int64_t nblk, int n_res, int nw, int s,
                                            int64_t& b_lo, int64_t& b_hi) {
  const int64_t fair = (nblk + (int64_t)RES_COST * n_res) / nw;
  int64_t b0 = nw == 1 ? nblk : fair - (int64_t)RES_COST * n_res;
  b0 = b0 < 0 ? 0 : b0 > nblk ? nblk : b0;
  if (s == 0) {
    b_lo = 0;
    b_hi = b0;
  } else {
    const int64_t rest = nblk - b0;
    b_lo = b0 + rest * (s - 1) / (nw - 1);
    b_hi = b0 + rest * s / (nw - 1);
  }
}
// PAGED: a paged cache (args.L.table set); its own instantiation, so that the block
// loop of a contiguous cache carries no page-table lookup.  VWIN: the per-token Value
// window (contiguous caches only); its own instantiation too, so that the mixed chunks'
// code and registers stay out of the other kernels.
template <int BITS, int GQA, int G, bool PAGED, bool VWIN>
__global__ __launch_bounds__(256 * waves_per_simd(BITS, GQA, G), 1) void decode_kernel(DecodeArgs args) {
  constexpr int NMT = (GQA + 3) / 4;
  constexpr int WAVES = 4 * waves_per_simd(BITS, GQA, G);
  constexpr int NTH = 64 * WAVES;
  // A wave's record of its blocks is written over its own WaveLds after its last block.
  __shared__ WaveLds<NMT> wl[WAVES];
  static_assert(sizeof(WaveLds<NMT>) >= GQA * PSTRIDE * sizeof(float), "block record in WaveLds");
  __shared__ alignas(16) float pw[WAVES][GQA * 32 + 4 * ((GQA + 3) / 4)];  // window probabilities
  __shared__ alignas(16) float comb[WAVES][GQA * PSTRIDE];      // window records
  __shared__ int counter;

  // workgroup -> (pair, s): uniform T: the nw workgroups of a pair are consecutive, so
  // the hardware's round-robin placement of workgroups on the 8 XCDs spreads each pair
  // over several of them (measured ~2% faster than keeping a pair on one XCD: the XCDs
  // stream at different rates); a ragged batch: ragged_assign
  tl_stamp(args.tl_slot, 0);
  int64_t pair = blockIdx.x / args.nw, slot0;
  int s = (int)(blockIdx.x % args.nw);
  DecodeArgs a = args;
  if (a.lens.p) {
    RaggedSlot rsl;
    if (!ragged_assign(a, rsl)) return;
    pair = rsl.pair;
    s = rsl.s;
    a.nw = rsl.nw;
    slot0 = rsl.slot0;
  } else {
    slot0 = pair * a.nw;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t b = pair / a.L.H, h = pair % a.L.H;
  if (a.lens.p) ragged_split(a, b);

  // this workgroup's share: window chunks (workgroup 0 only; first the mixed chunks of
  // the per-token Value window, if any), then blocks
  const int n_res_all = a.n_mix + (a.r + 31) / 32;
  int64_t b_lo, b_hi;
  block_share(a.nblk, n_res_all, a.nw, s, b_lo, b_hi);
  const int n_res = s == 0 ? n_res_all : 0;
  const int n_items = n_res + (int)(b_hi - b_lo);

  if (threadIdx.x == 0) counter = 0;
  // An appended token: workgroup 0 of the pair stores its rows into the window (read
  // by the next call; this one takes them from k_new / v_new).
  // (A fused step of the per-token Value window stores them in mixed_rows, after the
  // leaving Value has been read from that row.)
  if (a.new_slot >= 0 && !(VWIN && a.vt >= 0) && s == 0 && threadIdx.x < 2 * (D / 8)) {
    const int part = threadIdx.x / (D / 8), k = threadIdx.x % (D / 8);
    const __half* src = (part ? a.v_new : a.k_new) + pair * D;
    __half* dst = (part ? a.L.v_resid : a.L.k_resid) + pair * a.L.rs_pair() + (int64_t)a.new_slot * D;
    reinterpret_cast<uint4*>(dst)[k] = reinterpret_cast<const uint4*>(src)[k];
  }
  // Clear this workgroup's partial slot (each thread the words it stores at the end).
  const int n_parts = a.nw;
  const int64_t pair_floats = (int64_t)n_parts * GQA * PSTRIDE;
  const __amdgpu_buffer_rsrc_t parts =
      make_rsrc(a.part + slot0 * GQA * PSTRIDE, pair_floats * 4);
  const int my = s * GQA * PSTRIDE * 4;
  if (n_parts > 1) clear_partial<GQA, NTH>(parts, my);
  __syncthreads();

  // window chunks
  WaveItems witems(a.L.det ? nullptr : &counter, wave, WAVES, n_res, (int)(b_hi - b_lo));
  int item = witems.next();
  {
    ResidState<GQA> rs;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rs.m[i] = -INFINITY;
      rs.l[i] = 0.f;
    }
#pragma unroll
    for (int hd = 0; hd < GQA; ++hd) rs.acc[hd][0] = rs.acc[hd][1] = 0.f;
    if (item < n_res) {
      f16x8 aq[4];
      load_q_f16<GQA>(a.q + (b * a.L.H * GQA + h * GQA) * D, aq);
      while (item < n_res) {
        if (VWIN && item < a.n_mix) {
          if constexpr (VWIN)
            mixed_rows<BITS, GQA, G>(a, pair, a.Tq + 32 * (int64_t)item, aq, pw[wave], rs);
        } else {
          const int c0 = 32 * (item - a.n_mix);
          residual_rows<GQA>(a, pair, c0, a.r - c0 < 32 ? a.r - c0 : 32, aq, pw[wave], rs);
        }
        item = witems.next();
      }
    }
    residual_record<GQA>(rs, comb[wave]);
  }
  // blocks (an empty share leaves an empty record: m = -inf, l = 0)
  quantized_items<BITS, GQA, G, PAGED>(a, pair, item, n_res, n_items, b_lo, b_hi, &witems,
                                       wl[wave], reinterpret_cast<float*>(&wl[wave]));
  __syncthreads();
  tl_stamp(a.tl_slot, 1);

  float* o = a.out + (b * a.L.H * GQA + h * GQA) * D;
  finish_pair<GQA, NTH, 2 * WAVES>(
      [&](int i) {
        return i < WAVES ? reinterpret_cast<const float*>(&wl[i]) : (const float*)comb[i - WAVES];
      },
      parts, my, n_parts, a.counters + kCounterStride * pair, o, &comb[0][0], a.tl_slot);
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
  const TokenSplit ts = split_tokens(L, T);
  const int64_t Tq = ts.Tq;
  p.r = (int)ts.fp16_rows();          // sink rows and window tokens
  p.ring = ts.ring;
  p.n_groups = Tq / L.G;
  // with the per-token Value window the blocks stop at 64 * floor(Tqv / 64) and 32-row
  // mixed chunks cover the rest of the Key history
  const int64_t tblk = L.vwin ? ts.Tqv / BLK * BLK : Tq;
  p.tq_blocks = tblk;
  p.n_mix = (int)((Tq - tblk) / 32);
  const int64_t nblk = (tblk + BLK - 1) / BLK;
  const int64_t pairs = (int64_t)L.B * L.H;
  // default: one round of CU-sized workgroups over the 256 CUs, but no more workgroups
  // per pair than keep every wave busy with a block or window chunk (a chunk counting
  // RES_COST blocks): a small pair is cheaper in one workgroup than merged from
  // several.  At most one workgroup for the window and one per block.
  // The workspace holds partials for the count without that limit, which grows with T,
  // so a workspace sized for T serves every smaller T (the limited count does not: a
  // flush trades many window rows for a few blocks).
  int64_t room = n_split_req > 0 ? n_split_req : device_cus() / pairs;
  if (room > 1 + nblk) room = 1 + nblk;
  if (room < 1) room = 1;
  int64_t nw = room;
  if (n_split_req <= 0) {
    const int64_t waves = 4 * waves_per_simd(L.bits, gqa, L.G);
    const int64_t items = nblk + (int64_t)RES_COST * (p.n_mix + (p.r + 31) / 32);
    const int64_t busy = (items + waves - 1) / waves;
    if (nw > busy) nw = busy;
  }
  if (nw < 1) nw = 1;
  p.n_split = (int)nw;
  p.ws_counters = (size_t)pairs * kCounterStride * sizeof(uint32_t);
  p.ws_partials = room > 1 ? (size_t)pairs * room * gqa * PSTRIDE * sizeof(float) : 0;
  p.ws_partials = (p.ws_partials + 255) / 256 * 256;
  p.ws_total = p.ws_counters + p.ws_partials;
  return p;
}

hipError_t launch_decode(const LayerView& L, int q_heads, int64_t T, const __half* q,
                         float sm_scale, float* out, void* ws, const DecodePlan& plan,
                         const NewRow* new_row, Lens lens, hipStream_t s) {
  const int gqa = q_heads / L.H;
  DecodeArgs a;
  a.L = L;
  a.q = q;
  a.out = out;
  a.counters = reinterpret_cast<unsigned*>(ws);
  a.part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + plan.ws_counters);
  const TokenSplit ts = split_tokens(L, T);
  a.Tq = plan.tq_blocks;
  a.nblk = (a.Tq + BLK - 1) / BLK;
  a.Tqk = ts.Tq;
  a.Tqv = ts.Tqv;
  a.n_mix = plan.n_mix;
  a.r = plan.r;
  a.ring = plan.ring;
  a.nw = plan.n_split;
  a.qscale = sm_scale * 1.4426950408889634f;
  a.k_new = new_row ? new_row->k : nullptr;
  a.v_new = new_row ? new_row->v : nullptr;
  a.new_slot = new_row ? new_row->slot : -1;
  a.vt = new_row ? new_row->vt : -1;
#ifdef KIVI_TIMELINE
  static int tl_launches = 0;                      // launch i stamps slot i mod kTlSlots
  a.tl_slot = tl_launches++ % kTlSlots;
#else
  a.tl_slot = -1;
#endif
  a.lens = lens;
  const int64_t P = (int64_t)L.B * L.H;
  const dim3 grid((unsigned)(P * plan.n_split));
  bool ok = dispatch_decode(L.bits, gqa, L.G, [&](auto b, auto g, auto gg) {
    constexpr int B_ = decltype(b)::value, Q_ = decltype(g)::value, G_ = decltype(gg)::value;
    if (L.table)
      launch_decode_kernel(decode_kernel<B_, Q_, G_, true, false>, grid,
                           dim3(256 * waves_per_simd(B_, Q_, G_)), s, a);
    else if (L.vwin)
      launch_decode_kernel(decode_kernel<B_, Q_, G_, false, true>, grid,
                           dim3(256 * waves_per_simd(B_, Q_, G_)), s, a);
    else
      launch_decode_kernel(decode_kernel<B_, Q_, G_, false, false>, grid,
                           dim3(256 * waves_per_simd(B_, Q_, G_)), s, a);
    return true;
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kivi

#ifdef KIVI_TIMELINE
// Measurement build only: the stamps of the last kTlSlots launches, slot-major:
// [slot][workgroup < kTlWgs][mark < kTlMarks][real-time counter, shader clock counter].
extern "C" int kivi_timeline_read(void* host, size_t bytes) {
  const size_t need = sizeof(kivi::g_timeline);
  if (bytes < need) return 1;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(kivi::g_timeline), need) == hipSuccess ? 0 : 2;
}
extern "C" int kivi_timeline_geometry(int* slots, int* wgs, int* marks) {
  *slots = kivi::kTlSlots;
  *wgs = kivi::kTlWgs;
  *marks = kivi::kTlMarks;
  return 0;
}
#endif
