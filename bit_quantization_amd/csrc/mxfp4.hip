// MXFP4 KV codec: coding float16 Keys and Values as OCP MX blocks (32 four-bit E2M1
// elements sharing one power-of-two E8M0 scale), and decode attention over them.
//
// "KV Cache Quantization (KIVI & FP4)" §4, "Hardware Micro-Scaling": four-bit E2M1
// numbers (1 sign, 2 exponent, 1 mantissa bit) in blocks that share an 8-bit scale.
// The format is the OCP MX one the page names: blocks of 32 with scale X = 2^s,
// s = floor(log2 max|x|) - 2 (2 is E2M1's largest exponent), each element the E2M1
// value nearest to x / X, ties to the even code, saturating at 6, sign kept.  Blocks
// run along the channels of each token, so a token is coded on its own on arrival.
//
// Layout per (sequence, KV head): Key codes [T][64] bytes (channel 2i low nibble of
// byte i), Key scales [T][4]; Value codes in 32-token runs [T/32][128][16] bytes, run
// position p (nibble p & 1 of byte p / 2) holding token order[p] with the FP8 codec's
// order 0-3, 16-19, 4-7, 20-23, ...; Value scales [T/32][4][32] in the same order.
//
// Decode follows the FP8 kernel (S^T = K q^T and O^T = V^T P^T on the float16 matrix
// cores, probabilities kept in registers).  The E2M1 values widen to float16 exactly;
// a Key lane's 32 channels are one MX block of one token, so its scale is applied by
// the widening itself (v_cvt_scalef32_pk_f16_fp4); a Value lane holds 8 tokens of one
// channel, each with its own scale, applied by a packed float16 multiply (v_ldexp_f16
// when a scale is below float16's normal range).  Both are exact while
// the scaled value is a float16 number: always for the largest values of a block
// (s <= 13 for float16 inputs), and the values that fall below float16's range belong
// to blocks whose largest magnitude is under 2^-20.
#include <type_traits>

#include "decode_common.h"

namespace kivi {
namespace {

constexpr int kMxBlock = 32;       // elements per MX block
constexpr int kMxRun = 32;         // tokens per Value run
constexpr int kKRow = D / 2;       // Key code bytes per token
constexpr int kNBlk = D / kMxBlock;

// Position of token t of a 32-token run (inverse of 0-3, 16-19, 4-7, 20-23, ...).
__host__ __device__ __forceinline__ int mx_run_pos(int t) {
  return 8 * ((t & 15) >> 2) + 4 * (t >> 4) + (t & 3);
}

// s of a block from its largest magnitude (float32, from float16 values): the
// exponent of amax minus 2; a block of zeros gets -127.
__device__ __forceinline__ int mx_block_exponent(float amax) {
  if (!(amax > 0.f)) return -127;
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127;   // amax is normal
  const int s = e - 2;
  return s < -127 ? -127 : s > 127 ? 127 : s;
}

// E2M1 code of x / 2^s: with y = |x| 2^-s (exact) and its exponent clamped to
// [0, 2], the code is ((e + 1) << 1) + rint(y 2^(1 - e)) - 2: rint rounds half to
// even, a mantissa that rounds up carries into the exponent, below 1 the same formula
// gives the subnormal codes; codes past 7 (6.0) saturate.
__device__ __forceinline__ uint32_t e2m1_code(float x, int s) {
  const uint32_t sign = (__float_as_uint(x) >> 28) & 8u;
  const float y = __builtin_amdgcn_ldexpf(fabsf(x), -s);
  int e = (int)((__float_as_uint(y) >> 23) & 0xFF) - 127;
  e = e < 0 ? 0 : e > 2 ? 2 : e;
  const int r = (int)rintf(__builtin_amdgcn_ldexpf(y, 1 - e));
  const int code = ((e + 1) << 1) + r - 2;
  return sign | (uint32_t)(code > 7 ? 7 : code);
}

// ---- coding ---------------------------------------------------------------------------

// grid = (ceil(T / 32), B*H), 256 threads: one 32-token run of one (sequence, KV head).
// Thread (token tt, channels cc .. cc+15) codes half an MX block of its Key and Value
// row (the block's largest magnitude comes from the neighbouring thread); Key codes go
// straight to the row, Value codes to an LDS image of the run (one byte per code),
// packed into nibbles and written out whole (codes and scales of tokens >= T are 0).
__global__ __launch_bounds__(256) void mx_quantize_kernel(MxView L, const __half* __restrict__ k,
                                                          const __half* __restrict__ v,
                                                          int64_t ld, int64_t T) {
  __shared__ alignas(16) uint8_t vcode[D][kMxRun];      // [channel][run position]
  __shared__ alignas(16) uint8_t vscale[kNBlk][kMxRun];
  const int64_t pair = blockIdx.y;
  const int64_t run = blockIdx.x;
  const int tt = threadIdx.x >> 3, cc = (threadIdx.x & 7) * 16;
  const int64_t t = run * kMxRun + tt;
  reinterpret_cast<uint4*>(&vcode[0][0])[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
  if (threadIdx.x < 8) reinterpret_cast<uint4*>(&vscale[0][0])[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  const bool live = t < T;                               // uniform over each pair of threads
  float kx[16], vx[16];
  float kmax = 0.f, vmax = 0.f;
  if (live) {
    const uint4* kr = reinterpret_cast<const uint4*>(k + (pair * ld + t) * D + cc);
    const uint4* vr = reinterpret_cast<const uint4*>(v + (pair * ld + t) * D + cc);
    const uint4 kw[2] = {kr[0], kr[1]}, vw[2] = {vr[0], vr[1]};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t kword = (&kw[i / 8].x)[(i % 8) / 2], vword = (&vw[i / 8].x)[(i % 8) / 2];
      kx[i] = __half2float(__ushort_as_half((unsigned short)(kword >> (16 * (i & 1)))));
      vx[i] = __half2float(__ushort_as_half((unsigned short)(vword >> (16 * (i & 1)))));
      kmax = fmaxf(kmax, fabsf(kx[i]));
      vmax = fmaxf(vmax, fabsf(vx[i]));
    }
  }
  kmax = fmaxf(kmax, __shfl_xor(kmax, 1, 64));
  vmax = fmaxf(vmax, __shfl_xor(vmax, 1, 64));
  if (live) {
    const int sk = mx_block_exponent(kmax), sv = mx_block_exponent(vmax);
    const int p = mx_run_pos(tt);
    uint32_t kc[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      kc[i / 8] |= e2m1_code(kx[i], sk) << (4 * (i % 8));
      vcode[cc + i][p] = (uint8_t)e2m1_code(vx[i], sv);
    }
    *reinterpret_cast<uint2*>(L.k + pair * L.k_pair() + t * kKRow + cc / 2) = make_uint2(kc[0], kc[1]);
    if ((cc & 16) == 0) {
      L.k_scale[pair * L.ks_pair() + t * kNBlk + cc / kMxBlock] = (uint8_t)(sk + 127);
      vscale[cc / kMxBlock][p] = (uint8_t)(sv + 127);
    }
  }
  __syncthreads();
  // thread i packs channel i / 2, run positions 16 (i % 2) .. +15 into 8 bytes
  {
    const int c = threadIdx.x >> 1, h = threadIdx.x & 1;
    const uint4 b4 = *reinterpret_cast<const uint4*>(&vcode[c][16 * h]);
    const uint32_t w[4] = {b4.x, b4.y, b4.z, b4.w};
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint32_t code = (w[q / 4] >> (8 * (q % 4))) & 15u;
      packed[q / 8] |= code << (4 * (q % 8));
    }
    *reinterpret_cast<uint2*>(L.v + pair * L.v_pair() + run * D * (kMxRun / 2) + c * (kMxRun / 2) +
                              8 * h) = make_uint2(packed[0], packed[1]);
  }
  if (threadIdx.x < 32)
    reinterpret_cast<uint32_t*>(L.v_scale + pair * L.vs_pair() + run * kNBlk * kMxRun)[threadIdx.x] =
        reinterpret_cast<const uint32_t*>(&vscale[0][0])[threadIdx.x];
}

// Token t of one (sequence, KV head), coded by one wave: lane l codes channels 2l, 2l+1
// (16 lanes per MX block).  The Value nibbles are merged into their bytes, whose other
// nibble belongs to the run's neighbouring position.
__device__ __forceinline__ void mx_code_token(const MxView& L, int64_t pair,
                                              const __half* __restrict__ kn,
                                              const __half* __restrict__ vn, int64_t t) {
  const int lane = threadIdx.x & 63;
  const __half2 k2 = reinterpret_cast<const __half2*>(kn + pair * D)[lane];
  const __half2 v2 = reinterpret_cast<const __half2*>(vn + pair * D)[lane];
  const float k0 = __low2float(k2), k1 = __high2float(k2);
  const float v0 = __low2float(v2), v1 = __high2float(v2);
  float kmax = fmaxf(fabsf(k0), fabsf(k1)), vmax = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    kmax = fmaxf(kmax, __shfl_xor(kmax, o, 64));
    vmax = fmaxf(vmax, __shfl_xor(vmax, o, 64));
  }
  const int sk = mx_block_exponent(kmax), sv = mx_block_exponent(vmax);
  L.k[pair * L.k_pair() + t * kKRow + lane] = (uint8_t)(e2m1_code(k0, sk) | (e2m1_code(k1, sk) << 4));
  const int64_t run = t / kMxRun;
  const int p = mx_run_pos((int)(t % kMxRun));
  uint8_t* vrun = L.v + pair * L.v_pair() + run * D * (kMxRun / 2) + p / 2;
  const int shift = 4 * (p & 1);
  const uint32_t keep = 0xF0u >> shift;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    uint8_t* byte = vrun + (2 * lane + i) * (kMxRun / 2);
    const uint32_t code = e2m1_code(i ? v1 : v0, sv);
    *byte = (uint8_t)((*byte & keep) | (code << shift));
  }
  if ((lane & 15) == 0) {
    L.k_scale[pair * L.ks_pair() + t * kNBlk + lane / 16] = (uint8_t)(sk + 127);
    L.v_scale[pair * L.vs_pair() + run * kNBlk * kMxRun + (lane / 16) * kMxRun + p] = (uint8_t)(sv + 127);
  }
}

// grid = B*H, 64 threads: token t of each (sequence, KV head).
__global__ __launch_bounds__(64) void mx_append_kernel(MxView L, const __half* __restrict__ kn,
                                                       const __half* __restrict__ vn, int64_t t) {
  mx_code_token(L, blockIdx.x, kn, vn, t);
}

// ---- decode ---------------------------------------------------------------------------

struct MxDecodeArgs {
  MxView L;
  const __half* q;
  float* out;
  float* part;          // [P][nw][GQA][PSTRIDE]
  unsigned* counters;   // [P][kCounterStride]
  int64_t T;
  int64_t nblk;         // 32-token runs per pair
  int nw;               // workgroups per pair
  float qscale;         // sm_scale * log2(e)
  const __half* k_new;  // [P][D]: token new_t is coded by this launch (new_t >= 0)
  const __half* v_new;
  int64_t new_t;
};

constexpr int kMxWavesPerSimd = 4;

// The loads of one 32-token run of one lane.
struct MxRun {
  u32x4 kw[2];          // Key codes: tile nt, token t0 + 16nt + lo, MX block j (16 bytes)
  uint32_t ksc[2];      // that token's 4 Key scale codes
  uint32_t vw[8];       // Value codes: channel 16mt + lo, run positions 8j .. 8j+7
  u32x2 vsc[kNBlk];     // Value scale codes of positions 8j .. 8j+7, per MX block
};

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Four code bytes (8 E2M1 values) -> 8 float16, each times 2^(scale_code - 127).
__device__ __forceinline__ f16x8 widen8_scaled(uint32_t w, float scale) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 0);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 1);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 2);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 3);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// The scales 2^s of two Value positions as a float16 pair, from a word holding their
// E8M0 codes in bytes b and b + 1 (b = 0 or 2): the fields code - 112 shifted into the
// exponent bits.  Valid for codes 113 .. 142 (s in [-14, 15], the float16-normal
// powers of two); float16 inputs give codes of at most 140 (s <= 13).
template <int B>
__device__ __forceinline__ f16x2 pow2_pair(uint32_t codes) {
  const uint32_t spread = __builtin_amdgcn_perm(0u, codes, B == 0 ? 0x0C010C00u : 0x0C030C02u);
  return __builtin_bit_cast(f16x2, (spread - 0x00700070u) << 10);
}

// Online softmax, one head per lane group.  The reference maximum m of a head moves
// only when a run's maximum exceeds it by more than kLazyLog2 (base-2 units), so
// probabilities stay below 2^kLazyLog2 and the rescale of l and the accumulators runs
// on a few runs only (in a branch of its own: the empty asm keeps the compiler from
// flattening it into selects on every run).
// (m, l, acc) stay consistent for any reference, which is all the merge assumes.
constexpr float kLazyLog2 = 8.f;
__device__ __forceinline__ void lazy_rescale(float& m, float& l, f32x4 (&acc)[8], float mx) {
  const bool up = mx > m + kLazyLog2;
  if (__builtin_amdgcn_ballot_w64(up) != 0) {
    asm volatile("" ::: "memory");
    const float m_new = up ? mx : m;
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[mt] = acc[mt] * alpha;
  }
}
// p = 2^(z - m) for 8 logits as a float16 hi + lo pair per value (hi rounded toward
// zero, lo the float16 of the exact float32 remainder: 22 significant bits in all);
// returns the float32 sum of the p.
__device__ __forceinline__ float split_probabilities(const float (&z)[8], float m, f16x8& ph,
                                                     f16x8& pl) {
  float psum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const float p0 = __builtin_amdgcn_exp2f(z[e] - m), p1 = __builtin_amdgcn_exp2f(z[e + 1] - m);
    psum += p0 + p1;
    const auto hi = __builtin_amdgcn_cvt_pkrtz(p0, p1);
    const auto lo = __builtin_amdgcn_cvt_pkrtz(p0 - (float)hi[0], p1 - (float)hi[1]);
    ph[e] = hi[0];
    ph[e + 1] = hi[1];
    pl[e] = lo[0];
    pl[e + 1] = lo[1];
  }
  return psum;
}
// Token of the run that k-slot e (0..7) of lane group j supplies to P.V.
__device__ __forceinline__ int mx_slot_token(int j, int e) { return 4 * j + (e & 3) + 16 * (e >> 2); }

// One workgroup per CU; workgroup s of a pair takes runs [nblk*s/nw, nblk*(s+1)/nw),
// its waves take them from an LDS counter; each wave keeps an online softmax per head
// as the FP8 kernel does.
template <int GQA>
__global__ __launch_bounds__(256 * kMxWavesPerSimd, 1) void mx_decode_kernel(MxDecodeArgs a) {
  constexpr int WAVES = 4 * kMxWavesPerSimd;
  constexpr int NTH = 64 * WAVES;
  __shared__ alignas(16) float comb[WAVES][GQA * PSTRIDE];
  __shared__ int counter;

  const MxView& L = a.L;
  const int64_t P = (int64_t)L.B * L.H;
  const int64_t pair = blockIdx.x % P;
  const int s = (int)(blockIdx.x / P);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, lo = lane & 15, j = lane >> 4;
  const int64_t b = pair / L.H;
  const int h = (int)(pair % L.H);
  const int64_t b_lo = a.nblk * s / a.nw, b_hi = a.nblk * (s + 1) / a.nw;

  if (threadIdx.x == 0) counter = 0;
  // An appended token: its run is the pair's last, which only the last workgroup
  // reads; one of its waves codes the token before the barrier below.
  if (a.new_t >= 0 && s == a.nw - 1 && wave == 0) mx_code_token(L, pair, a.k_new, a.v_new, a.new_t);
  const int n_parts = a.nw;
  const int64_t pair_floats = (int64_t)n_parts * GQA * PSTRIDE;
  const __amdgpu_buffer_rsrc_t parts = make_rsrc(a.part + pair * pair_floats, pair_floats * 4);
  const int my = s * GQA * PSTRIDE * 4;
  if (n_parts > 1) clear_partial<GQA, NTH>(parts, my);
  __syncthreads();

  // q^T operand: lane (head lo, j) holds channels 32j + 8ks .. +7 for K-step ks, so lane
  // group j's K-steps cover MX block j
  f16x8 bq[4];
  const __half* qp = a.q + ((b * L.H + h) * GQA) * D;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    f16x8 v = {};
    if (lo < GQA) v = *reinterpret_cast<const f16x8*>(qp + lo * D + 32 * j + 8 * ks);
    bq[ks] = v;
  }
  const __amdgpu_buffer_rsrc_t kres = make_rsrc(L.k + pair * L.k_pair(), L.k_pair());
  const __amdgpu_buffer_rsrc_t ksres = make_rsrc(L.k_scale + pair * L.ks_pair(), L.ks_pair());
  const __amdgpu_buffer_rsrc_t vres = make_rsrc(L.v + pair * L.v_pair(), L.v_pair());
  const __amdgpu_buffer_rsrc_t vsres = make_rsrc(L.v_scale + pair * L.vs_pair(), L.vs_pair());

  float m = -INFINITY, l = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_run = [&](int64_t blk, MxRun& R) {
    const int64_t t0 = blk * kMxRun;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int64_t tok = t0 + 16 * nt + lo;
      R.kw[nt] = __builtin_amdgcn_raw_buffer_load_b128(kres, (int)(tok * kKRow + 16 * j), 0, 0);
      R.ksc[nt] = __builtin_amdgcn_raw_buffer_load_b32(ksres, (int)(tok * kNBlk), 0, 0);
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
      R.vw[mt] = __builtin_amdgcn_raw_buffer_load_b32(
          vres, (int)(blk * D * (kMxRun / 2) + (16 * mt + lo) * (kMxRun / 2) + 4 * j), 0, 0);
#pragma unroll
    for (int q = 0; q < kNBlk; ++q)
      R.vsc[q] = __builtin_amdgcn_raw_buffer_load_b64(
          vsres, (int)(blk * kNBlk * kMxRun + q * kMxRun + 8 * j), 0, 0);
  };
  // (Loading the next run before computing this one, at three waves per SIMD for the
  // registers, measured slower: 84.6 against 77.1 us per 32k step.)
  for (int item = grab_item(&counter); b_lo + item < b_hi; item = grab_item(&counter)) {
    const int64_t blk = b_lo + item;
    const int64_t t0 = blk * kMxRun;
    MxRun cur;
    load_run(blk, cur);
    const u32x4* kw = cur.kw;
    const uint32_t* ksc = cur.ksc;
    const uint32_t* vw = cur.vw;
    const u32x2* vsc = cur.vsc;

    // S^T = K q^T for the two 16-token tiles
    f32x4 d[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int sc = (int)((ksc[nt] >> (8 * j)) & 0xFF) - 127;
      const float kscale = __builtin_amdgcn_ldexpf(1.f, sc);
      d[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f16x8 kf = widen8_scaled(kw[nt][ks], kscale);
        d[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, bq[ks], d[nt], 0, 0, 0);
      }
    }
    // logits of head lo, tokens mx_slot_token(j, e), base 2; positions past T (the
    // pair's last run only) are masked in a branch of its own, so that full runs carry
    // no selects (the empty asm keeps the compiler from flattening it)
    float z[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = d[e >> 2][e & 3] * a.qscale;
    if (t0 + kMxRun > a.T) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (t0 + mx_slot_token(j, e) >= a.T) z[e] = -INFINITY;
    }
    float mx = z[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, z[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    lazy_rescale(m, l, acc, mx);
    f16x8 ph, pl;
    const float psum = split_probabilities(z, m, ph, pl);
    l += psum;
    // O^T += V^T P^T for the eight 16-channel tiles; a Value's scale is its token's
    // (positions past T hold code 0 and scale code 0: value 0).  Scale codes of 113 or
    // more (s >= -14, every block whose largest magnitude is 2^-12 or more) become
    // float16 pairs, one set per MX block, multiplied in packed form; a run with a
    // smaller one anywhere in the wave scales each value with v_ldexp_f16 instead
    // (exact down to float16's subnormals), in a branch of its own.
    bool fast = true;
#pragma unroll
    for (int q = 0; q < kNBlk; ++q)
      fast &= (((vsc[q][0] + 0x0F0F0F0Fu) & (vsc[q][1] + 0x0F0F0F0Fu) & 0x80808080u) == 0x80808080u);
    const bool all_fast = __builtin_amdgcn_ballot_w64(!fast) == 0;
#pragma unroll
    for (int q = 0; q < kNBlk; ++q) {
      if (all_fast) {
        const f16x2 s0 = pow2_pair<0>(vsc[q][0]), s1 = pow2_pair<2>(vsc[q][0]);
        const f16x2 s2 = pow2_pair<0>(vsc[q][1]), s3 = pow2_pair<2>(vsc[q][1]);
#pragma unroll
        for (int mt = 2 * q; mt < 2 * q + 2; ++mt) {
          const f16x8 vf = widen8_scaled(vw[mt], 1.f);
          const f16x2 v0 = f16x2{vf[0], vf[1]} * s0, v1 = f16x2{vf[2], vf[3]} * s1;
          const f16x2 v2 = f16x2{vf[4], vf[5]} * s2, v3 = f16x2{vf[6], vf[7]} * s3;
          const f16x8 vs = f16x8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vs, ph, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vs, pl, acc[mt], 0, 0, 0);
        }
      } else {
        // the scale words are made opaque here, so that their per-value extraction
        // stays in this branch
        u32x2 sw = vsc[q];
        asm volatile("" : "+v"(sw[0]), "+v"(sw[1]));
#pragma unroll
        for (int mt = 2 * q; mt < 2 * q + 2; ++mt) {
          f16x8 vf = widen8_scaled(vw[mt], 1.f);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int sc = (int)((sw[e / 4] >> (8 * (e % 4))) & 0xFF) - 127;
            vf[e] = __builtin_amdgcn_ldexph(vf[e], sc);
          }
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, ph, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pl, acc[mt], 0, 0, 0);
        }
      }
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
      for (int i = 0; i < 4; ++i) rec[16 * mt + 4 * j + i] = acc[mt][i];
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

}  // namespace

hipError_t launch_mx_quantize(const MxView& L, const __half* k, const __half* v, int64_t ld,
                              int64_t T, hipStream_t s) {
  const dim3 grid((unsigned)((T + kMxRun - 1) / kMxRun), (unsigned)(L.B * L.H));
  hipLaunchKernelGGL(mx_quantize_kernel, grid, dim3(256), 0, s, L, k, v, ld, T);
  return hipGetLastError();
}

hipError_t launch_mx_append(const MxView& L, const __half* k_new, const __half* v_new, int64_t t,
                            hipStream_t s) {
  hipLaunchKernelGGL(mx_append_kernel, dim3((unsigned)(L.B * L.H)), dim3(64), 0, s, L, k_new,
                     v_new, t);
  return hipGetLastError();
}

hipError_t launch_mx_decode(const MxView& L, int q_heads, int64_t T, const __half* q,
                            float sm_scale, float* out, void* ws, const Fp8Plan& plan,
                            const __half* k_new, const __half* v_new, hipStream_t s) {
  MxDecodeArgs a;
  a.L = L;
  a.q = q;
  a.out = out;
  a.counters = reinterpret_cast<unsigned*>(ws);
  a.part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + plan.ws_counters);
  a.T = T;
  a.nblk = (T + kMxRun - 1) / kMxRun;
  a.nw = plan.n_split;
  a.qscale = sm_scale * 1.4426950408889634f;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_t = k_new ? T - 1 : -1;
  const int gqa = q_heads / L.H;
  const dim3 grid((unsigned)((int64_t)L.B * L.H * plan.n_split));
  const dim3 block(256 * kMxWavesPerSimd);
  switch (gqa) {
    case 1: launch_decode_kernel(mx_decode_kernel<1>, grid, block, s, a); break;
    case 2: launch_decode_kernel(mx_decode_kernel<2>, grid, block, s, a); break;
    case 4: launch_decode_kernel(mx_decode_kernel<4>, grid, block, s, a); break;
    case 8: launch_decode_kernel(mx_decode_kernel<8>, grid, block, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kivi
