// The min/max asymmetric quantizer of one group, shared by the kernels that write
// codes: the prefill and append kernels, and the decode step that quantizes the Value
// leaving a per-token Value window.  "4.4 KV Cache quantization" §3.1; "09 — KV Cache
// Quantization", "KIVI — the reference paper": float16 scale = range / (2^b - 1) and
// zero = group minimum, code = clamp(rint((x - zero) / scale)).  Every kernel that
// writes codes calls these functions, so all of them write identical bytes.
#pragma once

#include "kivi_internal.h"

namespace kivi {
namespace {

struct GroupParams {
  float mn;      // group minimum (float32, exact float16 value)
  float s;       // float32 value of the stored float16 scale
  float inv;     // correctly rounded 1 / s (0 when s == 0)
  __half scale;
  __half zero;
};

__device__ __forceinline__ GroupParams group_params(float mn, float mx, int bits) {
#pragma clang fp contract(off)
  GroupParams p;
  const float qmax = (float)((1 << bits) - 1);
  const float rng = mx - mn;
  const float s32 = rng / qmax;          // IEEE division (correctly rounded)
  p.scale = __float2half_rn(s32);
  p.zero = __float2half_rn(mn);          // exact: mn is a float16 value
  p.mn = mn;
  p.s = __half2float(p.scale);
  p.inv = p.s == 0.0f ? 0.0f : 1.0f / p.s;
  return p;
}

// code = clamp(rint(RN((x - mn) / s)), 0, 2^b - 1), ties to even, with RN the
// correctly rounded float32 quotient (and code 0 when s == 0).  The quotient comes
// without a division: with inv = RN(1/s), q0 = RN(a * inv) is within one ulp of a/s,
// the remainder a - q0*s is exact in one FMA, and q0 + remainder*inv rounded once is
// RN(a/s) (Markstein's theorem on correctly rounded division from a correctly
// rounded reciprocal).  Here a = RN(x - mn) is 0 or at least 2^-24 and s a float16
// value, so nothing is subnormal; checked against IEEE division on the CPU for every
// positive float16 s, densely around every tie and code boundary.  With s == 0,
// inv == 0 gives q == 0: code 0 without a branch.  s is never infinite: the range of
// two float16 values is below 2^17, so s < 2^16.
//
// a = fma(x, 1, -mn) is RN(x - mn) (one rounding), with the float16 x converted inside
// the FMA.  q >= 0, and adding 1.5 * 2^23 to min(q, qmax) rounds it to an integer,
// ties to even, in the low mantissa bits: the low byte of the returned bit pattern
// is the code clamp(rint(q), 0, qmax).
constexpr float kRoundAdd = 12582912.0f;   // 1.5 * 2^23
template <int BITS>
__device__ __forceinline__ uint32_t quant_bits(__half x, const GroupParams& p) {
#pragma clang fp contract(off)
  constexpr float qmax = (float)((1 << BITS) - 1);
  const float a = fmaf(__half2float(x), 1.0f, -p.mn);
  const float q0 = a * p.inv;
  const float q = fmaf(fmaf(-q0, p.s, a), p.inv, q0);
  return __float_as_uint(fminf(q, qmax) + kRoundAdd);
}

}  // namespace
}  // namespace kivi
