// Per-element step of the per-token absmax 8-bit activation quantization,
// shared by k_act_quant and the fused decode kernel so that both produce the
// same bits.
//
// [SUM] 前置知识 > 1.58-bit BitNet 量化 and 方法步骤详情 step (3):
//   a_t = max_i |x[t,i]|,  x_q[t,i] = round-half-even(127 x[t,i] / a_t).
//
// Binary32 evaluation: x and a are first scaled by the same exact power of two
// so that a lands in [1, 2) (this keeps 127*x finite and a normal), then
// q = rint(fl(fl(127 x') / a')).  For bf16 inputs the exact quotient is either a
// half-integer or at least 2^-17 (relative) away from one, so the single
// binary32 rounding of the division cannot change the rounded integer: the
// result equals the exact round-half-even of 127 x / a.
#pragma once

#include "sbl_internal.h"

namespace sbl {

// Larger of the two 15-bit magnitudes of a bf16 pair (integer order equals
// magnitude order for finite bf16).
__device__ __forceinline__ uint32_t max_mag2(uint32_t w) {
  return max(w & 0x7FFFu, (w >> 16) & 0x7FFFu);
}

// Row scale set-up from the row maximum a > 0: a' = a 2^k in [1, 2) and
// c = fl(127 / a').
struct ActScale {
  int k;
  float as, c;
};
__device__ __forceinline__ ActScale act_scale(float a) {
  int e;
  (void)frexpf(a, &e);  // a = f * 2^e, f in [0.5, 1)
  ActScale s;
  s.k = 1 - e;
  s.as = ldexpf(a, s.k);
  s.c = 127.0f / s.as;
  return s;
}

// Fast path: qf = fl(x' * fl(127 / a')) differs from the exact quotient
// q = 127 x' / a' by less than |q| 2^-23 <= 2^-16 (|q| <= 127).  When qf is
// more than 2^-14 away from a half-integer, rint(qf) is therefore the integer
// nearest to q; otherwise (ties included) the element takes the division path,
// which is exact as stated above.
__device__ __forceinline__ int quant_one(uint32_t h16, int k, float as, float c) {
  const float xs = ldexpf(__uint_as_float(h16 << 16), k);
  const float qf = xs * c;
  float r = rintf(qf);
  if (__builtin_expect(fabsf(qf - r) > 0.5f - 0x1p-14f, 0)) r = rintf((127.0f * xs) / as);
  return (int)r;
}

// Four bf16 (two words) -> four int8 in one word, element order kept.
__device__ __forceinline__ uint32_t quant_word_pair(uint32_t w0, uint32_t w1, int k, float as, float c) {
  const int q0 = quant_one(w0 & 0xFFFFu, k, as, c);
  const int q1 = quant_one(w0 >> 16, k, as, c);
  const int q2 = quant_one(w1 & 0xFFFFu, k, as, c);
  const int q3 = quant_one(w1 >> 16, k, as, c);
  return (uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8) | ((uint32_t)(q2 & 0xFF) << 16) |
         ((uint32_t)(q3 & 0xFF) << 24);
}

// Eight bf16 (one 16-byte chunk) -> eight int8.
__device__ __forceinline__ uint2 quant_chunk(uint4 v, int k, float as, float c) {
  return make_uint2(quant_word_pair(v.x, v.y, k, as, c), quant_word_pair(v.z, v.w, k, as, c));
}

}  // namespace sbl
