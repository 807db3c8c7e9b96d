// Per-token absmax int8 activation quantization on gfx950.
//
// [SUM] 前置知识 > 1.58-bit BitNet 量化 (activations absmax-quantized to
// 8-bit integers) and 方法步骤详情 step (3):
//   a_t = max_i |x[t,i]|,  x_q[t,i] = round-half-even(127 x[t,i] / a_t).
//
// One wavefront per token row: the row is held in registers (up to NC 16-byte
// chunks per lane), the maximum is a wave reduction on the 15-bit magnitude
// bits (integer order equals magnitude order for finite bf16), then every
// element is quantized from registers.  Rows longer than 64*NC chunks re-read
// the remainder.
//
// Binary32 evaluation: x and a are first scaled by the same exact power of two
// so that a lands in [1, 2) (this keeps 127*x finite and a normal), then
// q = rint(fl(fl(127 x') / a')).  For bf16 inputs the exact quotient is either a
// half-integer or at least 2^-17 (relative) away from one, so the single
// binary32 rounding of the division cannot change the rounded integer: the
// result equals the exact round-half-even of 127 x / a.
#include "sbl_internal.h"

namespace sbl {

__device__ __forceinline__ uint32_t max_mag2(uint32_t w) {
  return max(w & 0x7FFFu, (w >> 16) & 0x7FFFu);
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

__device__ __forceinline__ uint32_t quant_word_pair(uint32_t w0, uint32_t w1, int k, float as, float c) {
  const int q0 = quant_one(w0 & 0xFFFFu, k, as, c);
  const int q1 = quant_one(w0 >> 16, k, as, c);
  const int q2 = quant_one(w1 & 0xFFFFu, k, as, c);
  const int q3 = quant_one(w1 >> 16, k, as, c);
  return (uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8) | ((uint32_t)(q2 & 0xFF) << 16) |
         ((uint32_t)(q3 & 0xFF) << 24);
}

__device__ __forceinline__ uint2 quant_chunk(uint4 v, int k, float as, float c) {
  return make_uint2(quant_word_pair(v.x, v.y, k, as, c), quant_word_pair(v.z, v.w, k, as, c));
}

// WPR waves per row (1: four rows per block of 256 threads; 4: one row per
// block, for long rows); each lane keeps NC 16-byte chunks of its row in
// registers: the row is read once.
template <int NC, int WPR>
__global__ __launch_bounds__(256) void k_act_quant(const uint16_t* __restrict__ x, int64_t T, int d_in,
                                                   int8_t* __restrict__ xq, float* __restrict__ absmax) {
  constexpr int kR = 64 * WPR;  // threads per row
  const int lane = threadIdx.x % kR;
  const int64_t t = (int64_t)blockIdx.x * (4 / WPR) + threadIdx.x / kR;
  __shared__ uint32_t wmax[4];
  if (WPR == 1 && t >= T) return;
  const int nch = d_in >> 3;  // 16-byte chunks per row
  const uint4* row = (const uint4*)(x + t * (int64_t)d_in);
  uint2* out = (uint2*)(xq + t * (int64_t)d_in);

  uint4 v[NC];
  uint32_t m = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int idx = lane + kR * c;
    if (idx < nch) {
      v[c] = row[idx];
      m = max(m, max(max_mag2(v[c].x), max_mag2(v[c].y)));
      m = max(m, max(max_mag2(v[c].z), max_mag2(v[c].w)));
    } else {
      v[c] = make_uint4(0, 0, 0, 0);
    }
  }
  for (int idx = lane + kR * NC; idx < nch; idx += kR) {  // rows longer than the register window
    const uint4 w = row[idx];
    m = max(m, max(max_mag2(w.x), max_mag2(w.y)));
    m = max(m, max(max_mag2(w.z), max_mag2(w.w)));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if constexpr (WPR > 1) {  // one row per block: maximum over its waves
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  }

  const float a = __uint_as_float(m << 16);
  if (lane == 0) absmax[t] = a;
  if (m == 0) {
    for (int idx = lane; idx < nch; idx += kR) out[idx] = make_uint2(0, 0);
    return;
  }
  int e;
  (void)frexpf(a, &e);  // a = f * 2^e, f in [0.5, 1)
  const int k = 1 - e;  // a * 2^k in [1, 2)
  const float as = ldexpf(a, k);
  const float c127 = 127.0f / as;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int idx = lane + kR * c;
    if (idx < nch) out[idx] = quant_chunk(v[c], k, as, c127);
  }
  for (int idx = lane + kR * NC; idx < nch; idx += kR) out[idx] = quant_chunk(row[idx], k, as, c127);
}

hipError_t launch_act_quant(const uint16_t* x, int64_t T, int64_t d_in, int8_t* xq, float* absmax, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int nch = (int)(d_in / 8);
  const dim3 rows4((unsigned)((T + 3) / 4)), rows1((unsigned)T), block(256);
  if (nch <= 64 * 4)
    hipLaunchKernelGGL((k_act_quant<4, 1>), rows4, block, 0, s, x, T, (int)d_in, xq, absmax);
  else if (nch <= 64 * 8)
    hipLaunchKernelGGL((k_act_quant<8, 1>), rows4, block, 0, s, x, T, (int)d_in, xq, absmax);
  else  // long rows: four waves per row
    hipLaunchKernelGGL((k_act_quant<8, 4>), rows1, block, 0, s, x, T, (int)d_in, xq, absmax);
  return hipGetLastError();
}

}  // namespace sbl
