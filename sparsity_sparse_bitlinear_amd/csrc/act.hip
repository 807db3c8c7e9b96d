// Per-token absmax int8 activation quantization on gfx950 ([SUM] 前置知识 >
// 1.58-bit BitNet 量化; 方法步骤详情 step (3)); the per-element arithmetic is in
// act_common.h.
//
// One wavefront per token row: the row is held in registers (up to NC 16-byte
// chunks per lane), the maximum is a wave reduction on the 15-bit magnitude
// bits (integer order equals magnitude order for finite bf16), then every
// element is quantized from registers.  Rows longer than 64*NC chunks re-read
// the remainder.
#include "act_common.h"

namespace sbl {

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
  const ActScale sc = act_scale(a);
  const int k = sc.k;
  const float as = sc.as, c127 = sc.c;
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
