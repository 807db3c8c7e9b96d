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

// Q_a(Norm(x)) ([SUM] 方法步骤详情 step (3)) with Norm = RMSNorm: one row per
// block of 256 threads, thread t holding chunks t, t + 256, ... in registers.
// The binary32 evaluation order is fixed so that x_q (an integer decision
// taken on the normalized value) is reproducible: squares of bf16 values are
// exact; each thread adds its chunks' squares one element at a time, the wave
// combines its lanes pairwise at distances 32 ... 1, and the block adds the
// wave sums as (w0 + w1) + (w2 + w3); r = 1 / sqrt(ss / d + eps) with
// correctly rounded division and square root; y = bf16((x r) g).  The only
// multiply-add the compiler may fuse, s + f * f, has an exact product (a bf16
// square), so fusing it rounds the same.  Then the act quant of y, as
// k_act_quant, from registers.
template <int NC>
__global__ __launch_bounds__(256) void k_rmsnorm_act_quant(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ g, float eps, int d_in,
                                                           int8_t* __restrict__ xq, float* __restrict__ absmax) {
  __shared__ float wsum[4];
  __shared__ uint32_t wmax[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int nch = d_in >> 3;
  const uint4* xr = (const uint4*)(x + row * (int64_t)d_in);
  const uint4* gr = (const uint4*)g;
  uint4 v[NC], gw[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int idx = tid + 256 * c;
    v[c] = idx < nch ? xr[idx] : make_uint4(0u, 0u, 0u, 0u);
    gw[c] = (g && idx < nch) ? gr[idx] : make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (tid + 256 * c < nch) {
      const uint32_t w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = __uint_as_float(e & 1 ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
        s = __fadd_rn(s, __fmul_rn(f, f));
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s = __fadd_rn(s, __shfl_xor(s, off, 64));
  if (lane == 0) wsum[wave] = s;
  __syncthreads();
  const float ss = __fadd_rn(__fadd_rn(wsum[0], wsum[1]), __fadd_rn(wsum[2], wsum[3]));
  // square root correctly rounded to binary32 through binary64 (53 >= 2 * 24 + 2 bits:
  // the second rounding cannot differ from a direct one); the single-precision
  // instruction alone is within 1 ulp, not correctly rounded
  const float var = __fadd_rn(__fdiv_rn(ss, (float)d_in), eps);
  const float r = __fdiv_rn(1.0f, (float)sqrt((double)var));
  uint32_t m = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint32_t w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
    const uint32_t q[4] = {gw[c].x, gw[c].y, gw[c].z, gw[c].w};
    uint32_t o[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float lo = __fmul_rn(__fmul_rn(__uint_as_float(w[h] << 16), r), __uint_as_float(q[h] << 16));
      const float hi = __fmul_rn(__fmul_rn(__uint_as_float(w[h] & 0xFFFF0000u), r), __uint_as_float(q[h] & 0xFFFF0000u));
      o[h] = cvt_pk_bf16(lo, hi);
    }
    v[c] = make_uint4(o[0], o[1], o[2], o[3]);
    if (tid + 256 * c < nch) m = max(m, max(max(max_mag2(o[0]), max_mag2(o[1])), max(max_mag2(o[2]), max_mag2(o[3]))));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if (lane == 0) wmax[wave] = m;
  __syncthreads();
  m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const float a = __uint_as_float(m << 16);
  if (tid == 0) absmax[row] = a;
  uint2* out = (uint2*)(xq + row * (int64_t)d_in);
  const ActScale qs = act_scale(m ? a : 1.0f);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int idx = tid + 256 * c;
    if (idx < nch) out[idx] = m ? quant_chunk(v[c], qs.k, qs.as, qs.c) : make_uint2(0u, 0u);
  }
}

bool rmsnorm_supported(int64_t d_in) { return d_in % 8 == 0 && d_in <= 256 * 8 * 8; }

hipError_t launch_rmsnorm_act_quant(const uint16_t* x, const uint16_t* g, float eps, int64_t T, int64_t d_in,
                                    int8_t* xq, float* absmax, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int nch = (int)(d_in / 8);
  const dim3 grid((unsigned)T), block(256);
  if (nch <= 256)
    hipLaunchKernelGGL(k_rmsnorm_act_quant<1>, grid, block, 0, s, x, g, eps, (int)d_in, xq, absmax);
  else if (nch <= 512)
    hipLaunchKernelGGL(k_rmsnorm_act_quant<2>, grid, block, 0, s, x, g, eps, (int)d_in, xq, absmax);
  else if (nch <= 1024)
    hipLaunchKernelGGL(k_rmsnorm_act_quant<4>, grid, block, 0, s, x, g, eps, (int)d_in, xq, absmax);
  else
    hipLaunchKernelGGL(k_rmsnorm_act_quant<8>, grid, block, 0, s, x, g, eps, (int)d_in, xq, absmax);
  return hipGetLastError();
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
