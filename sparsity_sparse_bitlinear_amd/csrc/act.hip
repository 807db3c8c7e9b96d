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
      v[c] = load_nt16(row + idx);
      m = max(m, max(max_mag2(v[c].x), max_mag2(v[c].y)));
      m = max(m, max(max_mag2(v[c].z), max_mag2(v[c].w)));
    } else {
      v[c] = make_uint4(0, 0, 0, 0);
    }
  }
  for (int idx = lane + kR * NC; idx < nch; idx += kR) {  // rows longer than the register window
    const uint4 w = row[idx];  // (read again below: cached)
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

// ---------------------------------------------------------------------------
// Q_a(Norm(x)) ([SUM] 方法步骤详情 step (3)) with Norm = RMSNorm:
//   ms = RN32(sum_i x_i^2 / d)   (the exact mean, rounded once)
//   r  = RN32(1 / sqrt(RN32(ms + eps)))
//   y  = bf16(RN32(RN32(x r) g)), then the act quant of y.
// Every step is one correctly rounded operation on exact values, so the result
// does not depend on how the sum is split over lanes and waves.
// ---------------------------------------------------------------------------

// Relative distance from a float64 estimate of ms to the nearest binary32
// rounding boundary below which the estimate is not trusted.  The float64 sum
// of at most 136 non-negative exact squares along any path of the reduction,
// then one division, is within 137 * 2^-53 * 1.01 < 2^-45.8 of the exact mean.
constexpr double kMsMargin = 0x1p-44;

// RN32 of a non-negative value known only as a float64 estimate q within a
// relative kMsMargin: true (with *out) when no binary32 rounding boundary lies
// within that distance of q, so that every value there rounds alike.
__device__ __forceinline__ bool rn32_certain(double q, float* out) {
  const float f = (float)q;  // round to nearest even; overflow gives +inf
  const double tol = q * kMsMargin;
  const double ovf = 0x1.ffffffp127;  // 2^128 - 2^103: the overflow threshold
  const uint32_t b = __float_as_uint(f);
  bool ok;
  if (b == 0x7F800000u) {
    ok = q - ovf > tol;
  } else {
    const double hi = b == 0x7F7FFFFFu ? ovf : 0.5 * ((double)f + (double)__uint_as_float(b + 1));
    const double lo = b == 0 ? -1.0 : 0.5 * ((double)f + (double)__uint_as_float(b - 1));
    ok = (hi - q > tol) && (q - lo > tol);
  }
  *out = f;
  return ok;
}

// Exact mean square from a histogram of squared significands by exponent
// (bins[s] = sum of sig^2 over elements with max(E, 1) - 1 = s, each square
// being sig^2 2^(2 s) units of 2^-266): the sum as a 17-word integer, divided
// by d, rounded once to binary32 (nearest even, subnormal and overflow ranges
// included).  One thread; big is scratch of 17 words in LDS.
__device__ __noinline__ float exact_mean_square(const uint32_t SBL_LDS* bins, uint32_t SBL_LDS* big, uint32_t d) {
  constexpr int kWords = 17;
  for (int i = 0; i < kWords; ++i) big[i] = 0u;
  for (int s = 0; s < 254; ++s) {
    const uint32_t v = bins[s];
    if (v == 0u) continue;
    const int pos = 2 * s, L = pos >> 5;
    const unsigned long long add = (unsigned long long)v << (pos & 31);
    unsigned long long t = (unsigned long long)big[L] + (uint32_t)add;
    big[L] = (uint32_t)t;
    t = (unsigned long long)big[L + 1] + (add >> 32) + (t >> 32);
    big[L + 1] = (uint32_t)t;
    for (int k = L + 2; (t >> 32) != 0u && k < kWords; ++k) {
      t = (unsigned long long)big[k] + (t >> 32);
      big[k] = (uint32_t)t;
    }
  }
  unsigned long long rem = 0;
  for (int L = kWords - 1; L >= 0; --L) {
    const unsigned long long cur = (rem << 32) | big[L];
    big[L] = (uint32_t)(cur / d);
    rem = cur % d;
  }
  int p = -1;
  for (int L = kWords - 1; L >= 0 && p < 0; --L)
    if (big[L]) p = 32 * L + 31 - __clz(big[L]);
  if (p < 0) return 0.0f;  // below 2^-266
  auto bit = [&](int i) -> uint32_t { return (big[i >> 5] >> (i & 31)) & 1u; };
  const int lsb = max(p - 23, 117);  // 2^-149 is bit 117 of a quantity in units of 2^-266
  uint32_t mant = 0;
  for (int i = p; i >= lsb; --i) mant = (mant << 1) | bit(i);
  const uint32_t guard = bit(lsb - 1);
  bool sticky = rem != 0;
  for (int i = lsb - 2; i >= 0 && !sticky; --i) sticky = bit(i) != 0u;
  if (guard && (sticky || (mant & 1u))) ++mant;
  // mant * 2^(lsb - 266): exponent field lsb - 116 with the leading one carried
  // into it (also a subnormal, lsb = 117, and a carry to the next binade)
  const uint32_t bits = ((uint32_t)(lsb - 116) << 23) + mant - (1u << 23);
  return bits >= 0x7F800000u ? __uint_as_float(0x7F800000u) : __uint_as_float(bits);
}

// Sign of m^2 v - 1 for a float64 m with at most 25 significant bits (m^2 is
// exact) and m^2 v within a factor 2 of 1: the product as hi + lo exactly
// (fma), hi - 1 exact by Sterbenz.
__device__ __forceinline__ double sq_times_minus_one(double m, double v) {
  const double p = m * m;
  const double hi = p * v;
  const double lo = fma(p, v, -hi);
  return (hi - 1.0) + lo;
}

// RN32(1 / sqrt(v)) for a binary32 v > 0 (+inf gives 0): a float64 estimate
// rounded to binary32 is within one place of the nearest value; it moves one
// place when the neighbouring midpoint m on that side has m^2 v on the wrong
// side of 1 (1/sqrt(v) is never a midpoint).  The result is always normal.
__device__ __forceinline__ float rsqrt_rn32(float v) {
  if (__float_as_uint(v) == 0x7F800000u) return 0.0f;
  const double vd = (double)v;
  float r = (float)(1.0 / sqrt(vd));
  const uint32_t b = __float_as_uint(r);
  const double rd = (double)r;
  const double up = 0.5 * (rd + (double)__uint_as_float(b + 1));
  const double dn = 0.5 * (rd + (double)__uint_as_float(b - 1));
  if (sq_times_minus_one(up, vd) < 0.0)
    r = __uint_as_float(b + 1);
  else if (sq_times_minus_one(dn, vd) > 0.0)
    r = __uint_as_float(b - 1);
  return r;
}

// Orders the LDS accesses of one wave's lanes around it (the wave's own
// instructions reach LDS in order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wave sum of a float64 value (every lane gets the total).
__device__ __forceinline__ double wave_sum_f64(double s) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  return s;
}

// WPR waves per row: 1 (four rows per block of 256 threads) or 4 (one row per
// block).  Each lane keeps NC 16-byte chunks of x (and of g) in registers: the
// row is read once.  The mean square is estimated in float64 (squares of bf16
// values are exact there) and rounded directly when the estimate is far from a
// binary32 rounding boundary; otherwise the row's squares are summed exactly
// (a per-exponent histogram in LDS, then exact_mean_square).  Then y in
// binary32 -> bf16 and the act quant of y, as k_act_quant.
template <int NC, int WPR>
__global__ __launch_bounds__(256) void k_rmsnorm_act_quant(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ g, float eps, int64_t T,
                                                           int d_in, int8_t* __restrict__ xq,
                                                           float* __restrict__ absmax, float* __restrict__ rstd) {
  constexpr int kR = 64 * WPR;  // threads per row
  constexpr int kRows = 4 / WPR;
  __shared__ double wsum[4];
  __shared__ uint32_t wmax[4];
  __shared__ uint32_t bins[kRows][256];
  __shared__ uint32_t big[kRows][20];
  __shared__ float ms_sh[kRows];
  const int tid = threadIdx.x, lane = tid % kR, wave = tid >> 6, rslot = tid / kR;
  const int64_t row = (int64_t)blockIdx.x * kRows + rslot;
  const bool live = row < T;  // WPR == 1: the last block may hold fewer rows
  const int nch = d_in >> 3;
  const uint4* xr = (const uint4*)(x + (live ? row : 0) * (int64_t)d_in);
  const uint4* gr = (const uint4*)g;
  uint4 v[NC], gw[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int idx = lane + kR * c;
    const bool in = live && idx < nch;
    v[c] = in ? xr[idx] : make_uint4(0u, 0u, 0u, 0u);
    gw[c] = (g && in) ? gr[idx] : make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
  }
  // float64 estimate of the sum of squares
  double s = 0.0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint32_t w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const double lo = (double)__uint_as_float(w[h] << 16);
      const double hi = (double)__uint_as_float(w[h] & 0xFFFF0000u);
      s = fma(lo, lo, s);
      s = fma(hi, hi, s);
    }
  }
  s = wave_sum_f64(s);
  if constexpr (WPR > 1) {
    if ((tid & 63) == 0) wsum[wave] = s;
    __syncthreads();
    s = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  }
  float ms;
  const bool certain = rn32_certain(s / (double)d_in, &ms);
  if (!certain) {  // uniform over the row's threads
    uint32_t SBL_LDS* hb = (uint32_t SBL_LDS*)bins[rslot];
    for (int i = lane; i < 256; i += kR) hb[i] = 0u;
    if constexpr (WPR > 1) __syncthreads(); else wave_sync();
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint32_t w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t m = (e & 1 ? w[e >> 1] >> 16 : w[e >> 1]) & 0x7FFFu;
        const uint32_t ex = m >> 7, fr = m & 0x7Fu;
        const uint32_t sig = ex ? (fr | 0x80u) : fr;
        if (sig) atomicAdd((uint32_t*)&bins[rslot][(ex ? ex : 1u) - 1u], sig * sig);
      }
    }
    if constexpr (WPR > 1) __syncthreads(); else wave_sync();
    if (lane == 0) ms_sh[rslot] = exact_mean_square(hb, (uint32_t SBL_LDS*)big[rslot], (uint32_t)d_in);
    if constexpr (WPR > 1) __syncthreads(); else wave_sync();
    ms = ms_sh[rslot];
  }
  const float r = rsqrt_rn32(__fadd_rn(ms, eps));
  if (live && lane == 0 && rstd) rstd[row] = r;

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
    m = max(m, max(max(max_mag2(o[0]), max_mag2(o[1])), max(max_mag2(o[2]), max_mag2(o[3]))));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if constexpr (WPR > 1) {
    if ((tid & 63) == 0) wmax[wave] = m;
    __syncthreads();
    m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  }
  if (!live) return;
  const float a = __uint_as_float(m << 16);
  if (lane == 0) absmax[row] = a;
  uint2* out = (uint2*)(xq + row * (int64_t)d_in);
  const ActScale qs = act_scale(m ? a : 1.0f);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int idx = lane + kR * c;
    if (idx < nch) out[idx] = m ? quant_chunk(v[c], qs.k, qs.as, qs.c) : make_uint2(0u, 0u);
  }
}

bool rmsnorm_supported(int64_t d_in) { return d_in % 8 == 0 && d_in <= 256 * 8 * 8; }

hipError_t launch_rmsnorm_act_quant(const uint16_t* x, const uint16_t* g, float eps, int64_t T, int64_t d_in,
                                    int8_t* xq, float* absmax, float* rstd, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int nch = (int)(d_in / 8);
  const dim3 rows4((unsigned)((T + 3) / 4)), rows1((unsigned)T), block(256);
  if (nch <= 64 * 4)
    hipLaunchKernelGGL((k_rmsnorm_act_quant<4, 1>), rows4, block, 0, s, x, g, eps, T, (int)d_in, xq, absmax, rstd);
  else if (nch <= 64 * 8)
    hipLaunchKernelGGL((k_rmsnorm_act_quant<8, 1>), rows4, block, 0, s, x, g, eps, T, (int)d_in, xq, absmax, rstd);
  else if (nch <= 256 * 4)
    hipLaunchKernelGGL((k_rmsnorm_act_quant<4, 4>), rows1, block, 0, s, x, g, eps, T, (int)d_in, xq, absmax, rstd);
  else if (nch <= 256 * 6)
    hipLaunchKernelGGL((k_rmsnorm_act_quant<6, 4>), rows1, block, 0, s, x, g, eps, T, (int)d_in, xq, absmax, rstd);
  else
    hipLaunchKernelGGL((k_rmsnorm_act_quant<8, 4>), rows1, block, 0, s, x, g, eps, T, (int)d_in, xq, absmax, rstd);
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
