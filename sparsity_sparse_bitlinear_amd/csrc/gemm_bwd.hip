// Dual-STE backward of Sparse-BitLinear on gfx950 bf16 matrix cores.
//
// [SUM] 前置知识 > Straight-Through Estimator (STE) (the Dual STE passes the
// gradient through both the ternary quantizer and the N:M selector), 核心方法
// (dense gradient flow to every master weight, masked ones included) and
// 方法步骤详情 step (7); [GIST] 2.2.  With y = x~ (gamma W_eff)^T:
//   dX[t,i] = gamma * sum_o dY[t,o] W_eff[o,i]     (k_bwd_dx)
//   dW[o,i] = sum_t dY[t,o] x~[t,i]                (k_bwd_dw, dense over (o,i))
//
// Both use v_mfma_f32_32x32x16_bf16 (lane l holds A[m = l%32][k = 8(l/32)+0..7]
// and B[k = 8(l/32)+0..7][n = l%32]).  Operands whose reduction index is not
// contiguous in memory are staged into LDS in their natural layout and read
// with ds_read_b64_tr_b16, which hands each lane 4 consecutive-k values of one
// column: in each 16-lane group, lane q addresses row kb + q/4, columns
// n0 + 4(q%4) .. +3, and lane i receives rows kb..kb+3 of column n0 + i.
//
//   dX: A = dY [T, d_out] (k = o contiguous, plain 16-byte fragment reads);
//       B = W_eff rows o, expanded from the code plane to bf16 {-1,0,+1}
//       (exact) in natural [o][i] layout, transposed by the tr16 read.
//   dW: A = dY^T, staged as [t][o]; B = x~ = x_q * a_t / 127 converted to bf16
//       while staging as [t][i]; both read with tr16.  Few output tiles: the
//       token range is split and the partial sums are added in a fixed order
//       by k_splitk_reduce (deterministic).
#include <algorithm>

#include "sbl_internal.h"

namespace sbl {

namespace {

constexpr int kBKb = 32;  // k elements per tile (bf16)

__device__ __forceinline__ int swz(int row, int c) { return row * 64 + 16 * (c ^ ((row >> 2) & 3)); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
}

// Two 2-bit codes (a 4-bit nibble) -> two bf16 values {0, +1 = 0x3F80, -1 = 0xBF80}.
__device__ __forceinline__ uint32_t code2_to_bf16x2(uint32_t nib) {
  const uint32_t s = (nib & 3u) | ((nib & 0xCu) << 14);
  return (s * 0x3F80u) | ((s & 0x20002u) << 7);
}

__device__ __forceinline__ uint4 code8_to_bf16x8(uint32_t c) {
  return make_uint4(code2_to_bf16x2(c), code2_to_bf16x2(c >> 4), code2_to_bf16x2(c >> 8),
                    code2_to_bf16x2(c >> 12));
}

__device__ __forceinline__ v4s tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((SBL_LDS v4s*)(SBL_LDS char*)p);
}

// 32x32x16 operand fragment (8 bf16 over k) from an LDS tile stored [k][mn] with
// pitch `pitch` bytes; k rows k0..k0+15, mn columns c0..c0+31.
__device__ __forceinline__ v8bf frag_tr(const char* base, int pitch, int k0, int c0, int lane) {
  const int g = lane >> 4, q = lane & 15;
  const int row = k0 + 8 * (g >> 1) + (q >> 2);
  const int col = c0 + 16 * (g & 1) + 4 * (q & 3);
  const char* p = base + row * pitch + col * 2;
  const v4s lo = tr16(p);
  const v4s hi = tr16(p + 4 * pitch);
  v8s r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(v8bf, r);
}

// ---------------------------------------------------------------------------
// dX = gamma * dY @ W_eff
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int OUT>
__global__ __launch_bounds__(256) void k_bwd_dx(const uint16_t* __restrict__ dY, const uint16_t* __restrict__ codes,
                                                const float* __restrict__ gamma_p, int T, int d_in, int d_out,
                                                void* __restrict__ dX) {
  static_assert((BM / WM) * (BN / WN) == 4, "4 waves per block");
  constexpr int MI = WM / 32, NJ = WN / 32;
  constexpr int CA = BM * 4 / 256;           // 16-byte chunks of A per thread
  constexpr int GB = BN / 8;                 // code groups per B row
  constexpr int RB = 256 / GB;               // B rows covered per pass
  constexpr int CB = kBKb / RB;              // passes
  constexpr int PB = (BN + 32) * 2;          // B pitch in bytes (== 64 mod 256)
  __shared__ __attribute__((aligned(16))) char lds[2 * BM * 64 + 2 * kBKb * PB];
  char* As = lds;
  char* Bs = lds + 2 * BM * 64;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm0 = (wave / (BN / WN)) * WM;
  const int wn0 = (wave % (BN / WN)) * WN;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int G = d_in >> 3;
  const int nk = (d_out + kBKb - 1) / kBKb;
  const bool a_vec = (d_out & 7) == 0;

  uint4 ra[CA];
  uint32_t rb[CB];

  auto load_tile = [&](int kt) {
    const int k0 = kt * kBKb;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int q = tid + 256 * i;
      const int row = q >> 2, c = q & 3;
      const int m = m0 + row, k = k0 + 8 * c;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m < T) {
        const uint16_t* p = dY + (int64_t)m * d_out + k;
        if (a_vec) {
          if (k < d_out) v = *(const uint4*)p;
        } else {
          uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (k + j < d_out) w[j >> 1] |= (uint32_t)p[j] << (16 * (j & 1));
          v = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
      ra[i] = v;
    }
#pragma unroll
    for (int s = 0; s < CB; ++s) {
      const int r = tid / GB + RB * s, gi = tid % GB;
      const int o = k0 + r, g = (n0 >> 3) + gi;
      rb[s] = (o < d_out && g < G) ? (uint32_t)codes[(int64_t)o * G + g] : 0u;
    }
  };
  auto store_tile = [&](int buf) {
    char* a = As + buf * BM * 64;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int q = tid + 256 * i;
      *(uint4*)(a + swz(q >> 2, q & 3)) = ra[i];
    }
    char* b = Bs + buf * kBKb * PB;
#pragma unroll
    for (int s = 0; s < CB; ++s) {
      const int r = tid / GB + RB * s, gi = tid % GB;
      *(uint4*)(b + r * PB + gi * 16) = code8_to_bf16x8(rb[s]);
    }
  };

  v16f acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tile(kt + 1);
    const char* a = As + buf * BM * 64;
    const char* b = Bs + buf * kBKb * PB;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int lc = 2 * ks + (lane >> 5);
      v8bf fa[MI], fb[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i) fa[i] = *(const v8bf*)(a + swz(wm0 + 32 * i + (lane & 31), lc));
#pragma unroll
      for (int j = 0; j < NJ; ++j) fb[j] = frag_tr(b, PB, 16 * ks, wn0 + 32 * j, lane);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float gamma = *gamma_p;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm0 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (m >= T) continue;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int n = n0 + wn0 + 32 * j + (lane & 31);
        if (n >= d_in) continue;
        const float v = acc[i][j][r] * gamma;
        const int64_t off = (int64_t)m * d_in + n;
        if constexpr (OUT == SBL_F32) ((float*)dX)[off] = v;
        else ((uint16_t*)dX)[off] = f32_to_bf16_rne(v);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dW = dY^T @ x~  (M = d_out, N = d_in, K = tokens)
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256) void k_bwd_dw(const uint16_t* __restrict__ dY, const int8_t* __restrict__ xq,
                                                const float* __restrict__ absmax, int T, int d_in, int d_out,
                                                int k_per_split, float* __restrict__ out) {
  static_assert((BM / WM) * (BN / WN) == 4, "4 waves per block");
  constexpr int MI = WM / 32, NJ = WN / 32;
  constexpr int PA = (BM + 32) * 2;
  constexpr int PB = (BN + 32) * 2;
  constexpr int CPA = BM / 8;                 // 16-byte chunks per A row (8 bf16)
  constexpr int CA = kBKb * CPA / 256;
  constexpr int CPB = BN / 16;                // 16-byte chunks per x_q row (16 int8)
  constexpr int CB = kBKb * CPB / 256;
  static_assert(CA >= 1 && CB >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) char lds[2 * kBKb * (PA + PB)];
  char* As = lds;
  char* Bs = lds + 2 * kBKb * PA;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm0 = (wave / (BN / WN)) * WM;
  const int wn0 = (wave % (BN / WN)) * WN;
  const int m0 = blockIdx.y * BM;   // output rows (o)
  const int n0 = blockIdx.x * BN;   // output cols (i)
  const int kbeg = blockIdx.z * k_per_split;
  const int kend = min(T, kbeg + k_per_split);
  const int nk = kend > kbeg ? (kend - kbeg + kBKb - 1) / kBKb : 0;
  const bool a_vec = (d_out & 7) == 0;
  const bool b_vec = (d_in & 15) == 0;

  uint4 ra[CA];
  uint4 rb[CB];
  float rs[CB];

  auto load_tile = [&](int kt) {
    const int t0 = kbeg + kt * kBKb;
#pragma unroll
    for (int s = 0; s < CA; ++s) {
      const int q = tid + 256 * s;
      const int r = q / CPA, c = q % CPA;
      const int t = t0 + r, o = m0 + 8 * c;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (t < kend) {
        const uint16_t* p = dY + (int64_t)t * d_out + o;
        if (a_vec) {
          if (o < d_out) v = *(const uint4*)p;
        } else {
          uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (o + j < d_out) w[j >> 1] |= (uint32_t)p[j] << (16 * (j & 1));
          v = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
      ra[s] = v;
    }
#pragma unroll
    for (int s = 0; s < CB; ++s) {
      const int q = tid + 256 * s;
      const int r = q / CPB, c = q % CPB;
      const int t = t0 + r, i = n0 + 16 * c;
      uint4 v = make_uint4(0, 0, 0, 0);
      float sc = 0.0f;
      if (t < kend) {
        sc = absmax[t] / 127.0f;
        const int8_t* p = xq + (int64_t)t * d_in + i;
        if (b_vec) {
          if (i < d_in) v = *(const uint4*)p;
        } else {
          if (i < d_in) { const uint2 h = *(const uint2*)p; v.x = h.x; v.y = h.y; }
          if (i + 8 < d_in) { const uint2 h = *(const uint2*)(p + 8); v.z = h.x; v.w = h.y; }
        }
      }
      rb[s] = v;
      rs[s] = sc;
    }
  };
  auto cvt4 = [](uint32_t w, float sc, uint32_t& lo, uint32_t& hi) {
    const float f0 = (float)(int)(int8_t)(w & 0xFFu) * sc;
    const float f1 = (float)(int)(int8_t)((w >> 8) & 0xFFu) * sc;
    const float f2 = (float)(int)(int8_t)((w >> 16) & 0xFFu) * sc;
    const float f3 = (float)(int)(int8_t)(w >> 24) * sc;
    lo = pack_bf16x2(f0, f1);
    hi = pack_bf16x2(f2, f3);
  };
  auto store_tile = [&](int buf) {
    char* a = As + buf * kBKb * PA;
#pragma unroll
    for (int s = 0; s < CA; ++s) {
      const int q = tid + 256 * s;
      *(uint4*)(a + (q / CPA) * PA + (q % CPA) * 16) = ra[s];
    }
    char* b = Bs + buf * kBKb * PB;
#pragma unroll
    for (int s = 0; s < CB; ++s) {
      const int q = tid + 256 * s;
      char* p = b + (q / CPB) * PB + (q % CPB) * 32;
      uint4 u0, u1;
      cvt4(rb[s].x, rs[s], u0.x, u0.y);
      cvt4(rb[s].y, rs[s], u0.z, u0.w);
      cvt4(rb[s].z, rs[s], u1.x, u1.y);
      cvt4(rb[s].w, rs[s], u1.z, u1.w);
      *(uint4*)p = u0;
      *(uint4*)(p + 16) = u1;
    }
  };

  v16f acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  if (nk > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tile(kt + 1);
    const char* a = As + buf * kBKb * PA;
    const char* b = Bs + buf * kBKb * PB;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8bf fa[MI], fb[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i) fa[i] = frag_tr(a, PA, 16 * ks, wm0 + 32 * i, lane);
#pragma unroll
      for (int j = 0; j < NJ; ++j) fb[j] = frag_tr(b, PB, 16 * ks, wn0 + 32 * j, lane);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tile(buf ^ 1);
    __syncthreads();
  }

  float* dst = out + (size_t)blockIdx.z * (size_t)d_out * (size_t)d_in;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm0 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (m >= d_out) continue;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int n = n0 + wn0 + 32 * j + (lane & 31);
        if (n < d_in) dst[(int64_t)m * d_in + n] = acc[i][j][r];
      }
    }
  }
}

// dW[idx] = sum_{z < S} part[z][idx], in order z = 0, 1, ..., S-1.
__global__ __launch_bounds__(256) void k_splitk_reduce(const float4* __restrict__ part, int64_t n4, int S,
                                                       float4* __restrict__ dW) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    float4 s = part[i];
    for (int z = 1; z < S; ++z) {
      const float4 v = part[(int64_t)z * n4 + i];
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    dW[i] = s;
  }
}

__global__ __launch_bounds__(256) void k_zero_f32(float* __restrict__ p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.0f;
}

// Tile configuration of the dW product.
constexpr int kDwBM = 256, kDwBN = 256;

int dw_splits(int64_t T, int64_t d_in, int64_t d_out) {
  const int64_t tiles = ((d_out + kDwBM - 1) / kDwBM) * ((d_in + kDwBN - 1) / kDwBN);
  if (T <= 0) return 1;
  int best = 1;
  double best_eff = 0.0;
  const int64_t max_s = std::max<int64_t>(1, std::min<int64_t>(32, T / 512));
  for (int s = 1; s <= max_s; ++s) {
    const int64_t w = tiles * s;
    const double eff = (double)w / (double)(256 * ((w + 255) / 256));
    // each extra split costs one more partial write + read; require a real gain
    if (eff > best_eff * 1.08) { best = s; best_eff = eff; }
  }
  return best;
}

}  // namespace

size_t backward_workspace_bytes(int64_t T, int64_t d_in, int64_t d_out, int flags) {
  if (!(flags & SBL_BWD_DW) || T == 0) return 0;
  const int S = dw_splits(T, d_in, d_out);
  if (S <= 1) return 0;
  return (size_t)S * (size_t)d_out * (size_t)d_in * sizeof(float);
}

hipError_t launch_backward(const uint16_t* codes, const float* gamma, const int8_t* xq, const float* absmax,
                           const uint16_t* dY, int64_t T, int64_t d_in, int64_t d_out, void* dX, int dx_dtype,
                           float* dW, int flags, void* ws, hipStream_t s) {
  if ((flags & SBL_BWD_DX) && T > 0) {
    const int64_t tiles256 = ((T + 255) / 256) * ((d_in + 255) / 256);
    if (tiles256 >= 512) {
      const dim3 grid((unsigned)((d_in + 255) / 256), (unsigned)((T + 255) / 256));
      if (dx_dtype == SBL_F32)
        hipLaunchKernelGGL((k_bwd_dx<256, 256, 128, 128, SBL_F32>), grid, dim3(256), 0, s, dY, codes, gamma, (int)T, (int)d_in, (int)d_out, dX);
      else
        hipLaunchKernelGGL((k_bwd_dx<256, 256, 128, 128, SBL_BF16>), grid, dim3(256), 0, s, dY, codes, gamma, (int)T, (int)d_in, (int)d_out, dX);
    } else {
      const dim3 grid((unsigned)((d_in + 127) / 128), (unsigned)((T + 127) / 128));
      if (dx_dtype == SBL_F32)
        hipLaunchKernelGGL((k_bwd_dx<128, 128, 64, 64, SBL_F32>), grid, dim3(256), 0, s, dY, codes, gamma, (int)T, (int)d_in, (int)d_out, dX);
      else
        hipLaunchKernelGGL((k_bwd_dx<128, 128, 64, 64, SBL_BF16>), grid, dim3(256), 0, s, dY, codes, gamma, (int)T, (int)d_in, (int)d_out, dX);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (flags & SBL_BWD_DW) {
    const int64_t n = d_out * d_in;
    if (T == 0) {
      hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 65536)), dim3(256), 0, s, dW, n);
      return hipGetLastError();
    }
    const int S = dw_splits(T, d_in, d_out);
    const int64_t kps = ((T + S - 1) / S + kBKb - 1) / kBKb * kBKb;
    const dim3 grid((unsigned)((d_in + kDwBN - 1) / kDwBN), (unsigned)((d_out + kDwBM - 1) / kDwBM), (unsigned)S);
    float* target = S > 1 ? (float*)ws : dW;
    hipLaunchKernelGGL((k_bwd_dw<kDwBM, kDwBN, 128, 128>), grid, dim3(256), 0, s, dY, xq, absmax, (int)T, (int)d_in,
                       (int)d_out, (int)kps, target);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (S > 1) {
      // d_out * d_in is a multiple of 8, so float4 covers it exactly
      const int64_t n4 = n / 4;
      hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)std::min<int64_t>((n4 + 255) / 256, 65536)), dim3(256), 0, s,
                         (const float4*)ws, n4, S, (float4*)dW);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace sbl
