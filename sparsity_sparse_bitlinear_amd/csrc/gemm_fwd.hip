// Forward product of Sparse-BitLinear on gfx950 int8 matrix cores.
//
// [SUM] 前置知识 > 半结构化 N:M 稀疏 (y = (W (.) M) x) and 方法步骤详情 step (6)
// (y ~= s * W_eff x~ with s absorbing the quantization scales):
//   acc[t,o] = sum_i x_q[t,i] * W_eff[o,i]   (exact int32)
//   y[t,o]   = acc[t,o] * gamma * a_t / 127
//
// C = A * B^T with A = x_q [T, d_in] (int8, K contiguous) and B = W_eff
// [d_out, d_in], streamed from the 2-bit code plane and expanded to int8
// {-1,0,+1} in LDS once per block tile, so every wave reads plain int8
// fragments.  v_mfma_i32_32x32x32_i8: lane l holds A[m = l%32][k = 16(l/32) +
// 0..15] and B[k = 16(l/32) + 0..15][n = l%32]; accumulator register r of
// lane l is C[8(r/4) + 4(l/32) + r%4][l%32].
//
// Tiles: block BM x BN over (tokens, outputs), K step 64 bytes, 4 waves in a
// 2 x 2 grid, double-buffered LDS with a register prefetch of the next tile.
// LDS rows are 64 bytes (4 chunks of 16); chunk c of row r is stored at
// c ^ ((r >> 2) & 3) so 16 consecutive rows reading the same chunk hit 16
// distinct 16-byte bank groups.
#include "sbl_internal.h"

namespace sbl {

namespace {

constexpr int kBK = 64;  // k bytes per tile

__device__ __forceinline__ int swz(int row, int c) { return row * 64 + 16 * (c ^ ((row >> 2) & 3)); }

// 16 two-bit codes (two groups) -> 16 int8 values in natural k order.
__device__ __forceinline__ uint32_t expand4(uint32_t byte4codes) {
  uint32_t x = byte4codes & 0xFFu;
  x = (x | (x << 12)) & 0x000F000Fu;
  x = (x | (x << 6)) & 0x03030303u;
  // byte selector 0 -> 0x00, 1 -> 0x01, 3 -> 0xFF
  return __builtin_amdgcn_perm(0u, 0xFF000100u, x);
}

__device__ __forceinline__ uint4 expand16(uint32_t w) {
  return make_uint4(expand4(w), expand4(w >> 8), expand4(w >> 16), expand4(w >> 24));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <int BM, int BN, int WM, int WN, int OUT>
__global__ __launch_bounds__(256) void k_fwd_i8(const int8_t* __restrict__ xq, const uint16_t* __restrict__ codes,
                                                const float* __restrict__ gamma_p,
                                                const float* __restrict__ absmax, int T, int d_in, int d_out,
                                                void* __restrict__ y) {
  static_assert((BM / WM) * (BN / WN) == 4, "4 waves per block");
  constexpr int MI = WM / 32, NJ = WN / 32;
  constexpr int CA = BM * 4 / 256;  // A chunks (16 B) per thread per tile
  __shared__ __attribute__((aligned(16))) char lds[2 * (BM + BN) * kBK];
  char* As = lds;
  char* Bs = lds + 2 * BM * kBK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm0 = (wave / (BN / WN)) * WM;
  const int wn0 = (wave % (BN / WN)) * WN;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int G = d_in >> 3;                  // code groups per row
  const int nk = (d_in + kBK - 1) / kBK;
  const bool a_vec = (d_in & 15) == 0;
  const bool b_vec = (G & 7) == 0;

  uint4 ra[CA];
  uint4 rb = make_uint4(0, 0, 0, 0);

  auto load_tile = [&](int kt) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int q = tid + 256 * i;
      const int row = q >> 2, c = q & 3;
      const int m = m0 + row, k = k0 + 16 * c;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m < T) {
        const int8_t* p = xq + (int64_t)m * d_in + k;
        if (a_vec) {
          if (k < d_in) v = *(const uint4*)p;
        } else {
          if (k < d_in) { const uint2 h = *(const uint2*)p; v.x = h.x; v.y = h.y; }
          if (k + 8 < d_in) { const uint2 h = *(const uint2*)(p + 8); v.z = h.x; v.w = h.y; }
        }
      }
      ra[i] = v;
    }
    if (tid < BN) {
      const int n = n0 + tid;
      const int g0 = kt * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (n < d_out) {
        const uint16_t* p = codes + (int64_t)n * G + g0;
        if (b_vec) {
          if (g0 < G) v = *(const uint4*)p;
        } else {
          uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (g0 + j < G) w[j >> 1] |= (uint32_t)p[j] << (16 * (j & 1));
          v = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
      rb = v;
    }
  };
  auto store_tile = [&](int buf) {
    char* a = As + buf * BM * kBK;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int q = tid + 256 * i;
      *(uint4*)(a + swz(q >> 2, q & 3)) = ra[i];
    }
    if (tid < BN) {
      char* b = Bs + buf * BN * kBK;
      *(uint4*)(b + swz(tid, 0)) = expand16(rb.x);
      *(uint4*)(b + swz(tid, 1)) = expand16(rb.y);
      *(uint4*)(b + swz(tid, 2)) = expand16(rb.z);
      *(uint4*)(b + swz(tid, 3)) = expand16(rb.w);
    }
  };

  v16i acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tile(kt + 1);
    const char* a = As + buf * BM * kBK;
    const char* b = Bs + buf * BN * kBK;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int lc = 2 * ks + (lane >> 5);
      v4i fa[MI], fb[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i) fa[i] = *(const v4i*)(a + swz(wm0 + 32 * i + (lane & 31), lc));
#pragma unroll
      for (int j = 0; j < NJ; ++j) fb[j] = *(const v4i*)(b + swz(wn0 + 32 * j + (lane & 31), lc));
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: y = acc * gamma * a_t / 127.
  const float gamma = *gamma_p;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm0 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (m >= T) continue;
      const float s = (gamma * absmax[m]) / 127.0f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int n = n0 + wn0 + 32 * j + (lane & 31);
        if (n >= d_out) continue;
        const int64_t off = (int64_t)m * d_out + n;
        if constexpr (OUT == SBL_I32) {
          ((int*)y)[off] = acc[i][j][r];
        } else if constexpr (OUT == SBL_F32) {
          ((float*)y)[off] = (float)acc[i][j][r] * s;
        } else {
          ((uint16_t*)y)[off] = f32_to_bf16_rne((float)acc[i][j][r] * s);
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_fwd_tiles(const uint16_t* codes, const float* gamma, const int8_t* xq, const float* absmax,
                            int64_t T, int64_t d_in, int64_t d_out, void* y, int y_dtype, hipStream_t s) {
  const dim3 grid((unsigned)((d_out + BN - 1) / BN), (unsigned)((T + BM - 1) / BM)), block(256);
  switch (y_dtype) {
    case SBL_F32:
      hipLaunchKernelGGL((k_fwd_i8<BM, BN, WM, WN, SBL_F32>), grid, block, 0, s, xq, codes, gamma, absmax, (int)T,
                         (int)d_in, (int)d_out, y);
      break;
    case SBL_BF16:
      hipLaunchKernelGGL((k_fwd_i8<BM, BN, WM, WN, SBL_BF16>), grid, block, 0, s, xq, codes, gamma, absmax, (int)T,
                         (int)d_in, (int)d_out, y);
      break;
    default:
      hipLaunchKernelGGL((k_fwd_i8<BM, BN, WM, WN, SBL_I32>), grid, block, 0, s, xq, codes, gamma, absmax, (int)T,
                         (int)d_in, (int)d_out, y);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward(const uint16_t* codes, const float* gamma, const int8_t* xq, const float* absmax,
                          int64_t T, int64_t d_in, int64_t d_out, void* y, int y_dtype, hipStream_t s) {
  if (T == 0) return hipSuccess;
  // Large problems: 256 x 256 tiles; otherwise 128 x 128 tiles keep more CUs busy.
  const int64_t tiles256 = ((T + 255) / 256) * ((d_out + 255) / 256);
  if (tiles256 >= 512) return launch_fwd_tiles<256, 256, 128, 128>(codes, gamma, xq, absmax, T, d_in, d_out, y, y_dtype, s);
  return launch_fwd_tiles<128, 128, 64, 64>(codes, gamma, xq, absmax, T, d_in, d_out, y, y_dtype, s);
}

}  // namespace sbl
