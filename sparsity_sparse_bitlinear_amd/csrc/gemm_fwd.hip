// Forward product of Sparse-BitLinear on gfx950 int8 matrix cores.
//
// [SUM] 前置知识 > 半结构化 N:M 稀疏 (y = (W (.) M) x) and 方法步骤详情 step (6)
// (y ~= s * W_eff x~ with s absorbing the quantization scales):
//   acc[t,o] = sum_i x_q[t,i] * W_eff[o,i]   (exact int32)
//   y[t,o]   = acc[t,o] * gamma * a_t / 127
//
// C = A * B^T with A = x_q [T, d_in] (int8, K contiguous) and B = W_eff
// [d_out, d_in], streamed from the 2-bit code plane and expanded to int8
// {-1,0,+1} while it is written to LDS (once per block tile), so every wave
// reads plain int8 fragments.  v_mfma_i32_32x32x32_i8: lane l holds
// A[m = l%32][k = 16(l/32) + 0..15] and B[k = 16(l/32) + 0..15][n = l%32];
// accumulator register r of lane l is C[8(r/4) + 4(l/32) + r%4][l%32].
// Block tile 256 tokens x 128 outputs, K step 64 bytes.  Global loads are
// buffer loads through a per-tile resource, so rows past the matrix end read
// as zero; they run two K steps ahead of the matrix work.
#include "gemm_common.h"

namespace sbl {

namespace {

using namespace gemm;

// 4 two-bit codes (one byte) -> 4 int8 values.
__device__ __forceinline__ uint32_t expand4(uint32_t byte4codes) {
  uint32_t x = byte4codes & 0xFFu;
  x = (x | (x << 12)) & 0x000F000Fu;
  x = (x | (x << 6)) & 0x03030303u;
  // byte selector 0 -> 0x00, 1 -> 0x01, 3 -> 0xFF
  return __builtin_amdgcn_perm(0u, 0xFF000100u, x);
}

// 16 codes (two groups, one 32-bit word) -> 16 int8 values in natural k order.
__device__ __forceinline__ uint4 expand16(uint32_t w) {
  return make_uint4(expand4(w), expand4(w >> 8), expand4(w >> 16), expand4(w >> 24));
}

// VEC: d_in % 64 == 0 (whole K steps, 16-byte aligned rows, 8-group code words).
template <int OUT, bool VEC>
__global__ __launch_bounds__(kThreads, 2) void k_fwd_i8(const int8_t* __restrict__ xq,
                                                        const uint16_t* __restrict__ codes,
                                                        const float* __restrict__ gamma_p,
                                                        const float* __restrict__ absmax, int T, int d_in,
                                                        int d_out, void* __restrict__ y) {
  constexpr int CA = kBM * 4 / kThreads;  // 16-byte A chunks per thread
  __shared__ __attribute__((aligned(16))) char lds[2 * (kBM + kBN) * kRow];
  char* As = lds;
  char* Bs = lds + 2 * kBM * kRow;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm0 = (wave >> 1) * kWM;
  const int wn0 = (wave & 1) * kWN;
  int mt, nt;
  xcd_tile(blockIdx.x, (T + kBM - 1) / kBM, (d_out + kBN - 1) / kBN, mt, nt);
  const int m0 = mt * kBM;
  const int n0 = nt * kBN;
  const int G = d_in >> 3;  // code groups per row
  const int nk = (d_in + 63) / 64;
  const int rows_a = min(kBM, T - m0);
  const int rows_b = min(kBN, d_out - n0);
  const int8_t* a_base = xq + (int64_t)m0 * d_in;
  const uint16_t* b_base = codes + (int64_t)n0 * G;

  // Lane offsets relative to the K-step base (fixed over the K loop).
  uint32_t a_off[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int q = tid + kThreads * i;
    a_off[i] = (uint32_t)((q >> 2) * d_in + 16 * (q & 3));
  }
  const int b_row = tid >> 1, b_half = tid & 1;  // code row, half (4 groups = 32 k)
  const uint32_t b_off = (uint32_t)(b_row * G * 2 + 8 * b_half);

  uint4 ra[2][CA];
  uint2 rb[2];

  auto load_tile = [&](int kt, int st) {
    const int k0 = kt * 64;
    const auto ar = make_rsrc(a_base + k0, clamp_bytes((int64_t)rows_a * d_in - k0));
    const auto br = make_rsrc(b_base + kt * 8, clamp_bytes(((int64_t)rows_b * G - kt * 8) * 2));
    if constexpr (VEC) {
#pragma unroll
      for (int i = 0; i < CA; ++i) ra[st][i] = bload16(ar, a_off[i]);
      rb[st] = bload8(br, b_off);
    } else {
      // K tail: 8-byte pieces of A and single code words past the row end read as zero
#pragma unroll
      for (int i = 0; i < CA; ++i) {
        const int k = k0 + 16 * ((tid + kThreads * i) & 3);
        const uint2 lo = bload8(ar, k < d_in ? a_off[i] : kOOB);
        const uint2 hi = bload8(ar, k + 8 < d_in ? a_off[i] + 8 : kOOB);
        ra[st][i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
      const int g0 = kt * 8 + 4 * b_half;
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = bload2(br, g0 + j < G ? b_off + 2 * j : kOOB);
      rb[st] = make_uint2(w[0] | (w[1] << 16), w[2] | (w[3] << 16));
    }
  };
  auto store_tile = [&](int buf, int st) {
    char* a = As + buf * kBM * kRow;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int q = tid + kThreads * i;
      *(uint4*)(a + swz(q >> 2, q & 3)) = ra[st][i];
    }
    char* b = Bs + buf * kBN * kRow;
    *(uint4*)(b + swz(b_row, 2 * b_half)) = expand16(rb[st].x);
    *(uint4*)(b + swz(b_row, 2 * b_half + 1)) = expand16(rb[st].y);
  };

  v16i acc[kMI][kNJ];
#pragma unroll
  for (int i = 0; i < kMI; ++i)
#pragma unroll
    for (int j = 0; j < kNJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  auto compute = [&](int buf) {
    const char* a = As + buf * kBM * kRow;
    const char* b = Bs + buf * kBN * kRow;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v4i fa[kMI], fb[kNJ];
#pragma unroll
      for (int i = 0; i < kMI; ++i) fa[i] = frag(a, wm0 + 32 * i, ks, lane);
#pragma unroll
      for (int j = 0; j < kNJ; ++j) fb[j] = frag(b, wn0 + 32 * j, ks, lane);
#pragma unroll
      for (int i = 0; i < kMI; ++i)
#pragma unroll
        for (int j = 0; j < kNJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };

  // Software pipeline over K steps: tile k sits in register stage k % 2 and LDS
  // buffer k % 2.  Each step issues the loads of tile k + 2, multiplies tile k
  // and writes tile k + 1 to LDS.  Tile indices past the end are clamped (the
  // extra loads and stores are never multiplied), keeping the loop body free
  // of conditionals.
  const int last = nk - 1;
  load_tile(0, 0);
  load_tile(min(1, last), 1);
  store_tile(0, 0);
  __syncthreads();
  int k = 0;
  for (; k + 2 <= nk; k += 2) {
    load_tile(min(k + 2, last), 0);
    compute(0);
    store_tile(1, 1);
    __syncthreads();
    load_tile(min(k + 3, last), 1);
    compute(1);
    store_tile(0, 0);
    __syncthreads();
  }
  if (k < nk) compute(0);

  // Epilogue: y = acc * gamma * a_t / 127 (or the raw int32 sums).
  const float g127 = *gamma_p * (1.0f / 127.0f);
#pragma unroll
  for (int i = 0; i < kMI; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm0 + 32 * i + acc_row(r, lane);
      if (m >= T) continue;
      const float s = g127 * absmax[m];
#pragma unroll
      for (int j = 0; j < kNJ; ++j) {
        const int n = n0 + wn0 + 32 * j + (lane & 31);
        if (n >= d_out) continue;
        const int64_t off = (int64_t)m * d_out + n;
        if constexpr (OUT == SBL_I32) {
          ((int*)y)[off] = acc[i][j][r];
        } else if constexpr (OUT == SBL_F32) {
          ((float*)y)[off] = (float)acc[i][j][r] * s;
        } else {
          ((__bf16*)y)[off] = (__bf16)((float)acc[i][j][r] * s);
        }
      }
    }
  }
}

template <bool VEC>
hipError_t launch_fwd_v(const uint16_t* codes, const float* gamma, const int8_t* xq, const float* absmax, int64_t T,
                        int64_t d_in, int64_t d_out, void* y, int y_dtype, hipStream_t s) {
  const int64_t nb = ((d_out + kBN - 1) / kBN) * ((T + kBM - 1) / kBM);
  const dim3 grid((unsigned)nb), block(kThreads);
  switch (y_dtype) {
    case SBL_F32:
      hipLaunchKernelGGL((k_fwd_i8<SBL_F32, VEC>), grid, block, 0, s, xq, codes, gamma, absmax, (int)T, (int)d_in,
                         (int)d_out, y);
      break;
    case SBL_BF16:
      hipLaunchKernelGGL((k_fwd_i8<SBL_BF16, VEC>), grid, block, 0, s, xq, codes, gamma, absmax, (int)T, (int)d_in,
                         (int)d_out, y);
      break;
    default:
      hipLaunchKernelGGL((k_fwd_i8<SBL_I32, VEC>), grid, block, 0, s, xq, codes, gamma, absmax, (int)T, (int)d_in,
                         (int)d_out, y);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward(const uint16_t* codes, const float* gamma, const int8_t* xq, const float* absmax,
                          int64_t T, int64_t d_in, int64_t d_out, void* y, int y_dtype, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (d_in % 64 == 0) return launch_fwd_v<true>(codes, gamma, xq, absmax, T, d_in, d_out, y, y_dtype, s);
  return launch_fwd_v<false>(codes, gamma, xq, absmax, T, d_in, d_out, y, y_dtype, s);
}

}  // namespace sbl
