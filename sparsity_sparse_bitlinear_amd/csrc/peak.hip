// Measurement helpers: the matrix-core and memory rates this GPU reaches
// outside the operator, so that achieved rates can be read against a measured
// ceiling as well as the datasheet one.  Not part of Sparse-BitLinear.
//
// k_mfma_peak: every wave keeps kChains independent accumulators and issues
// the operator's matrix instruction (int8 32x32x32 or bf16 32x32x16) on
// register operands, iters times per chain; nothing is loaded in the loop.
// k_read_peak: grid-stride 16-byte loads of a buffer, four in flight per lane,
// folded into one word per thread so that no load is dead.
#include "sbl_internal.h"

namespace sbl {

namespace {

constexpr int kChains = 4;

template <bool I8>
__global__ __launch_bounds__(256) void k_mfma_peak(int64_t iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  if constexpr (I8) {
    v4i a = {lane, lane + 1, lane + 2, lane + 3}, b = {3 * lane, lane ^ 5, 7, lane * lane};
    v16i acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[c][r] = 0;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[c][r];
    if (s == 0x7FFFFFFF) sink[blockIdx.x] = (float)s;  // keeps the loop live; never true in practice
  } else {
    v8bf a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (__bf16)(0.001f * (float)(lane + e));
      b[e] = (__bf16)(0.002f * (float)(lane - e));
    }
    v16f acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[c][r];
    if (s == 12345.678f) sink[blockIdx.x] = s;
  }
}

__global__ __launch_bounds__(256) void k_read_peak(const uint4* __restrict__ src, int64_t n16,
                                                   uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t x = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
    x ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
    x ^= v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (x == 0x9E3779B9u) sink[0] = x;
}

}  // namespace

hipError_t launch_mfma_peak(int kind, int64_t iters, int blocks, float* sink, hipStream_t s) {
  if (kind == 0)
    hipLaunchKernelGGL(k_mfma_peak<true>, dim3(blocks), dim3(256), 0, s, iters, sink);
  else
    hipLaunchKernelGGL(k_mfma_peak<false>, dim3(blocks), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

hipError_t launch_read_peak(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const int blocks = 256 * 16;
  hipLaunchKernelGGL(k_read_peak, dim3(blocks), dim3(256), 0, s, (const uint4*)src, n16, sink);
  return hipGetLastError();
}

}  // namespace sbl
