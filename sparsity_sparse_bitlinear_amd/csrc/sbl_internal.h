// Internal declarations shared by the HIP translation units of libsbl.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sbl.h"

namespace sbl {

// 16-byte load that is not kept in the caches (`nt`): for inputs read exactly once (x in the
// activation quantization, W in the packing's second pass), so that they do not push out of
// L2 and the last-level cache what the next kernels read again (x_q, the code plane).
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4*)p));
}


// ---------------------------------------------------------------------------
// Vector types used for MFMA operands and 16-byte memory traffic.
// ---------------------------------------------------------------------------
typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

#define SBL_LDS __attribute__((address_space(3)))

// Error reporting (thread-local detail text), implemented in api.hip.
void set_error(const char* fmt, ...);
int hip_fail(hipError_t e, const char* what);

// ---------------------------------------------------------------------------
// gamma: exact sum of |W| and its correctly rounded mean.
// ---------------------------------------------------------------------------

// Accumulation windows of the exact sum, by biased bf16 exponent E:
//   E in [kWinLo, kWinLo + 37]: summed in float64 per thread (every partial
//     sum of up to 256 such values is a multiple of 2^(kWinLo - 134) below
//     2^(kWinLo - 134 + 53), hence exact), flushed to a 128-bit integer in
//     units of 2^(kWinLo - 134) every 256 values;
//   E in [kWinLo, kWinLo + 56] (a group of 8 with any value outside the
//     float64 window): significand << (E - kWinLo) into the same integer;
//   anything else non-zero: an exact per-exponent histogram.
constexpr int kWinLo = 96;
constexpr int kWinHi = kWinLo + 56;
constexpr int kFastHi = kWinLo + 37;

// Partial results of one absum block (written to the workspace).
// Two float32 -> two bf16 (round to nearest even) in one word, lo in bits 0-15.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  typedef float v2f __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){lo, hi}, v2bf));
}

struct AbsumPartial {
  unsigned long long lo;    // 128-bit fast-window sum, low word
  unsigned long long hi;    // high word
  unsigned long long flag;  // non-zero iff the block has a histogram
  unsigned long long pad;
};

constexpr int kAbsumThreads = 256;
constexpr int kAbsumMaxBlocks = 1024;
constexpr int kPackBatchMax = 16;  // matrices per batched packing call

size_t quant_workspace_bytes(int64_t d_out, int64_t d_in);
int absum_blocks(int64_t n_vec8);

// N:M patterns with a packing kernel: M in {4, 8}, 1 <= N <= M.
bool mask_pattern_supported(int n_keep, int m_group);
hipError_t launch_quant_mask_pack(const uint16_t* W, int64_t d_out, int64_t d_in, int n_keep, int m_group,
                                  bool from_quantized, uint16_t* codes, uint8_t* mask, float* gamma, void* ws,
                                  hipStream_t s);
hipError_t launch_mask_grad(float* dW, const uint8_t* mask, int64_t d_out, int64_t d_in, hipStream_t s);

// Several matrices packed with three launches in all (quant.hip).
struct PackItem {
  const uint16_t* W;
  int64_t d_out, d_in;
  uint16_t* codes;
  uint8_t* mask;
  float* gamma;
};
size_t quant_batch_workspace_bytes(int count, const int64_t* n_weights);
hipError_t launch_quant_mask_pack_batch(int count, const PackItem* items, int n_keep, int m_group,
                                        bool from_quantized, void* ws, hipStream_t s);

// AdamW step + repack (quant.hip).  W, m, v updated in place.
struct AdamwArgs {
  float lr, beta1, beta2, eps, weight_decay, grad_scale;
  int64_t step;
};
hipError_t launch_adamw_repack(uint16_t* W, const float* g, float* m, float* v, int64_t d_out, int64_t d_in,
                               const AdamwArgs& a, int n_keep, int m_group, const uint8_t* mask_prev, uint8_t* mask,
                               uint16_t* codes, float* gamma, unsigned long long* flips, void* ws, hipStream_t s);

// Host/device: RN_float32(S * 2^-133 / count) for S given as 32-bit words.
__host__ __device__ float round_mean_words(const uint32_t* w, int nwords, unsigned long long count);

// ---------------------------------------------------------------------------
// activations, forward, backward launchers
// ---------------------------------------------------------------------------
hipError_t launch_act_quant(const uint16_t* x, int64_t T, int64_t d_in, int8_t* xq, float* absmax, hipStream_t s);
// RMSNorm + act quant (act.hip), d_in <= 16384.
bool rmsnorm_supported(int64_t d_in);
hipError_t launch_rmsnorm_act_quant(const uint16_t* x, const uint16_t* g, float eps, int64_t T, int64_t d_in,
                                    int8_t* xq, float* absmax, float* rstd, hipStream_t s);

// Compute units of the current device (cached per device).
int device_cus();

hipError_t launch_forward(const uint16_t* codes, const float* gamma, const int8_t* xq, const float* absmax,
                          int64_t T, int64_t d_in, int64_t d_out, void* y, int y_dtype, hipStream_t s);
// Forward on the kept-only 2:4 plane (2:8 and 2:4 masks; d_in % 128 == 0).
bool forward_sparse24_supported(int64_t d_in);
hipError_t launch_forward_sparse24(const uint8_t* plane, const float* gamma, const int8_t* xq, const float* absmax,
                                   int64_t T, int64_t d_in, int64_t d_out, void* y, int y_dtype, hipStream_t s);
// Code plane -> kept-only 2:4 plane (quant.hip); groups of 4 with more than 2
// non-zeros are counted into *bad (may be null).
hipError_t launch_pack_sparse24(const uint16_t* codes, int64_t d_out, int64_t d_in, uint8_t* plane,
                                unsigned long long* bad, hipStream_t s);

// Decode-size forward (decode.hip), T <= 64: the weights as the 2-bit code
// plane (SBL_PLANE_CODES, d_in % 64 == 0) or the pair plane (SBL_PLANE_PAIRS,
// d_in % 128 == 0; items[i].codes then points at bytes), up to
// kDecodeMultiMax matrices sharing one input.  fused: x is bf16 and the
// activation quantization runs in the launch (decode_fused_supported);
// otherwise x is x_q with absmax.
constexpr int kDecodeMultiMax = 4;
struct DecodeItem {
  const uint16_t* codes;
  const float* gamma;
  int64_t d_out;
  void* y;
};
bool decode_plane_supported(int format, int64_t T, int64_t d_in);
bool decode_fused_supported(int64_t T, int64_t d_in);
bool decode_fused_plane_supported(int format, int64_t T, int64_t d_in);
hipError_t launch_decode_plane(int format, int count, const DecodeItem* items, bool fused, const void* x,
                               const float* absmax, int64_t T, int64_t d_in, int y_dtype, hipStream_t s);
// Pair byte -> its 8 int8 values (bytes 252..255 are not produced: zeros).
__device__ inline uint2 pair_expand(uint32_t b) {
  if (b >= 252u) return make_uint2(0u, 0u);
  const uint32_t pr = b / 9u, cc = b - 9u * pr, d0 = cc / 3u, d1 = cc - 3u * d0;
  // pairs starting at a come after a (15 - a) / 2 others
  uint32_t p0 = 0;
  while (p0 < 6u && (p0 + 1u) * (14u - p0) / 2u <= pr) ++p0;
  const uint32_t p1 = pr - p0 * (15u - p0) / 2u + p0 + 1u;
  const unsigned long long v = ((unsigned long long)(d0 == 2u ? 0xFFu : d0) << (8u * p0)) |
                               ((unsigned long long)(d1 == 2u ? 0xFFu : d1) << (8u * p1));
  return make_uint2((uint32_t)v, (uint32_t)(v >> 32));
}

// The product of x_q for 17 to 64 tokens on the code plane or the pair plane
// (gemm_fwd.hip).
hipError_t launch_decode_codes_many(int count, const DecodeItem* items, bool pairs, const int8_t* xq,
                                    const float* absmax, int64_t T, int64_t d_in, int y_dtype, hipStream_t s);
// Code plane -> pair plane (masks keeping at most 2 of 8); groups with more
// than 2 non-zeros are written as 0 and counted into *bad (may be null).
hipError_t launch_pack_pairs(const uint16_t* codes, int64_t d_out, int64_t d_in, uint8_t* plane,
                             unsigned long long* bad, hipStream_t s);

// C[M, N] = alpha * A[M, K] B[N, K]^T, bf16 operands, float32 or bf16 output
// (gemm_nt.hip).  Only for shapes where gemm_nt_bf16_supported() holds.
// alpha == nullptr means 1.  With splits > 1 the K range is cut into pieces of
// k_per_split (a multiple of 64, none empty) and piece z writes its partial
// product to C + z * M * N.
bool gemm_nt_bf16_supported(int64_t M, int64_t N, int64_t K);
int64_t gemm_nt_bf16_tiles(int64_t M, int64_t N);
// AT != nullptr (splits == 1): also write A^T run-major, element (m, k) at
// (m / 8 * K + k) * 8 + m % 8 for m < at_ld (at_ld >= M, a multiple of 8; m
// from M to at_ld become zero); at_ld * K * 2 bytes must stay below 2 GiB.
hipError_t launch_gemm_nt_bf16(const uint16_t* A, const uint16_t* B, int64_t M, int64_t N, int64_t K,
                               const float* alpha, void* C, int out_dtype, hipStream_t s, int splits = 1,
                               int64_t k_per_split = 0, uint16_t* AT = nullptr, int64_t at_ld = 0);
// The same product (float32 C, alpha = 1) with B given run-major: B[n, k] at
// element (k / 8 * N + n) * 8 + k % 8 (K % 8 == 0), as written by k_xt_bf16
// (gemm_bwd.hip); with a_runs, A is run-major in the same way (as written by
// the AT side output below).  Only where gemm_nt_runs_supported() holds.
bool gemm_nt_runs_supported(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_nt_runs(const uint16_t* A, bool a_runs, const uint16_t* Brun, int64_t M, int64_t N, int64_t K,
                               void* C, hipStream_t s, int splits = 1, int64_t k_per_split = 0);
// The same product with B = W_eff^T given as the transposed 2-bit code plane of
// k_codes_t (gemm_bwd.hip): Bc [N, K64 / 16] words, K64 = K rounded up to 64.
// No split-K; AT as above.
// wscale != nullptr (with AT): the side output is scaled per row m, AT[k, m] =
// bf16(A[m, k] * wscale[m] * fl(1/127)).
hipError_t launch_gemm_nt_codes(const uint16_t* A, const uint32_t* Bc, int64_t M, int64_t N, int64_t K,
                                const float* alpha, void* C, int out_dtype, hipStream_t s, uint16_t* AT = nullptr,
                                int64_t at_ld = 0, const float* wscale = nullptr);
// The same product (float32 C, alpha = 1) with A run-major (as the scaled AT
// side output above writes it) and B given as int8 rows along K: Bq[k, n] =
// B[n, k], [kb_rows][N] row-major (rows kb_rows .. K read as zero), widened to
// bf16 exactly in registers.  Only where gemm_nt_q_supported() holds.
bool gemm_nt_q_supported(int64_t M, int64_t N, int64_t K, int64_t kb_rows);
// Split-K with a deeper split for the last tiles: the first `head` tiles of the
// grouped tile order take `splits` K ranges of k_per_split (a whole number of
// 256-block rounds), the rest take `tail_splits` ranges of tail_kps, partial
// product z of every tile in plane z of C (planes [max(splits, tail_splits)][M][N]),
// or, with `planes` set, plane 0 in C and plane z >= 1 at planes + (z - 1) M N.
// head == 0: every tile takes `splits` ranges.
struct SplitTail {
  int head, head_splits, tail_splits, tail_kps;
  float* planes;
};
hipError_t launch_gemm_nt_q(const uint16_t* Arun, const int8_t* Bq, int64_t M, int64_t N, int64_t K, int64_t kb_rows,
                            float* C, hipStream_t s, int splits = 1, int64_t k_per_split = 0,
                            SplitTail tail = SplitTail{0, 0, 0, 0, nullptr});

// Measurement helpers (peak.hip): the matrix instruction on register operands
// (kind 0: int8 32x32x32, 1: bf16 32x32x16; 4 chains per wave, iters each) and
// a streaming read of `bytes` bytes.
hipError_t launch_mfma_peak(int kind, int64_t iters, int blocks, float* sink, hipStream_t s);
hipError_t launch_read_peak(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s);

size_t backward_workspace_bytes(int64_t T, int64_t d_in, int64_t d_out, int flags);
hipError_t launch_backward(const uint16_t* codes, const float* gamma, const int8_t* xq, const float* absmax,
                           const uint16_t* dY, int64_t T, int64_t d_in, int64_t d_out, void* dX, int dx_dtype,
                           float* dW, int flags, void* ws, hipStream_t s);

}  // namespace sbl
