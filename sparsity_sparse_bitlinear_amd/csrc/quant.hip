// Weight side of Sparse-BitLinear on gfx950: gamma = mean|W| (exact), the N:8
// top-N mask on |W|, ternary codes and the packed planes.
//
// [SUM] 前置知识 > 1.58-bit BitNet 量化 defines gamma = ||W||_1 / (d_out d_in)
// and W_q = RoundClip(W/gamma, -1, 1); 前置知识 > 半结构化 N:M 稀疏 defines the
// N-of-M group mask; 核心方法 (i)-(iii) computes the mask from |W| of the
// master weight and applies it after quantization ([GIST] 2.2 likewise).
//
// Three launches, all on the caller's stream:
//   k_absum          pass 1 over W: exact partial sums of |W| per block (float64
//                    window sums flushed to 128-bit integers, integer fallback)
//   k_gamma_finalize one block: exact total, one correctly rounded division
//   k_mask_quant_pack pass 2 over W: per 8-group sorting network -> keep bits,
//                     threshold |w| > gamma/2 -> 2-bit codes, write both planes
//                     (N:8 for any N, N:4 such as 2:4 as two groups per word,
//                     and the mask-from-quantized-weight ablation)
// plus k_mask_grad, the mask-without-grad ablation on a dW buffer.
#include <cmath>

#include "sbl_internal.h"

namespace sbl {

// ---------------------------------------------------------------------------
// Exact rounding of the mean (host and device).
// ---------------------------------------------------------------------------

// Word idx of the little-endian word array (zero outside it).
__host__ __device__ static inline uint32_t word_at(const uint32_t* w, int nwords, int idx) {
  return (idx >= 0 && idx < nwords) ? w[idx] : 0u;
}

// 64 bits of S starting at bit position lo (lo may be negative; bits below 0
// read as zero).
__host__ __device__ static inline unsigned long long bits64(const uint32_t* w, int nwords, int lo) {
  const int q = lo >= 0 ? lo >> 5 : -((31 - lo) >> 5);  // floor(lo / 32)
  const int r = lo - 32 * q;                           // 0..31
  const unsigned long long w0 = word_at(w, nwords, q), w1 = word_at(w, nwords, q + 1);
  const unsigned long long w2 = word_at(w, nwords, q + 2);
  const unsigned long long low = w0 | (w1 << 32);
  return r ? ((low >> r) | (w2 << (64 - r))) : low;
}

// True iff any bit of S below position lo (exclusive) is set.
__host__ __device__ static inline bool any_below(const uint32_t* w, int nwords, int lo) {
  if (lo <= 0) return false;
  const int q = lo >> 5, r = lo & 31;
  for (int i = 0; i < q && i < nwords; ++i)
    if (w[i]) return true;
  return r && q < nwords && (w[q] & ((1u << r) - 1u));
}

// S = sum of nwords little-endian 32-bit words, in units of 2^-133.
// Returns the binary32 value nearest to S * 2^-133 / count (ties to even).
// Requires 1 <= count < 2^37 so that the 64-bit quotient below keeps at least
// 27 significant bits.
__host__ __device__ float round_mean_words(const uint32_t* w, int nwords, unsigned long long count) {
  int top = -1;
  for (int i = nwords - 1; i >= 0; --i) {
    if (w[i]) { top = i; break; }
  }
  if (top < 0) return 0.0f;
  const int p = top * 32 + 31 - __builtin_clz(w[top]);  // position of the leading one
  // M = bits [p-63, p] of S (left-aligned 64-bit window), sticky = any lower bit.
  const unsigned long long M = bits64(w, nwords, p - 63);
  bool sticky = any_below(w, nwords, p - 63);
  // value = (M + f) * 2^(p - 63 - 133) / count, f in [0, 1) (f > 0 iff sticky)
  const unsigned long long Q = M / count;
  const unsigned long long R = M % count;
  sticky = sticky || (R != 0);
  const int base_exp = p - 63 - 133;  // value = (Q + frac) * 2^base_exp, frac in [0,1)
  const int qb = 64 - __builtin_clzll(Q);
  const int e_top = qb - 1 + base_exp;
  int shift = (e_top >= -126) ? (qb - 24) : (-149 - base_exp);
  if (shift > 64) return 0.0f;  // below half of the smallest subnormal
  unsigned long long kept, rem, half;
  if (shift == 64) {
    kept = 0; rem = Q; half = 1ull << 63;
  } else {
    kept = Q >> shift;
    rem = Q & ((1ull << shift) - 1);
    half = 1ull << (shift - 1);
  }
  if (rem > half || (rem == half && (sticky || (kept & 1)))) kept += 1;
  return ldexpf((float)kept, shift + base_exp);
}

// ---------------------------------------------------------------------------
// Pass 1: exact partial sums of |W|.
// ---------------------------------------------------------------------------

struct U128 {
  unsigned long long lo, hi;
};

__device__ __forceinline__ void add128(U128& a, const U128& b) {
  const unsigned long long lo = a.lo + b.lo;
  a.hi += b.hi + (lo < a.lo ? 1ull : 0ull);
  a.lo = lo;
}

__device__ __forceinline__ void absum_half(uint32_t h, U128& acc, unsigned long long* hist, bool& any_hist) {
  const uint32_t mag = h & 0x7FFFu;
  const uint32_t e = mag >> 7;
  const uint32_t sig = (mag & 0x7Fu) | (e ? 0x80u : 0u);
  const uint32_t ee = e ? e : 1u;
  const uint32_t off = ee - (uint32_t)kWinLo;  // wraps for ee < kWinLo
  const bool in = off <= (uint32_t)(kWinHi - kWinLo);
  const unsigned long long v = (unsigned long long)(in ? sig : 0u) << (in ? off : 0u);
  const unsigned long long lo = acc.lo + v;
  acc.hi += (lo < acc.lo) ? 1ull : 0ull;
  acc.lo = lo;
  if (__builtin_expect(!in && sig != 0u, 0)) {
    atomicAdd(&hist[ee], (unsigned long long)sig);
    any_hist = true;
  }
}

// True iff every non-zero magnitude of the 8 values has its exponent in the
// float64 window [kWinLo, kFastHi].
__device__ __forceinline__ bool in_fast_window(const uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  bool ok = true;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t mag = (w[i] >> (16 * h)) & 0x7FFFu;
      ok = ok && (mag == 0u || ((mag >> 7) - (uint32_t)kWinLo) <= (uint32_t)(kFastHi - kWinLo));
    }
  }
  return ok;
}

// Block blk of nblk over one matrix: its exact partial sum into *part, its
// histogram (if any value fell outside the float64 window) into hist_out[0..256).
__device__ __forceinline__ void absum_body(const uint4* __restrict__ W, int64_t n_vec8, int nblk, int blk,
                                           AbsumPartial* __restrict__ part,
                                           unsigned long long* __restrict__ hist_out) {
  __shared__ unsigned long long hist[256];
  __shared__ U128 red[kAbsumThreads];
  __shared__ int block_any;
  const int tid = threadIdx.x;
  hist[tid] = 0;
  if (tid == 0) block_any = 0;
  __syncthreads();

  U128 acc = {0, 0};
  // kU independent float64 window sums, each exact while it holds at most 256
  // window values (flushed every 32 rounds of 8); kU loads in flight per round.
  constexpr int kU = 4;
  double fsum[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) fsum[u] = 0.0;
  int fcount = 0;
  bool any_hist = false;
  auto one = [&](const uint4 v, double& fs) {
    if (__builtin_expect(in_fast_window(v), 1)) {
      fs += (double)__uint_as_float((v.x & 0x7FFFu) << 16) + (double)__uint_as_float(v.x & 0x7FFF0000u);
      fs += (double)__uint_as_float((v.y & 0x7FFFu) << 16) + (double)__uint_as_float(v.y & 0x7FFF0000u);
      fs += (double)__uint_as_float((v.z & 0x7FFFu) << 16) + (double)__uint_as_float(v.z & 0x7FFF0000u);
      fs += (double)__uint_as_float((v.w & 0x7FFFu) << 16) + (double)__uint_as_float(v.w & 0x7FFF0000u);
    } else {
      absum_half(v.x & 0xFFFFu, acc, hist, any_hist);
      absum_half(v.x >> 16, acc, hist, any_hist);
      absum_half(v.y & 0xFFFFu, acc, hist, any_hist);
      absum_half(v.y >> 16, acc, hist, any_hist);
      absum_half(v.z & 0xFFFFu, acc, hist, any_hist);
      absum_half(v.z >> 16, acc, hist, any_hist);
      absum_half(v.w & 0xFFFFu, acc, hist, any_hist);
      absum_half(v.w >> 16, acc, hist, any_hist);
    }
  };
  // move the exact integers fsum * 2^(134 - kWinLo) < 2^53 into the 128-bit sum
  auto flush = [&]() {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const U128 f = {(unsigned long long)ldexp(fsum[u], 134 - kWinLo), 0ull};
      add128(acc, f);
      fsum[u] = 0.0;
    }
  };
  const int64_t stride = (int64_t)nblk * kAbsumThreads;
  int64_t i = (int64_t)blk * kAbsumThreads + tid;
  for (; i + (kU - 1) * stride < n_vec8; i += kU * stride) {
    uint4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = W[i + u * stride];
#pragma unroll
    for (int u = 0; u < kU; ++u) one(v[u], fsum[u]);
    if (++fcount == 32) {
      flush();
      fcount = 0;
    }
  }
  flush();
  for (; i < n_vec8; i += stride) one(W[i], fsum[0]);  // fewer than kU more: at most 24 values
  flush();
  if (any_hist) block_any = 1;  // benign race: every writer stores 1
  red[tid] = acc;
  __syncthreads();
  for (int s = kAbsumThreads / 2; s > 0; s >>= 1) {
    if (tid < s) {
      U128 a = red[tid];
      add128(a, red[tid + s]);
      red[tid] = a;
    }
    __syncthreads();
  }
  const int any = block_any;
  if (tid == 0) {
    AbsumPartial p;
    p.lo = red[0].lo;
    p.hi = red[0].hi;
    p.flag = (unsigned long long)any;
    p.pad = 0;
    *part = p;
  }
  if (any) hist_out[tid] = hist[tid];
}

__global__ __launch_bounds__(kAbsumThreads) void k_absum(const uint4* __restrict__ W, int64_t n_vec8,
                                                         AbsumPartial* __restrict__ part,
                                                         unsigned long long* __restrict__ hist_out) {
  absum_body(W, n_vec8, gridDim.x, blockIdx.x, part + blockIdx.x, hist_out + (size_t)blockIdx.x * 256);
}

// Adds v * 2^shift into the little-endian word array w[0..nw).
__device__ void add_shifted(uint32_t* w, int nw, unsigned long long v, int shift) {
  if (!v) return;
  int q = shift >> 5;
  const int r = shift & 31;
  uint32_t parts[3];
  parts[0] = (uint32_t)(v << r);
  parts[1] = (uint32_t)(r ? (v >> (32 - r)) : (v >> 32));
  parts[2] = (uint32_t)(r ? (v >> (64 - r)) : 0ull);
  unsigned long long carry = 0;
  for (int k = 0; q + k < nw; ++k) {
    const unsigned long long s = (unsigned long long)w[q + k] + (k < 3 ? parts[k] : 0u) + carry;
    w[q + k] = (uint32_t)s;
    carry = s >> 32;
    if (k >= 2 && carry == 0) break;
  }
}

constexpr int kSumWords = 10;  // 320 bits: enough for any finite bf16 matrix below 2^40 weights

__device__ __forceinline__ void finalize_body(const AbsumPartial* __restrict__ part,
                                              const unsigned long long* __restrict__ hist_in, int nblocks,
                                              unsigned long long count, float* __restrict__ gamma,
                                              unsigned long long* __restrict__ flips) {
  __shared__ U128 red[256];
  __shared__ unsigned long long fl[256];
  __shared__ unsigned long long bins[256];
  __shared__ int flags[256];
  __shared__ int any_flag;
  const int tid = threadIdx.x;
  if (tid == 0) any_flag = 0;
  __syncthreads();
  U128 acc = {0, 0};
  unsigned long long nflip = 0;
  int any = 0;
  for (int b = tid; b < nblocks; b += 256) {
    const AbsumPartial p = part[b];
    U128 v = {p.lo, p.hi};
    add128(acc, v);
    nflip += p.pad;
    any |= (p.flag != 0);
  }
  if (any) any_flag = 1;
  red[tid] = acc;
  fl[tid] = nflip;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) {
      U128 a = red[tid];
      add128(a, red[tid + s]);
      red[tid] = a;
      fl[tid] += fl[tid + s];
    }
    __syncthreads();
  }
  if (flips && tid == 0) *flips = fl[0];
  // Histogram bins of the blocks that have one: the flags are staged in LDS so
  // that the serial walk over blocks reads global memory only for flagged ones.
  unsigned long long bin = 0;
  if (any_flag) {
    for (int b0 = 0; b0 < nblocks; b0 += 256) {
      __syncthreads();
      flags[tid] = (b0 + tid < nblocks) ? (part[b0 + tid].flag != 0) : 0;
      __syncthreads();
      const int nb = min(256, nblocks - b0);
      for (int b = 0; b < nb; ++b)
        if (flags[b]) bin += hist_in[(size_t)(b0 + b) * 256 + tid];
    }
  }
  bins[tid] = bin;
  __syncthreads();
  if (tid == 0) {
    uint32_t w[kSumWords];
    for (int i = 0; i < kSumWords; ++i) w[i] = 0;
    // fast window: units of 2^(kWinLo - 134) = 2^(kWinLo - 1) * 2^-133
    add_shifted(w, kSumWords, red[0].lo, kWinLo - 1);
    add_shifted(w, kSumWords, red[0].hi, kWinLo - 1 + 64);
    // histogram bin e (biased exponent, >= 1): units of 2^(e - 134) = 2^(e - 1) * 2^-133
    if (any_flag)
      for (int e = 1; e < 255; ++e) add_shifted(w, kSumWords, bins[e], e - 1);
    *gamma = round_mean_words(w, kSumWords, count);
  }
}

__global__ __launch_bounds__(256) void k_gamma_finalize(const AbsumPartial* __restrict__ part,
                                                        const unsigned long long* __restrict__ hist_in,
                                                        int nblocks, unsigned long long count,
                                                        float* __restrict__ gamma,
                                                        unsigned long long* __restrict__ flips) {
  finalize_body(part, hist_in, nblocks, count, gamma, flips);
}

// ---------------------------------------------------------------------------
// Pass 2: mask, ternary codes, packing.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void cswap_desc(uint32_t& a, uint32_t& b) {
  const uint32_t hi = max(a, b), lo = min(a, b);
  a = hi;
  b = lo;
}

// One word of 8 bf16 values (4 words of the row).  Rank keys
// u_j = (key_j << 3) | (7 - j) are distinct and order slots by key, lower index
// first on ties; the key is the 15-bit |w| bit pattern (the mask
// Pi_{N:M}(|W|) of the master weight) or, for the "mask from quantized weight"
// ablation (FQ), |W_q| in {0, 1}.  M = 8: one group, an optimal 19-comparator
// network sorts the keys and the N-th largest is the keep threshold.  M = 4:
// two groups (slots 0-3 and 4-7), each sorted by a 5-comparator network.
// |w| > gamma/2  <=>  2|w| > gamma.  Both sides are non-negative binary32
// values, compared through their bit patterns (monotone for non-negative
// floats), so no floating-point mode (denormal flushing) can change the
// decision.  Doubling a magnitude in bit form: add one to the exponent of a
// normal value (values near the top become inf/NaN patterns, which still
// compare above every finite gamma), shift a subnormal left by one.
__device__ __forceinline__ bool above_half_gamma(uint32_t mag16, uint32_t gamma_bits) {
  const uint32_t b = mag16 << 16;
  const uint32_t twice = (b & 0x7F800000u) ? (b + 0x00800000u) : (b << 1);
  return twice > gamma_bits;
}

// N-th largest of 4 keys (descending network: (0,1) (2,3) (0,2) (1,3) (1,2)).
template <int N>
__device__ __forceinline__ uint32_t nth_of4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  cswap_desc(a, b); cswap_desc(c, d); cswap_desc(a, c); cswap_desc(b, d); cswap_desc(b, c);
  return N == 1 ? a : N == 2 ? b : N == 3 ? c : d;
}

// Keep bits (bit j = slot j) of N:M on the 8 rank keys u[j] (distinct).
template <int N, int M>
__device__ __forceinline__ uint32_t keep_bits(const uint32_t (&u)[8]) {
  uint32_t thr_lo = 0, thr_hi = 0;
  if constexpr (M == 8 && N < 8) {
    uint32_t s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = u[j];
    cswap_desc(s[0], s[2]); cswap_desc(s[1], s[3]); cswap_desc(s[4], s[6]); cswap_desc(s[5], s[7]);
    cswap_desc(s[0], s[4]); cswap_desc(s[1], s[5]); cswap_desc(s[2], s[6]); cswap_desc(s[3], s[7]);
    cswap_desc(s[0], s[1]); cswap_desc(s[2], s[3]); cswap_desc(s[4], s[5]); cswap_desc(s[6], s[7]);
    cswap_desc(s[2], s[4]); cswap_desc(s[3], s[5]);
    cswap_desc(s[1], s[4]); cswap_desc(s[3], s[6]);
    cswap_desc(s[1], s[2]); cswap_desc(s[3], s[4]); cswap_desc(s[5], s[6]);
    thr_lo = thr_hi = s[N - 1];
  } else if constexpr (M == 4 && N < 4) {
    thr_lo = nth_of4<N>(u[0], u[1], u[2], u[3]);
    thr_hi = nth_of4<N>(u[4], u[5], u[6], u[7]);
  }
  uint32_t mask = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) mask |= ((N == M) || (u[j] >= (j < 4 ? thr_lo : thr_hi)) ? 1u : 0u) << j;
  return mask;
}

// Rank keys of the magnitude mask: (15-bit |w| bits << 3) | (7 - j).
__device__ __forceinline__ void mag_keys(const uint32_t (&h)[8], uint32_t (&u)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) u[j] = ((h[j] & 0x7FFFu) << 3) | (uint32_t)(7 - j);
}

// 2-bit codes of the 8 slots: kept and |w| > gamma/2 -> sign code.
__device__ __forceinline__ uint16_t codes_of(const uint32_t (&h)[8], uint32_t mask, uint32_t gamma_bits) {
  uint32_t code = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bool nz = ((mask >> j) & 1u) && above_half_gamma(h[j] & 0x7FFFu, gamma_bits);
    code |= (nz ? ((h[j] & 0x8000u) ? 3u : 1u) : 0u) << (2 * j);
  }
  return (uint16_t)code;
}

template <int N, int M, bool FQ>
__device__ __forceinline__ void pack_group(const uint4 v, uint32_t gamma_bits, uint16_t& code_out,
                                           uint8_t& mask_out) {
  const uint32_t h[8] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16,
                         v.z & 0xFFFFu, v.z >> 16, v.w & 0xFFFFu, v.w >> 16};
  uint32_t u[8];
  if constexpr (FQ) {
#pragma unroll
    for (int j = 0; j < 8; ++j) u[j] = ((above_half_gamma(h[j] & 0x7FFFu, gamma_bits) ? 1u : 0u) << 3) | (uint32_t)(7 - j);
  } else {
    mag_keys(h, u);
  }
  const uint32_t mask = keep_bits<N, M>(u);
  code_out = codes_of(h, mask, gamma_bits);
  mask_out = (uint8_t)mask;
}

// A block takes 4 x 256 consecutive groups per round (each thread 4 groups,
// 256 apart, so every load and store instruction is contiguous); the four
// loads are issued before any group is packed.
template <int N, int M, bool FQ>
__device__ __forceinline__ void mqp_body(const uint4* __restrict__ W, int64_t n_groups,
                                         const float* __restrict__ gamma_p, uint16_t* __restrict__ codes,
                                         uint8_t* __restrict__ mask, int nblk, int blk) {
  constexpr int kU = 4;
  const uint32_t gamma_bits = __float_as_uint(*gamma_p);
  const int64_t stride = (int64_t)nblk * 256 * kU;
  for (int64_t g0 = (int64_t)blk * 256 * kU + threadIdx.x; g0 < n_groups; g0 += stride) {
    uint4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = g0 + 256 * u < n_groups ? load_nt16(W + g0 + 256 * u) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t g = g0 + 256 * u;
      if (g >= n_groups) break;
      uint16_t c;
      uint8_t m;
      pack_group<N, M, FQ>(v[u], gamma_bits, c, m);
      codes[g] = c;
      if (mask) mask[g] = m;
    }
  }
}

template <int N, int M, bool FQ>
__global__ __launch_bounds__(256) void k_mask_quant_pack(const uint4* __restrict__ W, int64_t n_groups,
                                                         const float* __restrict__ gamma_p,
                                                         uint16_t* __restrict__ codes, uint8_t* __restrict__ mask) {
  mqp_body<N, M, FQ>(W, n_groups, gamma_p, codes, mask, gridDim.x, blockIdx.x);
}

// ---------------------------------------------------------------------------
// Several matrices in one launch per pass (a layer's linears): the blocks of
// the grid are dealt to the matrices by the prefix sums in the descriptor, so
// the three launches cover every matrix and the small ones stop costing a
// launch each.
// ---------------------------------------------------------------------------
struct PackBatch {
  int count;
  const uint4* W[kPackBatchMax];
  int64_t n_groups[kPackBatchMax];
  uint16_t* codes[kPackBatchMax];
  uint8_t* mask[kPackBatchMax];
  float* gamma[kPackBatchMax];
  int absum_begin[kPackBatchMax + 1];  // absum blocks of matrix i: [absum_begin[i], absum_begin[i + 1])
  int pack_begin[kPackBatchMax + 1];   // packing blocks, likewise
};

__device__ __forceinline__ int batch_item(const int* begin, int count, int b) {
  int i = 0;
  while (i + 1 < count && b >= begin[i + 1]) ++i;
  return i;
}

__global__ __launch_bounds__(kAbsumThreads) void k_absum_batch(PackBatch pb, AbsumPartial* __restrict__ part,
                                                               unsigned long long* __restrict__ hist_out) {
  const int i = batch_item(pb.absum_begin, pb.count, blockIdx.x);
  absum_body(pb.W[i], pb.n_groups[i], pb.absum_begin[i + 1] - pb.absum_begin[i], blockIdx.x - pb.absum_begin[i],
             part + blockIdx.x, hist_out + (size_t)blockIdx.x * 256);
}

__global__ __launch_bounds__(256) void k_gamma_finalize_batch(PackBatch pb, const AbsumPartial* __restrict__ part,
                                                              const unsigned long long* __restrict__ hist_in) {
  const int i = blockIdx.x;
  const int b0 = pb.absum_begin[i];
  finalize_body(part + b0, hist_in + (size_t)b0 * 256, pb.absum_begin[i + 1] - b0,
                (unsigned long long)pb.n_groups[i] * 8ull, pb.gamma[i], nullptr);
}

template <int N, int M, bool FQ>
__global__ __launch_bounds__(256) void k_mask_quant_pack_batch(PackBatch pb) {
  const int i = batch_item(pb.pack_begin, pb.count, blockIdx.x);
  mqp_body<N, M, FQ>(pb.W[i], pb.n_groups[i], pb.gamma[i], pb.codes[i], pb.mask[i],
                     pb.pack_begin[i + 1] - pb.pack_begin[i], blockIdx.x - pb.pack_begin[i]);
}

// "Mask without grad" ablation: dW[o, i] = +0 where slot i of the mask plane
// is clear.  One thread per 8-slot group: two 16-byte loads and stores of dW,
// one mask byte.
__global__ __launch_bounds__(256) void k_mask_grad(float4* __restrict__ dW, const uint8_t* __restrict__ mask,
                                                   int64_t n_groups) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < n_groups; g += stride) {
    const uint32_t m = mask[g];
    float4 a = dW[2 * g], b = dW[2 * g + 1];
    a.x = (m & 1u) ? a.x : 0.0f;
    a.y = (m & 2u) ? a.y : 0.0f;
    a.z = (m & 4u) ? a.z : 0.0f;
    a.w = (m & 8u) ? a.w : 0.0f;
    b.x = (m & 16u) ? b.x : 0.0f;
    b.y = (m & 32u) ? b.y : 0.0f;
    b.z = (m & 64u) ? b.z : 0.0f;
    b.w = (m & 128u) ? b.w : 0.0f;
    dW[2 * g] = a;
    dW[2 * g + 1] = b;
  }
}

// ---------------------------------------------------------------------------
// Optimizer step + repack ([SUM] 方法步骤详情 step (8), then step (2) of the next
// step): AdamW on the bf16 master weight, and in the same pass over W the new
// mask, its flips against the previous one and the exact |W'| partial sums;
// gamma and the codes follow in the two launches after it.
// ---------------------------------------------------------------------------

// Host-folded hyper-parameters: m' = b1 m + c1 g, v' = b2 v + c2 g^2 (g scaled
// by gs), W' = W decay - step_size m' / (sqrt(v') / sqrt_bc2 + eps), the
// arithmetic of torch.optim.AdamW in float32 with one rounding of W' to bf16.
struct AdamHp {
  float b1, c1, b2, c2, gs, step_size, sqrt_bc2, eps, decay;
};

template <int N, int M>
__global__ __launch_bounds__(kAbsumThreads) void k_adamw_mask(uint4* __restrict__ W, const float4* __restrict__ g,
                                                              float4* __restrict__ mo, float4* __restrict__ vo,
                                                              int64_t n_groups, AdamHp hp,
                                                              const uint8_t* __restrict__ mask_prev,
                                                              uint8_t* __restrict__ mask,
                                                              AbsumPartial* __restrict__ part,
                                                              unsigned long long* __restrict__ hist_out) {
  __shared__ unsigned long long hist[256];
  __shared__ U128 red[kAbsumThreads];
  __shared__ unsigned long long fred[kAbsumThreads];
  __shared__ int block_any;
  const int tid = threadIdx.x;
  hist[tid] = 0;
  if (tid == 0) block_any = 0;
  __syncthreads();

  U128 acc = {0, 0};
  double fsum = 0.0;  // exact while it holds at most 256 window values
  int fcount = 0;
  bool any_hist = false;
  unsigned long long nflip = 0;
  const int64_t stride = (int64_t)gridDim.x * kAbsumThreads;
  for (int64_t i = (int64_t)blockIdx.x * kAbsumThreads + tid; i < n_groups; i += stride) {
    const uint4 w = W[i];
    const float4 g0 = g[2 * i], g1 = g[2 * i + 1];
    float4 m0 = mo[2 * i], m1 = mo[2 * i + 1], v0 = vo[2 * i], v1 = vo[2 * i + 1];
    const uint32_t prev = mask_prev ? mask_prev[i] : 0u;
    float wv[8] = {__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                   __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u),
                   __uint_as_float(w.z << 16), __uint_as_float(w.z & 0xFFFF0000u),
                   __uint_as_float(w.w << 16), __uint_as_float(w.w & 0xFFFF0000u)};
    const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    float mv[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
    float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float gj = gv[j] * hp.gs;
      mv[j] = hp.b1 * mv[j] + hp.c1 * gj;
      vv[j] = hp.b2 * vv[j] + hp.c2 * (gj * gj);
      const float denom = sqrtf(vv[j]) / hp.sqrt_bc2 + hp.eps;
      wv[j] = wv[j] * hp.decay - hp.step_size * (mv[j] / denom);
    }
    const uint4 wn = make_uint4(cvt_pk_bf16(wv[0], wv[1]), cvt_pk_bf16(wv[2], wv[3]), cvt_pk_bf16(wv[4], wv[5]),
                                cvt_pk_bf16(wv[6], wv[7]));
    W[i] = wn;
    mo[2 * i] = make_float4(mv[0], mv[1], mv[2], mv[3]);
    mo[2 * i + 1] = make_float4(mv[4], mv[5], mv[6], mv[7]);
    vo[2 * i] = make_float4(vv[0], vv[1], vv[2], vv[3]);
    vo[2 * i + 1] = make_float4(vv[4], vv[5], vv[6], vv[7]);
    // the next step's mask, from |W'|
    const uint32_t h[8] = {wn.x & 0xFFFFu, wn.x >> 16, wn.y & 0xFFFFu, wn.y >> 16,
                           wn.z & 0xFFFFu, wn.z >> 16, wn.w & 0xFFFFu, wn.w >> 16};
    uint32_t u[8];
    mag_keys(h, u);
    const uint32_t keep = keep_bits<N, M>(u);
    mask[i] = (uint8_t)keep;
    nflip += (unsigned long long)__popc((prev ^ keep) & 0xFFu);
    // exact partial sum of |W'| (as k_absum)
    if (__builtin_expect(in_fast_window(wn), 1)) {
#pragma unroll
      for (int j = 0; j < 8; ++j) fsum += (double)__uint_as_float((h[j] & 0x7FFFu) << 16);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) absum_half(h[j], acc, hist, any_hist);
    }
    if (++fcount == 32) {
      const U128 f = {(unsigned long long)ldexp(fsum, 134 - kWinLo), 0ull};
      add128(acc, f);
      fsum = 0.0;
      fcount = 0;
    }
  }
  {
    const U128 f = {(unsigned long long)ldexp(fsum, 134 - kWinLo), 0ull};
    add128(acc, f);
  }
  if (any_hist) block_any = 1;  // benign race: every writer stores 1
  red[tid] = acc;
  fred[tid] = nflip;
  __syncthreads();
  for (int st = kAbsumThreads / 2; st > 0; st >>= 1) {
    if (tid < st) {
      U128 a = red[tid];
      add128(a, red[tid + st]);
      red[tid] = a;
      fred[tid] += fred[tid + st];
    }
    __syncthreads();
  }
  const int any = block_any;
  if (tid == 0) {
    AbsumPartial p;
    p.lo = red[0].lo;
    p.hi = red[0].hi;
    p.flag = (unsigned long long)any;
    p.pad = fred[0];
    part[blockIdx.x] = p;
  }
  if (any) hist_out[(size_t)blockIdx.x * 256 + tid] = hist[tid];
}

// Codes of the updated W from its mask plane and gamma (pass 2).
__global__ __launch_bounds__(256) void k_codes_from_mask(const uint4* __restrict__ W, const uint8_t* __restrict__ mask,
                                                         int64_t n_groups, const float* __restrict__ gamma_p,
                                                         uint16_t* __restrict__ codes) {
  const uint32_t gamma_bits = __float_as_uint(*gamma_p);
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_groups; i += stride) {
    const uint4 w = W[i];
    const uint32_t h[8] = {w.x & 0xFFFFu, w.x >> 16, w.y & 0xFFFFu, w.y >> 16,
                           w.z & 0xFFFFu, w.z >> 16, w.w & 0xFFFFu, w.w >> 16};
    codes[i] = codes_of(h, mask[i], gamma_bits);
  }
}

// ---------------------------------------------------------------------------
// Kept-only 2:4 plane from the code plane (2:8 and 2:4 masks leave at most 2
// non-zeros in every group of 4 positions).  Per row and 64-wide step, for each
// half h (32 positions = 8 groups of 4): a word of 16 two-bit codes, slot 2 g + i
// holding the i-th stored value of group g, and a word of their positions
// (bits 4 g .. 4 g + 3: first | second << 2, first < second).  The group's
// non-zeros are stored in position order, padded with zeros at the next free
// positions (one non-zero at a: (a, a + 1), or (2, 3) for a = 3; none: (0, 1)).
// Bytes 0-3 codes of h = 0, 4-7 codes of h = 1, 8-11 and 12-15 positions.
// ---------------------------------------------------------------------------
// One group of 4 codes (8 bits) -> (2 stored codes, 4 position bits); *bad set
// for more than 2 non-zeros (the first two are kept).
__device__ __forceinline__ void sparse24_group(uint32_t c4, uint32_t& codes2, uint32_t& pos4, bool& bad) {
  int i0 = -1, i1 = -1, cnt = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if ((c4 >> (2 * i)) & 3u) {
      if (i0 < 0) i0 = i;
      else if (i1 < 0) i1 = i;
      ++cnt;
    }
  }
  bad = cnt > 2;
  if (i0 < 0) {
    i0 = 0;
    i1 = 1;
  } else if (i1 < 0) {
    if (i0 < 3) i1 = i0 + 1;
    else { i0 = 2; i1 = 3; }
  }
  codes2 = ((c4 >> (2 * i0)) & 3u) | (((c4 >> (2 * i1)) & 3u) << 2);
  pos4 = (uint32_t)i0 | ((uint32_t)i1 << 2);
}

// One thread per (row, 64-wide step): the step's 16 bytes of codes (8 code
// words of 8 positions; 32-bit word q = positions 16 q .. 16 q + 15).
__global__ __launch_bounds__(256) void k_pack_sparse24(const uint16_t* __restrict__ codes, int64_t items,
                                                       uint4* __restrict__ plane, unsigned long long* __restrict__ bad) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= items) return;
  const uint4 cw = *(const uint4*)(codes + id * 8);
  const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
  uint32_t out[4];
  unsigned long long nbad = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t cc = 0, ix = 0;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      uint32_t c2, p4;
      bool b;
      sparse24_group((w[2 * h + (g >> 2)] >> (8 * (g & 3))) & 0xFFu, c2, p4, b);
      cc |= c2 << (4 * g);
      ix |= p4 << (4 * g);
      nbad += b ? 1u : 0u;
    }
    out[h] = cc;
    out[2 + h] = ix;
  }
  plane[id] = make_uint4(out[0], out[1], out[2], out[3]);
  if (bad && nbad) atomicAdd(bad, nbad);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

int absum_blocks(int64_t n_vec8) {
  int64_t b = (n_vec8 + kAbsumThreads - 1) / kAbsumThreads;
  if (b < 1) b = 1;
  if (b > kAbsumMaxBlocks) b = kAbsumMaxBlocks;
  return (int)b;
}

size_t quant_workspace_bytes(int64_t d_out, int64_t d_in) {
  const int nb = absum_blocks(d_out * d_in / 8);
  return (size_t)nb * sizeof(AbsumPartial) + (size_t)nb * 256 * sizeof(unsigned long long);
}

using MqpKernel = void (*)(const uint4*, int64_t, const float*, uint16_t*, uint8_t*);

// k_mask_quant_pack instance for (N, M, FQ); nullptr outside 1 <= N <= M, M in {4, 8}.
static MqpKernel mqp_kernel(int n, int m, bool fq) {
#define SBL_MQP(NN, MM) (fq ? (MqpKernel)k_mask_quant_pack<NN, MM, true> : (MqpKernel)k_mask_quant_pack<NN, MM, false>)
  if (m == 8) {
    switch (n) {
      case 1: return SBL_MQP(1, 8);
      case 2: return SBL_MQP(2, 8);
      case 3: return SBL_MQP(3, 8);
      case 4: return SBL_MQP(4, 8);
      case 5: return SBL_MQP(5, 8);
      case 6: return SBL_MQP(6, 8);
      case 7: return SBL_MQP(7, 8);
      case 8: return SBL_MQP(8, 8);
    }
  } else if (m == 4) {
    switch (n) {
      case 1: return SBL_MQP(1, 4);
      case 2: return SBL_MQP(2, 4);
      case 3: return SBL_MQP(3, 4);
      case 4: return SBL_MQP(4, 4);
    }
  }
#undef SBL_MQP
  return nullptr;
}

bool mask_pattern_supported(int n_keep, int m_group) { return mqp_kernel(n_keep, m_group, false) != nullptr; }

hipError_t launch_quant_mask_pack(const uint16_t* W, int64_t d_out, int64_t d_in, int n_keep, int m_group,
                                  bool from_quantized, uint16_t* codes, uint8_t* mask, float* gamma, void* ws,
                                  hipStream_t s) {
  const MqpKernel pack = mqp_kernel(n_keep, m_group, from_quantized);
  if (!pack) return hipErrorInvalidValue;
  const int64_t n_groups = d_out * d_in / 8;
  const int nb = absum_blocks(n_groups);
  AbsumPartial* part = (AbsumPartial*)ws;
  unsigned long long* hist = (unsigned long long*)((char*)ws + (size_t)nb * sizeof(AbsumPartial));
  hipLaunchKernelGGL(k_absum, dim3(nb), dim3(kAbsumThreads), 0, s, (const uint4*)W, n_groups, part, hist);
  hipLaunchKernelGGL(k_gamma_finalize, dim3(1), dim3(256), 0, s, (const AbsumPartial*)part,
                     (const unsigned long long*)hist, nb, (unsigned long long)(d_out * d_in), gamma,
                     (unsigned long long*)nullptr);
  int64_t pb = (n_groups + 1023) / 1024;
  if (pb > 65536) pb = 65536;
  hipLaunchKernelGGL(pack, dim3((unsigned)pb), dim3(256), 0, s, (const uint4*)W, n_groups, (const float*)gamma, codes,
                     mask);
  return hipGetLastError();
}

using AdamKernel = void (*)(uint4*, const float4*, float4*, float4*, int64_t, AdamHp, const uint8_t*, uint8_t*,
                           AbsumPartial*, unsigned long long*);

static AdamKernel adam_kernel(int n, int m) {
  if (m == 8) {
    switch (n) {
      case 1: return k_adamw_mask<1, 8>;
      case 2: return k_adamw_mask<2, 8>;
      case 3: return k_adamw_mask<3, 8>;
      case 4: return k_adamw_mask<4, 8>;
      case 5: return k_adamw_mask<5, 8>;
      case 6: return k_adamw_mask<6, 8>;
      case 7: return k_adamw_mask<7, 8>;
      case 8: return k_adamw_mask<8, 8>;
    }
  } else if (m == 4) {
    switch (n) {
      case 1: return k_adamw_mask<1, 4>;
      case 2: return k_adamw_mask<2, 4>;
      case 3: return k_adamw_mask<3, 4>;
      case 4: return k_adamw_mask<4, 4>;
    }
  }
  return nullptr;
}

hipError_t launch_adamw_repack(uint16_t* W, const float* g, float* m, float* v, int64_t d_out, int64_t d_in,
                               const AdamwArgs& a, int n_keep, int m_group, const uint8_t* mask_prev, uint8_t* mask,
                               uint16_t* codes, float* gamma, unsigned long long* flips, void* ws, hipStream_t s) {
  const AdamKernel k1 = adam_kernel(n_keep, m_group);
  if (!k1) return hipErrorInvalidValue;
  // hyper-parameters folded in double, then float32 (as torch's scalars)
  const double bc1 = 1.0 - std::pow((double)a.beta1, (double)a.step);
  const double bc2 = 1.0 - std::pow((double)a.beta2, (double)a.step);
  AdamHp hp;
  hp.b1 = a.beta1;
  hp.c1 = (float)(1.0 - (double)a.beta1);
  hp.b2 = a.beta2;
  hp.c2 = (float)(1.0 - (double)a.beta2);
  hp.gs = a.grad_scale;
  hp.step_size = (float)((double)a.lr / bc1);
  hp.sqrt_bc2 = (float)std::sqrt(bc2);
  hp.eps = a.eps;
  hp.decay = (float)(1.0 - (double)a.lr * (double)a.weight_decay);
  const int64_t n_groups = d_out * d_in / 8;
  const int nb = absum_blocks(n_groups);
  AbsumPartial* part = (AbsumPartial*)ws;
  unsigned long long* hist = (unsigned long long*)((char*)ws + (size_t)nb * sizeof(AbsumPartial));
  hipLaunchKernelGGL(k1, dim3(nb), dim3(kAbsumThreads), 0, s, (uint4*)W, (const float4*)g, (float4*)m, (float4*)v,
                     n_groups, hp, mask_prev, mask, part, hist);
  hipLaunchKernelGGL(k_gamma_finalize, dim3(1), dim3(256), 0, s, (const AbsumPartial*)part,
                     (const unsigned long long*)hist, nb, (unsigned long long)(d_out * d_in), gamma,
                     mask_prev ? flips : (unsigned long long*)nullptr);
  int64_t pb = (n_groups + 255) / 256;
  if (pb > 65536) pb = 65536;
  hipLaunchKernelGGL(k_codes_from_mask, dim3((unsigned)pb), dim3(256), 0, s, (const uint4*)W, (const uint8_t*)mask,
                     n_groups, (const float*)gamma, codes);
  return hipGetLastError();
}

using MqpBatchKernel = void (*)(PackBatch);

static MqpBatchKernel mqp_batch_kernel(int n, int m, bool fq) {
#define SBL_MQPB(NN, MM) \
  (fq ? (MqpBatchKernel)k_mask_quant_pack_batch<NN, MM, true> : (MqpBatchKernel)k_mask_quant_pack_batch<NN, MM, false>)
  if (m == 8) {
    switch (n) {
      case 1: return SBL_MQPB(1, 8);
      case 2: return SBL_MQPB(2, 8);
      case 3: return SBL_MQPB(3, 8);
      case 4: return SBL_MQPB(4, 8);
      case 5: return SBL_MQPB(5, 8);
      case 6: return SBL_MQPB(6, 8);
      case 7: return SBL_MQPB(7, 8);
      case 8: return SBL_MQPB(8, 8);
    }
  } else if (m == 4) {
    switch (n) {
      case 1: return SBL_MQPB(1, 4);
      case 2: return SBL_MQPB(2, 4);
      case 3: return SBL_MQPB(3, 4);
      case 4: return SBL_MQPB(4, 4);
    }
  }
#undef SBL_MQPB
  return nullptr;
}

static int64_t pack_blocks(int64_t n_groups) {
  int64_t pb = (n_groups + 1023) / 1024;
  return pb > 65536 ? 65536 : (pb < 1 ? 1 : pb);
}

size_t quant_batch_workspace_bytes(int count, const int64_t* n_weights) {
  size_t total = 0;
  for (int i = 0; i < count; ++i) {
    const int nb = absum_blocks(n_weights[i] / 8);
    total += (size_t)nb * sizeof(AbsumPartial) + (size_t)nb * 256 * sizeof(unsigned long long);
  }
  return total;
}

hipError_t launch_quant_mask_pack_batch(int count, const PackItem* items, int n_keep, int m_group,
                                        bool from_quantized, void* ws, hipStream_t s) {
  const MqpBatchKernel pack = mqp_batch_kernel(n_keep, m_group, from_quantized);
  if (!pack || count < 1 || count > kPackBatchMax) return hipErrorInvalidValue;
  PackBatch pb{};
  pb.count = count;
  int64_t na = 0, np = 0;
  for (int i = 0; i < count; ++i) {
    const int64_t ng = items[i].d_out * items[i].d_in / 8;
    pb.W[i] = (const uint4*)items[i].W;
    pb.n_groups[i] = ng;
    pb.codes[i] = items[i].codes;
    pb.mask[i] = items[i].mask;
    pb.gamma[i] = items[i].gamma;
    pb.absum_begin[i] = (int)na;
    pb.pack_begin[i] = (int)np;
    na += absum_blocks(ng);
    np += pack_blocks(ng);
  }
  pb.absum_begin[count] = (int)na;
  pb.pack_begin[count] = (int)np;
  if (np > 0x7FFFFFFF) return hipErrorInvalidValue;
  AbsumPartial* part = (AbsumPartial*)ws;
  unsigned long long* hist = (unsigned long long*)((char*)ws + (size_t)na * sizeof(AbsumPartial));
  hipLaunchKernelGGL(k_absum_batch, dim3((unsigned)na), dim3(kAbsumThreads), 0, s, pb, part, hist);
  hipLaunchKernelGGL(k_gamma_finalize_batch, dim3((unsigned)count), dim3(256), 0, s, pb,
                     (const AbsumPartial*)part, (const unsigned long long*)hist);
  hipLaunchKernelGGL(pack, dim3((unsigned)np), dim3(256), 0, s, pb);
  return hipGetLastError();
}

hipError_t launch_pack_sparse24(const uint16_t* codes, int64_t d_out, int64_t d_in, uint8_t* plane,
                                unsigned long long* bad, hipStream_t s) {
  const int64_t items = d_out * (d_in / 64);
  if (items == 0) return hipSuccess;
  hipLaunchKernelGGL(k_pack_sparse24, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, codes, items,
                     (uint4*)plane, bad);
  return hipGetLastError();
}

hipError_t launch_mask_grad(float* dW, const uint8_t* mask, int64_t d_out, int64_t d_in, hipStream_t s) {
  const int64_t n_groups = d_out * d_in / 8;
  if (n_groups == 0) return hipSuccess;
  int64_t nb = (n_groups + 255) / 256;
  if (nb > 8192) nb = 8192;
  hipLaunchKernelGGL(k_mask_grad, dim3((unsigned)nb), dim3(256), 0, s, (float4*)dW, mask, n_groups);
  return hipGetLastError();
}

}  // namespace sbl
