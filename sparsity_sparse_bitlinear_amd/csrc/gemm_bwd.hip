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
// and B[k = 8(l/32)+0..7][n = l%32]) with fp32 accumulation.  All operands
// sit in LDS as K-contiguous rows (see gemm_common.h).  Operands whose
// reduction index is not contiguous in memory are transposed in registers
// while they are staged, in 4 x 4 or 4 x 8 blocks, and written with 8-byte
// LDS stores:
//   dX: A = dY [T, d_out] (k = o contiguous, a plain copy); B = W_eff^T: four
//       code words of consecutive rows o give, for each column i, four
//       consecutive-k bf16 values {-1,0,+1} (exact).
//   dW: A = dY^T: four rows t of dY give, for each o, four consecutive-k
//       values (byte permutes); B = x~^T: four rows t of x_q are widened,
//       scaled by a_t / 127 and rounded to bf16 pairwise along t.
// Global loads are buffer loads through per-K-step resources, so rows past a
// matrix edge read as zero.  dW with few output tiles splits the token range; the partial sums are added
// in a fixed order by k_splitk_reduce (deterministic).
#include <algorithm>
#include <cmath>

#include "gemm_common.h"

namespace sbl {

namespace {

using namespace gemm;

constexpr int kBK = 32;  // k elements (bf16) per LDS row


// Two 2-bit codes in bits 0-1 and 16-17 -> two bf16 values {0, +1 = 0x3F80, -1 = 0xBF80}.
__device__ __forceinline__ uint32_t code_pair_to_bf16x2(uint32_t s) {
  return (s * 0x3F80u) | ((s & 0x20002u) << 7);
}

// ---------------------------------------------------------------------------
// dX = gamma * dY @ W_eff      (M = tokens, N = d_in, K = d_out)
// ---------------------------------------------------------------------------
template <int OUT, bool VEC>
__global__ __launch_bounds__(kThreads, 2) void k_bwd_dx(const uint16_t* __restrict__ dY,
                                                        const uint16_t* __restrict__ codes,
                                                        const float* __restrict__ gamma_p, int T, int d_in,
                                                        int d_out, void* __restrict__ dX) {
  constexpr int CA = kBM * 4 / kThreads;
  __shared__ __attribute__((aligned(16))) char lds[2 * (kBM + kBN) * kRow];
  char* As = lds;
  char* Bs = lds + 2 * kBM * kRow;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm0 = (wave >> 1) * kWM;
  const int wn0 = (wave & 1) * kWN;
  int mt, nt;
  xcd_tile(blockIdx.x, (T + kBM - 1) / kBM, (d_in + kBN - 1) / kBN, mt, nt);
  const int m0 = mt * kBM;
  const int n0 = nt * kBN;
  const int G = d_in >> 3;
  const int nk = (d_out + kBK - 1) / kBK;

  const int rows_a = min(kBM, T - m0);
  const uint16_t* a_base = dY + (int64_t)m0 * d_out;
  uint32_t a_off[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int q = tid + kThreads * i;
    a_off[i] = (uint32_t)((q >> 2) * d_out * 2 + 16 * (q & 3));
  }
  // B: thread -> 4 consecutive code rows o (4 * og .. +3) x half a group (4 columns i);
  // the 32 lanes of a half-wave cover all 8 k-slots of 4 LDS rows (conflict-free stores)
  const int og = tid & 7;              // 0..7
  const int gh = tid >> 3;             // 16 groups x 2 halves
  const int bg = (n0 >> 3) + (gh >> 1);
  const int bh = gh & 1;
  // code word (row 4 * og + r, group bg) relative to the K-step base; groups past
  // the row end read as zero
  uint32_t b_off[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) b_off[r] = bg < G ? (uint32_t)(((4 * og + r) * G + (gh >> 1)) * 2) : kOOB;
  const uint16_t* b_base = codes + (n0 >> 3);

  uint4 ra[2][CA];
  uint32_t rb[2][4];

  // Buffer loads through per-K-step resources: token rows past T and code rows
  // past d_out read as zero.
  auto load_tile = [&](int kt, int st) {
    const int k0 = kt * kBK;
    const auto ar = make_rsrc(a_base + k0, clamp_bytes(((int64_t)rows_a * d_out - k0) * 2));
    const auto br = make_rsrc(b_base + (int64_t)k0 * G, clamp_bytes(((int64_t)(d_out - k0) * G - (n0 >> 3)) * 2));
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int k = k0 + 8 * ((tid + kThreads * i) & 3);
      if constexpr (VEC) {
        ra[st][i] = bload16(ar, k < d_out ? a_off[i] : kOOB);
      } else {
        uint32_t w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = bload2(ar, k + j < d_out ? a_off[i] + 2 * j : kOOB);
        ra[st][i] = make_uint4(w[0] | (w[1] << 16), w[2] | (w[3] << 16), w[4] | (w[5] << 16), w[6] | (w[7] << 16));
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) rb[st][r] = bload2(br, b_off[r]);
  };
  auto store_tile = [&](int buf, int st) {
    char* a = As + buf * kBM * kRow;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int q = tid + kThreads * i;
      *(uint4*)(a + swz(q >> 2, q & 3)) = ra[st][i];
    }
    char* b = Bs + buf * kBN * kRow;
    const uint32_t w01 = rb[st][0] | (rb[st][1] << 16);
    const uint32_t w23 = rb[st][2] | (rb[st][3] << 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int slot = 4 * bh + j;           // position i within the group
      const int row = 8 * (gh >> 1) + slot;  // LDS row = column i within the block tile
      uint2 v;
      v.x = code_pair_to_bf16x2((w01 >> (2 * slot)) & 0x00030003u);
      v.y = code_pair_to_bf16x2((w23 >> (2 * slot)) & 0x00030003u);
      *(uint2*)(b + swz(row, og >> 1) + 8 * (og & 1)) = v;
    }
  };

  v16f acc[kMI][kNJ];
#pragma unroll
  for (int i = 0; i < kMI; ++i)
#pragma unroll
    for (int j = 0; j < kNJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto compute = [&](int buf) {
    const char* a = As + buf * kBM * kRow;
    const char* b = Bs + buf * kBN * kRow;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8bf fa[kMI], fb[kNJ];
#pragma unroll
      for (int i = 0; i < kMI; ++i) fa[i] = __builtin_bit_cast(v8bf, frag(a, wm0 + 32 * i, ks, lane));
#pragma unroll
      for (int j = 0; j < kNJ; ++j) fb[j] = __builtin_bit_cast(v8bf, frag(b, wn0 + 32 * j, ks, lane));
#pragma unroll
      for (int i = 0; i < kMI; ++i)
#pragma unroll
        for (int j = 0; j < kNJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
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

  const float gamma = *gamma_p;
#pragma unroll
  for (int i = 0; i < kMI; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm0 + 32 * i + acc_row(r, lane);
      if (m >= T) continue;
#pragma unroll
      for (int j = 0; j < kNJ; ++j) {
        const int n = n0 + wn0 + 32 * j + (lane & 31);
        if (n >= d_in) continue;
        const float v = acc[i][j][r] * gamma;
        const int64_t off = (int64_t)m * d_in + n;
        if constexpr (OUT == SBL_F32) ((float*)dX)[off] = v;
        else ((__bf16*)dX)[off] = (__bf16)v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// W_eff^T for the direct-load dX product, still as 2-bit codes: the code plane
// [d_out, d_in / 8] transposed to one row per column i, in the word layout the
// product widens in registers (gemm_nt.hip, BC): per 64 rows o from o = 64 s,
// 4 words; word 2 h + w holds groups g = 4 w + 2 ss + h (ss = 0, 1) of 8
// consecutive o, the codes of o = 64 s + 8 g + 2 q and + 1 at bits 14 - 2p and
// 30 - 2p, p = 4 ss + q.  Rows are k64 / 4 bytes, k64 = d_out rounded up to
// 64; codes past d_out are 00 (zero).  A block takes 256 columns x 256 rows o
// through LDS (group-major, so a column's codes of 8 consecutive o are one
// 16-byte read) and writes 64 contiguous bytes per column.
// ---------------------------------------------------------------------------
constexpr int kCtI = 256, kCtO = 256;

__global__ __launch_bounds__(256) void k_codes_t(const uint16_t* __restrict__ codes, int d_out, int d_in, int k64,
                                                 uint32_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kCtI / 8][kCtO + 8];  // [group][o]
  const int G = d_in >> 3;
  const int i0 = blockIdx.x * kCtI, o0 = blockIdx.y * kCtO;
  const int g0 = i0 >> 3;
  const int tid = threadIdx.x;
  // 16-byte pieces (8 groups of one row o) where rows are 16-byte aligned and
  // the piece is inside the plane; single words elsewhere
#pragma unroll
  for (int u = 0; u < kCtO * (kCtI / 64) / 256; ++u) {
    const int e = tid + 256 * u;
    const int r = e / (kCtI / 64), gq = 8 * (e % (kCtI / 64));
    const int o = o0 + r, g = g0 + gq;
    uint16_t w[8];
    if ((G & 7) == 0 && o < d_out && g + 8 <= G) {
      const uint4 v = *(const uint4*)(codes + (int64_t)o * G + g);
      __builtin_memcpy(w, &v, 16);
    } else {
#pragma unroll
      for (int z = 0; z < 8; ++z) w[z] = (o < d_out && g + z < G) ? codes[(int64_t)o * G + g + z] : (uint16_t)0;
    }
#pragma unroll
    for (int z = 0; z < 8; ++z) tile[gq + z][r] = w[z];
  }
  __syncthreads();
  const int i = i0 + tid;
  if (i >= d_in) return;
  const int gl = tid >> 3, sh = 2 * (tid & 7);
  const int64_t row_words = k64 / 16;
#pragma unroll
  for (int st = 0; st < kCtO / 64; ++st) {
    const int ob = o0 + 64 * st;
    if (ob >= k64) break;
    uint32_t wv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const uint4 v = *(const uint4*)&tile[gl][64 * st + 8 * g];
      const uint32_t e2[4] = {v.x, v.y, v.z, v.w};  // o = 8 g + 2 q (low half) and + 1 (high half)
      const int ks = g >> 1, h = g & 1;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int p = 4 * (ks & 1) + q;
        const uint32_t c0 = (e2[q] >> sh) & 3u, c1 = (e2[q] >> (16 + sh)) & 3u;
        wv[2 * h + (ks >> 1)] |= (c0 << (14 - 2 * p)) | (c1 << (30 - 2 * p));
      }
    }
    *(uint4*)(out + (int64_t)i * row_words + ob / 16) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
}

size_t codes_t_bytes(int64_t d_in, int64_t d_out) { return (size_t)d_in * (size_t)(((d_out + 63) & ~63) / 4); }

hipError_t launch_codes_t(const uint16_t* codes, int64_t d_out, int64_t d_in, uint32_t* out, hipStream_t s) {
  const int64_t k64 = (d_out + 63) & ~(int64_t)63;
  const dim3 grid((unsigned)((d_in + kCtI - 1) / kCtI), (unsigned)((k64 + kCtO - 1) / kCtO));
  hipLaunchKernelGGL(k_codes_t, grid, dim3(256), 0, s, codes, (int)d_out, (int)d_in, (int)k64, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Token-contiguous operands for dW = dY^T x~ on the plain GEMM engine:
//   dYT[o, t] = dY[t, o]                          (bf16 copy)
//   xT [i, t] = bf16(x_q[t, i] * (a_t / 127))     (x~, rounded once to bf16)
// Both [C, T8] with T8 = T rounded up to 8; columns t >= T are zero.  A block
// moves a 128 x 128 tile through LDS: rows of the source are read in 16-byte
// (bf16) or 8-byte (int8) pieces, rows of the result are written as 16-byte
// runs of 8 consecutive t.
// ---------------------------------------------------------------------------
constexpr int kTT = 128;

template <bool DEQ, bool VEC>
__global__ __launch_bounds__(256) void k_token_major(const void* __restrict__ src, const float* __restrict__ absmax,
                                                     int T, int C, int T8, uint16_t* __restrict__ dst) {
  __shared__ uint32_t tile[kTT][kTT / 2 + 1];  // [t][c pair], bf16 pairs; odd pitch spreads the banks
  const int t0 = blockIdx.x * kTT, c0 = blockIdx.y * kTT;
  const int tid = threadIdx.x;
  // phase 1: 128 rows t x 16 pieces of 8 columns (256-byte bf16 / 128-byte int8 row segments)
#pragma unroll 4
  for (int e = tid; e < kTT * (kTT / 8); e += 256) {
    const int r = e >> 4, pc = e & 15;
    const int t = t0 + r, c = c0 + 8 * pc;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (t < T) {
      if constexpr (DEQ) {
        const int8_t* row = (const int8_t*)src + (int64_t)t * C;
        const float sc = absmax[t] * (1.0f / 127.0f);
        int8_t q[8];
        if (VEC && c + 8 <= C) {
          const uint2 v = *(const uint2*)(row + c);
          __builtin_memcpy(q, &v, 8);
        } else {
#pragma unroll
          for (int u = 0; u < 8; ++u) q[u] = c + u < C ? row[c + u] : (int8_t)0;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = cvt_pk_bf16((float)q[2 * u] * sc, (float)q[2 * u + 1] * sc);
      } else {
        const uint16_t* row = (const uint16_t*)src + (int64_t)t * C;
        if (VEC && c + 8 <= C) {
          const uint4 v = *(const uint4*)(row + c);
          w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint32_t lo = c + 2 * u < C ? row[c + 2 * u] : 0u;
            const uint32_t hi = c + 2 * u + 1 < C ? row[c + 2 * u + 1] : 0u;
            w[u] = lo | (hi << 16);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) tile[r][4 * pc + u] = w[u];
  }
  __syncthreads();
  // phase 2: 128 rows c x 16 runs of 8 t (256-byte row segments)
#pragma unroll 4
  for (int e = tid; e < kTT * (kTT / 8); e += 256) {
    const int cl = e >> 4, rt = e & 15;
    const int c = c0 + cl, t = t0 + 8 * rt;
    if (c >= C || t >= T8) continue;
    uint32_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t a = tile[8 * rt + 2 * u][cl >> 1], b = tile[8 * rt + 2 * u + 1][cl >> 1];
      v[u] = (cl & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
    }
    *(uint4*)(dst + (int64_t)c * T8 + t) = make_uint4(v[0], v[1], v[2], v[3]);
  }
}

// x~ for dW on the plain GEMM engine, token-contiguous in runs of 8 (the
// run-major B operand of launch_gemm_nt_runs): x~[t, i] = bf16(x_q[t, i] *
// (a_t / 127)) (the same values as k_token_major with DEQ) at element
// (t / 8 * C + i) * 8 + t % 8, t < T8; tokens t >= T are zero.  A block of 256
// threads takes 64 tokens x 256 columns: each thread issues its four 16-byte
// row pieces of x_q first, widens and scales them into an LDS tile [t][c] of
// bf16, and the tile is read back transposed with ds_read_b64_tr_b16 (16
// lanes exchange a 4 x 16 block: lane q addresses row q / 4, columns
// 4 (q % 4) .. + 3; lane i receives column i of the 4 rows).  Lane i of a wave
// then holds the run of 8 tokens of column 64 w + i, so a wave's store is
// 1 KB of contiguous memory.
constexpr int kXtT = 64, kXtC = 256;
constexpr int kXtPitch = 2 * kXtC + 32;  // bytes per LDS row; the pad spreads a 4-row read over the banks

// Y: the same for a bf16 source row-scaled, dst = bf16(y[t, c] * (a_t / 127))
// (the scaled dY that the int8 form of the dW product takes; C % 8 == 0).
template <bool Y>
__global__ __launch_bounds__(256) void k_xt_bf16(const void* __restrict__ src, const float* __restrict__ absmax, int T,
                                                 int C, int T8, uint16_t* __restrict__ dst) {
  __shared__ __attribute__((aligned(16))) char tile[kXtT * kXtPitch];
  const int t0 = blockIdx.x * kXtT, c0 = blockIdx.y * kXtC;
  const int tid = threadIdx.x;
  constexpr int kPc = Y ? 8 : 16;                   // columns per 16-byte source piece
  constexpr int kU = kXtT * kXtC / kPc / 256;       // pieces per thread (4 or 8)
  uint4 raw[kU];
  float sc[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int q = tid + 256 * u;
    const int r = q / (kXtC / kPc), c = c0 + kPc * (q % (kXtC / kPc));
    const int t = t0 + r;
    raw[u] = make_uint4(0u, 0u, 0u, 0u);
    sc[u] = 0.0f;
    if (t < T) {
      sc[u] = absmax[t] * (1.0f / 127.0f);
      if constexpr (Y) {
        const uint16_t* row = (const uint16_t*)src + (int64_t)t * C;
        if (c + 8 <= C) raw[u] = *(const uint4*)(row + c);
      } else {
        const int8_t* row = (const int8_t*)src + (int64_t)t * C;
        if ((C & 15) == 0 && c + 16 <= C) {
          raw[u] = *(const uint4*)(row + c);
        } else {
          int8_t b[16];
#pragma unroll
          for (int z = 0; z < 16; ++z) b[z] = c + z < C ? row[c + z] : (int8_t)0;
          __builtin_memcpy(&raw[u], b, 16);
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int q = tid + 256 * u;
    const int r = q / (kXtC / kPc), cc = q % (kXtC / kPc);
    char* p = tile + r * kXtPitch + 2 * kPc * cc;
    if constexpr (Y) {
      const uint32_t w4[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
      uint32_t w[4];
#pragma unroll
      for (int z = 0; z < 4; ++z)
        w[z] = cvt_pk_bf16(__uint_as_float(w4[z] << 16) * sc[u], __uint_as_float(w4[z] & 0xFFFF0000u) * sc[u]);
      *(uint4*)p = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      int8_t b[16];
      __builtin_memcpy(b, &raw[u], 16);
      uint32_t w[8];
#pragma unroll
      for (int z = 0; z < 8; ++z) w[z] = cvt_pk_bf16((float)b[2 * z] * sc[u], (float)b[2 * z + 1] * sc[u]);
      *(uint4*)p = make_uint4(w[0], w[1], w[2], w[3]);
      *(uint4*)(p + 16) = make_uint4(w[4], w[5], w[6], w[7]);
    }
  }
  __syncthreads();
  const int grp = tid >> 4, ql = tid & 15;  // 16-lane group: 16 consecutive columns
  const int cb = 16 * grp;                      // this group's first column in the tile
  const int c = c0 + cb + ql;                   // this lane's output row
  const int col_addr = cb + 4 * (ql & 3);       // first of the 4 columns lane ql addresses
#pragma unroll
  for (int tb = 0; tb < kXtT / 8; ++tb) {
    v4s part[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 8 * tb + 4 * h + (ql >> 2);
      part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SBL_LDS v4s*)(tile + row * kXtPitch + 2 * col_addr));
    }
    const int t = t0 + 8 * tb;
    if (c < C && t < T8)
      *(v8s*)(dst + ((int64_t)(t >> 3) * C + c) * 8) =
          (v8s){part[0][0], part[0][1], part[0][2], part[0][3], part[1][0], part[1][1], part[1][2], part[1][3]};
  }
}

bool dx_direct(int64_t T, int64_t d_in, int64_t d_out) {
  return T > 0 && d_out % 8 == 0 && gemm_nt_bf16_supported(T, d_in, d_out);
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

int64_t round8(int64_t t) { return (t + 7) & ~(int64_t)7; }

bool dw_direct(int64_t T, int64_t d_in, int64_t d_out) {
  return T > 0 && gemm_nt_bf16_supported(d_out, d_in, round8(T));
}

// dW on the int8 form: dW = (dY diag(a / 127))^T x_q, the scaled dY run-major
// (written by the dX product, or by k_xt_bf16<true>), x_q read as it is: no x~
// pass, and half the B bytes of the bf16 form.  Needs d_in % 16 == 0 (16-byte
// rows of x_q); otherwise x~ is made run-major and the bf16 form runs.
bool dw_q(int64_t T, int64_t d_in, int64_t d_out) {
  return dw_direct(T, d_in, d_out) && d_out % 8 == 0 && gemm_nt_q_supported(d_out, d_in, round8(T), T);
}

// K splits for the plain GEMM engine (one 256 x 256 block per CU): pick S to
// minimise rounds(tiles * S) / S of full-K block time plus the partial-sum
// traffic, with K pieces that are whole 64-token steps.
void nt_splits(int64_t M, int64_t N, int64_t K, int& S, int64_t& kps) {
  const int64_t tiles = gemm_nt_bf16_tiles(M, N);
  const double slots = 256.0;
  const double t_block = 2.0 * 256.0 * 256.0 * (double)K / 5.0e12;  // seconds per full-K block, ~half of peak
  const double t_byte = 1.0 / 5.0e12;                                 // seconds per byte of partial-sum traffic
  S = 1;
  double best = 1e300;
  const int max_s = (int)std::max<int64_t>(1, std::min<int64_t>(32, K / 512));
  for (int s = 1; s <= max_s; ++s) {
    const double rounds = std::ceil((double)tiles * s / slots);
    const double cost = rounds * t_block / s + (s > 1 ? (double)(s + 1) * 4.0 * (double)M * (double)N * t_byte : 0.0);
    if (cost < best * 0.97) { best = cost; S = s; }
  }
  kps = ((K + S - 1) / S + 63) / 64 * 64;  // whole 64-token K steps
  S = (int)((K + kps - 1) / kps);
}

// A split whose last round of blocks is partial (e.g. 344 tiles: 2 ranges
// make 688 blocks, rounds of 256, 256 and 176) can instead give the tiles that
// fill whole rounds fewer ranges and the remaining tiles a deeper split.  The
// plan with one range for the head writes the head tiles' sums into dW
// directly: 256 full-K blocks, then 88 tiles x 5 ranges (440 blocks of 1/5 the
// length) finish in 1.4 instead of 1.5 full-K rounds, and only the tail tiles
// have partial planes (plane 0 in dW, planes 1-4 in the workspace).  Same cost
// model as nt_splits; head == 0 keeps the uniform plan.
void nt_split_tail(int64_t M, int64_t N, int64_t K, int S, int64_t kps, SplitTail& tail) {
  tail = SplitTail{0, 0, 0, 0, nullptr};
  const int64_t tiles = gemm_nt_bf16_tiles(M, N);
  if (tiles <= 256 || M > 65535) return;
  const double t_block = 2.0 * 256.0 * 256.0 * (double)K / 5.0e12, t_byte = 1.0 / 5.0e12;
  const double tile_bytes = 256.0 * 256.0 * 4.0;
  const double base = std::ceil((double)tiles * S / 256.0) * t_block / S +
                      (S > 1 ? (S + 1) * 4.0 * (double)M * (double)N * t_byte : 0.0);
  double best = base * 0.97;
  const int max_s = (int)std::min<int64_t>(16, K / 512);
  const int64_t head = tiles / 256 * 256;  // one full-K block each: whole rounds
  const int64_t rest = tiles - head;
  if (rest <= 0) return;
  for (int sb = 2; sb <= max_s; ++sb) {
    const int64_t tkps = ((K + sb - 1) / sb + 63) / 64 * 64;
    const int sbe = (int)((K + tkps - 1) / tkps);  // ranges actually made (none empty)
    if (sbe < 2) continue;
    // head rounds, tail rounds; partial planes 1.. of the tail tiles written and read, plane 0 read
    const double cost = (double)(head / 256) * t_block + std::ceil((double)rest * sbe / 256.0) * t_block / sbe +
                        (2.0 * (sbe - 1) + 2.0) * (double)rest * tile_bytes * t_byte;
    if (cost < best) {
      best = cost;
      tail = SplitTail{(int)head, 1, sbe, (int)tkps, nullptr};
    }
  }
}

// ---------------------------------------------------------------------------
// dW = dY^T @ x~      (M = d_out, N = d_in, K = tokens)
// ---------------------------------------------------------------------------

// bf16 halves: low halves of a and b -> (a.lo, b.lo); high halves -> (a.hi, b.hi)
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

__device__ __forceinline__ float sbyte(uint32_t w, int b) { return (float)(int)(int8_t)((w >> (8 * b)) & 0xFFu); }

template <bool VEC>
__global__ __launch_bounds__(kThreads, 2) void k_bwd_dw(const uint16_t* __restrict__ dY,
                                                        const int8_t* __restrict__ xq,
                                                        const float* __restrict__ absmax, int T, int d_in,
                                                        int d_out, int k_per_split, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) char lds[2 * (kBM + kBN) * kRow];
  char* As = lds;
  char* Bs = lds + 2 * kBM * kRow;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm0 = (wave >> 1) * kWM;
  const int wn0 = (wave & 1) * kWN;
  const int gm = (d_out + kBM - 1) / kBM, gn = (d_in + kBN - 1) / kBN;
  const int split = blockIdx.x / (gm * gn);
  int mt, nt;
  xcd_tile(blockIdx.x - split * gm * gn, gm, gn, mt, nt);
  const int m0 = mt * kBM;  // output rows (o)
  const int n0 = nt * kBN;  // output cols (i)
  const int kbeg = split * k_per_split;
  const int kend = min(T, kbeg + k_per_split);
  const int nk = kend > kbeg ? (kend - kbeg + kBK - 1) / kBK : 0;

  // A: thread -> 4 consecutive tokens (4 * tg .. +3) x 8 consecutive o (8 * oc .. +7);
  // the 32 lanes of a half-wave cover all 8 k-slots of 4 LDS rows (conflict-free stores)
  const int tg = tid & 7;    // 0..7
  const int oc = tid >> 3;   // 0..31
  const int a_o = m0 + 8 * oc;
  // B: thread -> the same 4 tokens x 4 consecutive i (4 * oc .. +3)
  const int b_i = n0 + 4 * oc;
  // Lane offsets relative to the K-step base (token t0 = kbeg + 32 kt); columns
  // past the matrix edge read as zero.
  uint32_t a_off[4], b_off[4], s_off[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 4 * tg + r;
    a_off[r] = a_o < d_out ? (uint32_t)((t * d_out + 8 * oc) * 2) : kOOB;
    b_off[r] = b_i < d_in ? (uint32_t)(t * d_in + 4 * oc) : kOOB;
    s_off[r] = (uint32_t)(t * 4);
  }

  uint4 ra[2][4];
  uint32_t rb[2][4];
  float rs[2][4];

  // Buffer loads through per-K-step resources: tokens past the split end read
  // as zero (x_q = 0 and a_t = 0).
  auto load_tile = [&](int kt, int st) {
    const int t0 = kbeg + kt * kBK;
    const int64_t nt_ = kend - t0;
    const auto ar = make_rsrc(dY + (int64_t)t0 * d_out + m0, clamp_bytes((nt_ * d_out - m0) * 2));
    const auto br = make_rsrc(xq + (int64_t)t0 * d_in + n0, clamp_bytes(nt_ * d_in - n0));
    const auto sr = make_rsrc(absmax + t0, clamp_bytes(nt_ * 4));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (VEC) {
        ra[st][r] = bload16(ar, a_off[r]);
      } else {
        uint32_t w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = bload2(ar, a_o + j < d_out ? a_off[r] + 2 * j : kOOB);
        ra[st][r] = make_uint4(w[0] | (w[1] << 16), w[2] | (w[3] << 16), w[4] | (w[5] << 16), w[6] | (w[7] << 16));
      }
      rb[st][r] = bload4(br, b_off[r]);
      rs[st][r] = __uint_as_float(bload4(sr, s_off[r]));
    }
  };
  auto store_tile = [&](int buf, int st) {
    // A rows o (8 * oc + 2p, +1), k = 4 * tg .. +3
    char* a = As + buf * kBM * kRow;
    const uint32_t w0[4] = {ra[st][0].x, ra[st][0].y, ra[st][0].z, ra[st][0].w};
    const uint32_t w1[4] = {ra[st][1].x, ra[st][1].y, ra[st][1].z, ra[st][1].w};
    const uint32_t w2[4] = {ra[st][2].x, ra[st][2].y, ra[st][2].z, ra[st][2].w};
    const uint32_t w3[4] = {ra[st][3].x, ra[st][3].y, ra[st][3].z, ra[st][3].w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint2 lo, hi;
      lo.x = pack_lo(w0[p], w1[p]);
      lo.y = pack_lo(w2[p], w3[p]);
      hi.x = pack_hi(w0[p], w1[p]);
      hi.y = pack_hi(w2[p], w3[p]);
      const int row = 8 * oc + 2 * p;
      *(uint2*)(a + swz(row, tg >> 1) + 8 * (tg & 1)) = lo;
      *(uint2*)(a + swz(row + 1, tg >> 1) + 8 * (tg & 1)) = hi;
    }
    // B rows i (4 * oc + j), k = 4 * tg .. +3: x_q * a_t / 127 rounded to bf16
    char* b = Bs + buf * kBN * kRow;
    const float s0 = rs[st][0] * (1.0f / 127.0f), s1 = rs[st][1] * (1.0f / 127.0f);
    const float s2 = rs[st][2] * (1.0f / 127.0f), s3 = rs[st][3] * (1.0f / 127.0f);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint2 v;
      v.x = cvt_pk_bf16(sbyte(rb[st][0], j) * s0, sbyte(rb[st][1], j) * s1);
      v.y = cvt_pk_bf16(sbyte(rb[st][2], j) * s2, sbyte(rb[st][3], j) * s3);
      *(uint2*)(b + swz(4 * oc + j, tg >> 1) + 8 * (tg & 1)) = v;
    }
  };

  v16f acc[kMI][kNJ];
#pragma unroll
  for (int i = 0; i < kMI; ++i)
#pragma unroll
    for (int j = 0; j < kNJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto compute = [&](int buf) {
    const char* a = As + buf * kBM * kRow;
    const char* b = Bs + buf * kBN * kRow;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8bf fa[kMI], fb[kNJ];
#pragma unroll
      for (int i = 0; i < kMI; ++i) fa[i] = __builtin_bit_cast(v8bf, frag(a, wm0 + 32 * i, ks, lane));
#pragma unroll
      for (int j = 0; j < kNJ; ++j) fb[j] = __builtin_bit_cast(v8bf, frag(b, wn0 + 32 * j, ks, lane));
#pragma unroll
      for (int i = 0; i < kMI; ++i)
#pragma unroll
        for (int j = 0; j < kNJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };

  if (nk > 0) {
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
  }

  float* dst = out + (size_t)split * (size_t)d_out * (size_t)d_in;
#pragma unroll
  for (int i = 0; i < kMI; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm0 + 32 * i + acc_row(r, lane);
      if (m >= d_out) continue;
#pragma unroll
      for (int j = 0; j < kNJ; ++j) {
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

// The split-K sum of the tail tiles of a SplitTail plan with planes: plane 0
// is already in dW, planes z = 1 .. S_tail - 1 at part + (z - 1) M N are added
// to it in order (the head tiles' dW is final).  Block (t, y): tail tile t
// (grouped order, 4 tile rows per group), rows 4 y .. 4 y + 3 of it, one float4
// column per thread (N % 4 == 0).
__global__ __launch_bounds__(256) void k_splitk_add_tail(const float4* __restrict__ part, int M, int N, int head,
                                                         int S_tail, float4* __restrict__ dW) {
  const int gm = (M + 255) >> 8, gn = (N + 255) >> 8;
  int mt, nt;
  grouped_tile(head + (int)blockIdx.x, gm, gn, 4, mt, nt);
  const int m = mt * 256 + 4 * (int)blockIdx.y + ((int)threadIdx.x >> 6);
  const int c4 = nt * 64 + ((int)threadIdx.x & 63), n4r = N >> 2;
  if (m >= M || c4 >= n4r) return;
  const int64_t plane = (int64_t)M * n4r, i = (int64_t)m * n4r + c4;
  float4 s = dW[i];
  for (int z = 1; z < S_tail; ++z) {
    const float4 v = part[(int64_t)(z - 1) * plane + i];
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  dW[i] = s;
}

__global__ __launch_bounds__(256) void k_zero_f32(float* __restrict__ p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.0f;
}

// Token-range splits for dW: enough blocks to fill two slots on every CU, where a
// split earns its keep (each extra split adds a partial write and read of dW).
int dw_splits(int64_t T, int64_t d_in, int64_t d_out) {
  const int64_t tiles = ((d_out + kBM - 1) / kBM) * ((d_in + kBN - 1) / kBN);
  if (T <= 0) return 1;
  const int64_t slots = 512;  // 256 CUs x 2 resident blocks
  int best = 1;
  double best_cost = 1e300;
  const int64_t max_s = std::max<int64_t>(1, std::min<int64_t>(16, T / 1024));
  for (int s = 1; s <= max_s; ++s) {
    const int64_t w = tiles * s;
    const double rounds = (double)((w + slots - 1) / slots);
    // time ~ rounds * (work per block) + reduction traffic, in units of one full-K tile
    const double cost = rounds / s + (s > 1 ? 0.02 * s * (double)tiles / slots : 0.0);
    if (cost < best_cost * 0.97) { best = s; best_cost = cost; }
  }
  return best;
}

}  // namespace

// Workspace of the dW path: dY^T and x~^T ([d_out, T8] and [d_in, T8] bf16),
// then the split-K partial sums.  When dX and dW are computed in one call, the
// dX product writes dY^T itself, and W_eff^T (needed only by the dX product)
// sits where x~^T is written afterwards.
struct DwLayout {
  size_t dyt, xt, part, wt, total;
  int S;
  int64_t kps;
  bool q;          // int8 form: scaled dY^T and x_q as they are (no x~ copy)
  SplitTail tail;  // int8 form only: deeper split of the tiles after the whole rounds
};

// Workspace of dW (and, fused, of the dX code plane, which is dead before dW
// starts): dY^T [T8 x d_out] bf16, x~ [T8 x d_in] bf16 unless the int8 form is
// used, split-K partial sums.
DwLayout dw_layout(int64_t T, int64_t d_in, int64_t d_out, bool fused) {
  DwLayout L{};
  const int64_t T8 = round8(T);
  nt_splits(d_out, d_in, T8, L.S, L.kps);
  L.q = dw_q(T, d_in, d_out);
  L.tail = SplitTail{0, 0, 0, 0, nullptr};
  if (L.q) nt_split_tail(d_out, d_in, T8, L.S, L.kps, L.tail);
  if (L.tail.head > 0) {  // one range for the head tiles; planes 1.. of the tail in the workspace
    L.S = 1;
    L.kps = T8;
  }
  const int planes = L.tail.head > 0 ? L.tail.tail_splits - 1 : L.S > 1 ? L.S : 0;
  L.dyt = 0;
  L.xt = align256((size_t)d_out * (size_t)T8 * 2);
  L.part = L.xt + (L.q ? 0 : align256((size_t)d_in * (size_t)T8 * 2));
  L.total = L.part + (size_t)planes * (size_t)d_out * (size_t)d_in * sizeof(float);
  L.wt = L.xt;
  if (fused) L.total = std::max(L.total, L.wt + align256(codes_t_bytes(d_in, d_out)));
  return L;
}

bool fused_backward(int64_t T, int64_t d_in, int64_t d_out, int flags) {
  // dY^T leaves the dX product run-major, which the dW product reads as such
  return (flags & SBL_BWD_DX) && (flags & SBL_BWD_DW) && dx_direct(T, d_in, d_out) && dw_direct(T, d_in, d_out) &&
         gemm_nt_runs_supported(d_out, d_in, round8(T));
}

// dW on the plain GEMM engine from the layout L: dY^T (unless the dX product
// already wrote it), x~^T, the product, and the split-K sum.
hipError_t run_dw_direct(const int8_t* xq, const float* absmax, const uint16_t* dY, int64_t T, int64_t d_in,
                         int64_t d_out, float* dW, void* ws, const DwLayout& L, bool dyt_ready, hipStream_t s) {
  const int64_t T8 = round8(T);
  const int64_t n = d_out * d_in;
  uint16_t* dyt = (uint16_t*)((char*)ws + L.dyt);
  uint16_t* xt = (uint16_t*)((char*)ws + L.xt);
  float* target = L.S > 1 ? (float*)((char*)ws + L.part) : dW;  // one range (also the tail plan): dW itself
  hipError_t e;
  if (L.q) {
    if (!dyt_ready) {  // the dX product did not write the scaled dY^T
      const dim3 g((unsigned)((T8 + kXtT - 1) / kXtT), (unsigned)((d_out + kXtC - 1) / kXtC));
      hipLaunchKernelGGL(k_xt_bf16<true>, g, dim3(256), 0, s, dY, absmax, (int)T, (int)d_out, (int)T8, dyt);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    SplitTail tail = L.tail;
    if (tail.head > 0) tail.planes = (float*)((char*)ws + L.part);
    e = launch_gemm_nt_q(dyt, xq, d_out, d_in, T8, T, target, s, L.S, L.kps, tail);
    if (e != hipSuccess) return e;
    if (tail.head > 0) {
      const int64_t tiles = gemm_nt_bf16_tiles(d_out, d_in);
      const dim3 g((unsigned)(tiles - tail.head), 64);
      hipLaunchKernelGGL(k_splitk_add_tail, g, dim3(256), 0, s, (const float4*)tail.planes, (int)d_out, (int)d_in,
                         tail.head, tail.tail_splits, (float4*)dW);
      e = hipGetLastError();
    } else if (L.S > 1) {
      const int64_t n4 = n / 4;
      hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)std::min<int64_t>((n4 + 255) / 256, 65536)), dim3(256), 0,
                         s, (const float4*)target, n4, L.S, (float4*)dW);
      e = hipGetLastError();
    }
    return e;
  }
  if (!dyt_ready) {
    const dim3 g1((unsigned)((T8 + kTT - 1) / kTT), (unsigned)((d_out + kTT - 1) / kTT));
    if (d_out % 8 == 0)
      hipLaunchKernelGGL((k_token_major<false, true>), g1, dim3(256), 0, s, dY, nullptr, (int)T, (int)d_out, (int)T8, dyt);
    else
      hipLaunchKernelGGL((k_token_major<false, false>), g1, dim3(256), 0, s, dY, nullptr, (int)T, (int)d_out, (int)T8, dyt);
  }
  if (gemm_nt_runs_supported(d_out, d_in, T8)) {
    const dim3 g2((unsigned)((T8 + kXtT - 1) / kXtT), (unsigned)((d_in + kXtC - 1) / kXtC));
    hipLaunchKernelGGL(k_xt_bf16<false>, g2, dim3(256), 0, s, xq, absmax, (int)T, (int)d_in, (int)T8, xt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_gemm_nt_runs(dyt, dyt_ready, xt, d_out, d_in, T8, target, s, L.S, L.kps);
  } else {
    const dim3 g2((unsigned)((T8 + kTT - 1) / kTT), (unsigned)((d_in + kTT - 1) / kTT));
    hipLaunchKernelGGL((k_token_major<true, true>), g2, dim3(256), 0, s, xq, absmax, (int)T, (int)d_in, (int)T8, xt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_gemm_nt_bf16(dyt, xt, d_out, d_in, T8, nullptr, target, SBL_F32, s, L.S, L.kps);
  }
  if (e != hipSuccess) return e;
  if (L.S > 1) {
    const int64_t n4 = n / 4;
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)std::min<int64_t>((n4 + 255) / 256, 65536)), dim3(256), 0, s,
                       (const float4*)target, n4, L.S, (float4*)dW);
    e = hipGetLastError();
  }
  return e;
}

// The dX transpose plane and the dW buffers are used one after the other on
// the same stream, so they share the workspace.
size_t backward_workspace_bytes(int64_t T, int64_t d_in, int64_t d_out, int flags) {
  if (fused_backward(T, d_in, d_out, flags)) return dw_layout(T, d_in, d_out, true).total;
  size_t dx = 0, dw = 0;
  if ((flags & SBL_BWD_DX) && dx_direct(T, d_in, d_out)) dx = align256(codes_t_bytes(d_in, d_out));
  if ((flags & SBL_BWD_DW) && T > 0) {
    if (dw_direct(T, d_in, d_out)) {
      dw = dw_layout(T, d_in, d_out, false).total;
    } else {
      const int S = dw_splits(T, d_in, d_out);
      if (S > 1) dw = (size_t)S * (size_t)d_out * (size_t)d_in * sizeof(float);
    }
  }
  return std::max(dx, dw);
}

hipError_t launch_backward(const uint16_t* codes, const float* gamma, const int8_t* xq, const float* absmax,
                           const uint16_t* dY, int64_t T, int64_t d_in, int64_t d_out, void* dX, int dx_dtype,
                           float* dW, int flags, void* ws, hipStream_t s) {
  if (fused_backward(T, d_in, d_out, flags)) {
    // dX, leaving dY^T behind in the workspace, then dW from it
    const DwLayout L = dw_layout(T, d_in, d_out, true);
    uint32_t* WT = (uint32_t*)((char*)ws + L.wt);
    hipError_t e = launch_codes_t(codes, d_out, d_in, WT, s);
    if (e != hipSuccess) return e;
    // with the int8 form of dW the side output is dY scaled by a_t / 127
    e = launch_gemm_nt_codes(dY, WT, T, d_in, d_out, gamma, dX, dx_dtype, s, (uint16_t*)((char*)ws + L.dyt),
                             round8(T), L.q ? absmax : nullptr);
    if (e != hipSuccess) return e;
    return run_dw_direct(xq, absmax, dY, T, d_in, d_out, dW, ws, L, true, s);
  }
  if ((flags & SBL_BWD_DX) && dx_direct(T, d_in, d_out)) {
    uint32_t* WT = (uint32_t*)ws;
    hipError_t e = launch_codes_t(codes, d_out, d_in, WT, s);
    if (e != hipSuccess) return e;
    e = launch_gemm_nt_codes(dY, WT, T, d_in, d_out, gamma, dX, dx_dtype, s);
    if (e != hipSuccess) return e;
  } else if ((flags & SBL_BWD_DX) && T > 0) {
    const dim3 grid((unsigned)(((d_in + kBN - 1) / kBN) * ((T + kBM - 1) / kBM)));
    const bool vec = d_out % 8 == 0;
    if (dx_dtype == SBL_F32) {
      if (vec) hipLaunchKernelGGL((k_bwd_dx<SBL_F32, true>), grid, dim3(kThreads), 0, s, dY, codes, gamma, (int)T, (int)d_in, (int)d_out, dX);
      else hipLaunchKernelGGL((k_bwd_dx<SBL_F32, false>), grid, dim3(kThreads), 0, s, dY, codes, gamma, (int)T, (int)d_in, (int)d_out, dX);
    } else {
      if (vec) hipLaunchKernelGGL((k_bwd_dx<SBL_BF16, true>), grid, dim3(kThreads), 0, s, dY, codes, gamma, (int)T, (int)d_in, (int)d_out, dX);
      else hipLaunchKernelGGL((k_bwd_dx<SBL_BF16, false>), grid, dim3(kThreads), 0, s, dY, codes, gamma, (int)T, (int)d_in, (int)d_out, dX);
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
    if (dw_direct(T, d_in, d_out))
      return run_dw_direct(xq, absmax, dY, T, d_in, d_out, dW, ws, dw_layout(T, d_in, d_out, false), false, s);
    const int S = dw_splits(T, d_in, d_out);
    const int64_t kps = ((T + S - 1) / S + kBK - 1) / kBK * kBK;
    const int64_t tiles = ((d_in + kBN - 1) / kBN) * ((d_out + kBM - 1) / kBM);
    const dim3 grid((unsigned)(tiles * S));
    float* target = S > 1 ? (float*)ws : dW;
    // vector path: 16-byte dY rows (d_out % 8); x_q words are 4-byte aligned since d_in % 8 == 0
    if (d_out % 8 == 0)
      hipLaunchKernelGGL((k_bwd_dw<true>), grid, dim3(kThreads), 0, s, dY, xq, absmax, (int)T, (int)d_in, (int)d_out,
                         (int)kps, target);
    else
      hipLaunchKernelGGL((k_bwd_dw<false>), grid, dim3(kThreads), 0, s, dY, xq, absmax, (int)T, (int)d_in, (int)d_out,
                         (int)kps, target);
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
