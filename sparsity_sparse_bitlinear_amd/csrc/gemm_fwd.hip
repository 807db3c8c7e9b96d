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
#include <atomic>
#include <algorithm>

#include "gemm_common.h"
#include "act_common.h"

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

// ---------------------------------------------------------------------------
// Direct-load forward (d_in % 128 == 0): block tile 256 tokens x 256 outputs,
// 8 waves (2 along M x 4 along N, 128 x 64 each), one block per CU (NW = 8),
// or 128 x 256 with 4 waves, two blocks per CU (NW = 4, for small grids).  Per K
// step of 128: the x_q tile (256 or 128 rows x 128 bytes, swizzled as swz8) and the
// code tile (256 rows x 16 code words = 32 bytes) move to LDS with direct-to-
// LDS loads through two stages; each wave expands the code words of its own B
// fragments in registers (one 32-bit word = 16 codes = one MFMA operand of 16
// int8), one slice ahead of the matrix instructions that use them.
// ---------------------------------------------------------------------------
constexpr int kFBN = 256;                  // block cols (outputs)
constexpr int kFS = 2;                     // LDS stages
constexpr int kFK = 128;                   // k per step
constexpr int kFStageB = kFBN * 32;        // 8 KB of code words

// Byte offset of code word w (0..7, groups 2w and 2w + 1 of the step) of tile
// row n: the two 16-byte halves of a row swap places on rows with bit 3 set,
// which halves the bank conflicts of the 32 rows a fragment read touches.
__device__ __forceinline__ int code_word_at(int n, int w) { return 32 * n + 16 * ((w >> 2) ^ ((n >> 3) & 1)) + 4 * (w & 3); }

// SP: the weight operand is the kept-only 2:4 plane (2:8 and 2:4 masks) and the
// product runs on v_smfmac_i32_32x32x64_i8, whose first operand holds 2 of
// every 4 k: per lane 16 stored codes (a 32-bit word, expanded to 16 int8 as
// the dense code words are) and a 32-bit word of their positions.  Lane l
// holds output row l % 32 and the 8 groups of 4 at k 32 (l / 32) .. + 31 of a
// 64-wide slice; the x_q operand holds, for token l % 32, k 16 (l / 32) .. + 15
// and 32 + 16 (l / 32) .. + 15 (two 16-byte chunks), which is the pairing the
// instruction uses (established on the hardware with random operands).  A K
// step of 128 is then 2 slices instead of 4; loads, stages and the epilogue
// are those of the dense path (the plane has the code plane's size).
template <int OUT, bool SP, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void k_fwd_i8_direct(const int8_t* __restrict__ xq,
                                                         const uint16_t* __restrict__ codes,
                                                         const float* __restrict__ gamma_p,
                                                         const float* __restrict__ absmax, int T, int d_in,
                                                         int d_out, void* __restrict__ y) {
  // Operand stages, then a separate staging area for the output tile (8 KB per
  // wave), so that a tile's epilogue runs while the next tile's first two K
  // steps land in the stages.
  constexpr int kFT = 64 * NW;                 // threads
  constexpr int kFBM = NW == 8 ? 256 : 128;    // block rows (tokens)
  constexpr int kFStageA = kFBM * kRowK;       // x_q tile of a K step
  constexpr int kFStage = kFStageA + kFStageB;
  constexpr int kFDmaA = kFBM * 8 / kFT;       // 4 direct loads of x_q per thread per K step
  constexpr int kFDmaB = kFStageB / 16 / kFT;  // and 1 or 2 of code words
  constexpr int kFDmaStep = kFDmaA + kFDmaB;
  __shared__ __attribute__((aligned(1024))) char lds[kFS * kFStage + NW * 8192];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave >> 2) * kWM;
  const int wn0 = (wave & 3) * kWN;
  const int mtn = (T + kFBM - 1) / kFBM, ntn = (d_out + kFBN - 1) / kFBN;
  const int ntiles = mtn * ntn;
  const int G = d_in >> 3;
  const int nk = d_in / kFK;

  // Tiles blockIdx.x, + gridDim.x, ... in turn (the host launches one block per
  // tile, or, with nk >= 2, at most one per CU).  XCD-aware order as for a
  // grid of one block per tile, since gridDim.x is a multiple of the XCD count
  // whenever a block takes more than one tile.
  struct Tile {
    int m0, n0;
    __amdgpu_buffer_rsrc_t ar, br;
  };
  auto tile_at = [&](int t) {
    Tile r;
    int mt, nt;
    xcd_tile_grouped(t, mtn, ntn, 4, mt, nt);
    r.m0 = mt * kFBM;
    r.n0 = nt * kFBN;
    r.ar = make_rsrc(xq + (int64_t)r.m0 * d_in, clamp_bytes((int64_t)min(kFBM, T - r.m0) * d_in));
    r.br = make_rsrc(codes + (int64_t)r.n0 * G, clamp_bytes((int64_t)min(kFBN, d_out - r.n0) * G * 2));
    return r;
  };

  // x_q tile: LDS chunk position p holds row p / 8, logical chunk (p % 8) ^ ((row / 2) % 8)
  uint32_t a_off[kFDmaA];
#pragma unroll
  for (int i = 0; i < kFDmaA; ++i) {
    const int p = 64 * (kFDmaA * wave + i) + lane;
    const int r = p >> 3, c = (p & 7) ^ ((r >> 1) & 7);
    a_off[i] = (uint32_t)(r * d_in + 16 * c);
  }
  // code tile: chunk position p holds row p / 2, half (p % 2) ^ ((row / 8) % 2)
  uint32_t b_off[kFDmaB];
#pragma unroll
  for (int i = 0; i < kFDmaB; ++i) {
    const int p = 64 * (NW * i + wave) + lane;
    const int r = p >> 1, h = (p & 1) ^ ((r >> 3) & 1);
    b_off[i] = (uint32_t)(r * G * 2 + 16 * h);
  }

  // Load idx (0 .. kFDmaStep - 1) of the wave's loads of K step kt of tile tl into stage st.
  auto issue_one = [&](const Tile& tl, int kt, int st, int idx) {
    char* sa = lds + st * kFStage;
    if (idx < kFDmaA) dma16(tl.ar, sa + 1024 * (kFDmaA * wave + idx), a_off[idx], (uint32_t)kt * kFK);
    else dma16(tl.br, sa + kFStageA + 1024 * (NW * (idx - kFDmaA) + wave), b_off[idx - kFDmaA], (uint32_t)kt * (kFK / 4));
  };
  auto issue = [&](const Tile& tl, int kt, int st) {
#pragma unroll
    for (int i = 0; i < kFDmaStep; ++i) issue_one(tl, kt, st, i);
  };

  const float g127 = *gamma_p * (1.0f / 127.0f);
  // Output scales of this lane's rows, fetched a K loop ahead of the epilogue.
  float am[kMI];
  auto load_scales = [&](int m0) {
#pragma unroll
    for (int i = 0; i < kMI; ++i) {
      const int m = m0 + wm0 + 32 * i + (lane & 31);
      am[i] = m < T ? absmax[m] : 0.0f;
    }
  };

  v16i acc[kMI][kNJ];

  // K slice ks (32 of the 128 k of a step): A fragments, and the code word
  // (groups 4 ks + 2 (l / 32), +1) of output row wn0 + 32 j + l % 32.
  auto rd = [&](int st, int ks, v4i (&fa)[kMI], uint32_t (&wb)[kNJ]) {
    const char* a = lds + st * kFStage;
    const char* b = a + kFStageA;
#pragma unroll
    for (int i = 0; i < kMI; ++i) fa[i] = *(const v4i*)(a + swz8(wm0 + 32 * i + (lane & 31), 2 * ks + (lane >> 5)));
#pragma unroll
    for (int j = 0; j < kNJ; ++j)
      wb[j] = *(const uint32_t*)(b + code_word_at(wn0 + 32 * j + (lane & 31), 2 * ks + (lane >> 5)));
  };
  // The code fragment is the MFMA's first operand, so accumulator register r
  // of lane l holds C[m = l % 32][n = 8 (r / 4) + 4 (l / 32) + r % 4]: four
  // consecutive outputs of one token per group of four registers.
  auto mm = [&](const v4i (&fa)[kMI], const v4i (&fb)[kNJ]) {
#pragma unroll
    for (int i = 0; i < kMI; ++i)
#pragma unroll
      for (int j = 0; j < kNJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[j], fa[i], acc[i][j], 0, 0, 0);
  };
  auto mm_one = [&](int t, const v4i (&fa)[kMI], const v4i (&fb)[kNJ]) {
    acc[t / kNJ][t % kNJ] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[t % kNJ], fa[t / kNJ], acc[t / kNJ][t % kNJ], 0, 0, 0);
  };
  auto expand = [&](const uint32_t (&wb)[kNJ], v4i (&fb)[kNJ]) {
#pragma unroll
    for (int j = 0; j < kNJ; ++j) fb[j] = __builtin_bit_cast(v4i, expand16(wb[j]));
  };
  // SP: a K step is 2 slices of 64 k, each done as 2 units of 2 x_q fragments
  // (units 0-3 of a step: slice u / 2, fragments i = 2 (u % 2), + 1), so the
  // operand registers match the dense path's.  Unit u: the x_q chunks
  // 4 (u / 2) + h and 4 (u / 2) + 2 + h of rows wm0 + 32 i + l % 32.
  auto rd_fh = [&](int st, int u, v8i (&fh)[2]) {
    const char* a = lds + st * kFStage;
    const int h = lane >> 5, s2 = u >> 1;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = wm0 + 32 * (2 * (u & 1) + q) + (lane & 31);
      const v4i lo = *(const v4i*)(a + swz8(row, 4 * s2 + h));
      const v4i hi = *(const v4i*)(a + swz8(row, 4 * s2 + 2 + h));
      fh[q] = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
  };
  // SP: the stored-code word 4 s2 + h and the position word 4 s2 + 2 + h of slice s2.
  auto rd_cc = [&](int st, int s2, uint32_t (&cc)[kNJ], uint32_t (&ix)[kNJ]) {
    const char* b = lds + st * kFStage + kFStageA;
    const int h = lane >> 5;
#pragma unroll
    for (int j = 0; j < kNJ; ++j) {
      const int n = wn0 + 32 * j + (lane & 31);
      cc[j] = *(const uint32_t*)(b + code_word_at(n, 4 * s2 + h));
      ix[j] = *(const uint32_t*)(b + code_word_at(n, 4 * s2 + 2 + h));
    }
  };
  // SP: instruction q * kNJ + j of unit u.
  auto mm_sp_one = [&](int u, int t, const v8i (&fh)[2], const v4i (&fb)[kNJ], const uint32_t (&ix)[kNJ]) {
    const int i = 2 * (u & 1) + t / kNJ, j = t % kNJ;
    acc[i][j] = __builtin_amdgcn_smfmac_i32_32x32x64_i8(fb[j], fh[t / kNJ], acc[i][j], (int)ix[j], 0, 0);
  };
#define SBL_FWD_SLICE_ORDER(id)                                 \
  __builtin_amdgcn_sched_group_barrier(0x008, 1, id);           \
  __builtin_amdgcn_sched_group_barrier(0x100, kMI + kNJ, id);   \
  __builtin_amdgcn_sched_group_barrier(0x008, 3, id);           \
  __builtin_amdgcn_sched_group_barrier(0x002, 12, id);          \
  __builtin_amdgcn_sched_group_barrier(0x008, 1, id);           \
  __builtin_amdgcn_sched_group_barrier(0x002, 12, id);          \
  __builtin_amdgcn_sched_group_barrier(0x008, 1, id);           \
  __builtin_amdgcn_sched_group_barrier(0x002, 12, id);          \
  __builtin_amdgcn_sched_group_barrier(0x008, 1, id);           \
  __builtin_amdgcn_sched_group_barrier(0x002, 12, id);          \
  __builtin_amdgcn_sched_group_barrier(0x008, 1, id);           \
  __builtin_amdgcn_sched_barrier(0);
// SP: one unit = 2 kNJ sparse instructions with `nrd` LDS reads and `nva`
// vector instructions (the next slice's code expansion) placed between them.
#define SBL_FWD_SP_ORDER(id, nrd, nva)                       \
  __builtin_amdgcn_sched_group_barrier(0x008, 1, id);        \
  __builtin_amdgcn_sched_group_barrier(0x100, nrd, id);      \
  __builtin_amdgcn_sched_group_barrier(0x008, 1, id);        \
  __builtin_amdgcn_sched_group_barrier(0x002, nva, id);      \
  __builtin_amdgcn_sched_group_barrier(0x008, 2 * kNJ - 2, id); \
  __builtin_amdgcn_sched_barrier(0);

  // The K steps of all tiles of the block form one sequence with stage parity
  // running on across tiles.  Step k (its stage has landed): each of the 4
  // slices is read and its code words expanded while the previous slice is
  // multiplied.  Before the last slice: wait for this wave's loads of the
  // next step (of this tile, or the next tile's first) and its reads of this
  // stage, barrier, then refill this stage with the step after next (again
  // possibly the next tile's), its loads placed between the last slice's
  // matrix instructions.  A tile's epilogue follows its last step; the next
  // tile starts by reading its slice 0.
  v4i fa0[kMI], fa1[kMI], fb0[kNJ], fb1[kNJ];
  uint32_t wb0[kNJ], wb1[kNJ];
  v8i fh0[2], fh1[2];                               // SP: x_q operands of a unit
  uint32_t cc0[kNJ], cc1[kNJ], ix0[kNJ], ix1[kNJ];  // SP: stored-code and position words
  v4i fbs0[kNJ], fbs1[kNJ];                         // SP: expanded stored codes of a slice
  int t = blockIdx.x;
  Tile cur = tile_at(t);
  load_scales(cur.m0);
  Tile nxt = cur;
  bool has_next = t + (int)gridDim.x < ntiles;
  if (has_next) nxt = tile_at(t + gridDim.x);
  issue(cur, 0, 0);
  if (nk > 1) {
    issue(cur, 1, 1);
    wait_vmcnt<kFDmaStep>();
  } else {
    if (has_next) issue(nxt, 0, 1);
    wait_vmcnt<0>();
  }
  barrier_only();
  int sc = 0;
  for (;;) {
#pragma unroll
    for (int i = 0; i < kMI; ++i)
#pragma unroll
      for (int j = 0; j < kNJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;
    if constexpr (SP) {
      rd_cc(sc, 0, cc0, ix0);
      rd_fh(sc, 0, fh0);
      expand(cc0, fbs0);
      for (int k = 0; k < nk; ++k) {
        rd_fh(sc, 1, fh1);
        rd_cc(sc, 1, cc1, ix1);
#pragma unroll
        for (int t2 = 0; t2 < 2 * kNJ; ++t2) mm_sp_one(0, t2, fh0, fbs0, ix0);
        expand(cc1, fbs1);
        SBL_FWD_SP_ORDER(0, 4 + 2 * kNJ, 8)
        rd_fh(sc, 2, fh0);
#pragma unroll
        for (int t2 = 0; t2 < 2 * kNJ; ++t2) mm_sp_one(1, t2, fh1, fbs0, ix0);
        SBL_FWD_SP_ORDER(1, 4, 0)
        rd_fh(sc, 3, fh1);
#pragma unroll
        for (int t2 = 0; t2 < 2 * kNJ; ++t2) mm_sp_one(2, t2, fh0, fbs1, ix1);
        SBL_FWD_SP_ORDER(2, 4, 0)
        wait_vmcnt_lgkm0<0>();
        barrier_only();
        __builtin_amdgcn_sched_barrier(0);
        const bool in_tile = k + 2 < nk;
        const bool load = in_tile || (has_next && k + 2 - nk < nk);
        const Tile& lt = in_tile ? cur : nxt;
        const int kn = in_tile ? k + 2 : k + 2 - nk;
        // unit 3 restarts the pipe; the next step's slice-0 words and unit-0
        // fragments and this step's refill loads go between its instructions
        mm_sp_one(3, 0, fh1, fbs1, ix1);
        __builtin_amdgcn_sched_barrier(0);
        if (k + 1 < nk) {
          rd_cc(sc ^ 1, 0, cc0, ix0);
          rd_fh(sc ^ 1, 0, fh0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 1; u < 2 * kNJ; ++u) {
          mm_sp_one(3, u, fh1, fbs1, ix1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int d = 0; d < 2; ++d) {  // 5 or 6 loads over the 3 remaining slots
            const int li = 2 * (u - 1) + d;
            if (li < kFDmaStep && load) issue_one(lt, kn, sc, li);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int li = 2 * (2 * kNJ - 1); li < kFDmaStep; ++li)
          if (load) issue_one(lt, kn, sc, li);
        if (k + 1 < nk) expand(cc0, fbs0);
        __builtin_amdgcn_sched_barrier(0);
        sc ^= 1;
      }
    } else {
    rd(sc, 0, fa0, wb0);
    expand(wb0, fb0);
    for (int k = 0; k < nk; ++k) {
      rd(sc, 1, fa1, wb1);
      mm(fa0, fb0);
      expand(wb1, fb1);
      SBL_FWD_SLICE_ORDER(0)
      rd(sc, 2, fa0, wb0);
      mm(fa1, fb1);
      expand(wb0, fb0);
      SBL_FWD_SLICE_ORDER(1)
      rd(sc, 3, fa1, wb1);
      mm(fa0, fb0);
      expand(wb1, fb1);
      SBL_FWD_SLICE_ORDER(2)
      wait_vmcnt_lgkm0<0>();
      barrier_only();
      __builtin_amdgcn_sched_barrier(0);
      // the step after next: of this tile, or the next tile's (nk >= 2 when a
      // block takes more than one tile), or none
      const bool in_tile = k + 2 < nk;
      const bool load = in_tile || (has_next && k + 2 - nk < nk);
      const Tile& lt = in_tile ? cur : nxt;
      const int kn = in_tile ? k + 2 : k + 2 - nk;
      mm_one(0, fa1, fb1);
      __builtin_amdgcn_sched_barrier(0);
      if (k + 1 < nk) rd(sc ^ 1, 0, fa0, wb0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 1; u < kMI * kNJ; ++u) {
        mm_one(u, fa1, fb1);
        __builtin_amdgcn_sched_barrier(0);
        if (u - 1 < kFDmaStep && load) issue_one(lt, kn, sc, u - 1);
        if (u >= kMI * kNJ - kNJ && k + 1 < nk)
          fb0[u - (kMI * kNJ - kNJ)] = __builtin_bit_cast(v4i, expand16(wb0[u - (kMI * kNJ - kNJ)]));
        __builtin_amdgcn_sched_barrier(0);
      }
      sc ^= 1;
    }
    }

    // Epilogue of tile cur.
    const int m0 = cur.m0, n0 = cur.n0;
    float scl[kMI];
#pragma unroll
    for (int i = 0; i < kMI; ++i) scl[i] = g127 * am[i];
    // bf16 or float32 output with 16-byte aligned rows: the wave's 128 x 64
    // result goes through its staging area in rounds of 8 KB (64 rows of 128
    // bytes in bf16, 32 rows of 256 bytes in float32; 16-byte chunks swizzled
    // by row), so that each store instruction writes whole row segments of
    // the wave's 64 columns.
    bool staged = false;
    if constexpr (OUT == SBL_BF16 || OUT == SBL_F32) {
      if ((d_out & (OUT == SBL_F32 ? 3 : 7)) == 0) {
        staged = true;
        char* stg = lds + kFS * kFStage + wave * 8192;
        const int ml = lane & 31, h = lane >> 5;
        constexpr int kRB = OUT == SBL_F32 ? 256 : 128;   // bytes per staged row
        constexpr int kCh = kRB / 16;                     // 16-byte chunks per row
        constexpr int kIR = 8192 / kRB / 32;              // 32-row blocks per round
#pragma unroll
        for (int r = 0; r < kMI / kIR; ++r) {
#pragma unroll
          for (int ii = 0; ii < kIR; ++ii) {
            const int i = kIR * r + ii, row = 32 * ii + ml;
#pragma unroll
            for (int j = 0; j < kNJ; ++j)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const float v0 = (float)acc[i][j][4 * q] * scl[i], v1 = (float)acc[i][j][4 * q + 1] * scl[i];
                const float v2 = (float)acc[i][j][4 * q + 2] * scl[i], v3 = (float)acc[i][j][4 * q + 3] * scl[i];
                if constexpr (OUT == SBL_F32) {
                  const int c = 8 * j + 2 * q + h;
                  *(float4*)(stg + row * kRB + 16 * (c ^ (row & (kCh - 1)))) = make_float4(v0, v1, v2, v3);
                } else {
                  const int c = 4 * j + q;
                  *(uint2*)(stg + row * kRB + 16 * (c ^ (row & (kCh - 1))) + 8 * h) =
                      make_uint2(cvt_pk_bf16(v0, v1), cvt_pk_bf16(v2, v3));
                }
              }
          }
          const int c = lane & (kCh - 1);
          const int n = n0 + wn0 + c * (OUT == SBL_F32 ? 4 : 8);
#pragma unroll
          for (int u = 0; u < 32 * kIR * kCh / 64; ++u) {
            const int row = (64 / kCh) * u + lane / kCh;
            const uint4 v = *(const uint4*)(stg + row * kRB + 16 * (c ^ (row & (kCh - 1))));
            const int m = m0 + wm0 + 32 * kIR * r + row;
            if (m < T && n < d_out) store_nt16((char*)y + ((int64_t)m * d_out + n) * (OUT == SBL_F32 ? 4 : 2), v);
          }
        }
      }
    }
    if (!staged) {
      // each lane stores runs of 4 consecutive outputs of its token (8 or 16
      // bytes); element stores only where a run leaves the matrix or rows are
      // not 4-aligned
      const bool vec_out = (d_out & 3) == 0;
#pragma unroll
      for (int i = 0; i < kMI; ++i) {
        const int m = m0 + wm0 + 32 * i + (lane & 31);
        if (m >= T) continue;
        const float sv = scl[i];
#pragma unroll
        for (int j = 0; j < kNJ; ++j) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = n0 + wn0 + 32 * j + 8 * q + 4 * (lane >> 5);
            if (n >= d_out) continue;
            const int64_t off = (int64_t)m * d_out + n;
            const int a0 = acc[i][j][4 * q], a1 = acc[i][j][4 * q + 1], a2 = acc[i][j][4 * q + 2],
                      a3 = acc[i][j][4 * q + 3];
            if (vec_out && n + 4 <= d_out) {
              if constexpr (OUT == SBL_I32) {
                *(int4*)((int*)y + off) = make_int4(a0, a1, a2, a3);
              } else if constexpr (OUT == SBL_F32) {
                *(float4*)((float*)y + off) =
                    make_float4((float)a0 * sv, (float)a1 * sv, (float)a2 * sv, (float)a3 * sv);
              } else {
                *(uint2*)((__bf16*)y + off) = make_uint2(cvt_pk_bf16((float)a0 * sv, (float)a1 * sv),
                                                         cvt_pk_bf16((float)a2 * sv, (float)a3 * sv));
              }
            } else {
              const int av[4] = {a0, a1, a2, a3};
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                if (n + u >= d_out) break;
                if constexpr (OUT == SBL_I32) ((int*)y)[off + u] = av[u];
                else if constexpr (OUT == SBL_F32) ((float*)y)[off + u] = (float)av[u] * sv;
                else ((__bf16*)y)[off + u] = (__bf16)((float)av[u] * sv);
              }
            }
          }
        }
      }
    }

    if (!has_next) break;
    t += gridDim.x;
    cur = nxt;
    load_scales(cur.m0);
    has_next = t + (int)gridDim.x < ntiles;
    if (has_next) nxt = tile_at(t + gridDim.x);
  }
#undef SBL_FWD_SLICE_ORDER
#undef SBL_FWD_SP_ORDER
  // No direct loads may still target LDS when the block retires.
  wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------
// Decode-size forward for 17 to 64 tokens on the code plane (up to 16 tokens,
// and the pair plane, go through decode.hip).
// ---------------------------------------------------------------------------
// Decode forward (T <= 64, d_in % 64 == 0): the code plane is streamed once and
// every weight meets at most 64 tokens, so the kernel is bound by the code
// bytes and, at these sizes, by the latency of one round of loads, not by the
// matrix cores.  A block owns 16 output rows (8 on grids too small to fill
// the CUs, see DecBatch); its W waves split the K range
// (all of a wave's loads are issued before its first product) and each runs
// v_mfma_i32_16x16x64_i8 with the expanded code words as the first operand
// (lane l: row l % 16, k 16 (l / 16) + 0..15, one 32-bit word of 16 codes) and
// up to 4 tiles of 16 tokens as the second (rows past T read as zero).
// Accumulator register r of lane l then holds C[t = l % 16][o = 4 (l / 16) + r].
// The W partial sums are added in LDS in a fixed order (integers: exact) and
// scaled as in the large-T kernels.
// ---------------------------------------------------------------------------
constexpr int kDecRows = 16;
constexpr int kDecSteps = 8;  // 64-wide K steps per wave whose loads are all in flight at once (one token tile)

// K steps in flight per wave for NTT token tiles (register budget of 16-wave blocks).
template <int NTT>
constexpr int dec_steps() { return NTT == 1 ? kDecSteps : kDecSteps / 2; }

// Waves per block: 8 while the grid stays within about 4096 waves, else 4,
// and at least min_w.  Measured on the decode shapes (16 packed copies per
// graph): 16-wave blocks were slower everywhere (q at 64 tokens 13.1 us
// against 11.4 with 8), 8 beat 4 on the 128-block grids (down at one token
// 13.6 against 14.4 us), 4 and 8 tie on the 688-block grids.
inline int decode_waves(int64_t nblocks, int min_w) {
  const int w = nblocks * 8 <= 4096 ? 8 : 4;
  return w < min_w ? min_w : w;
}

// Sum of the W waves' accumulators (wave 0 keeps the total) and the scaled
// store of rows o0 .. o_end - 1 (RT tiles of 16 rows at most); accumulator
// i = NTT rt + tt holds row tile rt and token tile tt, and sc[tt] is the
// scale of this lane's token 16 tt + l % 16.
template <int NTT, int OUT, int W, int RT = 1>
__device__ __forceinline__ void decode_store(v4i (&acc)[RT * NTT], int (*red)[RT * NTT][4][64], int wave, int lane,
                                             int o0, int T, int d_out, int o_end, const float (&sc)[NTT],
                                             void* __restrict__ y) {
  constexpr int NA = RT * NTT;
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave - 1][i][r][lane] = acc[i][r];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll 1
  for (int w = 0; w < W - 1; ++w)
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][r] += red[w][i][r][lane];

  const int q = lane >> 4, r16 = lane & 15;
  const bool vec_out = (d_out & 3) == 0;
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int tt = i % NTT;
    const int t = 16 * tt + r16;
    const int o = o0 + 16 * (i / NTT) + 4 * q;
    if (t >= T || o >= o_end) continue;
    const float s = sc[tt];
    const int64_t off = (int64_t)t * d_out + o;
    const int a0 = acc[i][0], a1 = acc[i][1], a2 = acc[i][2], a3 = acc[i][3];
    if (vec_out && o + 4 <= o_end) {
      if constexpr (OUT == SBL_I32) {
        *(int4*)((int*)y + off) = make_int4(a0, a1, a2, a3);
      } else if constexpr (OUT == SBL_F32) {
        *(float4*)((float*)y + off) = make_float4((float)a0 * s, (float)a1 * s, (float)a2 * s, (float)a3 * s);
      } else {
        *(uint2*)((__bf16*)y + off) =
            make_uint2(cvt_pk_bf16((float)a0 * s, (float)a1 * s), cvt_pk_bf16((float)a2 * s, (float)a3 * s));
      }
    } else {
      const int av[4] = {a0, a1, a2, a3};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (o + u >= o_end) break;
        if constexpr (OUT == SBL_I32) ((int*)y)[off + u] = av[u];
        else if constexpr (OUT == SBL_F32) ((float*)y)[off + u] = (float)av[u] * s;
        else ((__bf16*)y)[off + u] = (__bf16)((float)av[u] * s);
      }
    }
  }
}

// Up to kDecodeMultiMax matrices that share one activation input (a layer's
// q, k and v, or gate and up) in one launch: the blocks are dealt to the
// matrices by the prefix sums of their row blocks, so each block owns rows of
// one matrix and computes exactly what a launch for that matrix alone
// computes.  A block owns 16 rows (one matrix-instruction tile), or 8 when
// the 16-row grid would leave half of the CUs idle (its other 8 tile rows
// read zero codes and are not stored): 128-block grids such as o and down of
// a 3B layer at one token gain (down 10.5 -> 8.5 us), 160-block ones lose.
struct DecBatch {
  int count;
  int rows;                        // output rows per block: 8, 16 or 32 (16 per row tile of k_fwd_decode<.., RT>)
  int begin[kDecodeMultiMax + 1];  // row blocks of matrix i: [begin[i], begin[i + 1])
  int d_out[kDecodeMultiMax];
  const uint16_t* codes[kDecodeMultiMax];
  const float* gamma[kDecodeMultiMax];
  void* y[kDecodeMultiMax];
};

__device__ __forceinline__ int dec_item(const DecBatch& db, int b) {
  int i = 0;
  while (i + 1 < db.count && b >= db.begin[i + 1]) ++i;
  return i;
}

// RT row tiles of 16 per block (RT = 2 on large grids with 4 token tiles:
// every block reads all of x_q, so 32-row blocks halve those re-reads).
// PAIRS: the weights as the pair plane (one byte per group of 8; a lane's 16 k
// of a step are 2 bytes, expanded through a table of the 252 bytes in LDS).
template <int NTT, int OUT, int W, int RT, bool PAIRS>
__global__ __launch_bounds__(64 * W) void k_fwd_decode(const int8_t* __restrict__ xq, const DecBatch db,
                                                       const float* __restrict__ absmax, int T, int d_in) {
  __shared__ int red[W - 1][RT * NTT][4][64];
  __shared__ uint2 table[PAIRS ? 256 : 1];
  if constexpr (PAIRS) {
    if (threadIdx.x < 256) table[threadIdx.x] = pair_expand(threadIdx.x);
    __syncthreads();
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int item = dec_item(db, blockIdx.x);
  const uint16_t* __restrict__ codes = db.codes[item];
  const float* __restrict__ gamma_p = db.gamma[item];
  const int d_out = db.d_out[item];
  void* __restrict__ y = db.y[item];
  const int o0 = (blockIdx.x - db.begin[item]) * db.rows;
  const int G = d_in >> 3;
  const int nks = d_in >> 6;
  const int per = (nks + W - 1) / W;
  const int s_begin = wave * per, s_end = min(nks, s_begin + per);
  const int rows = min(db.rows, d_out - o0);
  const int row_bytes = PAIRS ? G : 2 * G;
  constexpr int kStepBytes = PAIRS ? 8 : 16;  // bytes of a row per 64-wide K step
  const auto br = make_rsrc((const uint8_t*)codes + (int64_t)o0 * row_bytes, clamp_bytes((int64_t)rows * row_bytes));
  const auto xr = make_rsrc(xq, clamp_bytes((int64_t)T * d_in));
  const int q = lane >> 4, r16 = lane & 15;
  const uint32_t b_off = (uint32_t)(r16 * row_bytes + (PAIRS ? 2 : 4) * q);
  uint32_t x_off[NTT];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) x_off[tt] = (uint32_t)((16 * tt + r16) * d_in + 16 * q);

  v4i acc[RT * NTT];
#pragma unroll
  for (int i = 0; i < RT * NTT; ++i) acc[i] = (v4i){0, 0, 0, 0};
  constexpr int kS = dec_steps<NTT>();
  for (int s0 = s_begin; s0 < s_end; s0 += kS) {
    uint32_t wb[kS][RT];
    v4i fx[kS][NTT];
#pragma unroll
    for (int u = 0; u < kS; ++u) {
      const bool ok = s0 + u < s_end;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const uint32_t off = ok ? b_off + (uint32_t)(rt * 16 * row_bytes + (s0 + u) * kStepBytes) : kOOB;
        wb[u][rt] = PAIRS ? bload2(br, off) : bload4(br, off);
      }
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
        fx[u][tt] = __builtin_bit_cast(v4i, bload16(xr, ok ? x_off[tt] + (uint32_t)(s0 + u) * 64 : kOOB));
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the round is issued before the first product
    // Steps past the wave's range multiply zeros (their loads were out of
    // range); no early exit, which would let the compiler sink each load to
    // its use and serialize the round trips.
#pragma unroll
    for (int u = 0; u < kS; ++u)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        v4i fb;
        if constexpr (PAIRS) {
          const uint2 e0 = table[wb[u][rt] & 0xFFu], e1 = table[(wb[u][rt] >> 8) & 0xFFu];
          fb = (v4i){(int)e0.x, (int)e0.y, (int)e1.x, (int)e1.y};
        } else {
          fb = __builtin_bit_cast(v4i, expand16(wb[u][rt]));
        }
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
          acc[NTT * rt + tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fb, fx[u][tt], acc[NTT * rt + tt], 0, 0, 0);
      }
  }
  const float g127 = *gamma_p * (1.0f / 127.0f);
  float sc[NTT];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    const int t = 16 * tt + r16;
    sc[tt] = t < T ? g127 * absmax[t] : 0.0f;
  }
  decode_store<NTT, OUT, W, RT>(acc, red, wave, lane, o0, T, d_out, o0 + rows, sc, y);
}


template <int NTT, int W, int RT, bool PAIRS>
hipError_t launch_decode_w(const DecBatch& db, const int8_t* xq, const float* absmax, int64_t T, int64_t d_in,
                           int y_dtype, hipStream_t s) {
  const dim3 grid((unsigned)db.begin[db.count]), block(64 * W);
  switch (y_dtype) {
    case SBL_F32:
      hipLaunchKernelGGL((k_fwd_decode<NTT, SBL_F32, W, RT, PAIRS>), grid, block, 0, s, xq, db, absmax, (int)T,
                         (int)d_in);
      break;
    case SBL_BF16:
      hipLaunchKernelGGL((k_fwd_decode<NTT, SBL_BF16, W, RT, PAIRS>), grid, block, 0, s, xq, db, absmax, (int)T,
                         (int)d_in);
      break;
    default:
      hipLaunchKernelGGL((k_fwd_decode<NTT, SBL_I32, W, RT, PAIRS>), grid, block, 0, s, xq, db, absmax, (int)T,
                         (int)d_in);
      break;
  }
  return hipGetLastError();
}

template <int NTT, bool PAIRS>
hipError_t launch_decode(const DecBatch& db, const int8_t* xq, const float* absmax, int64_t T, int64_t d_in,
                         int y_dtype, hipStream_t s) {
  const int w = decode_waves(db.begin[db.count], 4);
  if constexpr (NTT == 4) {
    if (db.rows == 2 * kDecRows) {  // two row tiles: at most 8 waves (LDS of the partial sums)
      if (w >= 8) return launch_decode_w<NTT, 8, 2, PAIRS>(db, xq, absmax, T, d_in, y_dtype, s);
      return launch_decode_w<NTT, 4, 2, PAIRS>(db, xq, absmax, T, d_in, y_dtype, s);
    }
  }
  switch (w) {
    case 16: return launch_decode_w<NTT, 16, 1, PAIRS>(db, xq, absmax, T, d_in, y_dtype, s);
    case 8: return launch_decode_w<NTT, 8, 1, PAIRS>(db, xq, absmax, T, d_in, y_dtype, s);
    default: return launch_decode_w<NTT, 4, 1, PAIRS>(db, xq, absmax, T, d_in, y_dtype, s);
  }
}

// Descriptor of count matrices; false if the row blocks overflow an int.
// half: 8-row blocks allowed on small grids (one token tile, or rows of 8192
// and more: with four tiles of up to 64 tokens and shorter rows the doubled
// re-reads of x_q cost more than the extra blocks give; down of a 3B layer at
// 64 tokens gains); twin: 32-row blocks on grids of at least 4 blocks of 16
// rows per CU (four token tiles: halves the re-reads of x_q).
bool make_dec_batch(int count, const DecodeItem* items, bool half, bool twin, DecBatch& db) {
  if (count < 1 || count > kDecodeMultiMax) return false;
  db = DecBatch{};
  db.count = count;
  int64_t full = 0;
  for (int i = 0; i < count; ++i) full += (items[i].d_out + kDecRows - 1) / kDecRows;
  db.rows = half && 2 * full <= device_cus() ? kDecRows / 2 : twin && full >= 4 * device_cus() ? 2 * kDecRows : kDecRows;
  int64_t nb = 0;
  for (int i = 0; i < count; ++i) {
    db.begin[i] = (int)nb;
    db.d_out[i] = (int)items[i].d_out;
    db.codes[i] = items[i].codes;
    db.gamma[i] = items[i].gamma;
    db.y[i] = items[i].y;
    nb += (items[i].d_out + db.rows - 1) / db.rows;
    if (nb > 0x7FFFFFFF) return false;
  }
  db.begin[count] = (int)nb;
  return true;
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

int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// One block per tile, or with two or more K steps per tile at most one block
// per CU (a multiple of 8, the XCD count), each walking its tiles.  Grids of
// 256-token tiles that leave CUs idle take 128-token tiles of 4 waves, two
// blocks per CU, instead (k and v of a 3B layer: 0.035 -> 0.029 ms); on full
// grids the halved tiles measured 2-3% slower (more operand bytes per product).
template <bool SP, int NW>
static hipError_t launch_fwd_nw(const uint16_t* codes, const float* gamma, const int8_t* xq, const float* absmax,
                                int64_t T, int64_t d_in, int64_t d_out, void* y, int y_dtype, int64_t slots,
                                hipStream_t s) {
  constexpr int bm = NW == 8 ? 256 : 128;
  const int64_t nb = ((d_out + kFBN - 1) / kFBN) * ((T + bm - 1) / bm);
  const int64_t nblocks = d_in / kFK >= 2 && nb > slots ? slots : nb;
  const dim3 grid((unsigned)nblocks), block(64 * NW);
  switch (y_dtype) {
    case SBL_F32:
      hipLaunchKernelGGL((k_fwd_i8_direct<SBL_F32, SP, NW>), grid, block, 0, s, xq, codes, gamma, absmax, (int)T,
                         (int)d_in, (int)d_out, y);
      break;
    case SBL_BF16:
      hipLaunchKernelGGL((k_fwd_i8_direct<SBL_BF16, SP, NW>), grid, block, 0, s, xq, codes, gamma, absmax, (int)T,
                         (int)d_in, (int)d_out, y);
      break;
    default:
      hipLaunchKernelGGL((k_fwd_i8_direct<SBL_I32, SP, NW>), grid, block, 0, s, xq, codes, gamma, absmax, (int)T,
                         (int)d_in, (int)d_out, y);
      break;
  }
  return hipGetLastError();
}

template <bool SP>
static hipError_t launch_fwd_direct(const uint16_t* codes, const float* gamma, const int8_t* xq, const float* absmax,
                                    int64_t T, int64_t d_in, int64_t d_out, void* y, int y_dtype, hipStream_t s) {
  const int64_t cus = std::max(8, device_cus() / 8 * 8);
  const int64_t nb8 = ((d_out + kFBN - 1) / kFBN) * ((T + 255) / 256);
  if (nb8 < cus) return launch_fwd_nw<SP, 4>(codes, gamma, xq, absmax, T, d_in, d_out, y, y_dtype, 2 * cus, s);
  return launch_fwd_nw<SP, 8>(codes, gamma, xq, absmax, T, d_in, d_out, y, y_dtype, cus, s);
}

hipError_t launch_forward(const uint16_t* codes, const float* gamma, const int8_t* xq, const float* absmax,
                          int64_t T, int64_t d_in, int64_t d_out, void* y, int y_dtype, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (T <= 64 && decode_plane_supported(SBL_PLANE_CODES, T, d_in)) {
    const DecodeItem it{codes, gamma, d_out, y};
    return launch_decode_plane(SBL_PLANE_CODES, 1, &it, false, xq, absmax, T, d_in, y_dtype, s);
  }
  if (d_in % kFK == 0 && (int64_t)kBM * d_in <= kMaxRsrcBytes)
    return launch_fwd_direct<false>(codes, gamma, xq, absmax, T, d_in, d_out, y, y_dtype, s);
  if (d_in % 64 == 0) return launch_fwd_v<true>(codes, gamma, xq, absmax, T, d_in, d_out, y, y_dtype, s);
  return launch_fwd_v<false>(codes, gamma, xq, absmax, T, d_in, d_out, y, y_dtype, s);
}

bool forward_sparse24_supported(int64_t d_in) { return d_in % kFK == 0 && (int64_t)kBM * d_in <= kMaxRsrcBytes; }

hipError_t launch_forward_sparse24(const uint8_t* plane, const float* gamma, const int8_t* xq, const float* absmax,
                                   int64_t T, int64_t d_in, int64_t d_out, void* y, int y_dtype, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (!forward_sparse24_supported(d_in)) return hipErrorInvalidValue;
  return launch_fwd_direct<true>((const uint16_t*)plane, gamma, xq, absmax, T, d_in, d_out, y, y_dtype, s);
}

hipError_t launch_decode_codes_many(int count, const DecodeItem* items, bool pairs, const int8_t* xq,
                                    const float* absmax, int64_t T, int64_t d_in, int y_dtype, hipStream_t s) {
  if (T == 0) return hipSuccess;
  DecBatch db;
  if (T > 64 || d_in % 64 != 0 || !make_dec_batch(count, items, T <= 16 || d_in >= 8192, T > 16, db)) return hipErrorInvalidValue;
  if (T <= 16) return pairs ? launch_decode<1, true>(db, xq, absmax, T, d_in, y_dtype, s)
                            : launch_decode<1, false>(db, xq, absmax, T, d_in, y_dtype, s);
  return pairs ? launch_decode<4, true>(db, xq, absmax, T, d_in, y_dtype, s)
               : launch_decode<4, false>(db, xq, absmax, T, d_in, y_dtype, s);
}


}  // namespace sbl
