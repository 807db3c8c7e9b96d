// C = alpha * A B^T on gfx950 bf16 matrix cores, both operands K-contiguous.
//
//   C[m, n] = alpha * sum_k A[m, k] * B[n, k]     A [M, K], B [N, K] bf16 row-major,
//                                                  C [M, N] float32 or bf16
//
// This is the plain-GEMM engine behind both products of the Dual-STE backward
// ([SUM] 方法步骤详情 step (7)):
//   dX = gamma * dY W_eff      A = dY [T, d_out]; B = W_eff^T [d_in, d_out] as
//                              2-bit codes (transposed once per call, see
//                              BC below), widened to bf16 in registers
//   dW = dY^T x~               A = dY^T [d_out, T], B = x~^T [d_in, T]
//                              (both transposed once per call, token-contiguous)
//
// Operand tiles move from global memory to LDS with direct-to-LDS buffer loads
// (no register staging and no LDS store instructions) through two or three LDS
// stages of one K step (64 bf16) each: a step's loads are issued one or two
// steps ahead, in the middle of an earlier step.  Each lane of a direct load picks the
// global chunk that belongs at its LDS position, which is how the swizzle
// (see swz8) is applied without a store.  128-byte row pieces per K step let
// every load cover whole cache lines.
#include "gemm_common.h"

namespace sbl {

namespace {

using namespace gemm;

template <int S>
struct StageIdx {
  static constexpr int value = S;
};

// Block tile 256 x 256 computed by 8 waves (2 along M x 4 along N, 128 x 64
// each): one block per CU.  Loading 64 KB per K step for 4M multiply-adds
// halves the bytes each CU pulls through its L1 per matrix instruction
// compared with a 256 x 128 tile, which is what the L2-to-CU path can feed.

constexpr int kNT = 512;                  // threads per block
constexpr int kBNn = 256;                 // block cols (N) of the square tile (host-side tile counts)
constexpr int kStages = 2;                // LDS stages of one K step each
constexpr int kKStep = kRowK / 2;         // 64 bf16 per K step
// Per K step a stage holds kBM rows of A (128 bytes each) and kBNn rows of B:
// 128 bytes of bf16, 16 bytes of codes (BC) or, for BQ, 64 rows k x kBNn int8.

// B as codes (BC): row n of B holds, per K step of 64, 16 bytes = 4 words;
// word 2 h + w serves lane half h (k groups 2 ks + h of the four 16-wide
// slices ks) for slices 2 w and 2 w + 1.  In it, pair p = 4 (ks % 2) + q
// (k = 16 ks + 8 h + 2 q and + 1) has the 2-bit code of its first k at bits
// 14 - 2p, 15 - 2p and of its second at 30 - 2p, 31 - 2p, so that
// (word << 2p) & 0xC000C000 is the bf16 pair of 2 W_eff: the high byte of
// bf16 +2 is 0x40, of -2 is 0xC0 and of 0 is 0x00, i.e. code << 6 for the
// codes 01 (+1), 11 (-1) and 00 (0), with a zero low byte in all three.
// The product is therefore 2 A W_eff^T, exact, and alpha is halved.
__device__ __forceinline__ v8bf widen_codes(uint32_t u, int p0) {
  v4i r;
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = (int)((u << (2 * (p0 + q))) & 0xC000C000u);
  return __builtin_bit_cast(v8bf, r);
}

// Requires K % 8 == 0 (16-byte rows, K chunks never straddle a row end).
// A split-K grid has gridDim.y K ranges [kps * s, kps * (s + 1)); the blocks are
// dealt to (range, tile) pairs by xcd_split_order, and range s writes
// its partial product to C + s * M * N.  With tail.head > 0 (a one-row grid)
// the first tail.head tiles of the grouped order take tail.head_splits ranges
// of kps and the others tail.tail_splits ranges of tail.tail_kps, each range s
// again into plane s (with tail.planes: plane 0 in C, plane s >= 1 at
// tail.planes + (s - 1) M N).  alpha_p == nullptr means alpha = 1.
//
// WTA (no split-K): the A tiles staged in LDS are also written out transposed
// and run-major (see BR), AT[k, m] = A[m, k] at element (m / 8 * K + k) * 8 +
// m % 8 for m < at_ld (at_ld >= M, a multiple of 8; m from M to at_ld read as
// zero from the tile and are written as zeros).  With wscale != nullptr each
// row m is scaled on the way: AT[k, m] = bf16(A[m, k] * (wscale[m] / 127))
// (float32 product, the scale taken as wscale[m] * fl(1/127)).  This is how
// the dX product leaves dY^T behind for dW: every (m tile, K step) is written
// once, by the block whose column tile index equals the step modulo the number
// of column tiles, from the stage as soon as it has landed.
//
// BC: B is the code layout above with rows of K64 / 4 bytes (K64 = K rounded
// up to 64, codes past K are 00); no split-K.
//
// BR: B (bf16, K % 8 == 0) is run-major: the 8 values k = 8 j .. 8 j + 7 of
// row n sit in the 16 bytes at (j N + n) * 16, i.e. [K / 8][N][8], which its
// producer writes in whole contiguous pieces.  The B stage in LDS is then
// run-major too, [8 runs][256 rows][16 bytes]: a direct load fills 64
// consecutive rows of one run from 1 KB of contiguous memory, and fragment
// reads (32 consecutive rows of a run per half wave) need no swizzle.  B rows
// past N read whatever follows (or zero past the buffer); they only feed
// output columns that are not stored.
//
// AR: A is run-major in the same way ([K / 8][M][8]) and so is its LDS stage.
//
// BQ: B is given as int8 rows along K, Bq[k, n] = B[n, k] row-major [K][N]
// (N % 16 == 0; rows k >= kb_rows read as zero), and widened to bf16 in
// registers (exact).  Its LDS stage holds the 64 K rows of a step x 256
// columns, 16-byte chunks of row k at chunk position c ^ (2 (k % 8)); a B
// fragment (8 consecutive k of one n) is one ds_read_b64_tr_b8: in each
// 16-lane group, lane q addresses the 8 bytes of row q / 2 at columns
// 8 (q % 2) .. + 7 of a block of 8 rows x 16 columns, and lane i receives
// column i of the 8 rows.  The swizzle spreads those 8 rows over 8 even (or,
// for the odd chunk the neighbouring group reads, 8 odd) chunk positions, so
// two groups never share a bank.
//
// BN: block columns, 256 or 512 (codes B only); the block has BM = 65536 / BN
// rows, so the accumulators stay 128 per lane with 8 waves of 128 x 64 (2 x 4
// waves, or 1 x 8).  With the 2-bit B of dX a K step then loads 16 KB of A and
// 8 KB of codes instead of 32 KB and 4 KB: a third fewer bytes per product.
template <int BN, int OUT, bool WTA, bool BC, bool AR, bool BR, bool BQ>
__global__ __launch_bounds__(kNT, 1) void k_gemm_nt_bf16(const uint16_t* __restrict__ A,
                                                              const uint16_t* __restrict__ B, int M, int N, int K,
                                                              int kps, const float* __restrict__ alpha_p,
                                                              void* __restrict__ C, uint16_t* __restrict__ AT,
                                                              int at_ld, const float* __restrict__ wscale,
                                                              int kb_rows, SplitTail tail) {
  static_assert(BN == 256 || (BN == 512 && BC), "512-column blocks take the code-plane B only");
  constexpr int kBM = 65536 / BN, kBNn = BN;  // (hide the square tile's constants)
  constexpr int kWavesN = BN / 64;            // waves along N (each 64 columns)
  constexpr int kStageA = kBM * kRowK;
  constexpr int kStageB = kBNn * kRowK;
  constexpr int kStageBC = kBNn * 16;
  constexpr int kStageBQ = kKStep * kBNn;
  constexpr int kDmaA = kBM * 8 / kNT;        // A loads (1 KB) per wave and K step
  constexpr int kDmaB = kBNn * 8 / kNT;
  constexpr int kDmaStep = kDmaA + kDmaB;
  constexpr int kSt = kStageA + (BC ? kStageBC : BQ ? kStageBQ : kStageB);
  constexpr int kDmaBw = BC ? 1 : BQ ? 2 : kDmaB;  // B loads per wave and step (BC: waves below kWavesN only)
  // LDS stages of one K step each: three for the 128 x 512 code-plane form (3 x 24 KB,
  // loads two steps ahead), two elsewhere (a third 48 KB stage of the int8 B form
  // measured no faster).  Each stage is an LDS variable of its own and the K loop is
  // unrolled by the number of stages, so that every stage access names its variable: the
  // compiler then tells the direct loads into one stage from reads of another and makes a
  // read wait only for the loads of its own stage (with one array it waits for all of them).
  // The epilogue reuses the stages as 8 KB of staging per wave.
  constexpr int kS = BC && BN == 512 ? 3 : kStages;
  // (with two stages of less than 32 KB the third variable holds the rest of the staging)
  constexpr int kWpS = kSt / 8192;  // 8 KB staging areas per stage
  static_assert(kSt % 8192 == 0 && (kS == 3 ? 3 * kWpS >= 8 : true), "stages must hold the 8 staging areas");
  __shared__ __attribute__((aligned(1024))) char lds0[kSt];
  __shared__ __attribute__((aligned(1024))) char lds1[kSt];
  __shared__ __attribute__((aligned(1024))) char lds2[kS == 3 ? kSt : 2 * kWpS >= 8 ? 16 : (8 - 2 * kWpS) * 8192];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS targets live in SGPRs
  const int wm0 = (wave / kWavesN) * kWM;
  const int wn0 = (wave % kWavesN) * kWN;
  int mt, nt, split = 0;
  // 32 tiles resident per XCD: 4 x 8 of 256 x 256 tiles, 8 x 4 of 128 x 512 ones
  {
    const int gm = (M + kBM - 1) / kBM, gn = (N + kBNn - 1) / kBNn;
    if (tail.head > 0) {
      // the head's blocks (whole rounds) take kps-long K ranges; the blocks after
      // them serve the remaining tiles with the deeper split
      const int nh = tail.head * tail.head_splits;
      int t;
      if ((int)blockIdx.x < nh) {
        xcd_split_order(blockIdx.x, tail.head, tail.head_splits, split, t);
      } else {
        xcd_split_order(blockIdx.x - nh, gm * gn - tail.head, tail.tail_splits, split, t);
        t += tail.head;
        kps = tail.tail_kps;
      }
      grouped_tile(t, gm, gn, BN == 256 ? 4 : 8, mt, nt);
    } else if (gridDim.y > 1) {
      int t;
      xcd_split_order(blockIdx.x + blockIdx.y * gridDim.x, gridDim.x, gridDim.y, split, t);
      grouped_tile(t, gm, gn, BN == 256 ? 4 : 8, mt, nt);
    } else {
      xcd_tile_grouped(blockIdx.x, gm, gn, BN == 256 ? 4 : 8, mt, nt);
    }
  }
  const int m0 = mt * kBM;
  const int n0 = nt * kBNn;
  const int kbeg = split * kps;
  const int kend = min(K, kbeg + kps);
  const int nk = (kend - kbeg + kKStep - 1) / kKStep;  // >= 1: the host never makes an empty split
  const int rows_a = min(kBM, M - m0);
  const int rows_b = min(kBNn, N - n0);
  const uint16_t* a_base = A + (AR ? (int64_t)m0 * 8 : (int64_t)m0 * K);
  const int64_t b_row = BC ? (int64_t)((K + 63) & ~63) / 4 : (int64_t)K * 2;  // bytes per B row
  const char* b_base = (const char*)B + (BQ ? (int64_t)n0 : BR ? (int64_t)n0 * 16 : n0 * b_row);

  // Direct-load lanes: LDS chunk position p (16 bytes) of a stage holds row
  // p / 8, logical chunk (p % 8) ^ ((row / 2) % 8), i.e. swz8(row, c) = 16 p.
  // Wave w fills positions [64 (kDma w + i), +64) with its i-th load.
  uint32_t a_off[kDmaA], b_off[kDmaBw];
  int a_k[kDmaA], b_k[kDmaBw];
#pragma unroll
  for (int i = 0; i < kDmaA; ++i) {
    const int p = 64 * (kDmaA * wave + i) + lane;
    if constexpr (AR) {
      const int c = p >> 8, r = p & 255;
      a_off[i] = (uint32_t)((c * M + r) * 16);
      a_k[i] = 8 * c;
    } else {
      const int r = p >> 3, c = (p & 7) ^ ((r >> 1) & 7);
      a_off[i] = (uint32_t)(r * K * 2 + 16 * c);
      a_k[i] = 8 * c;
    }
  }
  if constexpr (BC) {
    b_off[0] = (uint32_t)((64 * (wave % kWavesN) + lane) * b_row);  // row 64 w + lane, one 16-byte piece
    b_k[0] = 0;
  } else if constexpr (BQ) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = 64 * (2 * wave + i) + lane;
      const int r = p >> 4, c = (p & 15) ^ ((r & 7) << 1);  // K row r, logical 16-column chunk c
      b_off[i] = (uint32_t)(r * N + 16 * c);
      b_k[i] = r;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kDmaB; ++i) {
      const int p = 64 * (kDmaB * wave + i) + lane;
      if constexpr (BR) {
        const int c = p >> 8, r = p & 255;
        b_off[i] = (uint32_t)((c * N + r) * 16);
        b_k[i] = 8 * c;
      } else {
        const int r = p >> 3, c = (p & 7) ^ ((r >> 1) & 7);
        b_off[i] = (uint32_t)(r * K * 2 + 16 * c);
        b_k[i] = 8 * c;
      }
    }
  }

  // Loads of K step kt into stage st.  The resources span the valid rows of the
  // block (rows past M or N read as zero) and the K offset rides in soffset;
  // chunks past K (last step only) are sent out of range explicitly.
  const auto ar = make_rsrc(a_base, clamp_bytes(AR ? ((int64_t)(K / 8) * M - m0) * 16 : (int64_t)rows_a * K * 2));
  const uint32_t a_soff_per_k = AR ? (uint32_t)M * 2 : 2u;  // soffset bytes per k
  const auto br = make_rsrc(b_base, clamp_bytes(BQ   ? (int64_t)kb_rows * N - n0
                                                : BR ? ((int64_t)(K / 8) * N - n0) * 16
                                                     : (int64_t)rows_b * b_row));
  const bool ktail = ((kend - kbeg) % kKStep) != 0;
  // BC: the waves that load the code rows of a step (one 1 KB piece each; all 8 with 512 columns)
  const bool b_loader = kWavesN == 8 || wave < kWavesN;
  auto issue = [&](int kt, char* sa) {
    const int k0 = kbeg + kt * kKStep;
    const uint32_t soff = (uint32_t)k0 * 2;
    char* sb = sa + kStageA;
#pragma unroll
    for (int i = 0; i < kDmaA; ++i)
      dma16(ar, sa + 1024 * (kDmaA * wave + i), ktail && k0 + a_k[i] >= kend ? kOOB : a_off[i],
            (uint32_t)k0 * a_soff_per_k);
    if constexpr (BC) {
      if (b_loader) dma16(br, sb + 1024 * wave, b_off[0], (uint32_t)k0 / 4);
    } else if constexpr (BQ) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        dma16(br, sb + 1024 * (2 * wave + i), k0 + b_k[i] >= kb_rows ? kOOB : b_off[i], (uint32_t)k0 * (uint32_t)N);
    } else {
#pragma unroll
      for (int i = 0; i < kDmaB; ++i)
        dma16(br, sb + 1024 * (kDmaB * wave + i), ktail && k0 + b_k[i] >= kend ? kOOB : b_off[i],
              BR ? (uint32_t)k0 * (uint32_t)N * 2 : soff);
    }
  };

  const float alpha = alpha_p ? *alpha_p : 1.0f;  // fetched before the K loop

  // One load (index idx of the wave's loads of a step) of K step kt into stage sa.
  constexpr int kNDma = BC ? kDmaA + 1 : BQ ? kDmaA + 2 : kDmaStep;
  auto issue_one = [&](int kt, char* sa, int idx) {
    const int k0 = kbeg + kt * kKStep;
    const uint32_t soff = (uint32_t)k0 * 2;
    char* sb = sa + kStageA;
    if (idx < kDmaA) {
      dma16(ar, sa + 1024 * (kDmaA * wave + idx), ktail && k0 + a_k[idx] >= kend ? kOOB : a_off[idx],
            (uint32_t)k0 * a_soff_per_k);
    } else if constexpr (BC) {
      if (b_loader) dma16(br, sb + 1024 * wave, b_off[0], (uint32_t)k0 / 4);
    } else if constexpr (BQ) {
      const int i = idx - kDmaA;
      dma16(br, sb + 1024 * (2 * wave + i), k0 + b_k[i] >= kb_rows ? kOOB : b_off[i], (uint32_t)k0 * (uint32_t)N);
    } else {
      const int i = idx - kDmaA;
      dma16(br, sb + 1024 * (kDmaB * wave + i), ktail && k0 + b_k[i] >= kend ? kOOB : b_off[i],
            BR ? (uint32_t)k0 * (uint32_t)N * 2 : soff);
    }
  };

  v16f acc[kMI][kNJ];
#pragma unroll
  for (int i = 0; i < kMI; ++i)
#pragma unroll
    for (int j = 0; j < kNJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Fragments of K slice ks (16 of the 64 k of a step) of a stage.  BC: the
  // code words of the whole step are read by rdc beforehand (at a point where
  // no direct loads are in flight: the compiler makes a read of them wait for
  // all outstanding loads) and widened per slice.
  uint2 wb[kNJ];
  auto rdc = [&](const char* st) {
    if constexpr (BC) {
      const char* b = st + kStageA;
#pragma unroll
      for (int j = 0; j < kNJ; ++j) wb[j] = *(const uint2*)(b + 16 * (wn0 + 32 * j + (lane & 31)) + 8 * (lane >> 5));
    }
  };
  // BQ: the int8 B fragments of a whole step (8 transposed reads), read by rdq
  // where rdc reads code words (the compiler would make these reads wait for
  // every load in flight) and widened per slice.
  v2i wq[BQ ? 4 : 1][kNJ];
  auto rdq = [&](const char* st) {
    if constexpr (BQ) {
      const char* b = st + kStageA;
      const int g = lane >> 4, q = lane & 15;
      const int r0 = 8 * (g >> 1) + (q >> 1);  // the K row this lane addresses in slice 0 (+16 per slice)
      // One opaque lane offset per column block, so that every read is the stage
      // variable plus two offsets: the compiler tags only short address chains
      // with their LDS variable, and an untagged read waits for every load in
      // flight (which matters once loads are in flight here, with three stages).
      int qo[kNJ];
#pragma unroll
      for (int j = 0; j < kNJ; ++j) {
        const int c = (wn0 + 32 * j + 16 * (g & 1)) >> 4;
        qo[j] = r0 * kBNn + 16 * (c ^ ((r0 & 7) << 1)) + 8 * (q & 1);
        asm volatile("" : "+v"(qo[j]));
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int j = 0; j < kNJ; ++j) {
          const SBL_LDS char* pa = (const SBL_LDS char*)(b + qo[j] + 16 * ks * kBNn);
          wq[ks][j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SBL_LDS v2i*)pa);
        }
      }
    }
  };
  auto cvtq = [&](int ks, int j, v8bf (&fb)[kNJ]) {
    if constexpr (BQ) {
      // byte e: one sign-extending byte-select convert each; the bf16 of an integer
      // of at most 8 significant bits is the high half of its float32 (the low half
      // is zero), so one byte permute packs two of them
      v4i r;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t d = (uint32_t)wq[ks][j][h];
        const float f0 = (float)(int)(signed char)d, f1 = (float)(int)(signed char)(d >> 8);
        const float f2 = (float)(int)(signed char)(d >> 16), f3 = (float)((int)d >> 24);
        r[2 * h] = (int)__builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
        r[2 * h + 1] = (int)__builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
      }
      fb[j] = __builtin_bit_cast(v8bf, r);
    }
  };
  auto rd = [&](const char* a, int ks, v8bf (&fa)[kMI], v8bf (&fb)[kNJ]) {
    const char* b = a + kStageA;
#pragma unroll
    for (int i = 0; i < kMI; ++i) {
      const int m = wm0 + 32 * i + (lane & 31), c = 2 * ks + (lane >> 5);
      fa[i] = __builtin_bit_cast(v8bf, *(const v4i*)(a + (AR ? 16 * (c * kBM + m) : swz8(m, c))));
    }
    if constexpr (BC) {
#pragma unroll
      for (int j = 0; j < kNJ; ++j) fb[j] = widen_codes(ks < 2 ? wb[j].x : wb[j].y, 4 * (ks & 1));
    } else if constexpr (BQ) {
      // widened by cvtq, spread between the matrix instructions
    } else {
#pragma unroll
      for (int j = 0; j < kNJ; ++j) {
        const int n = wn0 + 32 * j + (lane & 31), c = 2 * ks + (lane >> 5);
        fb[j] = __builtin_bit_cast(v8bf, *(const v4i*)(b + (BR ? 16 * (c * kBNn + n) : swz8(n, c))));
      }
    }
  };
  // Transposed copy of the A tile of stage st (K step k0): wave w takes 16
  // K-columns (16 (w % 4) ..) and kBM / 2 rows (from kBM / 2 (w / 4)) in rounds of 32;
  // in each round its 16-lane group g reads rows 8 g .. 8 g + 7 with two
  // ds_read_b64_tr_b16 (lane i: 4 rows of column i each) and stores them as
  // one 16-byte run of AT row k0 + column.
  const int gn = (N + kBNn - 1) / kBNn;
  __shared__ __attribute__((aligned(16))) float wsc[WTA ? kBM : 4];
  constexpr int kAtRounds = kBM / 64;  // 32-row rounds of each wave
  auto write_at_round = [&](const char* a, int k0, int r) {
    const int kb = 16 * (wave & 3), tb0 = 32 * kAtRounds * (wave >> 2);
    const int g = lane >> 4, q = lane & 15;
    const auto atr = make_rsrc(AT, clamp_bytes((int64_t)at_ld * K * 2));
    const int kc = kb + 4 * (q & 3);                    // first of the 4 columns lane q addresses
    {
      const int t0 = tb0 + 32 * r + 8 * g;              // first of this group's 8 rows
      v4s part[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = t0 + 4 * h + (q >> 2);
        const SBL_LDS char* p = (const SBL_LDS char*)(a + swz8(row, kc >> 3) + 2 * (kc & 7));
        part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SBL_LDS v4s*)p);
      }
      const int col = kb + q;                           // this lane's K column
      const bool ok = k0 + col < K && m0 + t0 < at_ld;
      v4i v = __builtin_bit_cast(v4i, (v8s){part[0][0], part[0][1], part[0][2], part[0][3],
                                             part[1][0], part[1][1], part[1][2], part[1][3]});
      if (wscale) {
        const float4 s0 = *(const float4*)(wsc + t0), s1 = *(const float4*)(wsc + t0 + 4);
        const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float lo = __uint_as_float((uint32_t)v[u] << 16) * sv[2 * u];
          const float hi = __uint_as_float((uint32_t)v[u] & 0xFFFF0000u) * sv[2 * u + 1];
          v[u] = (int)cvt_pk_bf16(lo, hi);
        }
      }
      __builtin_amdgcn_raw_buffer_store_b128(v, atr, ok ? (uint32_t)((((m0 + t0) >> 3) * K + k0 + col) * 16) : kOOB,
                                             0, 0);
    }
  };
  auto write_at = [&](const char* a, int k0) {
#pragma unroll
    for (int r = 0; r < kAtRounds; ++r) write_at_round(a, k0, r);
  };

  auto mm_one = [&](int t, const v8bf (&fa)[kMI], const v8bf (&fb)[kNJ]) {
    acc[t / kNJ][t % kNJ] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[t % kNJ], fa[t / kNJ], acc[t / kNJ][t % kNJ],
                                                                    0, 0, 0);
  };
  auto mm = [&](const v8bf (&fa)[kMI], const v8bf (&fb)[kNJ]) {
#pragma unroll
    for (int i = 0; i < kMI; ++i)
#pragma unroll
      for (int j = 0; j < kNJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
  };
  constexpr int kRdN = BC || BQ ? kMI : kMI + kNJ;  // LDS reads of a slice
// BQ: the widening of the next slice's B fragments (vector ALU) is spread
// over the slice's matrix instructions, 5 instructions after each.
#define ORDER_SLICE(id)                                              \
  if constexpr (BQ) {                                                \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, id);              \
    __builtin_amdgcn_sched_group_barrier(0x100, kRdN, id);           \
    for (int z_ = 0; z_ < kMI * kNJ - 1; ++z_) {                     \
      __builtin_amdgcn_sched_group_barrier(0x002, 5, id);            \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, id);            \
    }                                                                \
  } else {                                                           \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, id);              \
    __builtin_amdgcn_sched_group_barrier(0x100, kRdN, id);           \
    __builtin_amdgcn_sched_group_barrier(0x008, kMI * kNJ - 1, id);  \
  }

  // Step k (stage k % kS has landed; slice 0 is already in fa0/fb0): each of
  // the 4 slices is read while the previous one is multiplied.  Before the
  // last slice: wait for this wave's loads of step k + 1 (with three stages
  // those of step k + 2 stay in flight) and for its reads of stage k, barrier
  // (every wave's loads of step k + 1 landed, every wave done reading stage k),
  // refill stage k % kS with step k + kS, then read slice 0 of step k + 1 while
  // multiplying slice 3.  Past the last step the load index is clamped: the
  // redundant loads go to a stage nobody reads again.
  v8bf fa0[kMI], fb0[kNJ], fa1[kMI], fb1[kNJ];
  const int last = nk - 1;
  if constexpr (WTA) {
    // row scales of the side output (visible to all waves after the first barrier)
    if (wscale && tid < kBM) wsc[tid] = m0 + tid < M ? wscale[m0 + tid] * (1.0f / 127.0f) : 0.0f;
  }
  issue(0, lds0);
  issue(min(1, last), lds1);
  if constexpr (kS == 3) issue(min(2, last), lds2);
  if constexpr (BC) {  // (lgkmcnt too: the scale table above is read after the barrier)
    if (b_loader) wait_vmcnt_lgkm0<(kS - 1) * (kDmaA + 1)>();
    else wait_vmcnt_lgkm0<(kS - 1) * kDmaA>();
  } else {
    wait_vmcnt<(kS - 1) * kNDma>();  // this wave's loads of step 0 (those of the later steps may be in flight)
  }
  barrier_only();
  if constexpr (WTA) {
    if (nt == 0) write_at(lds0, kbeg);
  }
  rdc(lds0);
  rdq(lds0);
  rd(lds0, 0, fa0, fb0);
#pragma unroll
  for (int j = 0; j < kNJ; ++j) cvtq(0, j, fb0);
  // Step k out of stage S (a constant: see the LDS variables above).
  auto step = [&](auto stage, int k) {
    constexpr int S = decltype(stage)::value, X = (S + 1) % kS;  // stages of steps k and k + 1
    char* const cur = S == 0 ? lds0 : S == 1 ? lds1 : lds2;
    char* const nxt = X == 0 ? lds0 : X == 1 ? lds1 : lds2;
    rd(cur, 1, fa1, fb1);
#pragma unroll
    for (int j = 0; j < kNJ; ++j) cvtq(1, j, fb1);
    mm(fa0, fb0);
    ORDER_SLICE(0)
    __builtin_amdgcn_sched_barrier(0);
    rd(cur, 2, fa0, fb0);
#pragma unroll
    for (int j = 0; j < kNJ; ++j) cvtq(2, j, fb0);
    mm(fa1, fb1);
    ORDER_SLICE(1)
    __builtin_amdgcn_sched_barrier(0);
    rd(cur, 3, fa1, fb1);
#pragma unroll
    for (int j = 0; j < kNJ; ++j) cvtq(3, j, fb1);
    mm(fa0, fb0);
    ORDER_SLICE(2)
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kS == 3) {  // all but the newest step's loads (loads complete in order)
      if (BC && !b_loader) wait_vmcnt_lgkm0<kDmaA>();
      else wait_vmcnt_lgkm0<kNDma>();
    } else {
      wait_vmcnt_lgkm0<0>();
    }
    barrier_only();
    __builtin_amdgcn_sched_barrier(0);
    // this block writes the transposed copy of step k + 1's A tile (landed, and not refilled
    // before the next barrier), one round after each of the first matrix instructions below
    const bool wt = WTA && k + 1 < nk && (k + 1) % gn == nt;
    if constexpr (BC) {
      rdc(nxt);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (BQ) {
      rdq(nxt);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Slice 3 (its fragments are in registers) restarts the matrix pipe right
    // after the barrier; the reads of slice 0 of step k + 1 and the loads of
    // step k + kS go between its instructions, one load after each, into the
    // stage of step k, which every wave has finished reading.
    const int kn = min(k + kS, last);
    mm_one(0, fa1, fb1);
    __builtin_amdgcn_sched_barrier(0);
    rd(nxt, 0, fa0, fb0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < kMI * kNJ; ++t) {
      if (t > 0) mm_one(t, fa1, fb1);
      __builtin_amdgcn_sched_barrier(0);
      // (its LDS reads and stores overlap the matrix pipe: -0.3% on the backward against
      // writing it before the pipe restarts)
      if constexpr (WTA) {
        if (t < kAtRounds && wt) write_at_round(nxt, kbeg + (k + 1) * kKStep, t);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (t < kNDma) issue_one(kn, cur, t);
      // BQ: slice 0's B widening in the last slots, when its reads have landed
      if (t >= kMI * kNJ - kNJ) cvtq(0, t - (kMI * kNJ - kNJ), fb0);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = kMI * kNJ; t < kNDma; ++t) issue_one(kn, cur, t);
    __builtin_amdgcn_sched_barrier(0);
  };
  // Whole rounds of kS steps, then the remaining steps in straight code (an
  // exit from the middle of a round makes the compiler keep more registers
  // live across the loop).
  int k = 0;
  for (; k + kS <= nk; k += kS) {
    step(StageIdx<0>{}, k);
    step(StageIdx<1>{}, k + 1);
    if constexpr (kS == 3) step(StageIdx<2>{}, k + 2);
  }
  if (k < nk) step(StageIdx<0>{}, k);
  if constexpr (kS == 3) {
    if (k + 1 < nk) step(StageIdx<1>{}, k + 1);
  }
  // No direct loads may still target LDS when the block retires.
  wait_vmcnt<0>();

  // B is the MFMA's first operand, so accumulator register r of lane l holds
  // C[m = l % 32][n = 8 (r / 4) + 4 (l / 32) + r % 4]: each lane stores runs
  // of 4 consecutive outputs of one row (16 bytes in float32, 8 in bf16).
  constexpr float pre = BC ? 0.5f : 1.0f;  // BC: the sums are of 2 W_eff (halving is exact)
  // bf16 outputs (dX) stream past the caches: -0.5% on the backward; the float32 ones (dW, and
  // split-K planes that the sum reads back) measured the same either way and stay cached stores
  constexpr bool final_out = OUT == SBL_BF16;
  if (tail.planes && split > 0)
    C = (char*)tail.planes + (size_t)(split - 1) * (size_t)M * (size_t)N * (OUT == SBL_F32 ? 4 : 2);
  else
    C = (char*)C + (size_t)split * (size_t)M * (size_t)N * (OUT == SBL_F32 ? 4 : 2);

  // With 16-byte aligned output rows the wave's 128 x 64 result goes through
  // LDS, 8 KB per wave and round (64 rows of 128 bytes in bf16, 32 rows of 256
  // bytes in float32; 16-byte chunks swizzled by row), so that every store
  // instruction writes whole row segments of the wave's 64 columns.
  if ((N & (OUT == SBL_F32 ? 3 : 7)) == 0) {
    __syncthreads();  // every wave is done with the operand stages (no loads in flight)
    char* stg = wave < kWpS ? lds0 + wave * 8192
                : wave < 2 * kWpS ? lds1 + (wave - kWpS) * 8192 : lds2 + (wave - 2 * kWpS) * 8192;
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
            const float v0 = acc[i][j][4 * q] * pre * alpha, v1 = acc[i][j][4 * q + 1] * pre * alpha;
            const float v2 = acc[i][j][4 * q + 2] * pre * alpha, v3 = acc[i][j][4 * q + 3] * pre * alpha;
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
        if (m < M && n < N) {
          char* const p = (char*)C + ((int64_t)m * N + n) * (OUT == SBL_F32 ? 4 : 2);
          if (final_out) store_nt16(p, v);
          else *(uint4*)p = v;
        }
      }
    }
    return;
  }
  const bool vec_out = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < kMI; ++i) {
    const int m = m0 + wm0 + 32 * i + (lane & 31);
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < kNJ; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn0 + 32 * j + 8 * q + 4 * (lane >> 5);
        if (n >= N) continue;
        const int64_t off = (int64_t)m * N + n;
        const float v0 = acc[i][j][4 * q] * pre * alpha, v1 = acc[i][j][4 * q + 1] * pre * alpha;
        const float v2 = acc[i][j][4 * q + 2] * pre * alpha, v3 = acc[i][j][4 * q + 3] * pre * alpha;
        if (vec_out && n + 4 <= N) {
          if constexpr (OUT == SBL_F32) *(float4*)((float*)C + off) = make_float4(v0, v1, v2, v3);
          else *(uint2*)((__bf16*)C + off) = make_uint2(cvt_pk_bf16(v0, v1), cvt_pk_bf16(v2, v3));
        } else {
          const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (n + u >= N) break;
            if constexpr (OUT == SBL_F32) ((float*)C)[off + u] = vv[u];
            else ((__bf16*)C)[off + u] = (__bf16)vv[u];
          }
        }
      }
    }
  }
}

}  // namespace

bool gemm_nt_bf16_supported(int64_t M, int64_t N, int64_t K) {
  // K % 8: whole 16-byte chunks per row; the per-block resources must stay
  // below the 2 GiB range of a buffer offset.
  return M > 0 && N > 0 && K > 0 && K % 8 == 0 && (int64_t)kBM * K * 2 <= kMaxRsrcBytes &&
         (int64_t)kBNn * K * 2 <= kMaxRsrcBytes;
}

bool gemm_nt_runs_supported(int64_t M, int64_t N, int64_t K) {
  // a whole run-major operand is one buffer resource, and soffset = k0 * rows * 2
  return gemm_nt_bf16_supported(M, N, K) && K % 8 == 0 && (K / 8) * N * 16 <= kMaxRsrcBytes &&
         (K / 8) * M * 16 <= kMaxRsrcBytes;
}

int64_t gemm_nt_bf16_tiles(int64_t M, int64_t N) { return ((M + kBM - 1) / kBM) * ((N + kBNn - 1) / kBNn); }

hipError_t launch_gemm_nt_bf16(const uint16_t* A, const uint16_t* B, int64_t M, int64_t N, int64_t K,
                               const float* alpha, void* C, int out_dtype, hipStream_t s, int splits,
                               int64_t k_per_split, uint16_t* AT, int64_t at_ld) {
  if (splits < 1) splits = 1;
  if (splits == 1) k_per_split = K;
  if (AT && splits != 1) return hipErrorInvalidValue;
  const dim3 grid((unsigned)gemm_nt_bf16_tiles(M, N), (unsigned)splits), block(kNT);
  const bool f32 = out_dtype == SBL_F32;
  auto kern = AT ? (f32 ? k_gemm_nt_bf16<256, SBL_F32, true, false, false, false, false> : k_gemm_nt_bf16<256, SBL_BF16, true, false, false, false, false>)
                 : (f32 ? k_gemm_nt_bf16<256, SBL_F32, false, false, false, false, false> : k_gemm_nt_bf16<256, SBL_BF16, false, false, false, false, false>);
  hipLaunchKernelGGL(kern, grid, block, 0, s, A, B, (int)M, (int)N, (int)K, (int)k_per_split, alpha, C, AT,
                     (int)at_ld, nullptr, 0, SplitTail{0, 0, 0, 0, nullptr});
  return hipGetLastError();
}

hipError_t launch_gemm_nt_runs(const uint16_t* A, bool a_runs, const uint16_t* Brun, int64_t M, int64_t N, int64_t K,
                               void* C, hipStream_t s, int splits, int64_t k_per_split) {
  if (splits < 1) splits = 1;
  if (splits == 1) k_per_split = K;
  const dim3 grid((unsigned)gemm_nt_bf16_tiles(M, N), (unsigned)splits), block(kNT);
  auto kern = a_runs ? k_gemm_nt_bf16<256, SBL_F32, false, false, true, true, false> : k_gemm_nt_bf16<256, SBL_F32, false, false, false, true, false>;
  hipLaunchKernelGGL(kern, grid, block, 0, s, A, Brun, (int)M, (int)N, (int)K, (int)k_per_split, nullptr, C, nullptr,
                     0, nullptr, 0, SplitTail{0, 0, 0, 0, nullptr});
  return hipGetLastError();
}

bool gemm_nt_q_supported(int64_t M, int64_t N, int64_t K, int64_t kb_rows) {
  // run-major A and int8 B are each one buffer resource (soffset = k0 * rows * 2, k0 * N)
  return gemm_nt_bf16_supported(M, N, K) && K % 8 == 0 && N % 16 == 0 && (K / 8) * M * 16 <= kMaxRsrcBytes &&
         kb_rows * N <= kMaxRsrcBytes && K * N <= kMaxRsrcBytes;
}

hipError_t launch_gemm_nt_q(const uint16_t* Arun, const int8_t* Bq, int64_t M, int64_t N, int64_t K, int64_t kb_rows,
                            float* C, hipStream_t s, int splits, int64_t k_per_split, SplitTail tail) {
  if (splits < 1) splits = 1;
  if (splits == 1) k_per_split = K;
  const int64_t tiles = gemm_nt_bf16_tiles(M, N);
  dim3 grid((unsigned)tiles, (unsigned)splits);
  if (tail.head > 0) {
    // the head's blocks must fill whole rounds (the tail's order starts a round)
    if (tail.head >= tiles || tail.head_splits != splits || (tail.head * splits) % 256 != 0 ||
        tail.tail_splits < 1 || tail.tail_kps < 64 || tail.tail_kps % 64 != 0 || (splits > 1 && k_per_split % 64 != 0))
      return hipErrorInvalidValue;
    grid = dim3((unsigned)(tail.head * splits + (tiles - tail.head) * tail.tail_splits), 1);
  }
  hipLaunchKernelGGL((k_gemm_nt_bf16<256, SBL_F32, false, false, true, false, true>), grid, dim3(kNT), 0, s, Arun,
                     (const uint16_t*)Bq, (int)M, (int)N, (int)K, (int)k_per_split, nullptr, (void*)C, nullptr, 0,
                     nullptr, (int)kb_rows, tail);
  return hipGetLastError();
}

hipError_t launch_gemm_nt_codes(const uint16_t* A, const uint32_t* Bc, int64_t M, int64_t N, int64_t K,
                                const float* alpha, void* C, int out_dtype, hipStream_t s, uint16_t* AT,
                                int64_t at_ld, const float* wscale) {
  // 128 x 512 blocks: a third fewer operand bytes per product than 256 x 256 with a 2-bit B
  const dim3 grid((unsigned)(((M + 127) / 128) * ((N + 511) / 512))), block(kNT);
  const bool f32 = out_dtype == SBL_F32;
  auto kern = AT ? (f32 ? k_gemm_nt_bf16<512, SBL_F32, true, true, false, false, false> : k_gemm_nt_bf16<512, SBL_BF16, true, true, false, false, false>)
                 : (f32 ? k_gemm_nt_bf16<512, SBL_F32, false, true, false, false, false> : k_gemm_nt_bf16<512, SBL_BF16, false, true, false, false, false>);
  hipLaunchKernelGGL(kern, grid, block, 0, s, A, (const uint16_t*)Bc, (int)M, (int)N, (int)K, (int)K, alpha, C, AT,
                     (int)at_ld, wscale, 0, SplitTail{0, 0, 0, 0, nullptr});
  return hipGetLastError();
}

}  // namespace sbl
