// Decode forward (T <= 64 tokens on pre-packed weights, [SUM] Table 3 decode
// rows): y[t, o] = (sum_k x_q[t, k] W_eff[o, k]) * gamma * a_t / 127 with the
// int32 sums exact, from either weight plane:
//
//   code plane  2 bits per weight (00 = 0, 01 = +1, 11 = -1), any N:8;
//   pair plane  one byte per group of 8 for masks keeping at most 2 of 8:
//               9 * rank(p0, p1) + 3 * digit(v0) + digit(v1), half the bytes.
//
// At these token counts the launch is bound by the weight bytes and by memory
// latency, not by the matrix cores, so the kernel is laid out for bytes in
// flight:
// * every lane loads whole 16-byte chunks of a weight row (64 weights of the
//   code plane, 128 of the pair plane); a wave's load covers 16 rows x 4
//   consecutive chunks, and all of a wave's loads for a tile are issued before
//   its first product;
// * the instruction is v_mfma_i32_16x16x64_i8 with the weights as the first
//   operand.  Its 64-wide K is four quadrants of 16 (lane l: row l % 16,
//   quadrant l / 16); quadrant q of instruction u takes the 16 k starting at
//   16 u inside the chunk that lane's load brought (chunk 4 j + q), and the
//   token operand takes the same k from the activation tile, so each lane
//   expands only what it loaded;
// * blocks are few and long-lived: a block stages the activations once (the
//   int8 tile copied from x_q, or x itself quantized with the act-quant
//   arithmetic) and then walks tile groups; a tile is 16 (or 8) output rows,
//   its K range split over wpt waves whose partial sums are added in LDS in a
//   fixed order (integers: exact).
// Accumulator register r of lane l holds C[o = 4 (l / 16) + r][t = l % 16].
#include <algorithm>

#include "act_common.h"
#include "gemm_common.h"

namespace sbl {

namespace {

using namespace gemm;

constexpr int kDecTile = 16;  // rows of one matrix instruction

// Dispatch plan of one launch: up to kDecodeMultiMax matrices sharing the
// activations, their tiles numbered by prefix sums.
struct DecPlan {
  int count;
  int tile_begin[kDecodeMultiMax + 1];
  int d_out[kDecodeMultiMax];
  const uint8_t* plane[kDecodeMultiMax];
  const float* gamma[kDecodeMultiMax];
  void* y[kDecodeMultiMax];
  int rows;    // output rows per tile: 16, or 8 on small grids (the instruction's other 8 read zeros)
  int wpt;     // waves per tile (K split)
  int per;     // chunk quads per wave
  int nchunk;  // 16-byte chunks per weight row
  int groups;  // tile groups: W / wpt tiles each
};

// LDS layout (bytes): activation tile [T][d_in + 16] int8, token scales, row
// maxima, pair table [256] x 8 bytes, partial sums [W][NTT][4][64] int32.
struct DecLds {
  int xs, amax, rmax, table, red, total;
};
__host__ __device__ inline DecLds dec_lds(int T, int d_in, int W, int NTT, bool pairs, bool stage) {
  DecLds L;
  L.xs = 0;
  L.amax = stage ? ((T * (d_in + 16) + 15) & ~15) : 0;
  L.rmax = L.amax + 64 * 4;
  L.table = L.rmax + 64 * 4;
  L.red = L.table + (pairs ? 256 * 8 : 0);
  L.total = L.red + W * NTT * 4 * 64 * 4;
  return L;
}

// The weight stream: every plane byte is read once per call, and a model reads a layer's planes
// again only after every other layer's, so they are not kept in the caches (`nt`, cache-policy
// bit 1 of the buffer load): a layer at one token -2% when the planes stream from HBM.
__device__ __forceinline__ uint4 bload16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}

// 4 two-bit codes (one byte) -> 4 int8 values (00 -> 0, 01 -> 1, 11 -> -1).
__device__ __forceinline__ uint32_t codes4(uint32_t byte4codes) {
  uint32_t x = byte4codes & 0xFFu;
  x = (x | (x << 12)) & 0x000F000Fu;
  x = (x | (x << 6)) & 0x03030303u;
  return __builtin_amdgcn_perm(0u, 0xFF000100u, x);
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// XS: where the token operand comes from: 0 x_q in global memory, 1 x_q
// copied into LDS, 2 bf16 x quantized into LDS (the activation quantization
// fused in; each thread keeps up to kFuseRegs 16-byte chunks).
constexpr int kFuseRegs = 16;
constexpr int kQ = 8;  // chunk quads whose loads a wave keeps in flight

template <int OUT, int W, int NTT, bool PAIRS, int XS>
__global__ __launch_bounds__(64 * W) void k_decode(const void* __restrict__ xin, const float* __restrict__ absmax_in,
                                                   const DecPlan p, int T, int d_in) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int KC = PAIRS ? 128 : 64;  // weights per 16-byte chunk
  constexpr int U = KC / 16;            // matrix instructions per chunk
  constexpr int UH = PAIRS ? 4 : U;     // instructions whose token operands are loaded together (XS = 0)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r16 = lane & 15;
  const int ld = d_in + 16;
  const DecLds L = dec_lds(T, d_in, W, NTT, PAIRS, XS > 0);
  char* xs = smem + L.xs;
  float* amax = (float*)(smem + L.amax);
  uint32_t* rmax = (uint32_t*)(smem + L.rmax);
  const uint2* table = (const uint2*)(smem + L.table);
  int* red = (int*)(smem + L.red);

  const int tpg = W / p.wpt;
  const int slot = wave / p.wpt, ks = wave - slot * p.wpt;
  const int nquad = (p.nchunk + 3) >> 2;
  const int qbeg = ks * p.per, qend = min(nquad, qbeg + p.per);
  const int row_bytes = PAIRS ? d_in >> 3 : d_in >> 2;
  const int ntiles = p.tile_begin[p.count];
  int* my_red = red + (size_t)wave * NTT * 256;

  // Tile of group g for this wave, and the loads of its chunk quads qb .. qb + kQ - 1.
  struct TileRef {
    int item, row0, rows;
    __amdgpu_buffer_rsrc_t br;
  };
  auto tile_ref = [&](int g) {
    TileRef t;
    const int tile = g * tpg + slot;
    t.item = 0;
    while (t.item + 1 < p.count && tile >= p.tile_begin[t.item + 1]) ++t.item;
    t.row0 = (tile - p.tile_begin[t.item]) * p.rows;
    t.rows = tile < ntiles ? min(p.rows, p.d_out[t.item] - t.row0) : 0;
    t.br = make_rsrc(p.plane[t.item] + (int64_t)(t.rows > 0 ? t.row0 : 0) * row_bytes,
                     clamp_bytes((int64_t)t.rows * row_bytes));
    return t;
  };
  uint4 cw[kQ];
  auto issue = [&](const TileRef& t, int qb) {
    const int nq = min(kQ, qend - qb);  // wave-uniform
#pragma unroll
    for (int j = 0; j < kQ; ++j) {
      const int chunk = 4 * (qb + j) + q;
      cw[j] = make_uint4(0u, 0u, 0u, 0u);
      if (j < nq)
        cw[j] = bload16_nt(t.br, chunk < p.nchunk && r16 < t.rows ? (uint32_t)(r16 * row_bytes + 16 * chunk) : kOOB);
    }
  };

  // XS == 2: this thread's activation chunks (kc consecutive 16-byte chunks, so that a
  // thread's chunks mostly lie in one row) are loaded first, then the first group's weights;
  // vector memory returns in issue order, so the quantization below waits for the
  // activations only and runs while the weight bytes are in flight.
  uint4 xv[XS == 2 ? kFuseRegs : 1];
  int kc = 0;
  if constexpr (XS == 2) {
    const int total = T * (d_in >> 3);
    kc = (total + 64 * W - 1) / (64 * W);  // <= kFuseRegs (checked by the launcher)
    const auto xr0 = make_rsrc(xin, clamp_bytes((int64_t)total * 16));
#pragma unroll
    for (int i = 0; i < kFuseRegs; ++i) {
      const int c = tid * kc + i;
      xv[i] = make_uint4(0u, 0u, 0u, 0u);
      if (i < kc) xv[i] = bload16(xr0, c < total ? (uint32_t)c * 16u : kOOB);  // block-uniform test
    }
  }
  TileRef ti = tile_ref(blockIdx.x);
  if constexpr (XS == 2) {
    // exactly kQ loads whatever the wave's share (slots past it read zero without touching
    // memory), so that the compiler can wait for the activations with vmcnt(kQ)
    const bool on = blockIdx.x < p.groups && qbeg < qend;
    const int nq = on ? min(kQ, qend - qbeg) : 0;
#pragma unroll
    for (int j = 0; j < kQ; ++j) {
      const int chunk = 4 * (qbeg + j) + q;
      cw[j] = bload16_nt(ti.br, j < nq && chunk < p.nchunk && r16 < ti.rows ? (uint32_t)(r16 * row_bytes + 16 * chunk)
                                                                         : kOOB);
    }
  } else {
    if (blockIdx.x < p.groups && qbeg < qend) issue(ti, qbeg);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- set-up: pair table, activation tile and token scales
  if constexpr (PAIRS) {
    if (tid < 256) ((uint2*)(smem + L.table))[tid] = pair_expand((uint32_t)tid);
  }
  if constexpr (XS == 2) {
    // x bf16 [T][d_in]: T * d_in / 8 chunks over the block, kc consecutive ones per thread
    const int nch = d_in >> 3, total = T * nch;
    if (tid < T) rmax[tid] = 0u;
    __syncthreads();
    const auto cmax = [&](const uint4& v) {
      return max(max(max_mag2(v.x), max_mag2(v.y)), max(max_mag2(v.z), max_mag2(v.w)));
    };
    if (kc == 1) {  // (block-uniform) one chunk per thread: chunk tid
      const bool in = tid < total;
      const int t = in ? tid / nch : 0;
      if (in) atomicMax(&rmax[t], cmax(xv[0]));  // integer maximum: the order does not matter
      __syncthreads();
      if (tid < T) amax[tid] = __uint_as_float(rmax[tid] << 16);
      if (in) {
        const uint32_t m = rmax[t];
        const ActScale qs = act_scale(m ? __uint_as_float(m << 16) : 1.0f);
        *(uint2*)(xs + t * ld + 8 * (tid - t * nch)) = m ? quant_chunk(xv[0], qs.k, qs.as, qs.c) : make_uint2(0u, 0u);
      }
    } else {
      {  // row maxima: a running maximum per thread, one LDS atomic per row it touches
        uint32_t m = 0;
        int trow = -1;
#pragma unroll
        for (int i = 0; i < kFuseRegs; ++i) {
          const int c = tid * kc + i;
          if (i < kc && c < total) {
            const int t = c / nch;
            if (t != trow) {
              if (trow >= 0) atomicMax(&rmax[trow], m);
              trow = t;
              m = 0;
            }
            m = max(m, cmax(xv[i]));
          }
        }
        if (trow >= 0) atomicMax(&rmax[trow], m);
      }
      __syncthreads();
      if (tid < T) amax[tid] = __uint_as_float(rmax[tid] << 16);
      {  // the row scale set-up once per row a thread touches
        int srow = -1;
        uint32_t m = 0;
        ActScale qs = {0, 1.0f, 1.0f};
#pragma unroll
        for (int i = 0; i < kFuseRegs; ++i) {
          const int c = tid * kc + i;
          if (i < kc && c < total) {
            const int t = c / nch, j = c - t * nch;
            if (t != srow) {
              srow = t;
              m = rmax[t];
              qs = act_scale(m ? __uint_as_float(m << 16) : 1.0f);
            }
            *(uint2*)(xs + t * ld + 8 * j) = m ? quant_chunk(xv[i], qs.k, qs.as, qs.c) : make_uint2(0u, 0u);
          }
        }
      }
    }
  } else if constexpr (XS == 1) {
    const int n16 = d_in >> 4, total = T * n16;
    for (int c = tid; c < total; c += 64 * W) {
      const int t = c / n16, j = c - t * n16;
      *(uint4*)(xs + t * ld + 16 * j) = ((const uint4*)xin)[c];
    }
    if (tid < T) amax[tid] = absmax_in[tid];
  } else {
    if (tid < T) amax[tid] = absmax_in[tid];
  }
  __syncthreads();

  const auto xr = make_rsrc(xin, clamp_bytes((int64_t)T * d_in));

  for (int g = blockIdx.x; g < p.groups; g += gridDim.x) {
    const bool tile_ok = ti.rows > 0;
    const int item = ti.item, row0 = ti.row0, rows = ti.rows;
    const int d_out = p.d_out[item];
    // two accumulators per token tile, alternating over the instructions, so that
    // consecutive matrix instructions do not wait on each other (integer sums: exact)
    v4i acc[NTT], acc2[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[tt] = acc2[tt] = (v4i){0, 0, 0, 0};

    // rounds of up to kQ chunk quads (the first one already in flight)
    for (int qb = qbeg; qb < qend; qb += kQ) {
      if (qb != qbeg) {
        issue(ti, qb);
        __builtin_amdgcn_sched_barrier(0);
      }
      const int nq = min(kQ, qend - qb);  // wave-uniform
#pragma unroll
      for (int j = 0; j < kQ; ++j) {
        if (j >= nq) break;  // wave-uniform
        const int chunk = min(4 * (qb + j) + q, p.nchunk - 1);  // past the row: zero weights, any x
#pragma unroll
        for (int h = 0; h < U; h += UH) {
          // this part's token operands (global memory or the LDS tile) and weight operands
          // (expanded codes, or pair-table entries from LDS), all read before its first
          // matrix instruction so that their latencies overlap
          v4i bx[UH][NTT], av[UH];
#pragma unroll
          for (int u = 0; u < UH; ++u)
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
              const int t = 16 * tt + r16;
              const int kb = chunk * KC + 16 * (h + u);
              if constexpr (XS == 0)
                bx[u][tt] = __builtin_bit_cast(v4i, bload16(xr, t < T ? (uint32_t)(t * d_in + kb) : kOOB));
              else
                bx[u][tt] = t < T ? *(const v4i*)(xs + t * ld + kb) : (v4i){0, 0, 0, 0};
            }
#pragma unroll
          for (int u = 0; u < UH; ++u) {
            if constexpr (PAIRS) {
              const uint32_t w = word_of(cw[j], (h + u) >> 1) >> (16 * ((h + u) & 1));
              const uint2 e0 = table[w & 0xFFu], e1 = table[(w >> 8) & 0xFFu];
              av[u] = (v4i){(int)e0.x, (int)e0.y, (int)e1.x, (int)e1.y};
            } else {
              const uint32_t w = word_of(cw[j], h + u);
              av[u] = (v4i){(int)codes4(w), (int)codes4(w >> 8), (int)codes4(w >> 16), (int)codes4(w >> 24)};
            }
          }
#pragma unroll
          for (int u = 0; u < UH; ++u)
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
              if (u & 1) acc2[tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[u], bx[u][tt], acc2[tt], 0, 0, 0);
              else acc[tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[u], bx[u][tt], acc[tt], 0, 0, 0);
            }
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[tt] += acc2[tt];
    // the next group's first loads go out before this one's sums are stored
    if (g + (int)gridDim.x < p.groups) {
      ti = tile_ref(g + gridDim.x);
      if (qbeg < qend) issue(ti, qbeg);
    }
    __builtin_amdgcn_sched_barrier(0);

    // partial sums of a tile's waves, added in the order ks = 1, 2, ...
    if (p.wpt > 1) {
      if (ks > 0) {
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
          for (int r = 0; r < 4; ++r) my_red[(tt * 4 + r) * 64 + lane] = acc[tt][r];
      }
      __syncthreads();
      if (ks == 0) {
        for (int k = 1; k < p.wpt; ++k) {
          const int* o = red + (size_t)(wave + k) * NTT * 256;
#pragma unroll
          for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[tt][r] += o[(tt * 4 + r) * 64 + lane];
        }
      }
    }
    if (ks == 0 && tile_ok) {
      const float g127 = *p.gamma[item] * (1.0f / 127.0f);
      void* __restrict__ y = p.y[item];
      const bool vec_out = (d_out & 3) == 0;
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
        const int t = 16 * tt + r16;
        const int o = row0 + 4 * q;
        if (t >= T || 4 * q >= rows) continue;
        const float s = g127 * amax[t];
        const int64_t off = (int64_t)t * d_out + o;
        const int a0 = acc[tt][0], a1 = acc[tt][1], a2 = acc[tt][2], a3 = acc[tt][3];
        if (vec_out && 4 * q + 4 <= rows) {
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
            if (4 * q + u >= rows) break;
            if constexpr (OUT == SBL_I32) ((int*)y)[off + u] = av[u];
            else if constexpr (OUT == SBL_F32) ((float*)y)[off + u] = (float)av[u] * s;
            else ((__bf16*)y)[off + u] = (__bf16)((float)av[u] * s);
          }
        }
      }
    }
    if (p.wpt > 1) __syncthreads();  // the partial sums are read before the next group writes them
  }
}

// Pair plane from the code plane: one thread per group of 8.  A group with
// more than 2 non-zeros has no pair byte: it is written as 0 and counted.
__global__ __launch_bounds__(256) void k_pack_pairs(const uint16_t* __restrict__ codes, int64_t n,
                                                    uint8_t* __restrict__ plane, unsigned long long* __restrict__ bad) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  unsigned long long nbad = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint32_t c = codes[i];
    uint32_t nz = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) nz |= ((c >> (2 * j)) & 3u) ? (1u << j) : 0u;
    const int cnt = __popc(nz);
    uint32_t b = 0;
    if (cnt > 2) {
      ++nbad;
    } else {
      uint32_t p0, p1;
      if (cnt == 2) {
        p0 = __ffs(nz) - 1;
        p1 = 31 - __clz(nz);
      } else if (cnt == 1) {
        const uint32_t a = __ffs(nz) - 1;
        p0 = 0;
        p1 = a == 0 ? 1u : a;
      } else {
        p0 = 0;
        p1 = 1;
      }
      auto digit = [](uint32_t code) { return code == 1u ? 1u : code == 3u ? 2u : 0u; };
      const uint32_t rank = p0 * (15u - p0) / 2u + (p1 - p0 - 1u);
      b = 9u * rank + 3u * digit((c >> (2 * p0)) & 3u) + digit((c >> (2 * p1)) & 3u);
    }
    plane[i] = (uint8_t)b;
  }
  if (bad) {
    // one atomic per wave, only when a group was refused
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) nbad += __shfl_xor(nbad, off, 64);
    if ((threadIdx.x & 63) == 0 && nbad) atomicAdd(bad, nbad);
  }
}

template <int OUT, int W, int NTT, bool PAIRS, int XS>
hipError_t launch_k(const DecPlan& p, const void* x, const float* absmax, int64_t T, int64_t d_in, int grid,
                    size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((k_decode<OUT, W, NTT, PAIRS, XS>), dim3(grid), dim3(64 * W), lds, s, x, absmax, p, (int)T,
                     (int)d_in);
  return hipGetLastError();
}

template <int OUT, int W, int NTT, bool PAIRS>
hipError_t launch_xs(const DecPlan& p, int xs, const void* x, const float* absmax, int64_t T, int64_t d_in, int grid,
                     size_t lds, hipStream_t s) {
  if (xs == 2) {
    if constexpr (NTT == 1) return launch_k<OUT, W, NTT, PAIRS, 2>(p, x, absmax, T, d_in, grid, lds, s);
    return hipErrorInvalidValue;
  }
  if (xs == 1) return launch_k<OUT, W, NTT, PAIRS, 1>(p, x, absmax, T, d_in, grid, lds, s);
  return launch_k<OUT, W, NTT, PAIRS, 0>(p, x, absmax, T, d_in, grid, lds, s);
}

template <int OUT, int W, bool PAIRS>
hipError_t launch_ntt(const DecPlan& p, int xs, int ntt, const void* x, const float* absmax, int64_t T, int64_t d_in,
                      int grid, size_t lds, hipStream_t s) {
  // one 16-token tile: more than 16 tokens take the row-tile kernel of the forward
  if (ntt != 1) return hipErrorInvalidValue;
  return launch_xs<OUT, W, 1, PAIRS>(p, xs, x, absmax, T, d_in, grid, lds, s);
}

template <int OUT, bool PAIRS>
hipError_t launch_w(const DecPlan& p, int W, int xs, int ntt, const void* x, const float* absmax, int64_t T,
                    int64_t d_in, int grid, size_t lds, hipStream_t s) {
  if (W == 4) return launch_ntt<OUT, 4, PAIRS>(p, xs, ntt, x, absmax, T, d_in, grid, lds, s);
  return launch_ntt<OUT, 8, PAIRS>(p, xs, ntt, x, absmax, T, d_in, grid, lds, s);
}

constexpr int kLdsMax = 64 * 1024;  // dynamic LDS of one block

}  // namespace

bool decode_plane_supported(int format, int64_t T, int64_t d_in) {
  const int64_t kc = format == SBL_PLANE_PAIRS ? 128 : 64;
  return T >= 0 && T <= 64 && d_in % kc == 0 && d_in >= kc && (int64_t)T * d_in <= kMaxRsrcBytes;
}

static bool fused_fits(bool pairs, int64_t T, int64_t d_in) {
  // x fits the registers of an 8-wave block (kFuseRegs chunks per thread), and the
  // LDS tile with the largest partial-sum area (8 waves)
  return T >= 1 && T <= 16 && d_in % (pairs ? 128 : 64) == 0 && T * (d_in / 8) <= 64 * 8 * kFuseRegs &&
         dec_lds((int)T, (int)d_in, 8, 1, pairs, true).total <= kLdsMax;
}

bool decode_fused_supported(int64_t T, int64_t d_in) { return fused_fits(false, T, d_in); }
bool decode_fused_plane_supported(int format, int64_t T, int64_t d_in) {
  return fused_fits(format == SBL_PLANE_PAIRS, T, d_in);
}

hipError_t launch_decode_plane(int format, int count, const DecodeItem* items, bool fused, const void* x,
                               const float* absmax, int64_t T, int64_t d_in, int y_dtype, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (count < 1 || count > kDecodeMultiMax || !decode_plane_supported(format, T, d_in)) return hipErrorInvalidValue;
  const bool pairs = format == SBL_PLANE_PAIRS;
  if (fused && !fused_fits(pairs, T, d_in)) return hipErrorInvalidValue;
  if (!fused && T > 16)  // every block re-reads x_q there: the kernel with row-tile pairs
    return launch_decode_codes_many(count, items, pairs, (const int8_t*)x, absmax, T, d_in, y_dtype, s);
  const int cus = device_cus();
  DecPlan p{};
  p.count = count;
  p.nchunk = (int)(d_in / (pairs ? 128 : 64));
  const int nquad = (p.nchunk + 3) / 4;
  int64_t rows16 = 0;
  for (int i = 0; i < count; ++i) rows16 += (items[i].d_out + kDecTile - 1) / kDecTile;
  // 8-row tiles (half of each instruction idle) only where 16-row tiles leave CUs idle and the
  // quantization of x is not repeated in every block
  p.rows = rows16 < cus && !fused ? kDecTile / 2 : kDecTile;
  int64_t nt = 0;
  for (int i = 0; i < count; ++i) {
    p.tile_begin[i] = (int)nt;
    p.d_out[i] = (int)items[i].d_out;
    p.plane[i] = (const uint8_t*)items[i].codes;
    p.gamma[i] = items[i].gamma;
    p.y[i] = items[i].y;
    nt += (items[i].d_out + p.rows - 1) / p.rows;
    if (nt > 0x3FFFFFFF) return hipErrorInvalidValue;
  }
  p.tile_begin[count] = (int)nt;
  // waves per tile: enough to keep at most 8 chunk loads per lane, and to give
  // the grid about 4 waves per CU when the tiles alone do not
  int wpt = 1;
  while (wpt < 8 && ((nquad + wpt - 1) / wpt > kQ || (nt * wpt < 4LL * cus && (nquad + wpt - 1) / wpt > 1))) wpt *= 2;
  int W = std::max(4, wpt);
  if (fused) {  // the block's threads hold x in registers, kFuseRegs 16-byte chunks each, and
                // more than 4 each are spread over 8 waves (the quantization runs before any product)
    while (W < 8 && (int64_t)64 * W * 4 < T * (d_in / 8)) W *= 2;
    if ((int64_t)64 * W * kFuseRegs < T * (d_in / 8)) return hipErrorInvalidValue;
  }
  p.wpt = wpt;
  p.per = (nquad + wpt - 1) / wpt;
  const int tpg = W / wpt;
  p.groups = (int)((nt + tpg - 1) / tpg);
  const int ntt = 1;  // T <= 16 from here on (fused: checked above; otherwise the kernel above took T > 16)
  int xs = fused ? 2 : 1;  // x_q staged in LDS when the tile fits, else read from global memory
  DecLds L = dec_lds((int)T, (int)d_in, W, ntt, pairs, true);
  if (!fused && L.total > kLdsMax) {
    xs = 0;
    L = dec_lds((int)T, (int)d_in, W, ntt, pairs, false);
  }
  if (L.total > kLdsMax) return hipErrorInvalidValue;
  // resident blocks: LDS and about 16 waves per CU
  const int per_cu = std::max(1, std::min(kLdsMax / std::max(L.total, 1), 16 / W));  // about 16 waves per CU
  const int grid = (int)std::min<int64_t>(p.groups, (int64_t)cus * per_cu);
  const size_t lds = (size_t)L.total;
  if (pairs) {
    switch (y_dtype) {
      case SBL_F32: return launch_w<SBL_F32, true>(p, W, xs, ntt, x, absmax, T, d_in, grid, lds, s);
      case SBL_BF16: return launch_w<SBL_BF16, true>(p, W, xs, ntt, x, absmax, T, d_in, grid, lds, s);
      default: return launch_w<SBL_I32, true>(p, W, xs, ntt, x, absmax, T, d_in, grid, lds, s);
    }
  }
  switch (y_dtype) {
    case SBL_F32: return launch_w<SBL_F32, false>(p, W, xs, ntt, x, absmax, T, d_in, grid, lds, s);
    case SBL_BF16: return launch_w<SBL_BF16, false>(p, W, xs, ntt, x, absmax, T, d_in, grid, lds, s);
    default: return launch_w<SBL_I32, false>(p, W, xs, ntt, x, absmax, T, d_in, grid, lds, s);
  }
}

hipError_t launch_pack_pairs(const uint16_t* codes, int64_t d_out, int64_t d_in, uint8_t* plane,
                             unsigned long long* bad, hipStream_t s) {
  const int64_t n = d_out * (d_in / 8);
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 65536);
  hipLaunchKernelGGL(k_pack_pairs, dim3((unsigned)blocks), dim3(256), 0, s, codes, n, plane, bad);
  return hipGetLastError();
}

}  // namespace sbl
