// Shared pieces of the matrix-core kernels (forward int8, backward bf16).
//
// Every kernel computes one BM x BN output tile per block of 256 threads
// (4 waves in a 2 x 2 grid, 128 x 64 per wave, 32 x 32 MFMA tiles).  Both
// operands live in LDS as K-contiguous rows of 64 bytes (32 bf16 or 64 int8
// values per K step), 4 chunks of 16 bytes per row, swizzled (see swz) so
// that fragment reads and staging stores are free of bank conflicts.  A fragment is
// one ds_read_b128: lane l reads row (base + l % 32), chunk (2 ks + l / 32),
// which is the MFMA operand layout (row = l % 32, k = 8 or 16 per l / 32).
// 128 accumulator registers per wave keep two blocks resident per CU, so one
// block's loads, barriers and epilogue overlap the other's matrix work.
#pragma once

#include "sbl_internal.h"

namespace sbl {
namespace gemm {

constexpr int kThreads = 256;
constexpr int kBM = 256;      // block rows (M)
constexpr int kBN = 128;      // block cols (N)
constexpr int kWM = 128;      // wave rows
constexpr int kWN = 64;       // wave cols
constexpr int kMI = kWM / 32; // MFMA tiles per wave along M
constexpr int kNJ = kWN / 32; // MFMA tiles per wave along N
constexpr int kRow = 64;      // bytes per LDS row (one K step)


// LDS address of chunk c (16 bytes) of K-row `row`.  LDS reads are served in
// groups of 16 lanes over 64 banks of 4 bytes (256 bytes per cycle); a 64-byte
// row fills a quarter of the banks, so 16 consecutive rows reading the same
// chunk cover all 64 banks once when chunk c of row r is stored at position
// c ^ ((r >> 2) & 3).  The staging stores (16-byte rows copies, and 8-byte
// transposed stores whose 32 lanes cover all 8 k-slots of 4 rows) are also
// conflict-free under this layout.
__device__ __forceinline__ int swz(int row, int c) { return row * kRow + 16 * (c ^ ((row >> 2) & 3)); }

__device__ __forceinline__ v4i frag(const char* base, int row0, int ks, int lane) {
  return *(const v4i*)(base + swz(row0 + (lane & 31), 2 * ks + (lane >> 5)));
}

// Wide K steps (direct-load kernels): LDS rows of kRowK = 128 bytes, 8 chunks.
// A fragment read is 16 lanes on 16 consecutive rows, same chunk: the 8 even
// rows then sit in banks 0-31 and the 8 odd rows in banks 32-63, and
// c ^ ((row / 2) % 8) gives each of the 8 a different 16-byte bank group, so
// the read is conflict-free.  Direct loads fill whole 1 KB runs (8 rows).
constexpr int kRowK = 128;
__device__ __forceinline__ int swz8(int row, int c) { return row * kRowK + 16 * (c ^ ((row >> 1) & 7)); }

// Block index -> (m tile, n tile).  Blocks are dispatched round-robin over
// the 8 XCDs (b % 8); XCD x gets a contiguous range of tiles in row-major
// order (n fastest), so the tiles resident on one XCD share A rows in its L2.
__device__ __forceinline__ void xcd_tile(int b, int gm, int gn, int& mt, int& nt) {
  const int nb = gm * gn;
  int tile = b;
  if (nb >= 8) {
    const int x = b & 7, local = b >> 3;
    const int q = nb >> 3, r = nb & 7;
    tile = x * q + min(x, r) + local;
  }
  mt = tile / gn;
  nt = tile - mt * gn;
}

// Same split over the XCDs, but each XCD walks its range in groups of GM tile
// rows, column by column inside a group: the blocks resident on an XCD at one
// time then cover about a GM x (resident / GM) patch of the output, so both
// operands are shared in its L2 instead of one of them streaming through.
__device__ __forceinline__ void grouped_tile(int tile, int gm, int gn, int GM, int& mt, int& nt) {
  const int g = tile / (GM * gn);
  const int rem = tile - g * GM * gn;
  const int rows = min(GM, gm - g * GM);
  mt = g * GM + rem % rows;
  nt = rem / rows;
}
__device__ __forceinline__ void xcd_tile_grouped(int b, int gm, int gn, int GM, int& mt, int& nt) {
  const int nb = gm * gn;
  int tile = b;
  if (nb >= 8) {
    const int x = b & 7, local = b >> 3;
    const int q = nb >> 3, r = nb & 7;
    tile = x * q + min(x, r) + local;
  }
  grouped_tile(tile, gm, gn, GM, mt, nt);
}

// Split-K grids (S K ranges of T tiles, block L = x + T y in launch order):
// with one block per CU an XCD holds 32 blocks at a time, so the blocks are
// dealt in rounds of 256, and in each full round XCD x takes 32 consecutive
// work items.  Work items run over chunks of 32 consecutive tiles of the
// grouped order, each chunk once per K range (chunk-major), so that a full
// round gives every XCD one chunk (a 4 x 8 patch of 256 x 256 tiles) at one K
// range: its operand rows are shared by all 32 resident blocks.  The last,
// partial round is dealt evenly.  Returns the K range s and the tile index t
// in grouped order; every (s, t) is taken by exactly one block.
__device__ __forceinline__ void xcd_split_order(int L, int T, int S, int& s, int& t) {
  const int total = T * S;
  const int x = L & 7, local = L >> 3;
  const int base = 256 * (local >> 5), j = local & 31;
  const int R = min(256, total - base);
  const int item = R == 256 ? base + 32 * x + j : base + x * (R >> 3) + min(x, R & 7) + j;
  const int c = item / (32 * S), rem = item - c * 32 * S;
  const int cs = min(32, T - 32 * c);
  s = rem / cs;
  t = 32 * c + (rem - s * cs);
}

// Buffer resource for raw (unformatted) loads of `bytes` bytes at `base`.
// Accesses at offsets at or beyond `bytes` return zero, which is how tile rows
// past the end of a matrix are zero-filled without per-lane selects.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Lane offset that is always out of range (reads return zero): resources are
// never larger than kMaxRsrcBytes, and valid lane offsets stay below it.
constexpr uint32_t kOOB = 0x80000000u;
constexpr int64_t kMaxRsrcBytes = 0x7FFFFFF0LL;

// Clamp a byte count to [0, kMaxRsrcBytes].
__device__ __forceinline__ uint32_t clamp_bytes(int64_t b) {
  return b <= 0 ? 0u : (b >= kMaxRsrcBytes ? (uint32_t)kMaxRsrcBytes : (uint32_t)b);
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// Direct-to-LDS loads.  One buffer_load_dwordx4 ... lds per wave moves 64
// lanes x 16 bytes from arbitrary per-lane global offsets into 1 KB of LDS
// starting at a wave-uniform address (lane l lands at +16 l), without passing
// through registers.  Out-of-range offsets write zeros.  Completion is tracked
// by vmcnt, so a consumer waits on vmcnt and then meets the other waves at a
// barrier; nothing else orders these writes.
// ---------------------------------------------------------------------------
// soff (wave-uniform) is added to every lane's offset.  Callers size the
// resource so that in-range accesses stay below num_records with or without
// soff, and send out-of-range lanes to kOOB.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* lds_wave_base, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (SBL_LDS void*)lds_wave_base, 16, voff, soff, 0, 0);
}

// 16-byte store that is not kept in the caches (the `nt` store): for the large outputs (y, dX,
// the final dW) that nothing in the same call reads again; streaming them past the caches
// leaves L2 and the last-level cache to the operands.
__device__ __forceinline__ void store_nt16(void* p, uint4 v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), (u32x4*)p);
}

// 4-byte variant: lane l lands at +4 l (256 bytes per wave).
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, char* lds_wave_base, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (SBL_LDS void*)lds_wave_base, 4, voff, soff, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their maxima so they are not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Same, and also wait for all LDS reads of this wave (lgkmcnt = 0).
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every outstanding load, including the prefetches still in flight).
// The empty asm keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Row index (within the wave tile) of accumulator register r of lane l.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

}  // namespace gemm
}  // namespace sbl
