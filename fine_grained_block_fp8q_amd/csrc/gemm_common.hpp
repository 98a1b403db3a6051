// Pieces shared by the block-scaled FP8 GEMM kernels (gfx950): LDS row
// swizzle, explicit waits, buffer resources, MFMA operand fragments from LDS,
// tile arguments and the XCD-aware tile order.
#pragma once

#include "fp8q_device.hpp"

namespace fp8q {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ lds_ptr_t to_lds(uint8_t* p) { return (lds_ptr_t)(p); }

// Physical 16-byte column of logical column c in LDS row r.  A fragment read
// has 16 lanes on 16 consecutive 128-byte rows at one logical column.  With
// f(r) = (r/2 mod 8) ^ 4*(r&1), the 8 even rows and the 8 odd rows each take
// all 8 columns, so the 16 lanes hit 16 distinct 16-byte slots of a 256-byte
// bank window, and each 8-row half also takes 8 distinct columns: the
// ds_read_b128 is bank-conflict free with 32 or 64 four-byte banks.  XOR with
// a per-row constant is an involution, so the same map locates and fetches.
__device__ __forceinline__ int swz(int r, int c) { return c ^ (((r >> 1) & 7) ^ ((r & 1) << 2)); }

// s_waitcnt vmcnt(N) with expcnt/lgkmcnt left at their maxima (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that orders LDS accesses but does not drain global loads
// still in flight (those are waited for explicitly with vmcnt).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

struct TileArgs {
  const uint8_t* A;     // rows of A (absolute row index)
  const float* SA;      // SA[g * sa_ld + row]
  const uint8_t* W;     // [w_rows][K]
  const float* SW;      // [w_rows/128][K/128]
  int64_t a_row0;       // first A row of the tile
  int64_t a_rows;       // exclusive end of the valid A rows
  int64_t w_row0;       // first W row (= output column) of the tile
  int64_t w_rows;       // N
  int64_t K;
  int64_t sa_ld;        // leading dimension of SA (total rows)
  int64_t sw_ld;        // row-scaled weight operand: leading dimension of SW = [K/128][sw_ld]
  void* C;              // output base
  int64_t ldc;          // N
  int out_bf16;
};

// Buffer resource over [base, base + bytes) for raw loads (gfx9 word 3:
// 32-bit untyped data); offsets past `bytes` read as zero instead of faulting.
constexpr int kRawRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes < 0xFFFFFFFFll ? (uint32_t)bytes : 0xFFFFFFFFu;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n,
                                           kRawRsrcWord3);
}

// MFMA operand fragment: LDS row r, 16-byte pieces q and q+4 of its 128-byte
// K chunk.  A and B fragments use the same (q, byte) -> K mapping, so every
// product pairs matching K indices, and each 8-byte group the matrix core
// sums together is still 8 consecutive K.  Pieces (q, q+4) rather than
// (2q, 2q+1): with the row swizzle swz, the 64 lanes of each read then
// spread over all LDS banks in every lane group the LDS serves together
// (measured: 1.55x the read throughput of the (2q, 2q+1) assignment).
__device__ __forceinline__ v8i load_frag(const uint8_t* base, int r, int q) {
  const v4i lo = *reinterpret_cast<const v4i*>(base + r * 128 + swz(r, q) * 16);
  const v4i hi = *reinterpret_cast<const v4i*>(base + r * 128 + swz(r, q + 4) * 16);
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Workgroup id -> output tile.  Workgroups are dispatched round-robin over
// the 8 XCDs (id mod 8), each with its own L2.  Give each XCD a contiguous
// run of tile ids, and walk tiles in groups of kGroupM tile rows (tile row
// fastest), so an XCD's tiles form a compact kGroupM x (run / kGroupM) block
// that shares A row bands and W column bands in that XCD's L2.
constexpr int kXcds = 8;
constexpr int kGroupM = 4;

__device__ __forceinline__ void xcd_tile(int bid, int nblocks, int tiles_n, int& tm, int& tn) {
  int id = bid;
  if (nblocks % kXcds == 0) id = (bid % kXcds) * (nblocks / kXcds) + bid / kXcds;
  const int tiles_m = nblocks / tiles_n;
  const int per_group = kGroupM * tiles_n;
  const int grp = id / per_group;
  const int first_m = grp * kGroupM;
  const int gm = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
  const int in = id - grp * per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}

}  // namespace fp8q
