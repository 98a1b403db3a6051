// Ring-streaming probe (measurement support, not part of the method): the
// rate at which the grouped GEMM's operand pipeline alone can stream expert
// weights, for the ring depths and activation-row counts its tiles use.
// Built into libfp8q_probe.so; bench.py --ring-probe calls it.
//
// One workgroup of 8 waves per CU walks `tiles_per_wg` tiles.  Tile t reads
// 256 weight rows of its own (rows 256 t .. 256 t + 255 of W, wrapping) and
// RA activation rows shared by the `tiles_per_expert` consecutive tiles of
// one expert.  Tiles are handed out as the grouped GEMM hands out its own:
// each XCD (workgroup id mod 8) walks a contiguous run of tile ids, its
// workgroups taking consecutive ids in each round, so an expert's tiles run
// together on one XCD and share its activation rows in that XCD's L2.  Each
// tile moves 128 bytes of each row per K chunk into an LDS ring of S
// stages with the GEMM's 16-byte direct-to-LDS buffer loads (1 KiB per
// instruction: 8 rows of 128 bytes; A rows first, then W rows), instruction
// 8 j + w of a chunk going to wave w as in the GEMM's loader, so every wave
// issues its share of A rows, then of W rows.  Per chunk: issue chunk
// g + S - 1, wait until chunk g has landed, one barrier.  No MFMA and no LDS
// reads: what it measures is the streaming ceiling of the tile shape, S - 1
// chunks in flight per CU.
//
// The reads variant adds, after each chunk's barrier, RD 16-byte LDS reads
// per lane of every wave from the stage of the chunk that just landed (1 KiB
// per instruction, consumed into a running XOR), the GEMM main loop's
// fragment-read volume with no MFMA: it measures how LDS reads slow the
// direct-to-LDS stream beside them.  (The reads race with the loads refilling
// other stages and with the next refill of their own; their values are
// never used.)
//
// The split variant gives the activation rows a ring of SA stages and the
// weight rows one of SW >= SA stages: per chunk every wave issues its loads
// of activation chunk g + SA - 1, then of weight chunk g + SW - 1 (the same
// counts in every wave), waits until activation and weight chunk g have
// landed, and passes one barrier.  Loads complete in issue order, so the
// wait for activation chunk g leaves the weight loads issued after it in
// flight: the weights get SW - 1 chunks of lead, the activation rows (which
// come from L2) SA - 1.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.hpp"

namespace fp8q_ring_probe {

using fp8q::make_rsrc;
using fp8q::to_lds;
using fp8q::v4i;
using fp8q::wait_vmcnt;

constexpr int kWRows = 256;

template <int RA, int S>
struct Ring {
  static constexpr int A_INSTR = RA / 8;              // 1 KiB instructions per chunk
  static constexpr int W_INSTR = kWRows / 8;
  static constexpr int INSTR = A_INSTR + W_INSTR;
  static constexpr int PER_WAVE = (INSTR + 7) / 8;    // the last ones repeat A loads
  static constexpr int STAGE = INSTR * 1024;
  // at least 96 KiB, so that a second workgroup never shares the CU
  static constexpr int LDS = S * STAGE > 96 * 1024 ? S * STAGE : 96 * 1024;
  static_assert(RA % 8 == 0 && RA <= 256 && S >= 2, "shape");
  static_assert(LDS <= 160 * 1024, "LDS");
  static_assert(PER_WAVE * (S - 1) < 64, "vmcnt range");
};

// Chunk g's loads of this wave into its stage (chunks past the end re-fetch
// the last one).
template <int RA, int S>
__device__ __forceinline__ void issue_chunk(uint8_t* lds, __amdgpu_buffer_rsrc_t ra,
                                            __amdgpu_buffer_rsrc_t rw, const uint32_t* voff,
                                            const int* dst, const bool* is_a, int64_t g,
                                            int64_t G) {
  using R = Ring<RA, S>;
  const int64_t gc = g < G ? g : G - 1;
  uint8_t* stage = lds + (int)(g % S) * R::STAGE;
#pragma unroll
  for (int j = 0; j < R::PER_WAVE; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a[j] ? ra : rw, to_lds(stage + dst[j]), 16,
                                             voff[j], (int)(gc * 128), 0, 0);
}

// Tile id of round i of this workgroup: XCD blockIdx.x mod 8 owns tile ids
// [x R, x R + R), R = gridDim.x / 8 * tiles_per_wg, and its workgroups take
// consecutive ids in each round.
__device__ __forceinline__ int64_t tile_of(int i, int tiles_per_wg) {
  const int per_xcd = gridDim.x / 8;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  return ((int64_t)xcd * tiles_per_wg + i) * per_xcd + slot;
}

template <int RA, int S, int RD = 0>
__global__ __launch_bounds__(512) void ring_kernel(const uint8_t* __restrict__ W, int64_t w_rows,
                                                   const uint8_t* __restrict__ A, int64_t a_rows,
                                                   int64_t K, int tiles_per_wg,
                                                   int tiles_per_expert, int* __restrict__ sink) {
  using R = Ring<RA, S>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[R::LDS];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t G = K / 128;
  v4i seen = v4i{0, 0, 0, 0};
  for (int i = 0; i < tiles_per_wg; ++i) {
    const int64_t tile = tile_of(i, tiles_per_wg);
    const int64_t w0 = (tile * kWRows) % w_rows;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + w0 * K, kWRows * K);
    __amdgpu_buffer_rsrc_t ra = rw;
    if constexpr (RA > 0) {
      const int64_t a0 = ((tile / tiles_per_expert) * RA) % a_rows;
      ra = make_rsrc(A + a0 * K, RA * K);
    }
    uint32_t voff[R::PER_WAVE];
    int dst[R::PER_WAVE];
    bool is_a[R::PER_WAVE];
#pragma unroll
    for (int j = 0; j < R::PER_WAVE; ++j) {
      const int m = (j * 8 + wave) % R::INSTR;
      is_a[j] = m < R::A_INSTR;
      const int r = (is_a[j] ? m : m - R::A_INSTR) * 8 + (lane >> 3);
      voff[j] = (uint32_t)(r * K) + (uint32_t)((lane & 7) * 16);
      dst[j] = m * 1024;
    }
#pragma unroll
    for (int s = 0; s < S - 1; ++s) issue_chunk<RA, S>(lds, ra, rw, voff, dst, is_a, s, G);
    for (int64_t g = 0; g < G; ++g) {
      issue_chunk<RA, S>(lds, ra, rw, voff, dst, is_a, g + S - 1, G);
      wait_vmcnt<R::PER_WAVE * (S - 1)>();  // chunk g landed
      __builtin_amdgcn_s_barrier();
      if constexpr (RD > 0) {
        const uint8_t* stage = lds + (int)(g % S) * R::STAGE;
#pragma unroll
        for (int r = 0; r < RD; ++r) {
          const int off = ((wave * RD + r) * 1024 + lane * 16) % R::STAGE;
          seen ^= *reinterpret_cast<const v4i*>(stage + off);
        }
      }
    }
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
  }
  // Keeps the reads: a store the host never asks for (sink is null).
  if (sink != nullptr && (seen[0] ^ seen[1] ^ seen[2] ^ seen[3]) == 0x5a5a5a5a)
    sink[blockIdx.x] = threadIdx.x;
}

template <int RA, int S, int RD = 0>
hipError_t launch(const uint8_t* W, int64_t w_rows, const uint8_t* A, int64_t a_rows, int64_t K,
                  int blocks, int tiles_per_wg, int tiles_per_expert, hipStream_t stream) {
  ring_kernel<RA, S, RD><<<dim3(blocks), dim3(512), 0, stream>>>(
      W, w_rows, A, a_rows, K, tiles_per_wg, tiles_per_expert, nullptr);
  return hipGetLastError();
}

// Split rings: RA activation rows in SA stages, kWRows weight rows in SW.
template <int RA, int SA, int SW>
struct Split {
  static constexpr int A_PW = RA / 64;       // 1 KiB instructions per wave and chunk
  static constexpr int W_PW = kWRows / 64;
  static constexpr int A_STAGE = RA * 128;
  static constexpr int W_STAGE = kWRows * 128;
  static constexpr int BYTES = SA * A_STAGE + SW * W_STAGE;
  static constexpr int LDS = BYTES > 96 * 1024 ? BYTES : 96 * 1024;
  // Loads a wave has issued after the last one the wait for chunk g needs:
  // with SA < SW that is activation chunk g, issued SA - 1 iterations back
  // and followed in its iteration by that iteration's weight loads; with
  // SA == SW it is weight chunk g, at the end of its iteration.
  static constexpr int AFTER =
      SA < SW ? W_PW + (A_PW + W_PW) * (SA - 1) : (A_PW + W_PW) * (SA - 1);
  static_assert(RA % 64 == 0 && RA > 0 && RA <= 256 && SA >= 2 && SW >= SA, "shape");
  static_assert(LDS <= 160 * 1024, "LDS");
  static_assert(AFTER < 64, "vmcnt range");
};

template <int N>
__device__ __forceinline__ void issue_rows(uint8_t* stage, __amdgpu_buffer_rsrc_t r,
                                           const uint32_t* voff, int wave, int64_t g, int64_t G) {
  const int64_t gc = g < G ? g : G - 1;
#pragma unroll
  for (int j = 0; j < N; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, to_lds(stage + (wave * N + j) * 1024), 16,
                                             voff[j], (int)(gc * 128), 0, 0);
}

template <int RA, int SA, int SW>
__global__ __launch_bounds__(512) void split_ring_kernel(const uint8_t* __restrict__ W,
                                                         int64_t w_rows,
                                                         const uint8_t* __restrict__ A,
                                                         int64_t a_rows, int64_t K,
                                                         int tiles_per_wg, int tiles_per_expert) {
  using R = Split<RA, SA, SW>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[R::LDS];
  uint8_t* const lds_w = lds + SA * R::A_STAGE;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t G = K / 128;
  uint32_t va[R::A_PW], vw[R::W_PW];
#pragma unroll
  for (int j = 0; j < R::A_PW; ++j)
    va[j] = (uint32_t)(((wave * R::A_PW + j) * 8 + (lane >> 3)) * K) + (uint32_t)((lane & 7) * 16);
#pragma unroll
  for (int j = 0; j < R::W_PW; ++j)
    vw[j] = (uint32_t)(((wave * R::W_PW + j) * 8 + (lane >> 3)) * K) + (uint32_t)((lane & 7) * 16);
  for (int i = 0; i < tiles_per_wg; ++i) {
    const int64_t tile = tile_of(i, tiles_per_wg);
    const int64_t w0 = (tile * kWRows) % w_rows;
    const int64_t a0 = ((tile / tiles_per_expert) * RA) % a_rows;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + w0 * K, kWRows * K);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + a0 * K, RA * K);
    // the iterations before chunk 0, in steady-state order
#pragma unroll
    for (int s = 1 - SW; s < 0; ++s) {
      if (s + SA - 1 >= 0)
        issue_rows<R::A_PW>(lds + ((s + SA - 1) % SA) * R::A_STAGE, ra, va, wave, s + SA - 1, G);
      issue_rows<R::W_PW>(lds_w + ((s + SW - 1) % SW) * R::W_STAGE, rw, vw, wave, s + SW - 1, G);
    }
    for (int64_t g = 0; g < G; ++g) {
      issue_rows<R::A_PW>(lds + (int)((g + SA - 1) % SA) * R::A_STAGE, ra, va, wave, g + SA - 1, G);
      issue_rows<R::W_PW>(lds_w + (int)((g + SW - 1) % SW) * R::W_STAGE, rw, vw, wave, g + SW - 1,
                          G);
      wait_vmcnt<R::AFTER>();  // activation and weight chunk g landed
      __builtin_amdgcn_s_barrier();
    }
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
  }
}

template <int RA, int SA, int SW>
hipError_t launch_split(const uint8_t* W, int64_t w_rows, const uint8_t* A, int64_t a_rows,
                        int64_t K, int blocks, int tiles_per_wg, int tiles_per_expert,
                        hipStream_t stream) {
  split_ring_kernel<RA, SA, SW><<<dim3(blocks), dim3(512), 0, stream>>>(
      W, w_rows, A, a_rows, K, tiles_per_wg, tiles_per_expert);
  return hipGetLastError();
}

}  // namespace fp8q_ring_probe

using fp8q_ring_probe::kWRows;
using fp8q_ring_probe::launch;
using fp8q_ring_probe::launch_split;

extern "C" {

// Streams tiles through the ring described above on one workgroup per CU of
// the current device.  W: device [w_rows][K] bytes, w_rows a multiple of 256;
// A: device [a_rows][K] bytes, a_rows a multiple of ra (A unused when ra is
// 0); K a multiple of 128 with 256 * K < 2^31; (ra, stages) one of (0, 2),
// (0, 3), (0, 4), (64, 3), (128, 3), (160, 3), (192, 2), (256, 2): the
// grouped GEMM's row buckets with their ring depths, and weights alone.  Returns 0, -1 for
// unsupported arguments, or the HIP error code.  Asynchronous on `stream`.
int fp8q_probe_ring(const void* W, int64_t w_rows, const void* A, int64_t a_rows, int64_t K,
                    int ra, int stages, int tiles_per_wg, int tiles_per_expert,
                    hipStream_t stream) {
  if (!W || w_rows <= 0 || w_rows % kWRows || K <= 0 || K % 128 || kWRows * K >= (1ll << 31) ||
      tiles_per_wg <= 0 || tiles_per_expert <= 0 ||
      (ra > 0 && (!A || a_rows < ra || a_rows % ra || (int64_t)ra * K >= (1ll << 31))))
    return -1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return (int)hipGetLastError();
  if (cus % 8) return -1;   // the tile hand-out assumes 8 XCDs of equal size
  const uint8_t* w = static_cast<const uint8_t*>(W);
  const uint8_t* a = static_cast<const uint8_t*>(A);
  hipError_t e;
  if (ra == 0 && stages == 2) e = launch<0, 2>(w, w_rows, a, a_rows, K, cus, tiles_per_wg, tiles_per_expert, stream);
  else if (ra == 0 && stages == 3) e = launch<0, 3>(w, w_rows, a, a_rows, K, cus, tiles_per_wg, tiles_per_expert, stream);
  else if (ra == 0 && stages == 4) e = launch<0, 4>(w, w_rows, a, a_rows, K, cus, tiles_per_wg, tiles_per_expert, stream);
  else if (ra == 64 && stages == 3) e = launch<64, 3>(w, w_rows, a, a_rows, K, cus, tiles_per_wg, tiles_per_expert, stream);
  else if (ra == 128 && stages == 3) e = launch<128, 3>(w, w_rows, a, a_rows, K, cus, tiles_per_wg, tiles_per_expert, stream);
  else if (ra == 160 && stages == 3) e = launch<160, 3>(w, w_rows, a, a_rows, K, cus, tiles_per_wg, tiles_per_expert, stream);
  else if (ra == 192 && stages == 2) e = launch<192, 2>(w, w_rows, a, a_rows, K, cus, tiles_per_wg, tiles_per_expert, stream);
  else if (ra == 256 && stages == 2) e = launch<256, 2>(w, w_rows, a, a_rows, K, cus, tiles_per_wg, tiles_per_expert, stream);
  else return -1;
  return (int)e;
}

// The reads variant: the kernel's ring for (ra, stages) as in fp8q_probe_ring,
// plus `reads` 16-byte LDS reads per lane of every wave per chunk; (ra,
// stages, reads) one of (0, 2, 24), (128, 3, 12), (128, 3, 24), (256, 2, 24)
// (24 reads per wave are the 256 x 256 tile's fragment reads per chunk; the
// 128-row tile's 4 live waves make 12 per wave on average).  Arguments
// otherwise as for fp8q_probe_ring; returns 0, -1 for unsupported arguments,
// or the HIP error code.  Asynchronous on `stream`.
int fp8q_probe_ring_reads(const void* W, int64_t w_rows, const void* A, int64_t a_rows,
                          int64_t K, int ra, int stages, int reads, int tiles_per_wg,
                          int tiles_per_expert, hipStream_t stream) {
  using Launch = hipError_t (*)(const uint8_t*, int64_t, const uint8_t*, int64_t, int64_t, int,
                                int, int, hipStream_t);
  Launch f = nullptr;
  if (ra == 0 && stages == 2 && reads == 24) f = launch<0, 2, 24>;
  else if (ra == 128 && stages == 3 && reads == 12) f = launch<128, 3, 12>;
  else if (ra == 128 && stages == 3 && reads == 24) f = launch<128, 3, 24>;
  else if (ra == 256 && stages == 2 && reads == 24) f = launch<256, 2, 24>;
  if (!f || !W || w_rows <= 0 || w_rows % kWRows || K <= 0 || K % 128 ||
      kWRows * K >= (1ll << 31) || tiles_per_wg <= 0 || tiles_per_expert <= 0 ||
      (ra > 0 && (!A || a_rows < ra || a_rows % ra || (int64_t)ra * K >= (1ll << 31))))
    return -1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return (int)hipGetLastError();
  if (cus % 8) return -1;   // the tile hand-out assumes 8 XCDs of equal size
  return (int)f(static_cast<const uint8_t*>(W), w_rows, static_cast<const uint8_t*>(A), a_rows,
                K, cus, tiles_per_wg, tiles_per_expert, stream);
}

// The split-ring variant: ra activation rows in a ring of a_stages stages,
// 256 weight rows in one of w_stages.  Arguments as for fp8q_probe_ring, with
// ra > 0; (ra, a_stages, w_stages) one of (64, 2, 4), (128, 2, 3), (128, 2, 4),
// (128, 3, 3), (192, 2, 2), (192, 2, 3), (256, 2, 2), (256, 2, 3).  Returns 0,
// -1 for unsupported arguments, or the HIP error code.  Asynchronous on `stream`.
int fp8q_probe_ring_split(const void* W, int64_t w_rows, const void* A, int64_t a_rows,
                          int64_t K, int ra, int a_stages, int w_stages, int tiles_per_wg,
                          int tiles_per_expert, hipStream_t stream) {
  using Launch = hipError_t (*)(const uint8_t*, int64_t, const uint8_t*, int64_t, int64_t, int,
                                int, int, hipStream_t);
  Launch f = nullptr;
  const int sa = a_stages, sw = w_stages;
  if (ra == 64 && sa == 2 && sw == 4) f = launch_split<64, 2, 4>;
  else if (ra == 128 && sa == 2 && sw == 3) f = launch_split<128, 2, 3>;
  else if (ra == 128 && sa == 2 && sw == 4) f = launch_split<128, 2, 4>;
  else if (ra == 128 && sa == 3 && sw == 3) f = launch_split<128, 3, 3>;
  else if (ra == 192 && sa == 2 && sw == 2) f = launch_split<192, 2, 2>;
  else if (ra == 192 && sa == 2 && sw == 3) f = launch_split<192, 2, 3>;
  else if (ra == 256 && sa == 2 && sw == 2) f = launch_split<256, 2, 2>;
  else if (ra == 256 && sa == 2 && sw == 3) f = launch_split<256, 2, 3>;
  if (!f || !W || !A || w_rows <= 0 || w_rows % kWRows || K <= 0 || K % 128 ||
      kWRows * K >= (1ll << 31) || tiles_per_wg <= 0 || tiles_per_expert <= 0 ||
      a_rows < ra || a_rows % ra || (int64_t)ra * K >= (1ll << 31))
    return -1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return (int)hipGetLastError();
  if (cus % 8) return -1;   // the tile hand-out assumes 8 XCDs of equal size
  return (int)f(static_cast<const uint8_t*>(W), w_rows, static_cast<const uint8_t*>(A), a_rows, K,
                cus, tiles_per_wg, tiles_per_expert, stream);
}

}  // extern "C"
