// Block-scaled FP8 GEMM with FP32 promotion every 128 K, dense and grouped.
//
// Method: why-be.co.kr as_center post 57820, promotion passage (at the end of
// every N_C interval the partial result leaves the matrix unit, is multiplied
// by the scaling factors and added into FP32 registers on the general ALUs);
// pkd.ac.th webboard post 78017, increased-precision accumulation passage
// (N_C = 128); the-good.kr free board post 2169793 (per-group scaling along K,
// dequantized on the general ALUs).
//
// MI355X mapping.  One v_mfma_f32_16x16x128_f8f6f4 consumes exactly one
// 128-wide K chunk of a 16x16 output block, so each chunk's partial P_g is a
// single MFMA started from zero; the promotion acc = fma(P_g, s_a*s_w, acc) is
// four VALU FMAs per MFMA.  Two waves share each SIMD, so one wave's FMAs
// overlap the other wave's MFMAs (the role the pages give to two alternating
// warpgroups on Hopper).
//
// Workgroup tile BM x BN with 8 waves (4 along M x 2 along N), wave tile
// 64 x 128: each wave's 128 columns are one weight block, so s_w is a single
// wave-uniform scalar per chunk.  Operands move HBM/L2 -> LDS with 16-byte
// direct-to-LDS loads (no VGPR staging), double-buffered over K chunks with
// one barrier per chunk.  LDS rows are 128 bytes (one chunk of K) with the
// 16-byte column index XOR-swizzled by (row & 7) so MFMA fragment reads are
// bank-conflict free.

#include "fp8q_device.hpp"

namespace fp8q {

namespace gemm_cfg {
constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 128;                       // one promotion interval
constexpr int WAVES_M = 4;
constexpr int WAVES_N = 2;
constexpr int NWAVES = WAVES_M * WAVES_N;     // 8
constexpr int THREADS = NWAVES * 64;          // 512
constexpr int WM = BM / WAVES_M;              // 64
constexpr int WN = BN / WAVES_N;              // 128 = one weight block
constexpr int MB = WM / 16;                   // 4 MFMA row blocks per wave
constexpr int NB = WN / 16;                   // 8 MFMA column blocks per wave
constexpr int A_BYTES = BM * BK;              // 32 KiB
constexpr int B_BYTES = BN * BK;              // 32 KiB
constexpr int SA_BYTES = BM * 4;              // 1 KiB
constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES;
constexpr int STAGES = 2;
constexpr int LDS_BYTES = STAGE * STAGES;     // 130 KiB of the 160 KiB
static_assert(WN == 128, "a wave's columns must be one 128-wide weight block");
}  // namespace gemm_cfg

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ lds_ptr_t to_lds(uint8_t* p) {
  return (lds_ptr_t)(p);
}

// Physical 16-byte column of logical column c in LDS row r.
__device__ __forceinline__ int swz(int r, int c) { return c ^ (r & 7); }

// Issue the direct-to-LDS loads of one K chunk (A tile, W tile, A scales).
// Each load instruction moves 64 lanes x 16 B = 8 LDS rows of 128 B; lane i
// of the instruction lands at LDS byte 16*i, i.e. row i/8, physical column
// i%8, and therefore fetches logical column swz(row, i%8) from global memory.
// Rows past the matrix edge are clamped to the last row (their results are
// never stored).
__device__ __forceinline__ void issue_chunk(uint8_t* stage, const uint8_t* __restrict__ A,
                                            const float* __restrict__ SA,
                                            const uint8_t* __restrict__ W, int64_t a_row0,
                                            int64_t a_rows, int64_t w_row0, int64_t w_rows,
                                            int64_t K, int64_t sa_ld, int64_t g, int wave,
                                            int lane) {
  using namespace gemm_cfg;
  const int sub_r = lane >> 3;
  const int pc = lane & 7;
  constexpr int A_INSTR = A_BYTES / 1024;  // 32
  constexpr int B_INSTR = B_BYTES / 1024;  // 32
#pragma unroll
  for (int j = 0; j < A_INSTR / NWAVES; ++j) {
    const int blk = wave * (A_INSTR / NWAVES) + j;
    const int r = blk * 8 + sub_r;
    int64_t gr = a_row0 + r;
    gr = gr < a_rows ? gr : a_rows - 1;
    const uint8_t* src = A + gr * K + g * BK + swz(r, pc) * 16;
    __builtin_amdgcn_global_load_lds(src, to_lds(stage + blk * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < B_INSTR / NWAVES; ++j) {
    const int blk = wave * (B_INSTR / NWAVES) + j;
    const int r = blk * 8 + sub_r;
    int64_t gr = w_row0 + r;
    gr = gr < w_rows ? gr : w_rows - 1;
    const uint8_t* src = W + gr * K + g * BK + swz(r, pc) * 16;
    __builtin_amdgcn_global_load_lds(src, to_lds(stage + A_BYTES + blk * 1024), 16, 0, 0);
  }
  // A scales of this chunk: BM floats, 64 per dword-load instruction.
  if (wave < BM / 64) {
    const int r = wave * 64 + lane;
    int64_t gr = a_row0 + r;
    gr = gr < a_rows ? gr : a_rows - 1;
    const float* src = SA + g * sa_ld + gr;
    __builtin_amdgcn_global_load_lds(src, to_lds(stage + A_BYTES + B_BYTES + wave * 256), 4, 0,
                                     0);
  }
}

struct TileArgs {
  const uint8_t* A;     // [a_rows][K] rows of this problem
  const float* SA;      // SA[g * sa_ld + row]
  const uint8_t* W;     // [w_rows][K]
  const float* SW;      // [w_rows/128][K/128]
  int64_t a_row0;       // first A row of the tile
  int64_t a_rows;       // rows of A valid for this tile (exclusive end, absolute)
  int64_t w_row0;       // first W row (= output column) of the tile
  int64_t w_rows;       // N
  int64_t K;
  int64_t sa_ld;        // leading dimension of SA (M_total)
  void* C;              // output base
  int64_t ldc;          // N
  int out_bf16;
};

// Computes one BM x BN output tile.  All 512 lanes of the workgroup call it.
__device__ __forceinline__ void gemm_tile(const TileArgs& t, uint8_t* smem) {
  using namespace gemm_cfg;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave_m = wave / WAVES_N;
  const int wave_n = wave % WAVES_N;
  const int r16 = lane & 15;   // fragment row (A) / column (B) within a 16-block
  const int q = lane >> 4;     // which 32-byte slice of the 128-byte chunk
  const int64_t G = t.K / BK;
  const int64_t KB = G;

  // Output column block of this wave and its weight-scale row.
  int64_t wblk = (t.w_row0 + wave_n * WN) / 128;
  const int64_t last_wblk = t.w_rows / 128 - 1;
  wblk = wblk < last_wblk ? wblk : last_wblk;
  const float* sw_row = t.SW + wblk * KB;

  // Waves whose rows are all past the valid range skip the MFMA work.
  const bool wave_live = (t.a_row0 + wave_m * WM) < t.a_rows;

  v4f acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  issue_chunk(smem, t.A, t.SA, t.W, t.a_row0, t.a_rows, t.w_row0, t.w_rows, t.K, t.sa_ld, 0,
              wave, lane);

  for (int64_t g = 0; g < G; ++g) {
    uint8_t* cur = smem + (g & 1) * STAGE;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's chunk-g loads landed
    __syncthreads();                     // every wave's loads landed; stage g+1 free
    if (g + 1 < G)
      issue_chunk(smem + ((g + 1) & 1) * STAGE, t.A, t.SA, t.W, t.a_row0, t.a_rows, t.w_row0,
                  t.w_rows, t.K, t.sa_ld, g + 1, wave, lane);
    if (!wave_live) continue;

    const uint8_t* As = cur;
    const uint8_t* Bs = cur + A_BYTES;
    const float* SAs = reinterpret_cast<const float*>(cur + A_BYTES + B_BYTES);
    const float sw = sw_row[g];

    v8i a[MB];
    v4f mult[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int r = wave_m * WM + i * 16 + r16;
      const v4i lo = *reinterpret_cast<const v4i*>(As + r * BK + swz(r, 2 * q) * 16);
      const v4i hi = *reinterpret_cast<const v4i*>(As + r * BK + swz(r, 2 * q + 1) * 16);
      a[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const v4f sa = *reinterpret_cast<const v4f*>(SAs + wave_m * WM + i * 16 + 4 * q);
      mult[i] = sa * sw;
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int r = wave_n * WN + j * 16 + r16;
      const v4i lo = *reinterpret_cast<const v4i*>(Bs + r * BK + swz(r, 2 * q) * 16);
      const v4i hi = *reinterpret_cast<const v4i*>(Bs + r * BK + swz(r, 2 * q + 1) * 16);
      const v8i b = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            a[i], b, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
        acc[i][j][0] = __builtin_fmaf(p[0], mult[i][0], acc[i][j][0]);
        acc[i][j][1] = __builtin_fmaf(p[1], mult[i][1], acc[i][j][1]);
        acc[i][j][2] = __builtin_fmaf(p[2], mult[i][2], acc[i][j][2]);
        acc[i][j][3] = __builtin_fmaf(p[3], mult[i][3], acc[i][j][3]);
      }
    }
  }

  // Epilogue: lane holds rows 4q..4q+3, column r16 of every 16x16 block.
  if (!wave_live) return;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t row = t.a_row0 + wave_m * WM + i * 16 + 4 * q + v;
      if (row >= t.a_rows) continue;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int64_t col = t.w_row0 + wave_n * WN + j * 16 + r16;
        if (col >= t.w_rows) continue;
        if (t.out_bf16)
          reinterpret_cast<uint16_t*>(t.C)[row * t.ldc + col] =
              (uint16_t)f32_to_bf16_bits(acc[i][j][v]);
        else
          reinterpret_cast<float*>(t.C)[row * t.ldc + col] = acc[i][j][v];
      }
    }
  }
}

__global__ __launch_bounds__(gemm_cfg::THREADS) void gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ SA, const uint8_t* __restrict__ W,
    const float* __restrict__ SW, int64_t M, int64_t N, int64_t K, void* __restrict__ C,
    int out_bf16, int tiles_n) {
  using namespace gemm_cfg;
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
  const int tile = blockIdx.x;
  const int tm = tile / tiles_n;
  const int tn = tile % tiles_n;
  TileArgs t;
  t.A = A;
  t.SA = SA;
  t.W = W;
  t.SW = SW;
  t.a_row0 = (int64_t)tm * BM;
  t.a_rows = M;
  t.w_row0 = (int64_t)tn * BN;
  t.w_rows = N;
  t.K = K;
  t.sa_ld = M;
  t.C = C;
  t.ldc = N;
  t.out_bf16 = out_bf16;
  gemm_tile(t, smem);
}

// Grouped variant.  The grid over-provisions tiles; each workgroup maps its id
// to (expert, m-tile, n-tile) by a prefix sum of ceil(M_e / BM) over the device
// offsets, held in LDS.  Workgroups past the last tile exit.
constexpr int kMaxExpertsLds = 1024;

__global__ __launch_bounds__(gemm_cfg::THREADS) void grouped_gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ SA, int64_t M_total,
    const int32_t* __restrict__ off, int G, const uint8_t* __restrict__ W,
    const float* __restrict__ SW, int64_t N, int64_t K, void* __restrict__ C, int out_bf16,
    int tiles_n) {
  using namespace gemm_cfg;
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
  int* mt_prefix = reinterpret_cast<int*>(smem);  // [G + 1], reused before the mainloop

  // Prefix over experts of the number of BM-row tiles (serial chunks of
  // THREADS experts with a block scan each).
  const int tid = threadIdx.x;
  int running = 0;
  if (tid == 0) mt_prefix[0] = 0;
  for (int base = 0; base < G; base += THREADS) {
    const int e = base + tid;
    int cnt = 0;
    if (e < G) {
      const int rows = off[e + 1] - off[e];
      cnt = rows > 0 ? (rows + BM - 1) / BM : 0;
    }
    // inclusive scan across the workgroup through LDS (Hillis-Steele)
    int* scan = mt_prefix + kMaxExpertsLds + 1;
    scan[tid] = cnt;
    __syncthreads();
    for (int d = 1; d < THREADS; d <<= 1) {
      const int add = tid >= d ? scan[tid - d] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    if (e < G) mt_prefix[e + 1] = running + scan[tid];
    running += scan[THREADS - 1];
    __syncthreads();
  }
  const int total_mtiles = running;
  const int tile = blockIdx.x;
  const int mt_global = tile / tiles_n;
  const int tn = tile % tiles_n;
  if (mt_global >= total_mtiles) return;
  // binary search: expert e with prefix[e] <= mt_global < prefix[e+1]
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (mt_prefix[mid] <= mt_global) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int mt = mt_global - mt_prefix[e];
  const int64_t r0 = off[e];
  const int64_t r1 = off[e + 1];
  __syncthreads();  // mt_prefix is overwritten by the mainloop

  TileArgs t;
  t.A = A;
  t.SA = SA;
  t.W = W + (int64_t)e * N * K;
  t.SW = SW + (int64_t)e * (N / 128) * (K / 128);
  t.a_row0 = r0 + (int64_t)mt * BM;
  t.a_rows = r1;
  t.w_row0 = (int64_t)tn * BN;
  t.w_rows = N;
  t.K = K;
  t.sa_ld = M_total;
  t.C = C;
  t.ldc = N;
  t.out_bf16 = out_bf16;
  gemm_tile(t, smem);
}

hipError_t launch_gemm(const uint8_t* a_q, const float* a_s, const uint8_t* w_q,
                       const float* w_s, int64_t M, int64_t N, int64_t K, void* c, int out_bf16,
                       hipStream_t stream) {
  using namespace gemm_cfg;
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t tiles_m = (M + BM - 1) / BM;
  const int64_t tiles_n = (N + BN - 1) / BN;
  const int64_t tiles = tiles_m * tiles_n;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_kernel, dim3((unsigned)tiles), dim3(THREADS), 0, stream, a_q, a_s, w_q,
                     w_s, M, N, K, c, out_bf16, (int)tiles_n);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const uint8_t* a_q, const float* a_s, int64_t M_total,
                               const int32_t* off, int G, const uint8_t* w_q, const float* w_s,
                               int64_t N, int64_t K, void* c, int out_bf16,
                               hipStream_t stream) {
  using namespace gemm_cfg;
  if (M_total == 0 || N == 0) return hipSuccess;
  if (G > kMaxExpertsLds) return hipErrorInvalidValue;
  const int64_t tiles_n = (N + BN - 1) / BN;
  // sum_e ceil(M_e / BM) <= floor(M_total / BM) + G
  const int64_t max_mtiles = M_total / BM + G;
  const int64_t tiles = max_mtiles * tiles_n;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(grouped_gemm_kernel, dim3((unsigned)tiles), dim3(THREADS), 0, stream, a_q,
                     a_s, M_total, off, G, w_q, w_s, N, K, c, out_bf16, (int)tiles_n);
  return hipGetLastError();
}

}  // namespace fp8q
