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
// four VALU FMAs per MFMA.  Inside a wave the column blocks are software
// pipelined: the MFMAs of block j run on the matrix core while the VALU folds
// block j-1's partials into the accumulators (the role the pages give to two
// alternating warpgroups on Hopper).
//
// Each wave owns a 64 x 128 output tile: its 128 columns are one weight
// block, so s_w is one wave-uniform scalar per chunk, and its 64 row scales are
// one 256-byte LDS slot per chunk.  Operands move HBM/L2 -> LDS with 16-byte
// direct-to-LDS loads (no VGPR staging) through a ring of STAGES K chunks, one
// barrier per chunk.  LDS rows are 128 bytes (one K chunk) with the 16-byte
// column index XOR-swizzled per row so fragment reads are bank-conflict free.

#include "fp8q_device.hpp"

namespace fp8q {

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_, int ROWS_ = BM_>
struct GemmCfg {
  static constexpr int BM = BM_;
  static constexpr int BN = BN_;
  static constexpr int BK = 128;                    // one promotion interval
  static constexpr int WAVES_M = WAVES_M_;
  static constexpr int WAVES_N = WAVES_N_;
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = NWAVES * 64;
  static constexpr int WM = BM / WAVES_M;
  static constexpr int WN = BN / WAVES_N;
  static constexpr int MB = WM / 16;                // MFMA row blocks per wave
  static constexpr int NB = WN / 16;                // MFMA column blocks per wave
  static constexpr int ROWS = ROWS_;                // A rows staged per chunk (<= BM)
  static constexpr int A_BYTES = ROWS * BK;
  static constexpr int B_BYTES = BN * BK;
  static constexpr int SA_BYTES = NWAVES * 256;     // 64 row scales per wave
  static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES;
  static constexpr int STAGES = STAGES_;
  static constexpr int LDS_BYTES = STAGE * STAGES;
  static constexpr int A_BLK = A_BYTES / 1024;      // 1 KiB load instructions for A
  static constexpr int OP_BLK = A_BLK + B_BYTES / 1024;
  static constexpr int PER_WAVE = OP_BLK / NWAVES;  // operand loads per wave per chunk
  static constexpr int LOADS = PER_WAVE + 1;        // + the scale slot
  static_assert(WM == 64, "a wave's rows are 64 (one 256-byte scale slot)");
  static_assert(WN == 128, "a wave's columns must be one 128-wide weight block");
  static_assert(ROWS % 64 == 0 && ROWS <= BM, "staged rows cover whole waves");
  static_assert(OP_BLK % NWAVES == 0, "tile loads must split evenly over the waves");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(STAGES >= 2 && STAGES <= 6 && LOADS * (STAGES - 2) < 64, "vmcnt range");
};

// Dense configuration: 256 x 256 tiles, 8 waves (two per SIMD, so one wave's
// promotion FMAs overlap the other's MFMAs), 2 stages (130 KiB of LDS).
using DenseCfg = GemmCfg<256, 256, 4, 2, 2>;
// Grouped configurations: 256-row tiles cover an expert's tokens (decode
// batches hold at most 256) so each expert's weights stream once per n-tile.
// Only the tile's live rows (rounded up to 64) are staged, and the LDS this
// frees deepens the ring: 6 / 4 / 3 / 3 stages for 64 / 128 / 192 / 256 rows,
// i.e. up to 80 KiB of weights in flight per CU.
template <int ROWS, int S>
using GroupedCfg = GemmCfg<256, 128, 4, 1, S, ROWS>;

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

// Wait until at most `after` chunks' loads (issued after the one needed) are
// still outstanding for this wave (after <= MAXA <= 4).
template <int LOADS, int MAXA>
__device__ __forceinline__ void wait_chunk(int after) {
  if (MAXA >= 4 && after >= 4) wait_vmcnt<LOADS * 4>();
  else if (MAXA >= 3 && after >= 3) wait_vmcnt<LOADS * 3>();
  else if (MAXA >= 2 && after >= 2) wait_vmcnt<LOADS * 2>();
  else if (MAXA >= 1 && after >= 1) wait_vmcnt<LOADS>();
  else wait_vmcnt<0>();
}

// Issue the direct-to-LDS loads of one K chunk (A rows, W rows, row scales).
// The operand tiles are cut into 1 KiB load instructions (8 rows of 128 B):
// instructions 0 .. A_BLK-1 carry A rows, the rest W rows, and wave w issues
// instructions w*PER_WAVE .. w*PER_WAVE + PER_WAVE - 1.  Lane i of an
// instruction lands at LDS byte 16*i, i.e. row i/8, physical column i%8, and
// therefore fetches logical column swz(row, i%8) from global memory.  Rows past
// the valid range are clamped to the last valid row (their results are never
// stored).  Every wave issues exactly Cfg::LOADS instructions per chunk.
template <class Cfg>
__device__ __forceinline__ void issue_one(uint8_t* stage, const uint8_t* __restrict__ A,
                                          const uint8_t* __restrict__ W, int64_t a_row0,
                                          int64_t a_rows, int64_t w_row0, int64_t w_rows,
                                          int64_t K, int64_t g, int wave, int lane, int j) {
  const int sub_r = lane >> 3;
  const int pc = lane & 7;
  const int m = wave * Cfg::PER_WAVE + j;
  if (m < Cfg::A_BLK) {
    const int r = m * 8 + sub_r;
    int64_t gr = a_row0 + r;
    gr = gr < a_rows ? gr : a_rows - 1;
    const uint8_t* src = A + gr * K + g * Cfg::BK + swz(r, pc) * 16;
    __builtin_amdgcn_global_load_lds(src, to_lds(stage + m * 1024), 16, 0, 0);
  } else {
    const int mb = m - Cfg::A_BLK;
    const int r = mb * 8 + sub_r;
    int64_t gr = w_row0 + r;
    gr = gr < w_rows ? gr : w_rows - 1;
    const uint8_t* src = W + gr * K + g * Cfg::BK + swz(r, pc) * 16;
    __builtin_amdgcn_global_load_lds(src, to_lds(stage + Cfg::A_BYTES + mb * 1024), 16, 0, 0);
  }
}

template <class Cfg>
__device__ __forceinline__ void issue_scales(uint8_t* stage, const float* __restrict__ SA,
                                             int64_t a_row0, int64_t a_rows, int64_t sa_ld,
                                             int64_t g, int wave, int wave_m, int lane) {
  int64_t gr = a_row0 + wave_m * 64 + lane;
  gr = gr < a_rows ? gr : a_rows - 1;
  const float* src = SA + g * sa_ld + gr;
  __builtin_amdgcn_global_load_lds(src, to_lds(stage + Cfg::A_BYTES + Cfg::B_BYTES + wave * 256),
                                   4, 0, 0);
}

template <class Cfg>
__device__ __forceinline__ void issue_chunk(uint8_t* stage, const uint8_t* __restrict__ A,
                                            const float* __restrict__ SA,
                                            const uint8_t* __restrict__ W, int64_t a_row0,
                                            int64_t a_rows, int64_t w_row0, int64_t w_rows,
                                            int64_t K, int64_t sa_ld, int64_t g, int wave,
                                            int wave_m, int lane) {
#pragma unroll
  for (int j = 0; j < Cfg::PER_WAVE; ++j)
    issue_one<Cfg>(stage, A, W, a_row0, a_rows, w_row0, w_rows, K, g, wave, lane, j);
  issue_scales<Cfg>(stage, SA, a_row0, a_rows, sa_ld, g, wave, wave_m, lane);
}

// MFMA operand fragment: LDS row r, the 32-byte slice q of its 128-byte K
// chunk (two swizzled 16-byte columns).  A and B fragments use the same
// (q, byte) -> K mapping, so every product pairs matching K indices.
__device__ __forceinline__ v8i load_frag(const uint8_t* base, int r, int q) {
  const v4i lo = *reinterpret_cast<const v4i*>(base + r * 128 + swz(r, 2 * q) * 16);
  const v4i hi = *reinterpret_cast<const v4i*>(base + r * 128 + swz(r, 2 * q + 1) * 16);
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Promotion of one 16x16 chunk partial: acc += P * (s_a[row] * s_w).
__device__ __forceinline__ void promote(v4f& acc, const v4f& p, const v4f& mult) {
  acc[0] = __builtin_fmaf(p[0], mult[0], acc[0]);
  acc[1] = __builtin_fmaf(p[1], mult[1], acc[1]);
  acc[2] = __builtin_fmaf(p[2], mult[2], acc[2]);
  acc[3] = __builtin_fmaf(p[3], mult[3], acc[3]);
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
  void* C;              // output base
  int64_t ldc;          // N
  int out_bf16;
};

// Computes one BM x BN output tile.  All lanes of the workgroup call it.
template <class Cfg>
__device__ __forceinline__ void gemm_tile(const TileArgs& t, uint8_t* smem) {
  constexpr int MB = Cfg::MB, NB = Cfg::NB, S = Cfg::STAGES;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave_m = wave / Cfg::WAVES_N;
  const int wave_n = wave % Cfg::WAVES_N;
  const int r16 = lane & 15;   // fragment row (A) / column (B) within a 16-block
  const int q = lane >> 4;     // which 32-byte slice of the 128-byte chunk
  const int64_t G = t.K / Cfg::BK;

  // Weight-scale row of this wave's 128 columns.
  int64_t wblk = (t.w_row0 + wave_n * Cfg::WN) / 128;
  const int64_t last_wblk = t.w_rows / 128 - 1;
  wblk = wblk < last_wblk ? wblk : last_wblk;
  const float* sw_row = t.SW + wblk * G;

  // Waves whose rows are all past the valid range skip the MFMA work.
  const bool wave_live =
      (wave_m * Cfg::WM < Cfg::ROWS) && (t.a_row0 + wave_m * Cfg::WM) < t.a_rows;

  v4f acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < G)
      issue_chunk<Cfg>(smem + s * Cfg::STAGE, t.A, t.SA, t.W, t.a_row0, t.a_rows, t.w_row0,
                       t.w_rows, t.K, t.sa_ld, s, wave, wave_m, lane);

  int cur_stage = 0;
  for (int64_t g = 0; g < G; ++g) {
    // This wave's loads of chunk g have landed once at most the chunks issued
    // after it (up to S-2 of them) are still outstanding.
    {
      const int64_t left = G - 1 - g;
      wait_chunk<Cfg::LOADS, S - 2>(left < S - 2 ? (int)left : S - 2);
    }
    lds_barrier();  // every wave's chunk g landed; chunk g-1's stage is free
    // The loads of chunk g+S-1 go into the stage chunk g-1 used (free after
    // the barrier).
    {
      const int64_t gn = g + S - 1;
      if (gn < G) {
        int st = cur_stage + S - 1;
        st = st >= S ? st - S : st;
        issue_chunk<Cfg>(smem + st * Cfg::STAGE, t.A, t.SA, t.W, t.a_row0, t.a_rows, t.w_row0,
                         t.w_rows, t.K, t.sa_ld, gn, wave, wave_m, lane);
      }
    }
    const uint8_t* As = smem + cur_stage * Cfg::STAGE;
    const uint8_t* Bs = As + Cfg::A_BYTES;
    const float* SAs = reinterpret_cast<const float*>(As + Cfg::A_BYTES + Cfg::B_BYTES + wave * 256);
    cur_stage = cur_stage + 1 == S ? 0 : cur_stage + 1;
    if (!wave_live) continue;

    const float sw = sw_row[g];
    v8i a[MB];
    v4f mult[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      a[i] = load_frag(As, wave_m * Cfg::WM + i * 16 + r16, q);
      const v4f sa = *reinterpret_cast<const v4f*>(SAs + i * 16 + 4 * q);
      mult[i] = sa * sw;
    }
    // Software pipeline over the MB x NB blocks (row block fastest, so one B
    // fragment serves MB MFMAs): block k's partial is folded by the VALU two
    // MFMAs after it was issued, when its result is surely back, so the
    // matrix core and the VALU overlap without dependency stalls; block j+1's
    // B fragment is read from LDS while block j's MFMAs run.
    constexpr int LAG = 2;
    v8i b[2];
    v4f p[LAG + 1];
    b[0] = load_frag(Bs, wave_n * Cfg::WN + r16, q);
#pragma unroll
    for (int k = 0; k < MB * NB + LAG; ++k) {
      if (k < MB * NB) {
        const int i = k % MB, j = k / MB;
        if (i == 0 && j + 1 < NB)
          b[(j + 1) & 1] = load_frag(Bs, wave_n * Cfg::WN + (j + 1) * 16 + r16, q);
        p[k % (LAG + 1)] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            a[i], b[j & 1], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
      }
      const int kp = k - LAG;
      if (kp >= 0) promote(acc[kp % MB][kp / MB], p[kp % (LAG + 1)], mult[kp % MB]);
    }
  }

  // Epilogue: lane holds rows 4q..4q+3, column r16 of every 16x16 block.
  if (!wave_live) return;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t row = t.a_row0 + wave_m * Cfg::WM + i * 16 + 4 * q + v;
      if (row >= t.a_rows) continue;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int64_t col = t.w_row0 + wave_n * Cfg::WN + j * 16 + r16;
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

template <class Cfg>
__global__ __launch_bounds__(Cfg::THREADS) void gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ SA, const uint8_t* __restrict__ W,
    const float* __restrict__ SW, int64_t M, int64_t N, int64_t K, void* __restrict__ C,
    int out_bf16, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::LDS_BYTES];
  int tm, tn;
  xcd_tile(blockIdx.x, gridDim.x, tiles_n, tm, tn);
  TileArgs t;
  t.A = A;
  t.SA = SA;
  t.W = W;
  t.SW = SW;
  t.a_row0 = (int64_t)tm * Cfg::BM;
  t.a_rows = M;
  t.w_row0 = (int64_t)tn * Cfg::BN;
  t.w_rows = N;
  t.K = K;
  t.sa_ld = M;
  t.C = C;
  t.ldc = N;
  t.out_bf16 = out_bf16;
  gemm_tile<Cfg>(t, smem);
}

// Grouped variant.  The grid over-provisions tiles; each workgroup maps its id
// to (expert, m-tile, n-tile) by a prefix sum of ceil(M_e / 256) over the device
// offsets, held in LDS.  Workgroups past the last real tile exit.  Real tiles
// are numbered (expert, m-tile)-major, n-tile fastest, and handed to XCDs in
// contiguous runs (workgroup id mod 8 is its XCD), so the n-tiles of one
// expert share that expert's rows of A in one L2.  Each tile then runs the
// instantiation for its live row count.
constexpr int kMaxExpertsLds = 1024;
constexpr int kGroupedThreads = 256;
constexpr int kGroupedLds =
    GroupedCfg<64, 6>::LDS_BYTES > GroupedCfg<128, 4>::LDS_BYTES
        ? (GroupedCfg<64, 6>::LDS_BYTES > GroupedCfg<256, 3>::LDS_BYTES
               ? GroupedCfg<64, 6>::LDS_BYTES
               : GroupedCfg<256, 3>::LDS_BYTES)
        : GroupedCfg<128, 4>::LDS_BYTES;
static_assert(GroupedCfg<192, 3>::LDS_BYTES <= kGroupedLds, "grouped LDS sizing");
static_assert(GroupedCfg<64, 6>::THREADS == kGroupedThreads &&
                  GroupedCfg<256, 3>::THREADS == kGroupedThreads,
              "all grouped configurations use the same workgroup");

__global__ __launch_bounds__(kGroupedThreads) void grouped_gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ SA, int64_t M_total,
    const int32_t* __restrict__ off, int G, const uint8_t* __restrict__ W,
    const float* __restrict__ SW, int64_t N, int64_t K, void* __restrict__ C, int out_bf16,
    int tiles_n) {
  constexpr int T = kGroupedThreads;
  constexpr int BM = 256;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kGroupedLds];
  static_assert((kMaxExpertsLds + 1 + T) * 4 <= kGroupedLds, "prefix scratch fits in LDS");
  int* mt_prefix = reinterpret_cast<int*>(smem);  // [G + 1], reused before the mainloop
  int* scan = mt_prefix + kMaxExpertsLds + 1;     // [T]

  // Prefix over experts of the number of BM-row tiles (chunks of T experts,
  // each with a Hillis-Steele block scan).
  const int tid = threadIdx.x;
  int running = 0;
  if (tid == 0) mt_prefix[0] = 0;
  for (int base = 0; base < G; base += T) {
    const int e = base + tid;
    int cnt = 0;
    if (e < G) {
      const int rows = off[e + 1] - off[e];
      cnt = rows > 0 ? (rows + BM - 1) / BM : 0;
    }
    scan[tid] = cnt;
    __syncthreads();
    for (int d = 1; d < T; d <<= 1) {
      const int add = tid >= d ? scan[tid - d] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    if (e < G) mt_prefix[e + 1] = running + scan[tid];
    running += scan[T - 1];
    __syncthreads();
  }
  const int total = running * tiles_n;  // real tiles
  const int bid = blockIdx.x;
  if (bid >= total) return;
  // XCD-contiguous numbering of the real tiles: bid -> id is a bijection on
  // [0, total); XCD x (= bid mod 8) receives ids [x*q + min(x, r), ...).
  const int q8 = total / kXcds, r8 = total % kXcds;
  const int x = bid % kXcds;
  const int id = x * q8 + (x < r8 ? x : r8) + bid / kXcds;
  const int mt_global = id / tiles_n;
  const int tn = id % tiles_n;
  // expert e with prefix[e] <= mt_global < prefix[e+1]
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
  t.w_row0 = (int64_t)tn * 128;
  t.w_rows = N;
  t.K = K;
  t.sa_ld = M_total;
  t.C = C;
  t.ldc = N;
  t.out_bf16 = out_bf16;
  const int64_t live = r1 - t.a_row0;  // 1 .. (>= 256 when more m-tiles follow)
  if (live <= 64)
    gemm_tile<GroupedCfg<64, 6>>(t, smem);
  else if (live <= 128)
    gemm_tile<GroupedCfg<128, 4>>(t, smem);
  else if (live <= 192)
    gemm_tile<GroupedCfg<192, 3>>(t, smem);
  else
    gemm_tile<GroupedCfg<256, 3>>(t, smem);
}

hipError_t launch_gemm(const uint8_t* a_q, const float* a_s, const uint8_t* w_q,
                       const float* w_s, int64_t M, int64_t N, int64_t K, void* c, int out_bf16,
                       hipStream_t stream) {
  using Cfg = DenseCfg;
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t tiles_m = (M + Cfg::BM - 1) / Cfg::BM;
  const int64_t tiles_n = (N + Cfg::BN - 1) / Cfg::BN;
  const int64_t tiles = tiles_m * tiles_n;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_kernel<Cfg>, dim3((unsigned)tiles), dim3(Cfg::THREADS), 0, stream, a_q,
                     a_s, w_q, w_s, M, N, K, c, out_bf16, (int)tiles_n);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const uint8_t* a_q, const float* a_s, int64_t M_total,
                               const int32_t* off, int G, const uint8_t* w_q, const float* w_s,
                               int64_t N, int64_t K, void* c, int out_bf16,
                               hipStream_t stream) {
  if (M_total == 0 || N == 0) return hipSuccess;
  if (G > kMaxExpertsLds) return hipErrorInvalidValue;
  const int64_t tiles_n = (N + 127) / 128;
  // sum_e ceil(M_e / 256) <= floor(M_total / 256) + G
  const int64_t max_mtiles = M_total / 256 + G;
  const int64_t tiles = max_mtiles * tiles_n;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(grouped_gemm_kernel, dim3((unsigned)tiles), dim3(kGroupedThreads), 0,
                     stream, a_q, a_s, M_total, off, G, w_q, w_s, N, K, c, out_bf16,
                     (int)tiles_n);
  return hipGetLastError();
}

}  // namespace fp8q
