// Online fine-grained quantizers: BF16 -> OCP E4M3 with one scale per 1x128
// activation group or per 128x128 weight block.
//
// Method: the-good.kr free board post 2169793, fine-grained quantization
// passage (max-abs taken online per 1x128 activation tile / 128x128 weight
// block, scaling factor derived from it so the max-abs maps to the largest
// FP8 value, then the cast to FP8); power-of-two scales: why-be.co.kr
// as_center post 72410 (scaling factors that are integral powers of 2).
//
// Both kernels are HBM-streaming: every input byte is read once with 16-byte
// loads, the group max-abs is reduced in registers (DPP within a 16-lane row
// for activations, plus LDS across waves for weight blocks), and the codes are
// written with 8-byte non-temporal stores, 128 contiguous bytes per group row.
//
// Arithmetic (bit-exact contract): the group rule and conversion in
// quant_rules.hpp; this file is built without fast math and without FP
// contraction.

#include "quant_rules.hpp"

namespace fp8q {

// 8 code bytes, stored non-temporally: the codes are read back by a GEMM
// launch later, not by this one, so they need not displace cached lines on the
// way out (measured on back-to-back launches over rotating buffers: weight
// quantizer 18.8 -> 14.4 us, activation quantizer 18.0 -> 16.9 us at
// 4096 x 7168; a whole quantize + quantize + GEMM step is unchanged).
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_codes(uint8_t* dst, const uint2 o) {
  __builtin_nontemporal_store(v2u{o.x, o.y}, reinterpret_cast<v2u*>(dst));
}

// ---------------------------------------------------------------------------
// Activations.  A workgroup of 256 lanes covers 16 rows x 2 groups: each
// 16-lane DPP row owns one activation row and walks 2 consecutive groups, one
// 16-byte load per lane per group (16 lanes x 16 B = one 128-element group).
// Blocks are ordered group-block fastest so neighbouring workgroups stream
// neighbouring bytes of the same rows.  (2 groups per workgroup measured
// 4% faster than 4 at 4096 x 7168 and 2% at 32768 x 7168; 1 and 8 slower.)
constexpr int kActRows = 16;
constexpr int kActGroupsPerBlock = 2;

// Max-abs of 8 BF16 values by a packed 16-bit integer max of the magnitude
// bits (for non-negative floats the integer order of the bit patterns is the
// numeric order, so this is exactly the max of |x|), widened to float: fewer
// VALU instructions than unpacking to floats first.
typedef uint16_t v2u16 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float absmax8_pk(const uint4 v) {
  const uint32_t m = 0x7FFF7FFFu;
  auto h = [](uint32_t w) { return __builtin_bit_cast(v2u16, w); };
  const v2u16 r = __builtin_elementwise_max(__builtin_elementwise_max(h(v.x & m), h(v.y & m)),
                                            __builtin_elementwise_max(h(v.z & m), h(v.w & m)));
  const uint32_t b = r[0] > r[1] ? r[0] : r[1];
  return __uint_as_float(b << 16);
}

template <int MODE>
__global__ __launch_bounds__(256) void quantize_act_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, uint8_t* __restrict__ q,
    float* __restrict__ s, int64_t n_gblk) {
  const int64_t G = K / kGroup;
  const int64_t bid = blockIdx.x;
  const int64_t gb = bid % n_gblk;
  const int64_t rb = bid / n_gblk;
  const int unit = threadIdx.x >> 4;
  const int l16 = threadIdx.x & 15;
  const int64_t m = rb * kActRows + unit;
  const bool row_ok = m < M;

  uint4 v[kActGroupsPerBlock];
#pragma unroll
  for (int j = 0; j < kActGroupsPerBlock; ++j) {
    const int64_t g = gb * kActGroupsPerBlock + j;
    if (row_ok && g < G)
      v[j] = *reinterpret_cast<const uint4*>(x + m * K + g * kGroup + l16 * 8);
    else
      v[j] = make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int j = 0; j < kActGroupsPerBlock; ++j) {
    const int64_t g = gb * kActGroupsPerBlock + j;
    const float amax = row16_max(absmax8_pk(v[j]));
    const GroupRule r = group_rule<MODE>(amax);
    if (row_ok && g < G) {
      store_codes(q + m * K + g * kGroup + l16 * 8, convert8<MODE>(v[j], r));
      if (l16 == j) s[g * M + m] = r.s;
    }
  }
}

// ---------------------------------------------------------------------------
// Weights.  One 256-lane workgroup per 128x128 block: lane (r0 = t/16,
// c = t%16) loads rows r0, r0+16, ..., r0+112 at byte column 16c, so all
// eight 16-byte loads are in flight before the reduction.  The block max is
// reduced across each DPP row, across the 4 rows of a wave by readlane, and
// across the 4 waves through LDS.
template <int MODE>
__global__ __launch_bounds__(256) void quantize_weight_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t K, uint8_t* __restrict__ q,
    float* __restrict__ s, int64_t KB) {
  __shared__ float red[4];
  const int64_t bid = blockIdx.x;
  const int64_t nb = bid / KB;
  const int64_t kb = bid % KB;
  const int t = threadIdx.x;
  const int l16 = t & 15;
  const int r0 = t >> 4;
  const int lane = t & 63;
  const int wave = t >> 6;

  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = nb * kGroup + r0 + 16 * i;
    v[i] = *reinterpret_cast<const uint4*>(w + row * K + kb * kGroup + l16 * 8);
  }
  float a = absmax8(v[0]);
#pragma unroll
  for (int i = 1; i < 8; ++i) a = fmaxf(a, absmax8(v[i]));
  a = row16_max(a);
  a = fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 0)),
                  __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 16))),
            fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 32)),
                  __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 48))));
  if (lane == 0) red[wave] = a;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const GroupRule r = group_rule<MODE>(amax);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = nb * kGroup + r0 + 16 * i;
    store_codes(q + row * K + kb * kGroup + l16 * 8, convert8<MODE>(v[i], r));
  }
  if (t == 0) s[nb * KB + kb] = r.s;
  (void)N;
}

// ---------------------------------------------------------------------------
// Transposed quantizers for the backward GEMMs.  The weight-gradient GEMM
// (dW = dY^T X) contracts over the tokens, so its operands dY^T and X^T are
// quantized in groups of 128 consecutive rows of one column of dY and X; the
// activation-gradient GEMM (dX = dY W) takes W^T, whose 128x128 blocks are
// those of W with their codes transposed.  Both kernels write the codes of
// the transposed matrix directly.

// BF16 element j (0..7) of a 16-byte load, as float.
__device__ __forceinline__ float bf16_at(const uint4& v, int j) {
  const uint32_t w = j < 2 ? v.x : j < 4 ? v.y : j < 6 ? v.z : v.w;
  return (j & 1) ? bf16_hi(w) : bf16_lo(w);
}

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_piece(uint8_t* dst, const uint4 o) {
  __builtin_nontemporal_store(v4u{o.x, o.y, o.z, o.w}, reinterpret_cast<v4u*>(dst));
}

// Activations, transposed: x[M][K] -> q_t[K][M], s_t[M/128][K].  A workgroup
// covers 128 rows (one group of tokens) x 64 columns.  Lane (rq = t/8,
// cp = t%8) loads rows 4rq .. 4rq+3 at columns 8cp .. 8cp+7, so 8 lanes read a
// row's 128 contiguous bytes.  A column's max-abs is reduced over the lane's
// 4 rows, across the 8 lanes of the wave that share cp (shuffles), then
// across the 4 waves through LDS.  The lane packs the codes of its 4
// consecutive rows of each column into one word of the tile's transposed copy
// in LDS (64 output rows of 128 bytes); the workgroup then stores that copy
// with one 16-byte store per lane and piece, 8 lanes per 128-byte output row.
// (Storing the words straight to HBM, 32-byte runs per row and wave, ran at
// half the rate.)
constexpr int kTRow = 144;  // bytes per row of a transposed code tile in LDS (16-byte aligned)

template <int MODE>
__global__ __launch_bounds__(256) void quantize_act_t_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, uint8_t* __restrict__ qt,
    float* __restrict__ st, int64_t n_kblk) {
  __shared__ float red[4][64];
  __shared__ __attribute__((aligned(16))) uint8_t tile[64 * kTRow];
  const int64_t bid = blockIdx.x;
  const int64_t kb = bid % n_kblk;  // 64-column block (fastest: neighbours share rows)
  const int64_t mb = bid / n_kblk;  // group of 128 rows
  const int t = threadIdx.x;
  const int rq = t >> 3, cp = t & 7;
  const int wave = t >> 6;
  const int64_t m0 = mb * kGroup + 4 * rq;
  const int64_t k0 = kb * 64 + 8 * cp;
  uint4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const uint4*>(x + (m0 + i) * K + k0);
  float a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = fmaxf(fmaxf(fabsf(bf16_at(v[0], j)), fabsf(bf16_at(v[1], j))),
                 fmaxf(fabsf(bf16_at(v[2], j)), fabsf(bf16_at(v[3], j))));
#pragma unroll
    for (int d = 8; d < 64; d <<= 1) a[j] = fmaxf(a[j], __shfl_xor(a[j], d));
  }
  if ((t & 63) < 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) red[wave][8 * cp + j] = a[j];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = 8 * cp + j;
    const float amax = fmaxf(fmaxf(red[0][c], red[1][c]), fmaxf(red[2][c], red[3][c]));
    const GroupRule r = group_rule<MODE>(amax);
    if (rq == 0) st[mb * K + k0 + j] = r.s;
    const uint32_t w = pack_e4m3x4(apply<MODE>(bf16_at(v[0], j), r), apply<MODE>(bf16_at(v[1], j), r),
                                   apply<MODE>(bf16_at(v[2], j), r), apply<MODE>(bf16_at(v[3], j), r));
    *reinterpret_cast<uint32_t*>(tile + c * kTRow + 4 * rq) = w;
  }
  __syncthreads();
  // 64 rows x 128 bytes = 512 pieces of 16 bytes, 2 per lane.
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int p = t + 256 * u;
    const int row = p >> 3, piece = p & 7;
    const uint4 o = *reinterpret_cast<const uint4*>(tile + row * kTRow + 16 * piece);
    store_piece(qt + (kb * 64 + row) * M + mb * kGroup + 16 * piece, o);
  }
}

// Weights, transposed: w[N][K] -> q_t[K][N], s_t[K/128][N/128].  One 256-lane
// workgroup per 128x128 block: lane (rq = t/16, cp = t%16) loads rows
// 8rq .. 8rq+7 at columns 8cp .. 8cp+7 (16 lanes read a row's 256 bytes).
// The block max is reduced as in quantize_weight_kernel (each DPP row is one
// rq); each lane then writes the codes of its 8 consecutive rows of each of
// its 8 columns (8 bytes) into the block's transposed copy in LDS, which the
// workgroup stores with 16-byte pieces, 8 lanes per 128-byte output row.
template <int MODE>
__global__ __launch_bounds__(256) void quantize_weight_t_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t K, uint8_t* __restrict__ qt,
    float* __restrict__ st, int64_t KB) {
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) uint8_t tile[128 * kTRow];
  const int64_t bid = blockIdx.x;
  const int64_t nb = bid / KB;
  const int64_t kb = bid % KB;
  const int t = threadIdx.x;
  const int rq = t >> 4, cp = t & 15;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int64_t n0 = nb * kGroup + 8 * rq;
  const int64_t k0 = kb * kGroup + 8 * cp;
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const uint4*>(w + (n0 + i) * K + k0);
  float a = absmax8(v[0]);
#pragma unroll
  for (int i = 1; i < 8; ++i) a = fmaxf(a, absmax8(v[i]));
  a = row16_max(a);
  a = fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 0)),
                  __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 16))),
            fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 32)),
                  __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 48))));
  if (lane == 0) red[wave] = a;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const GroupRule r = group_rule<MODE>(amax);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint2 o;
    o.x = pack_e4m3x4(apply<MODE>(bf16_at(v[0], j), r), apply<MODE>(bf16_at(v[1], j), r),
                      apply<MODE>(bf16_at(v[2], j), r), apply<MODE>(bf16_at(v[3], j), r));
    o.y = pack_e4m3x4(apply<MODE>(bf16_at(v[4], j), r), apply<MODE>(bf16_at(v[5], j), r),
                      apply<MODE>(bf16_at(v[6], j), r), apply<MODE>(bf16_at(v[7], j), r));
    *reinterpret_cast<uint2*>(tile + (8 * cp + j) * kTRow + 8 * rq) = o;
  }
  if (t == 0) st[kb * (N / kGroup) + nb] = r.s;
  __syncthreads();
  // 128 rows x 128 bytes = 1024 pieces of 16 bytes, 4 per lane.
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int p = t + 256 * u;
    const int row = p >> 3, piece = p & 7;
    const uint4 o = *reinterpret_cast<const uint4*>(tile + row * kTRow + 16 * piece);
    store_piece(qt + (kb * kGroup + row) * N + nb * kGroup + 16 * piece, o);
  }
}

hipError_t launch_quantize_act_t(const void* x, int64_t M, int64_t K, uint8_t* qt, float* st,
                                 int mode, hipStream_t stream) {
  const int64_t n_kblk = K / 64;
  const int64_t blocks = (M / kGroup) * n_kblk;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(256);
  if (mode == 0)
    hipLaunchKernelGGL(quantize_act_t_kernel<0>, grid, block, 0, stream,
                       static_cast<const uint16_t*>(x), M, K, qt, st, n_kblk);
  else
    hipLaunchKernelGGL(quantize_act_t_kernel<1>, grid, block, 0, stream,
                       static_cast<const uint16_t*>(x), M, K, qt, st, n_kblk);
  return hipGetLastError();
}

hipError_t launch_quantize_weight_t(const void* w, int64_t N, int64_t K, uint8_t* qt,
                                    float* st, int mode, hipStream_t stream) {
  const int64_t KB = K / kGroup;
  const int64_t blocks = (N / kGroup) * KB;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(256);
  if (mode == 0)
    hipLaunchKernelGGL(quantize_weight_t_kernel<0>, grid, block, 0, stream,
                       static_cast<const uint16_t*>(w), N, K, qt, st, KB);
  else
    hipLaunchKernelGGL(quantize_weight_t_kernel<1>, grid, block, 0, stream,
                       static_cast<const uint16_t*>(w), N, K, qt, st, KB);
  return hipGetLastError();
}

hipError_t launch_quantize_act(const void* x, int64_t M, int64_t K, uint8_t* q, float* s,
                               int mode, hipStream_t stream) {
  const int64_t G = K / kGroup;
  const int64_t n_gblk = (G + kActGroupsPerBlock - 1) / kActGroupsPerBlock;
  const int64_t n_rblk = (M + kActRows - 1) / kActRows;
  const int64_t blocks = n_gblk * n_rblk;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(256);
  if (mode == 0)
    hipLaunchKernelGGL(quantize_act_kernel<0>, grid, block, 0, stream,
                       static_cast<const uint16_t*>(x), M, K, q, s, n_gblk);
  else
    hipLaunchKernelGGL(quantize_act_kernel<1>, grid, block, 0, stream,
                       static_cast<const uint16_t*>(x), M, K, q, s, n_gblk);
  return hipGetLastError();
}

hipError_t launch_quantize_weight(const void* w, int64_t N, int64_t K, uint8_t* q, float* s,
                                  int mode, hipStream_t stream) {
  const int64_t KB = K / kGroup;
  const int64_t blocks = (N / kGroup) * KB;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(256);
  if (mode == 0)
    hipLaunchKernelGGL(quantize_weight_kernel<0>, grid, block, 0, stream,
                       static_cast<const uint16_t*>(w), N, K, q, s, KB);
  else
    hipLaunchKernelGGL(quantize_weight_kernel<1>, grid, block, 0, stream,
                       static_cast<const uint16_t*>(w), N, K, q, s, KB);
  return hipGetLastError();
}

}  // namespace fp8q
