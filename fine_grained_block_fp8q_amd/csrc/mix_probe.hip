// Instruction-mix probe (measurement support, not part of the method): how
// much of a SIMD's matrix-core time survives the other instructions a
// block-scaled GEMM main loop issues between its MFMAs.  Built into
// libfp8q_probe.so; bench.py --mix-probe calls it.
//
// One workgroup of 8 waves per CU (its LDS allocation keeps a second one
// out), two waves per SIMD as in the GEMM kernels.  Each wave runs `iters`
// iterations; an iteration is 4 output blocks of 16x16 over one 128-K chunk:
//   FP8 mode   4 x v_mfma_scale_f32_16x16x128_f8f6f4   (the fp8q_gemm step)
//   FP16 mode 16 x v_mfma_f32_16x16x32_f16, 4 chained per block
//                                                    (the precise-mode step)
// and, per the bits of `kind`,
//   kReads  3 x 16-byte LDS reads per iteration whose data become the next
//           iteration's MFMA operands (the GEMM's 0.75 fragment reads per
//           FP8 MFMA, operands rotating as in the GEMM);
//   kPromote the blocks start from zero and 16 FP32 FMAs per iteration fold
//           the partials into accumulators (the promotion), each block's
//           two steps after its MFMA; without it the blocks chain through
//           the C operand;
//   kWiden  (FP16 mode, with kReads) the 12 code words read are widened to
//           FP16 by 24 v_cvt_scalef32_pk_f16_fp8, 1.5 per FP16 MFMA as in the
//           precise GEMM, each read's words one step after the read.
//   kScaled (FP8 mode) the MFMAs take E8M0 operand scales from registers
//           (byte 127 = 1.0 on both operands): the block-scaled form that
//           fp8q_gemm_mfma_scaled issues.
// The result of every lane is stored, so nothing is dead code.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kReads = 1, kPromote = 2, kWiden = 4, kFp16 = 8, kScaled = 16;
constexpr int kLdsBytes = 96 * 1024;   // > 80 KiB: one workgroup per CU
constexpr int kWindow = 64 * 1024;     // the reads cycle through 64 KiB

__device__ __forceinline__ v4i rd16(const uint8_t* lds, uint32_t off) {
  return *reinterpret_cast<const v4i*>(lds + (off & (kWindow - 1)));
}

__device__ __forceinline__ v4i widen(int w) {
  // two code words -> four FP16 pairs; scale operand 1.0 leaves values as is
  v4i o;
  o[0] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  o[1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
  o[2] = o[0] ^ 0x00010001;
  o[3] = o[1] ^ 0x00010001;
  return o;
}

template <int KIND>
__global__ __launch_bounds__(512) void mix_kernel(float* __restrict__ out, int iters) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // finite E4M3 codes of magnitude 2^-2 .. 2^1 with both signs
  for (int i = threadIdx.x; i < kLdsBytes / 4; i += 512)
    reinterpret_cast<uint32_t*>(lds)[i] = 0x30b83038u ^ ((uint32_t)i * 0x01030507u & 0x0f0f0f0fu);
  __syncthreads();

  const uint32_t base = (uint32_t)(wave * 64 + lane) * 16;
  constexpr bool FP16 = KIND & kFp16;
  v4f acc[4], p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
    p[j] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  const float s = 1.0f + (float)lane * 1e-7f;
  // E8M0 1.0 in every byte, from memory so the compiler keeps the scaled form
  const int one = 0x7f7f7f7f ^ (int)(reinterpret_cast<const uint32_t*>(lds)[0] & 0u);
  v4i r0 = rd16(lds, base), r1 = rd16(lds, base + 1024), r2 = rd16(lds, base + 2048);
  v8i a = v8i{r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
  v8i b = v8i{r2[0], r2[1], r2[2], r2[3], r0[0], r0[1], r0[2], r0[3]};
  v16i wa, wb;  // FP16 operands (FP16 mode)
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const v4i x = widen(a[2 * h]), y = widen(b[2 * h]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wa[4 * h + e] = x[e];
      wb[4 * h + e] = y[e];
    }
  }

  // Steps j = 0..3 of an iteration (one output block each), fenced so the
  // compiler keeps the GEMM's order: the block's MFMA(s); the LDS read of
  // step j (j < 3) and the widening of step j-1's read; the promotion of
  // block j-2 (two blocks behind its MFMA, as in the GEMM kernels).
  v4i rw[3] = {r0, r1, r2};
  for (int it = 0; it < iters; ++it) {
    v4f pn[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v4f c0 = (KIND & kPromote) ? v4f{0.f, 0.f, 0.f, 0.f} : p[j];
      if constexpr (FP16) {
        v4f c = c0;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const v4i qa = v4i{wa[4 * h], wa[4 * h + 1], wa[4 * h + 2], wa[4 * h + 3]};
          const int hb = (h + j) & 3;
          const v4i qb = v4i{wb[4 * hb], wb[4 * hb + 1], wb[4 * hb + 2], wb[4 * hb + 3]};
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, qa),
                                                    __builtin_bit_cast(v8h, qb), c, 0, 0, 0);
        }
        pn[j] = c;
      } else if constexpr (KIND & kScaled) {
        pn[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            j & 1 ? b : a, j & 2 ? a : b, c0, 0, 0, 0, one, 1, one);
      } else {
        pn[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            j & 1 ? b : a, j & 2 ? a : b, c0, 0, 0, 0, 0, 0, 0);
      }
      if constexpr (KIND & kReads) {
        if (j < 3) rw[j] = rd16(lds, base + (uint32_t)it * 3072u + (uint32_t)j * 1024u);
        if constexpr (FP16 && (KIND & kWiden)) {
          // step j widens the 4 code words read at step j-1 (8 conversions)
          if (j >= 1) {
            const v4i w = rw[j - 1];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              const int lo = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[d], 1.0f, false));
              const int hi = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[d], 1.0f, true));
              if (j == 1) { wa[2 * d] = lo; wa[2 * d + 1] = hi; }
              if (j == 2) { wa[8 + 2 * d] = lo; wa[8 + 2 * d + 1] = hi; }
              if (j == 3) { wb[2 * d] = lo; wb[2 * d + 1] = hi; }
            }
          }
        }
      }
      if constexpr (KIND & kPromote) {
        const int bj = (j + 2) & 3;   // block j-2 of this iteration, or of the previous
        const v4f src = j >= 2 ? pn[j - 2] : p[bj];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[bj][e] = __builtin_fmaf(src[e], s, acc[bj][e]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (KIND & kReads) {
      if constexpr (FP16 && !(KIND & kWiden)) {
        // rotate the read words into the operands without converting them
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wa[e] = rw[0][e];
          wa[4 + e] = rw[1][e];
          wb[e] = rw[2][e];
        }
      } else if constexpr (!FP16) {
        a = v8i{rw[0][0], rw[0][1], rw[0][2], rw[0][3], rw[1][0], rw[1][1], rw[1][2], rw[1][3]};
        b = v8i{rw[2][0], rw[2][1], rw[2][2], rw[2][3], b[0], b[1], b[2], b[3]};
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = pn[j];
  }
  float r = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) r += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3] + p[j][0] + p[j][3];
  out[blockIdx.x * 512 + threadIdx.x] = r;
}

template <int KIND>
void launch(float* out, int blocks, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mix_kernel<KIND>, dim3(blocks), dim3(512), 0, stream, out, iters);
}

}  // namespace

extern "C" {

// Runs the mix `kind` (a combination of 1 = reads, 2 = promotion, 4 = widening,
// 8 = FP16 mode, 16 = E8M0-scaled FP8 MFMAs; widening needs reads and the FP16
// mode) on one workgroup of
// 8 waves per CU of the current device, each wave `iters` iterations.
// out: device float[cus * 512].  Returns 0, -1 for an unsupported kind or
// bad arguments, or the HIP error code.  Asynchronous on `stream`.
int fp8q_probe_mix(int kind, int iters, float* out, hipStream_t stream) {
  if (!out || iters <= 0) return -1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return (int)hipGetLastError();
  switch (kind) {
    case 0: launch<0>(out, cus, iters, stream); break;
    case 1: launch<1>(out, cus, iters, stream); break;
    case 2: launch<2>(out, cus, iters, stream); break;
    case 3: launch<3>(out, cus, iters, stream); break;
    case 16: launch<16>(out, cus, iters, stream); break;
    case 19: launch<19>(out, cus, iters, stream); break;
    case 8: launch<8>(out, cus, iters, stream); break;
    case 9: launch<9>(out, cus, iters, stream); break;
    case 10: launch<10>(out, cus, iters, stream); break;
    case 11: launch<11>(out, cus, iters, stream); break;
    case 13: launch<13>(out, cus, iters, stream); break;
    case 15: launch<15>(out, cus, iters, stream); break;
    default: return -1;
  }
  return (int)hipGetLastError();
}

// Number of compute units of the current device (the workgroups one
// fp8q_probe_mix launch runs), or -1.
int fp8q_probe_cus(void) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  return cus;
}

}  // extern "C"
