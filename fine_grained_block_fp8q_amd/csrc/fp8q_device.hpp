// Device helpers shared by the fp8q kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Largest finite OCP E4M3 magnitude: (1 + 6/8) * 2^8.
constexpr float kE4M3Max = 448.0f;
constexpr int kGroup = 128;  // 1x128 activation groups, 128x128 weight blocks

// DPP controls (row = 16 lanes).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_fmax(float v) {
  int o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false);
  return fmaxf(v, __int_as_float(o));
}

// Max over the 16 lanes of a DPP row; every lane of the row gets the result.
// Inputs are non-negative magnitudes.
__device__ __forceinline__ float row16_max(float v) {
  v = dpp_fmax<kDppQuadXor1>(v);
  v = dpp_fmax<kDppQuadXor2>(v);
  v = dpp_fmax<kDppRowHalfMirror>(v);
  v = dpp_fmax<kDppRowMirror>(v);
  return v;
}

// Two BF16 values packed in a 32-bit word -> floats (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Four floats -> four OCP E4M3 bytes (round to nearest even), a in byte 0.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// float -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace fp8q
