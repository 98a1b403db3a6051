// The quantization rule of one 1x128 group or 128x128 block (max-abs ->
// multiplier and stored scale) and the BF16 -> E4M3 conversion, shared by the
// quantizer kernels and the GEMM that quantizes its activation operand on the
// way into LDS, so both produce the same codes and scales bit for bit.
//
// Method: the-good.kr free board post 2169793, fine-grained quantization
// passage (the max-abs of a group maps to the largest FP8 value); powers of
// two: why-be.co.kr as_center post 72410.  FP32 mode: inv = 448/amax and
// s = amax/448 with IEEE-correct division, code = cvt_e4m3_rne(x * inv); a
// non-finite inv flushes the group (s = 0, codes signed zero).  Pow2 mode:
// s = 2^e for the smallest e with 448 * 2^e >= amax, code = cvt(ldexp(x, -e)).
// None of these expressions has a multiply feeding an add, so FP contraction
// cannot change them; IEEE division is HIP's default.
#pragma once

#include "fp8q_device.hpp"

namespace fp8q {

struct GroupRule {
  float mul;   // FP32 mode: x * mul
  int neg_e;   // pow2 mode: ldexp(x, neg_e)
  float s;     // stored dequantization scale
};

// Smallest e with 448 * 2^e >= a (a > 0, finite), from the bits of a.
// a = f * 2^E with f in [1, 2); 448 = 1.75 * 2^8, so e = E - 8 if f <= 1.75
// and e = E - 7 otherwise.  An FP32 subnormal (a BF16 subnormal widened) is
// first scaled by 2^64, exactly, so that its exponent field holds E + 64.
// (Straight-line code: selects, no branch.)
__device__ __forceinline__ int pow2_exponent(float a) {
  const bool sub = a < 0x1p-126f;
  const uint32_t b = __float_as_uint(sub ? a * 0x1p64f : a);
  const int E = (int)(b >> 23) - 127 - (sub ? 64 : 0);
  return ((b & 0x7FFFFFu) <= 0x600000u) ? E - 8 : E - 7;
}

__device__ __forceinline__ float exp2_int(int e) {  // 2^e for e in [-149, 127]
  return (e >= -126) ? __uint_as_float((uint32_t)(e + 127) << 23)
                     : __uint_as_float(1u << (e + 149));
}

template <int MODE>
__device__ __forceinline__ GroupRule group_rule(float amax) {
  GroupRule r;
  if (MODE == 0) {
    const float inv = kE4M3Max / amax;
    const bool flushed = !__builtin_isfinite(inv);
    r.mul = flushed ? 0.0f : inv;
    r.s = flushed ? 0.0f : amax / kE4M3Max;
    r.neg_e = 0;
  } else {
    // (e is computed for amax = 0 too and then discarded: no branch)
    const bool pos = amax > 0.0f;
    const int e_any = pow2_exponent(amax);
    const int e = pos ? e_any : 0;
    r.neg_e = -e;
    r.s = pos ? exp2_int(e) : 0.0f;
    r.mul = 0.0f;
  }
  return r;
}

template <int MODE>
__device__ __forceinline__ float apply(float x, const GroupRule& r) {
  return MODE == 0 ? x * r.mul : __builtin_ldexpf(x, r.neg_e);
}

// 8 BF16 values (one 16-byte load) -> 8 E4M3 bytes.
template <int MODE>
__device__ __forceinline__ uint2 convert8(const uint4 v, const GroupRule& r) {
  uint2 o;
  o.x = pack_e4m3x4(apply<MODE>(bf16_lo(v.x), r), apply<MODE>(bf16_hi(v.x), r),
                    apply<MODE>(bf16_lo(v.y), r), apply<MODE>(bf16_hi(v.y), r));
  o.y = pack_e4m3x4(apply<MODE>(bf16_lo(v.z), r), apply<MODE>(bf16_hi(v.z), r),
                    apply<MODE>(bf16_lo(v.w), r), apply<MODE>(bf16_hi(v.w), r));
  return o;
}

__device__ __forceinline__ float absmax8(const uint4 v) {
  // |bf16| as float: clear the sign bits, then widen.
  const uint32_t m = 0x7FFF7FFFu;
  const uint32_t a = v.x & m, b = v.y & m, c = v.z & m, d = v.w & m;
  float r = fmaxf(bf16_lo(a), bf16_hi(a));
  r = fmaxf(r, fmaxf(bf16_lo(b), bf16_hi(b)));
  r = fmaxf(r, fmaxf(bf16_lo(c), bf16_hi(c)));
  r = fmaxf(r, fmaxf(bf16_lo(d), bf16_hi(d)));
  return r;
}

}  // namespace fp8q
