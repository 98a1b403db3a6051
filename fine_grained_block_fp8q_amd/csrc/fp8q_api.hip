// C ABI of libfp8q: host-side validation and launch (declared in include/fp8q.h).
//
// Validation runs entirely on the host and before any HIP call, in the order
// the header documents, so every error path can be exercised without a GPU.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "fp8q.h"

namespace fp8q {
hipError_t launch_quantize_act(const void* x, int64_t M, int64_t K, uint8_t* q, float* s,
                               int mode, hipStream_t stream);
hipError_t launch_quantize_weight(const void* w, int64_t N, int64_t K, uint8_t* q, float* s,
                                  int mode, hipStream_t stream);
hipError_t launch_gemm(const uint8_t* a_q, const float* a_s, const uint8_t* w_q,
                       const float* w_s, int64_t M, int64_t N, int64_t K, void* c, int out_bf16,
                       int mode, hipStream_t stream);
hipError_t launch_grouped_gemm(const uint8_t* a_q, const float* a_s, int64_t M_total,
                               const int32_t* off, int G, const uint8_t* w_q, const float* w_s,
                               int64_t N, int64_t K, void* c, int out_bf16, int precise,
                               hipStream_t stream);
hipError_t launch_gemm_bf16(const void* a, const void* w, int64_t M, int64_t N, int64_t K,
                            void* c, int out_bf16, hipStream_t stream);
hipError_t launch_quantize_act_t(const void* x, int64_t M, int64_t K, uint8_t* qt, float* st,
                                 int mode, hipStream_t stream);
hipError_t launch_quantize_weight_t(const void* w, int64_t N, int64_t K, uint8_t* qt,
                                    float* st, int mode, hipStream_t stream);
hipError_t launch_gemm_rowscaled(const uint8_t* a_q, const float* a_s, const uint8_t* b_q,
                                 const float* b_s, int64_t M, int64_t N, int64_t K, void* c,
                                 int out_bf16, int precise, hipStream_t stream);
hipError_t launch_gemm_cast(const void* x, const uint8_t* w_q, const float* w_s, int64_t M,
                            int64_t N, int64_t K, void* c, int out_bf16, int mode,
                            hipStream_t stream);
hipError_t launch_grouped_gemm_cast(const void* x, int64_t M_total, const int32_t* off, int G,
                                    const uint8_t* w_q, const float* w_s, int64_t N, int64_t K,
                                    void* c, int out_bf16, int mode, hipStream_t stream);
#ifdef FP8Q_DEBUG_CHECKS
hipError_t offsets_error_take(hipStream_t stream, int* flag);
#endif
}  // namespace fp8q

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other architecture
std::atomic<int> g_arch_cache[kMaxDevices];

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The current device must be a gfx950.  Cached per device ordinal.
fp8q_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return FP8Q_ERR_DEVICE;
  }
  if (dev < kMaxDevices) {
    const int c = g_arch_cache[dev].load(std::memory_order_relaxed);
    if (c == 1) return FP8Q_OK;
    if (c == 2) return FP8Q_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return FP8Q_ERR_DEVICE;
  }
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_cache[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? FP8Q_OK : FP8Q_ERR_DEVICE;
}

fp8q_status launched(hipError_t e) {
  if (e == hipSuccess) return FP8Q_OK;
  (void)hipGetLastError();
  return FP8Q_ERR_LAUNCH;
}

// A grouped launch's status.  Debug builds (FP8Q_DEBUG_CHECKS) synchronize
// the stream and report the kernel's verdict on the device offsets.
fp8q_status grouped_launched(hipError_t e, hipStream_t stream) {
  const fp8q_status st = launched(e);
#ifdef FP8Q_DEBUG_CHECKS
  if (st == FP8Q_OK) {
    int flag = 0;
    if (fp8q::offsets_error_take(stream, &flag) != hipSuccess) return launched(hipErrorUnknown);
    if (flag) return FP8Q_ERR_OFFSETS;
  }
#else
  (void)stream;
#endif
  return st;
}

bool valid_mode(int m) { return m == FP8Q_SCALE_F32 || m == FP8Q_SCALE_POW2; }
bool valid_out(int o) { return o == FP8Q_OUT_F32 || o == FP8Q_OUT_BF16; }

}  // namespace

extern "C" {

int fp8q_abi_version(void) { return FP8Q_ABI_VERSION; }

int fp8q_debug_checks(void) {
#ifdef FP8Q_DEBUG_CHECKS
  return 1;
#else
  return 0;
#endif
}

const char* fp8q_status_string(fp8q_status st) {
  switch (st) {
    case FP8Q_OK: return "FP8Q_OK";
    case FP8Q_ERR_NULL: return "FP8Q_ERR_NULL: a required pointer is NULL";
    case FP8Q_ERR_SHAPE:
      return "FP8Q_ERR_SHAPE: negative size, K or N not a multiple of 128, or G < 1";
    case FP8Q_ERR_ALIGN:
      return "FP8Q_ERR_ALIGN: data pointer not 16-byte aligned or scale/offset pointer not "
             "4-byte aligned";
    case FP8Q_ERR_ENUM: return "FP8Q_ERR_ENUM: unknown scale mode or output dtype";
    case FP8Q_ERR_DEVICE: return "FP8Q_ERR_DEVICE: no current HIP device, or it is not gfx950";
    case FP8Q_ERR_LAUNCH: return "FP8Q_ERR_LAUNCH: kernel launch failed";
    case FP8Q_ERR_UNSUPPORTED: return "FP8Q_ERR_UNSUPPORTED: valid request outside what the library implements";
    case FP8Q_ERR_OFFSETS:
      return "FP8Q_ERR_OFFSETS: device offsets not 0 = off[0] <= ... <= off[G] <= M_total "
             "(reported by FP8Q_DEBUG_CHECKS builds)";
  }
  return "FP8Q_ERR_UNKNOWN: not a status code";
}

fp8q_status fp8q_quantize_act(const void* x_bf16, int64_t M, int64_t K, uint8_t* q, float* s,
                              fp8q_scale_mode mode, hipStream_t stream) {
  const bool empty = (M == 0 || K == 0);
  if (!empty && (!x_bf16 || !q || !s)) return FP8Q_ERR_NULL;
  if (M < 0 || K < 0 || K % 128 != 0) return FP8Q_ERR_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(q, 16) || !aligned(s, 4)) return FP8Q_ERR_ALIGN;
  if (!valid_mode(mode)) return FP8Q_ERR_ENUM;
  if (empty) return FP8Q_OK;
  const fp8q_status d = check_device();
  if (d != FP8Q_OK) return d;
  return launched(fp8q::launch_quantize_act(x_bf16, M, K, q, s, (int)mode, stream));
}

fp8q_status fp8q_quantize_weight(const void* w_bf16, int64_t N, int64_t K, uint8_t* q, float* s,
                                 fp8q_scale_mode mode, hipStream_t stream) {
  const bool empty = (N == 0 || K == 0);
  if (!empty && (!w_bf16 || !q || !s)) return FP8Q_ERR_NULL;
  if (N < 0 || K < 0 || N % 128 != 0 || K % 128 != 0) return FP8Q_ERR_SHAPE;
  if (!aligned(w_bf16, 16) || !aligned(q, 16) || !aligned(s, 4)) return FP8Q_ERR_ALIGN;
  if (!valid_mode(mode)) return FP8Q_ERR_ENUM;
  if (empty) return FP8Q_OK;
  const fp8q_status d = check_device();
  if (d != FP8Q_OK) return d;
  return launched(fp8q::launch_quantize_weight(w_bf16, N, K, q, s, (int)mode, stream));
}

// The GEMM kernels address a tile's operands with 32-bit buffer offsets
// (row-in-tile * K + chunk offset) and a chunk's row scales with a 31-bit
// scalar offset (chunk * rows * 4): K up to 2^22 and rows * K/128 * 4 below
// 2^31 keep every offset in range.
static bool gemm_extent_ok(int64_t rows, int64_t K) {
  if (K > (int64_t(1) << 22)) return false;
  return rows <= int64_t(0x7FFFFFFF) / 4 / (K / 128);
}

static fp8q_status gemm_call(const uint8_t* a_q, const float* a_s, const uint8_t* w_q,
                             const float* w_s, int64_t M, int64_t N, int64_t K, void* c,
                             fp8q_out_dtype out, int mode, hipStream_t stream) {
  const bool empty_out = (M == 0 || N == 0);
  const bool empty_k = (K == 0);
  if (!empty_out && !c) return FP8Q_ERR_NULL;
  if (!empty_out && !empty_k && (!a_q || !a_s || !w_q || !w_s)) return FP8Q_ERR_NULL;
  if (M < 0 || N < 0 || K < 0 || N % 128 != 0 || K % 128 != 0) return FP8Q_ERR_SHAPE;
  if (!aligned(a_q, 16) || !aligned(w_q, 16) || !aligned(c, 16) || !aligned(a_s, 4) ||
      !aligned(w_s, 4))
    return FP8Q_ERR_ALIGN;
  if (!valid_out(out)) return FP8Q_ERR_ENUM;
  if (empty_out) return FP8Q_OK;
  if (empty_k) return FP8Q_ERR_UNSUPPORTED;  // C = 0 would need a fill kernel
  if (!gemm_extent_ok(M, K)) return FP8Q_ERR_UNSUPPORTED;
  const fp8q_status d = check_device();
  if (d != FP8Q_OK) return d;
  return launched(
      fp8q::launch_gemm(a_q, a_s, w_q, w_s, M, N, K, c, out == FP8Q_OUT_BF16, mode, stream));
}

fp8q_status fp8q_gemm(const uint8_t* a_q, const float* a_s, const uint8_t* w_q,
                      const float* w_s, int64_t M, int64_t N, int64_t K, void* c,
                      fp8q_out_dtype out, hipStream_t stream) {
  return gemm_call(a_q, a_s, w_q, w_s, M, N, K, c, out, 0, stream);
}

fp8q_status fp8q_gemm_precise(const uint8_t* a_q, const float* a_s, const uint8_t* w_q,
                              const float* w_s, int64_t M, int64_t N, int64_t K, void* c,
                              fp8q_out_dtype out, hipStream_t stream) {
  return gemm_call(a_q, a_s, w_q, w_s, M, N, K, c, out, 1, stream);
}

fp8q_status fp8q_gemm_mfma_scaled(const uint8_t* a_q, const float* a_s, const uint8_t* w_q,
                                  const float* w_s, int64_t M, int64_t N, int64_t K, void* c,
                                  fp8q_out_dtype out, hipStream_t stream) {
  return gemm_call(a_q, a_s, w_q, w_s, M, N, K, c, out, 2, stream);
}

static fp8q_status grouped_call(const uint8_t* a_q, const float* a_s, int64_t M_total,
                                const int32_t* off, int32_t G, const uint8_t* w_q,
                                const float* w_s, int64_t N, int64_t K, void* c,
                                fp8q_out_dtype out, int precise, hipStream_t stream) {
  const bool empty_out = (M_total == 0 || N == 0);
  if (!off) return FP8Q_ERR_NULL;
  if (!empty_out && !c) return FP8Q_ERR_NULL;
  if (!empty_out && K != 0 && (!a_q || !a_s || !w_q || !w_s)) return FP8Q_ERR_NULL;
  if (M_total < 0 || N < 0 || K < 0 || G < 1 || N % 128 != 0 || K % 128 != 0)
    return FP8Q_ERR_SHAPE;
  if (G > 1024) return FP8Q_ERR_UNSUPPORTED;
  if (M_total > 0x7FFFFFFF) return FP8Q_ERR_SHAPE;  // offsets are int32
  if (!aligned(a_q, 16) || !aligned(w_q, 16) || !aligned(c, 16) || !aligned(a_s, 4) ||
      !aligned(w_s, 4) || !aligned(off, 4))
    return FP8Q_ERR_ALIGN;
  if (!valid_out(out)) return FP8Q_ERR_ENUM;
  if (empty_out) return FP8Q_OK;
  if (K == 0) return FP8Q_ERR_UNSUPPORTED;
  if (!gemm_extent_ok(M_total, K)) return FP8Q_ERR_UNSUPPORTED;
  const fp8q_status d = check_device();
  if (d != FP8Q_OK) return d;
  return grouped_launched(fp8q::launch_grouped_gemm(a_q, a_s, M_total, off, G, w_q, w_s, N, K,
                                                    c, out == FP8Q_OUT_BF16, precise, stream),
                          stream);
}

fp8q_status fp8q_grouped_gemm(const uint8_t* a_q, const float* a_s, int64_t M_total,
                              const int32_t* off, int32_t G, const uint8_t* w_q,
                              const float* w_s, int64_t N, int64_t K, void* c,
                              fp8q_out_dtype out, hipStream_t stream) {
  return grouped_call(a_q, a_s, M_total, off, G, w_q, w_s, N, K, c, out, 0, stream);
}

fp8q_status fp8q_grouped_gemm_precise(const uint8_t* a_q, const float* a_s, int64_t M_total,
                                      const int32_t* off, int32_t G, const uint8_t* w_q,
                                      const float* w_s, int64_t N, int64_t K, void* c,
                                      fp8q_out_dtype out, hipStream_t stream) {
  return grouped_call(a_q, a_s, M_total, off, G, w_q, w_s, N, K, c, out, 1, stream);
}

fp8q_status fp8q_quantize_act_t(const void* x_bf16, int64_t M, int64_t K, uint8_t* q_t,
                                float* s_t, fp8q_scale_mode mode, hipStream_t stream) {
  const bool empty = (M == 0 || K == 0);
  if (!empty && (!x_bf16 || !q_t || !s_t)) return FP8Q_ERR_NULL;
  if (M < 0 || K < 0 || M % 128 != 0 || K % 128 != 0) return FP8Q_ERR_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(q_t, 16) || !aligned(s_t, 4)) return FP8Q_ERR_ALIGN;
  if (!valid_mode(mode)) return FP8Q_ERR_ENUM;
  if (empty) return FP8Q_OK;
  const fp8q_status d = check_device();
  if (d != FP8Q_OK) return d;
  return launched(fp8q::launch_quantize_act_t(x_bf16, M, K, q_t, s_t, (int)mode, stream));
}

fp8q_status fp8q_quantize_weight_t(const void* w_bf16, int64_t N, int64_t K, uint8_t* q_t,
                                   float* s_t, fp8q_scale_mode mode, hipStream_t stream) {
  const bool empty = (N == 0 || K == 0);
  if (!empty && (!w_bf16 || !q_t || !s_t)) return FP8Q_ERR_NULL;
  if (N < 0 || K < 0 || N % 128 != 0 || K % 128 != 0) return FP8Q_ERR_SHAPE;
  if (!aligned(w_bf16, 16) || !aligned(q_t, 16) || !aligned(s_t, 4)) return FP8Q_ERR_ALIGN;
  if (!valid_mode(mode)) return FP8Q_ERR_ENUM;
  if (empty) return FP8Q_OK;
  const fp8q_status d = check_device();
  if (d != FP8Q_OK) return d;
  return launched(fp8q::launch_quantize_weight_t(w_bf16, N, K, q_t, s_t, (int)mode, stream));
}

static fp8q_status rowscaled_call(const uint8_t* a_q, const float* a_s, const uint8_t* b_q,
                                  const float* b_s, int64_t M, int64_t N, int64_t K, void* c,
                                  fp8q_out_dtype out, int precise, hipStream_t stream) {
  const bool empty_out = (M == 0 || N == 0);
  if (!empty_out && !c) return FP8Q_ERR_NULL;
  if (!empty_out && K != 0 && (!a_q || !a_s || !b_q || !b_s)) return FP8Q_ERR_NULL;
  if (M < 0 || N < 0 || K < 0 || N % 128 != 0 || K % 128 != 0) return FP8Q_ERR_SHAPE;
  if (!aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(c, 16) || !aligned(a_s, 4) ||
      !aligned(b_s, 4))
    return FP8Q_ERR_ALIGN;
  if (!valid_out(out)) return FP8Q_ERR_ENUM;
  if (empty_out) return FP8Q_OK;
  if (K == 0) return FP8Q_ERR_UNSUPPORTED;
  if (!gemm_extent_ok(M, K) || !gemm_extent_ok(N, K)) return FP8Q_ERR_UNSUPPORTED;
  const fp8q_status d = check_device();
  if (d != FP8Q_OK) return d;
  return launched(fp8q::launch_gemm_rowscaled(a_q, a_s, b_q, b_s, M, N, K, c,
                                              out == FP8Q_OUT_BF16, precise, stream));
}

fp8q_status fp8q_gemm_rowscaled(const uint8_t* a_q, const float* a_s, const uint8_t* b_q,
                                const float* b_s, int64_t M, int64_t N, int64_t K, void* c,
                                fp8q_out_dtype out, hipStream_t stream) {
  return rowscaled_call(a_q, a_s, b_q, b_s, M, N, K, c, out, 0, stream);
}

fp8q_status fp8q_gemm_rowscaled_precise(const uint8_t* a_q, const float* a_s,
                                        const uint8_t* b_q, const float* b_s, int64_t M,
                                        int64_t N, int64_t K, void* c, fp8q_out_dtype out,
                                        hipStream_t stream) {
  return rowscaled_call(a_q, a_s, b_q, b_s, M, N, K, c, out, 1, stream);
}

fp8q_status fp8q_gemm_bf16(const void* a, const void* w, int64_t M, int64_t N, int64_t K,
                           void* c, fp8q_out_dtype out, hipStream_t stream) {
  const bool empty_out = (M == 0 || N == 0);
  if (!empty_out && !c) return FP8Q_ERR_NULL;
  if (!empty_out && K != 0 && (!a || !w)) return FP8Q_ERR_NULL;
  if (M < 0 || N < 0 || K < 0 || N % 128 != 0 || K % 128 != 0) return FP8Q_ERR_SHAPE;
  if (!aligned(a, 16) || !aligned(w, 16) || !aligned(c, 16)) return FP8Q_ERR_ALIGN;
  if (!valid_out(out)) return FP8Q_ERR_ENUM;
  if (empty_out) return FP8Q_OK;
  if (K == 0) return FP8Q_ERR_UNSUPPORTED;
  if (K > (int64_t(1) << 21)) return FP8Q_ERR_UNSUPPORTED;
  const fp8q_status d = check_device();
  if (d != FP8Q_OK) return d;
  return launched(fp8q::launch_gemm_bf16(a, w, M, N, K, c, out == FP8Q_OUT_BF16, stream));
}

// The fused GEMMs read 2K-byte BF16 activation rows through 32-bit buffer
// offsets (row-in-tile * 2K): K up to 2^21, as for the BF16 GEMM.
fp8q_status fp8q_gemm_fused(const void* x_bf16, const uint8_t* w_q, const float* w_s,
                            int64_t M, int64_t N, int64_t K, void* c, fp8q_out_dtype out,
                            fp8q_scale_mode mode, hipStream_t stream) {
  const bool empty_out = (M == 0 || N == 0);
  if (!empty_out && !c) return FP8Q_ERR_NULL;
  if (!empty_out && K != 0 && (!x_bf16 || !w_q || !w_s)) return FP8Q_ERR_NULL;
  if (M < 0 || N < 0 || K < 0 || N % 128 != 0 || K % 128 != 0) return FP8Q_ERR_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(w_q, 16) || !aligned(c, 16) || !aligned(w_s, 4))
    return FP8Q_ERR_ALIGN;
  if (!valid_out(out) || !valid_mode(mode)) return FP8Q_ERR_ENUM;
  if (empty_out) return FP8Q_OK;
  if (K == 0) return FP8Q_ERR_UNSUPPORTED;
  if (K > (int64_t(1) << 21)) return FP8Q_ERR_UNSUPPORTED;
  const fp8q_status d = check_device();
  if (d != FP8Q_OK) return d;
  return launched(fp8q::launch_gemm_cast(x_bf16, w_q, w_s, M, N, K, c, out == FP8Q_OUT_BF16,
                                         (int)mode, stream));
}

fp8q_status fp8q_grouped_gemm_fused(const void* x_bf16, int64_t M_total, const int32_t* off,
                                    int32_t G, const uint8_t* w_q, const float* w_s, int64_t N,
                                    int64_t K, void* c, fp8q_out_dtype out, fp8q_scale_mode mode,
                                    hipStream_t stream) {
  const bool empty_out = (M_total == 0 || N == 0);
  if (!off) return FP8Q_ERR_NULL;
  if (!empty_out && !c) return FP8Q_ERR_NULL;
  if (!empty_out && K != 0 && (!x_bf16 || !w_q || !w_s)) return FP8Q_ERR_NULL;
  if (M_total < 0 || N < 0 || K < 0 || G < 1 || N % 128 != 0 || K % 128 != 0)
    return FP8Q_ERR_SHAPE;
  if (G > 1024) return FP8Q_ERR_UNSUPPORTED;
  if (M_total > 0x7FFFFFFF) return FP8Q_ERR_SHAPE;  // offsets are int32
  if (!aligned(x_bf16, 16) || !aligned(w_q, 16) || !aligned(c, 16) || !aligned(w_s, 4) ||
      !aligned(off, 4))
    return FP8Q_ERR_ALIGN;
  if (!valid_out(out) || !valid_mode(mode)) return FP8Q_ERR_ENUM;
  if (empty_out) return FP8Q_OK;
  if (K == 0) return FP8Q_ERR_UNSUPPORTED;
  if (K > (int64_t(1) << 21)) return FP8Q_ERR_UNSUPPORTED;
  const fp8q_status d = check_device();
  if (d != FP8Q_OK) return d;
  return grouped_launched(fp8q::launch_grouped_gemm_cast(x_bf16, M_total, off, G, w_q, w_s, N,
                                                         K, c, out == FP8Q_OUT_BF16, (int)mode,
                                                         stream),
                          stream);
}

}  // extern "C"
