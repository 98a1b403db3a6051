// Streaming-bandwidth probe (measurement support, not part of the method): the
// ceiling the HBM-bound quantizers are judged against at their own sizes, and
// the known-size kernel that calibrates the FETCH_SIZE / WRITE_SIZE counters.
// Built into libfp8q_probe.so; bench.py --copy-probe calls it.
//
// ratio 1: dst[i] = src[i], 16 bytes per lane (a plain copy);
// ratio 2: 16 bytes read, 8 written per lane (the quantizers' 2:1 traffic,
//          BF16 in, one code byte out).  Non-temporal loads and stores, a
//          grid-stride loop over 16-byte pieces.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(256) void copy_kernel(const v4u* __restrict__ src, v4u* __restrict__ dst,
                                                   int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(256) void halve_kernel(const v4u* __restrict__ src, v2u* __restrict__ dst,
                                                    int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const v4u v = __builtin_nontemporal_load(src + i);
    __builtin_nontemporal_store(v2u{v[0] ^ v[2], v[1] ^ v[3]}, dst + i);
  }
}

}  // namespace

extern "C" {

// Reads src_bytes (a multiple of 16) from src and writes src_bytes / ratio to
// dst (ratio 1 or 2); device pointers, 16-byte aligned, asynchronous on
// `stream`.  Returns 0, or -1 for invalid arguments, or the HIP error code.
int fp8q_probe_stream(const void* src, void* dst, int64_t src_bytes, int ratio,
                      hipStream_t stream) {
  if (!src || !dst || src_bytes <= 0 || src_bytes % 16 || (ratio != 1 && ratio != 2) ||
      (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16)
    return -1;
  const int64_t n = src_bytes / 16;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return (int)hipGetLastError();
  int64_t blocks = (n + 255) / 256;
  const int64_t cap = (int64_t)cus * 16;  // enough resident waves to hide latency
  if (blocks > cap) blocks = cap;
  if (ratio == 1)
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const v4u*>(src), static_cast<v4u*>(dst), n);
  else
    hipLaunchKernelGGL(halve_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const v4u*>(src), static_cast<v2u*>(dst), n);
  return (int)hipGetLastError();
}

}  // extern "C"
