// Test kernels for the device's fp32 square root and division, compiled with
// libzshard's own flags (correctly rounded divide and square root, no
// contraction, fp32 denormals kept) and written the way the library's AdamW
// update writes them (__builtin_sqrtf, the / operator).  The tests compare
// every result with the host's IEEE binary32 operations.  Test
// infrastructure; not part of the library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ void sqrt_kernel(uint32_t first, int64_t n, float* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = __builtin_sqrtf(__uint_as_float(first + (uint32_t)i));
}

__global__ void div_kernel(const float* __restrict__ a, const float* __restrict__ b, int64_t n,
                           float* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) out[i] = a[i] / b[i];
}

int grid(int64_t n) {
  const int64_t g = (n + 255) / 256;
  return (int)(g < 1 ? 1 : g > 65536 ? 65536 : g);
}

}  // namespace

extern "C" {

// out[i] = sqrt(float with encoding first + i), i < n; first + n must not pass 2^32.
__attribute__((visibility("default"))) int zs_devmath_sqrt(uint32_t first, int64_t n, float* out, void* stream) {
  if (n < 0 || !out || (uint64_t)first + (uint64_t)n > (1ull << 32)) return 1;
  if (n == 0) return 0;
  sqrt_kernel<<<dim3(grid(n)), dim3(256), 0, (hipStream_t)stream>>>(first, n, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// out[i] = a[i] / b[i], i < n.
__attribute__((visibility("default"))) int zs_devmath_div(const float* a, const float* b, int64_t n, float* out,
                                                          void* stream) {
  if (n < 0 || (n > 0 && (!a || !b || !out))) return 1;
  if (n == 0) return 0;
  div_kernel<<<dim3(grid(n)), dim3(256), 0, (hipStream_t)stream>>>(a, b, n, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
