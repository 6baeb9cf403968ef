// Seeded synthetic inputs, device side.
//
// Shared test/bench plumbing: fills device buffers with the same numbers the
// host generator (synth_host.c) draws, so that inputs of 100+ GB never cross
// PCIe.  Same definition, written again for the device; a GPU test checks the
// two produce identical bits.  No optimizer arithmetic lives here.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t mix(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float normal_f32(uint64_t key, uint64_t i, double sigma, int absval) {
  uint64_t s = 0;
#pragma unroll
  for (uint64_t j = 0; j < 3; ++j) {
    uint64_t w = mix(key + 4u * i + j);
    s += (w & 0xFFFFu) + ((w >> 16) & 0xFFFFu) + ((w >> 32) & 0xFFFFu) + (w >> 48);
  }
  double z = ((double)(int64_t)s - 393210.0) * (1.0 / 65536.0);
  if (absval) z = fabs(z);
  return (float)(sigma * z);
}

__global__ void fill_normal_f32(uint64_t key, uint64_t offset, int64_t n, double sigma, int absval,
                                float* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n; t += stride)
    out[t] = normal_f32(key, offset + (uint64_t)t, sigma, absval);
}

__global__ void fill_normal_bf16(uint64_t key, uint64_t offset, int64_t n, double sigma, uint64_t mask_key,
                                 uint64_t mask_thresh, uint16_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n; t += stride) {
    uint64_t i = offset + (uint64_t)t;
    uint16_t h = (uint16_t)(__float_as_uint(normal_f32(key, i, sigma, 0)) >> 16);
    if (mask_thresh && mix(mask_key + 4u * i) < mask_thresh) h = 0;
    out[t] = h;
  }
}

int grid_for(int64_t n) {
  int64_t b = (n + 255) / 256;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return (int)b;
}

}  // namespace

extern "C" {

int synth_dev_fill_normal_f32(uint64_t key, uint64_t offset, int64_t n, double sigma, int absval, float* out,
                              void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(fill_normal_f32, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, key, offset, n, sigma,
                     absval, out);
  return (int)hipGetLastError();
}

int synth_dev_fill_normal_bf16(uint64_t key, uint64_t offset, int64_t n, double sigma, uint64_t mask_key,
                               uint64_t mask_thresh, uint16_t* out, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(fill_normal_bf16, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, key, offset, n, sigma,
                     mask_key, mask_thresh, out);
  return (int)hipGetLastError();
}

}  // extern "C"
