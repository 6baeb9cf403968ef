// Host AdamW for the optimizer-offload path: the fp32 master, momentum and
// variance live in host memory and the update runs on the CPU (ZeRO-Offload,
// named in "Почему training 70B модели требует optimizer sharding (ZeRO-3)?",
// §6 and §7, and configured in its §8 DeepSpeed example: offload_optimizer to
// the CPU with pinned memory).
//
// Same operation sequence as the GPU kernels, one IEEE binary32 rounding per
// operation and no fused multiply-add: the AVX2 path uses only vector add,
// sub, mul, div and sqrt (each correctly rounded) and is built without FMA, so
// results are bit-identical to the device update.  A scalar path covers CPUs
// without AVX2 and the tails.
#include <immintrin.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "zs_cpu_adam.h"

namespace zs {
namespace {

inline uint16_t bf16_rne(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);  // quiet NaN
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

void range_scalar(const float* g, int64_t lo, int64_t hi, float* P, float* M, float* V, uint16_t* B,
                  const HostScalars& c) {
  for (int64_t i = lo; i < hi; ++i) {
    const float gi = g[i] * c.k;
    const float m1 = c.b1 * M[i] + c.c1 * gi;
    const float v1 = c.b2 * V[i] + c.c2 * (gi * gi);
    const float d = std::sqrt(v1) * c.rb + c.e;
    const float u = m1 / d;
    const float p1 = c.dk * P[i] - c.ss * u;
    P[i] = p1;
    M[i] = m1;
    V[i] = v1;
    B[i] = bf16_rne(p1);
  }
}

__attribute__((target("avx2"))) void range_avx2(const float* g, int64_t lo, int64_t hi, float* P, float* M,
                                                 float* V, uint16_t* B, const HostScalars& c) {
  const __m256 b1 = _mm256_set1_ps(c.b1), c1 = _mm256_set1_ps(c.c1), b2 = _mm256_set1_ps(c.b2),
               c2 = _mm256_set1_ps(c.c2), e = _mm256_set1_ps(c.e), ss = _mm256_set1_ps(c.ss),
               rb = _mm256_set1_ps(c.rb), dk = _mm256_set1_ps(c.dk), kk = _mm256_set1_ps(c.k);
  const __m256i abs_mask = _mm256_set1_epi32(0x7FFFFFFF), inf = _mm256_set1_epi32(0x7F800000),
                round = _mm256_set1_epi32(0x7FFF), one = _mm256_set1_epi32(1),
                quiet = _mm256_set1_epi32(0x0040);
  // The bf16 output is write-only: stream it past the cache when it is 16-byte aligned.
  const bool stream_b = ((reinterpret_cast<uintptr_t>(B + lo) & 15) == 0);
  int64_t i = lo;
  for (; i + 8 <= hi; i += 8) {
    const __m256 gi = _mm256_mul_ps(_mm256_loadu_ps(g + i), kk);
    const __m256 m1 = _mm256_add_ps(_mm256_mul_ps(b1, _mm256_loadu_ps(M + i)), _mm256_mul_ps(c1, gi));
    const __m256 v1 =
        _mm256_add_ps(_mm256_mul_ps(b2, _mm256_loadu_ps(V + i)), _mm256_mul_ps(c2, _mm256_mul_ps(gi, gi)));
    const __m256 d = _mm256_add_ps(_mm256_mul_ps(_mm256_sqrt_ps(v1), rb), e);
    const __m256 u = _mm256_div_ps(m1, d);
    const __m256 p1 = _mm256_sub_ps(_mm256_mul_ps(dk, _mm256_loadu_ps(P + i)), _mm256_mul_ps(ss, u));
    _mm256_storeu_ps(P + i, p1);
    _mm256_storeu_ps(M + i, m1);
    _mm256_storeu_ps(V + i, v1);
    // bf16, round to nearest even; NaN -> quiet NaN
    const __m256i w = _mm256_castps_si256(p1);
    const __m256i lsb = _mm256_and_si256(_mm256_srli_epi32(w, 16), one);
    __m256i r = _mm256_srli_epi32(_mm256_add_epi32(_mm256_add_epi32(w, round), lsb), 16);
    const __m256i is_nan = _mm256_cmpgt_epi32(_mm256_and_si256(w, abs_mask), inf);
    r = _mm256_blendv_epi8(r, _mm256_or_si256(_mm256_srli_epi32(w, 16), quiet), is_nan);
    // eight 16-bit values (each < 2^16, so the unsigned-saturating pack is exact) into 16 bytes
    const __m256i packed = _mm256_permute4x64_epi64(_mm256_packus_epi32(r, r), 0x08);
    const __m128i b8 = _mm256_castsi256_si128(packed);
    if (stream_b)
      _mm_stream_si128(reinterpret_cast<__m128i*>(B + i), b8);
    else
      _mm_storeu_si128(reinterpret_cast<__m128i*>(B + i), b8);
  }
  if (stream_b) _mm_sfence();  // streamed stores are visible before the caller reads or copies B
  range_scalar(g, i, hi, P, M, V, B, c);
}

bool have_avx2() {
  static const bool yes = __builtin_cpu_supports("avx2");
  return yes;
}

}  // namespace

void cpu_adam(const float* g, int64_t n, float* P, float* M, float* V, uint16_t* B, const HostScalars& c,
              int threads) {
  if (n <= 0) return;
  if (threads < 1) threads = 1;
  const int64_t min_per_thread = 1 << 16;
  threads = (int)std::min<int64_t>(threads, std::max<int64_t>(1, n / min_per_thread));
  auto body = [&](int64_t lo, int64_t hi) {
    if (have_avx2())
      range_avx2(g, lo, hi, P, M, V, B, c);
    else
      range_scalar(g, lo, hi, P, M, V, B, c);
  };
  if (threads == 1) {
    body(0, n);
    return;
  }
  std::vector<std::thread> pool;
  pool.reserve(threads);  // may throw before any element is touched
  for (int t = 0; t < threads; ++t) {
    // 8-aligned split points keep the vector path on whole groups
    const int64_t lo = (n * t / threads) & ~int64_t(7), hi = t + 1 == threads ? n : (n * (t + 1) / threads) & ~int64_t(7);
    bool started = false;
    try {
      pool.emplace_back(body, lo, hi);
      started = true;
    } catch (...) {
    }
    if (!started) body(lo, hi);  // no thread to spare: this range runs here
  }
  for (auto& th : pool) th.join();
}

}  // namespace zs
