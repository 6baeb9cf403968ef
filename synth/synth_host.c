/*
 * Seeded synthetic inputs, host side.
 *
 * This file is shared test/bench plumbing: it draws the numbers that both the
 * CPU oracle and the GPU library consume.  It contains none of the optimizer's
 * arithmetic.  Its device twin (synth_dev.hip) implements the same generator
 * from the same definition and must produce identical bits; a GPU test checks
 * that on a prefix of every stream.
 *
 * Definition (counter-based, so any element can be drawn on its own):
 *   mix(x)        = SplitMix64 finaliser (Steele, Lea & Flood, "Fast splittable
 *                   pseudorandom number generators", OOPSLA 2014): add the
 *                   golden gamma 0x9E3779B97F4A7C15, then xor-shift-multiply
 *                   with 0xBF58476D1CE4E5B9 (>>30) and 0x94D049BB133111EB (>>27),
 *                   final xor-shift >>31.
 *   key(seed, s)  = mix(mix(seed) ^ s)
 *   word(k, i, j) = mix(k + 4*i + j)            j = 0, 1, 2
 *   normal(k, i)  = sum of the twelve 16-bit fields of word(k,i,0..2)  (an
 *                   Irwin-Hall sum, integer, exact), centred by 393210 and
 *                   scaled by 2^-16 -> z, exact in double; x = (float)(sigma*z)
 *                   with one double multiply and one round-to-nearest-even.
 *                   Mean 0, standard deviation sigma*(1-2^-32)^(1/2), bounded
 *                   by +-6 sigma.
 *   |normal|      = (float)(sigma*|z|)
 *   bf16 normal   = upper 16 bits of the float's encoding (truncation; this is
 *                   only how the inputs are drawn, not a rounding the method does)
 *   mask(k, i)    = word(k, i, 0) < threshold   (Bernoulli(threshold / 2^64))
 *   uniform(k, i) = (word(k, i, 0) >> 11) * 2^-53  in [0, 1)
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t mix(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline double irwin_hall_z(uint64_t key, uint64_t i) {
  uint64_t s = 0;
  for (uint64_t j = 0; j < 3; ++j) {
    uint64_t w = mix(key + 4u * i + j);
    s += (w & 0xFFFFu) + ((w >> 16) & 0xFFFFu) + ((w >> 32) & 0xFFFFu) + (w >> 48);
  }
  return ((double)(int64_t)s - 393210.0) * (1.0 / 65536.0);
}

static inline float normal_f32(uint64_t key, uint64_t i, double sigma, int absval) {
  double z = irwin_hall_z(key, i);
  if (absval) z = fabs(z);
  return (float)(sigma * z);
}

static inline uint16_t upper16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  return (uint16_t)(u >> 16);
}

uint64_t synth_key(uint64_t seed, uint64_t stream) { return mix(mix(seed) ^ stream); }

uint64_t synth_word(uint64_t key, uint64_t i, int j) { return mix(key + 4u * i + (uint64_t)j); }

/* out[t] = normal(key, offset + t), t in [0, n) */
void synth_normal_f32(uint64_t key, uint64_t offset, int64_t n, double sigma, int absval, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n; ++t) out[t] = normal_f32(key, offset + (uint64_t)t, sigma, absval);
}

/* out[t] = normal(key, idx[t]) */
void synth_normal_f32_at(uint64_t key, const int64_t* idx, int64_t n, double sigma, int absval, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n; ++t) out[t] = normal_f32(key, (uint64_t)idx[t], sigma, absval);
}

/* bf16 draws; when mask_thresh != 0, positions where mask(mask_key, i) holds are +0. */
void synth_normal_bf16(uint64_t key, uint64_t offset, int64_t n, double sigma, uint64_t mask_key,
                       uint64_t mask_thresh, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n; ++t) {
    uint64_t i = offset + (uint64_t)t;
    uint16_t h = upper16(normal_f32(key, i, sigma, 0));
    if (mask_thresh && mix(mask_key + 4u * i) < mask_thresh) h = 0;
    out[t] = h;
  }
}

void synth_normal_bf16_at(uint64_t key, const int64_t* idx, int64_t n, double sigma, uint64_t mask_key,
                          uint64_t mask_thresh, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n; ++t) {
    uint64_t i = (uint64_t)idx[t];
    uint16_t h = upper16(normal_f32(key, i, sigma, 0));
    if (mask_thresh && mix(mask_key + 4u * i) < mask_thresh) h = 0;
    out[t] = h;
  }
}

void synth_uniform_f64(uint64_t key, uint64_t offset, int64_t n, double* out) {
  for (int64_t t = 0; t < n; ++t) out[t] = (double)(mix(key + 4u * (offset + (uint64_t)t)) >> 11) * 0x1.0p-53;
}

int synth_abi_version(void) { return 1; }
