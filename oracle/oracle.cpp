// CPU oracle for one ZeRO rank's optimizer-side step.
//
// TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
// CPU-baseline leg may load this library.  The GPU library shares no code with
// it, and this file includes nothing from the GPU library.
//
// What it computes, for one rank's shard of n parameters and N data-parallel
// replicas (all arithmetic is IEEE binary32 with round-to-nearest-even, one
// rounding per operation, no fused multiply-add, evaluated in exactly the order
// written below; build with -ffp-contract=off and without -ffast-math):
//
//  1. Reduce half of the gradient reduce-scatter: the rank keeps the average of
//     the N replicas' gradients for its shard.  Averaging: "Data Parallelism
//     数据并行（二）", section 数据并行训练（DP）, gradient-synchronisation
//     equation (the sum over nodes divided by the node count; its summation
//     bound read as N terms, ranks 0..N-1).  Reduce-scatter of the grads and the
//     per-shard update: "Почему training 70B модели требует optimizer sharding
//     (ZeRO-3)?", §5, ZeRO-3 step algorithm, steps 2 and 3.  The same section of
//     the Data Parallelism page notes floating-point addition is not
//     associative, so the order is fixed: rank 0 first, then 1, ..., N-1.
//       s = f32(G_0[i]);  s = s + f32(G_r[i]) for r = 1..N-1;  g = s / N
//  2. Mixed-precision Adam with decoupled weight decay on the shard, state per
//     parameter as laid out in the Data Parallelism page's appendix (DNN 训练的
//     内存需求): fp32 master, bf16 working copy, bf16 gradient, fp32 momentum,
//     fp32 variance, 16 bytes in all.  The pages name the optimizer (AdamW,
//     betas 0.9/0.999, eps 1e-8 in the ZeRO-3 page's §8 DeepSpeed config) but
//     print no update equations; these follow Kingma & Ba, "Adam: A Method for
//     Stochastic Optimization" (2015), Algorithm 1 (bias-corrected moments,
//     eps added after the square root), with the decay of Loshchilov & Hutter,
//     "Decoupled Weight Decay Regularization" (2019), scaled by the learning
//     rate.  With scalars folded once in double and rounded once to fp32:
//       b1 = f(beta1)  c1 = f(1-beta1)  b2 = f(beta2)  c2 = f(1-beta2)  e = f(eps)
//       ss = f(lr / (1 - beta1^t))  rb = f(1 / sqrt(1 - beta2^t))  dk = f(1 - lr*wd)
//     per element:
//       m1 = b1*M + c1*g
//       v1 = b2*V + c2*(g*g)
//       d  = sqrt(v1)*rb + e
//       u  = m1 / d
//       p1 = dk*P - ss*u
//  3. bf16 re-cast of the new master (round to nearest even; NaN stays NaN):
//     the working copy the next parameter all-gather would ship (ZeRO-3 page,
//     §5, forward all-gather of every layer's shards).
//
// Two-pass form (global-norm gradient clipping and fp16 dynamic loss scaling,
// both set in the ZeRO-3 page's §8 DeepSpeed config: gradient_clipping, and the
// fp16 block with a dynamic loss scale):
//  pass 1  g_i = (s_i / N) * u, s_i the rank-ordered sum above, u = f32(1/S)
//          for loss scale S (1 when not scaling); gradients bf16 or fp16.
//          total_sq = sum over i of (double)g_i^2, in double, index order.
//  pass 2  if total_sq is not finite (overflow) the step is skipped: nothing
//          changes.  Otherwise, with c = max_norm / (sqrt(total_sq) + 1e-6) in
//          double and k = f32(min(c, 1)) (k = 1 without clipping), the update
//          above runs on g_i * k (one fp32 multiply) and writes the working copy
//          as bf16 or fp16 (round to nearest even).
//  scaler  dynamic loss scale: an overflow skips the step; the scale halves
//          (not below the minimum) on every overflow from the `hysteresis`-th
//          one counted since the budget was last restored.  The budget is
//          restored only when the scale grows: after `window` consecutive
//          clean steps the scale doubles and the count restarts.  A halving
//          does not restore it, nor does a clean step short of the window.
//          This is how DeepSpeed's dynamic loss scaler, the system whose fp16
//          block the ZeRO-3 page's §8 prints, spends its hysteresis by
//          default; the page itself does not define the knob.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

extern "C" {

typedef struct oracle_hp {
  double lr, beta1, beta2, eps, weight_decay;
} oracle_hp;

}  // extern "C"

namespace {

float widen(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

uint16_t to_bf16(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0) return 0x7FC0;  // NaN
  uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

// IEEE binary16 -> binary32 (exact).
float half_to_f32(uint16_t h) {
  const uint32_t sign = (uint32_t)(h >> 15) << 31;
  const int exp = (h >> 10) & 0x1F;
  const uint32_t man = h & 0x3FF;
  uint32_t u;
  if (exp == 0x1F) {
    u = sign | 0x7F800000u | (man << 13);  // Inf or NaN
  } else if (exp != 0) {
    u = sign | ((uint32_t)(exp - 15 + 127) << 23) | (man << 13);
  } else if (man == 0) {
    u = sign;
  } else {  // subnormal: value = man * 2^-24
    float f = (float)man * 0x1p-24f;
    std::memcpy(&u, &f, 4);
    u |= sign;
  }
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// binary32 -> binary16, round to nearest even (overflow to Inf, NaN stays NaN).
uint16_t to_f16(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return (uint16_t)(sign | 0x7E00u);  // NaN
  if (a >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u);  // rounds to >= 65520: Inf
  if (a < 0x38800000u) {                                     // below 2^-14: subnormal or zero in binary16
    // value / 2^-24, rounded to nearest even integer
    float f;
    std::memcpy(&f, &a, 4);
    const float q = f * 0x1p24f;  // exact: a power-of-two scale of a normal or subnormal binary32
    float r = std::nearbyint(q);  // default rounding mode: to nearest even
    return (uint16_t)(sign | (uint16_t)r);
  }
  // normal binary16: drop 13 mantissa bits with round to nearest even, re-bias the exponent
  const uint32_t lsb = (a >> 13) & 1u;
  const uint32_t r = (a + 0xFFFu + lsb) >> 13;  // may carry into the exponent
  return (uint16_t)(sign | (uint16_t)(r - ((uint32_t)(127 - 15) << 10)));
}

float widen_fmt(uint16_t h, int fmt) { return fmt ? half_to_f32(h) : widen(h); }

struct Folded {
  float b1, c1, b2, c2, e, ss, rb, dk;
};

Folded fold(const oracle_hp& hp, int64_t t) {
  Folded f;
  f.b1 = (float)hp.beta1;
  f.c1 = (float)(1.0 - hp.beta1);
  f.b2 = (float)hp.beta2;
  f.c2 = (float)(1.0 - hp.beta2);
  f.e = (float)hp.eps;
  f.ss = (float)(hp.lr / (1.0 - std::pow(hp.beta1, (double)t)));
  f.rb = (float)(1.0 / std::sqrt(1.0 - std::pow(hp.beta2, (double)t)));
  f.dk = (float)(1.0 - hp.lr * hp.weight_decay);
  return f;
}

float reduce_mean(const uint16_t* const* G, int32_t N, int64_t i) {
  float s = widen(G[0][i]);
  for (int32_t r = 1; r < N; ++r) s = s + widen(G[r][i]);
  return s / (float)N;
}

void step_range(const uint16_t* const* G, int32_t N, int64_t lo, int64_t hi, float* P, float* M, float* V,
                uint16_t* B, const Folded& f) {
  for (int64_t i = lo; i < hi; ++i) {
    float g = reduce_mean(G, N, i);
    float m1 = f.b1 * M[i] + f.c1 * g;
    float v1 = f.b2 * V[i] + f.c2 * (g * g);
    float d = std::sqrt(v1) * f.rb + f.e;
    float u = m1 / d;
    float p1 = f.dk * P[i] - f.ss * u;
    P[i] = p1;
    M[i] = m1;
    V[i] = v1;
    B[i] = to_bf16(p1);
  }
}

template <class F>
void parallel_ranges(int64_t n, int32_t threads, F body) {
  if (threads <= 0) threads = (int32_t)std::thread::hardware_concurrency();
  if (threads < 1) threads = 1;
  if ((int64_t)threads > n) threads = (int32_t)(n > 0 ? n : 1);
  if (threads == 1) {
    body(0, n);
    return;
  }
  std::vector<std::thread> pool;
  for (int32_t k = 0; k < threads; ++k) {
    int64_t lo = n * k / threads, hi = n * (k + 1) / threads;
    pool.emplace_back([=] { body(lo, hi); });
  }
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

// Folded fp32 scalars in the order b1, c1, b2, c2, e, ss, rb, dk.
void oracle_fold(const oracle_hp* hp, int64_t t, float* out8) {
  Folded f = fold(*hp, t);
  const float v[8] = {f.b1, f.c1, f.b2, f.c2, f.e, f.ss, f.rb, f.dk};
  std::memcpy(out8, v, sizeof v);
}

uint16_t oracle_f32_to_bf16(float x) { return to_bf16(x); }

void oracle_f32_to_bf16_array(const float* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = to_bf16(x[i]);
}

// gbar[i] = average of the N replicas' grads (step 1 only).
int oracle_reduce_mean(const uint16_t* const* G, int32_t N, int64_t n, float* gbar, int32_t threads) {
  if (N < 1 || n < 0) return 1;
  parallel_ranges(n, threads, [&](int64_t lo, int64_t hi) {
    for (int64_t i = lo; i < hi; ++i) gbar[i] = reduce_mean(G, N, i);
  });
  return 0;
}

// The whole step on a flat shard: updates P, M, V in place and writes B.
// G is an array of N pointers to n bf16 values each.  t is the 1-based index of
// this update.  Returns 0, or 1 for N < 1, n < 0 or t < 1.
int oracle_reduce_adam(const uint16_t* const* G, int32_t N, int64_t n, float* P, float* M, float* V, uint16_t* B,
                       const oracle_hp* hp, int64_t t, int32_t threads) {
  if (N < 1 || n < 0 || t < 1) return 1;
  const Folded f = fold(*hp, t);
  parallel_ranges(n, threads, [&](int64_t lo, int64_t hi) { step_range(G, N, lo, hi, P, M, V, B, f); });
  return 0;
}

// Bytes of model and optimizer state one parameter holds on its owning rank
// (the Data Parallelism page's appendix; the same 16 as the 2+2+4+4+4 of the
// Distributed-training chapter's §2): fp32 master + bf16 working copy + bf16
// gradient + fp32 momentum + fp32 variance.
uint16_t oracle_f32_to_f16(float x) { return to_f16(x); }
float oracle_f16_to_f32(uint16_t h) { return half_to_f32(h); }

void oracle_f32_to_f16_array(const float* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = to_f16(x[i]);
}

// Pass 1: gbar[i] = (s_i / N) * f32(1/loss_scale); fmt 0 = bf16 grads, 1 = fp16.
int oracle_reduce_unscale(const uint16_t* const* G, int32_t N, int64_t n, int32_t fmt, double loss_scale,
                          float* gbar, int32_t threads) {
  if (N < 1 || n < 0 || !(loss_scale > 0)) return 1;
  const float inv = (float)(1.0 / loss_scale);
  parallel_ranges(n, threads, [&](int64_t lo, int64_t hi) {
    for (int64_t i = lo; i < hi; ++i) {
      float s = widen_fmt(G[0][i], fmt);
      for (int32_t r = 1; r < N; ++r) s = s + widen_fmt(G[r][i], fmt);
      gbar[i] = (s / (float)N) * inv;
    }
  });
  return 0;
}

// Squared L2 norm of gbar: sum of (double)gbar[i]^2 in double, in index order.
double oracle_sqnorm(const float* gbar, int64_t n) {
  double acc = 0.0;
  for (int64_t i = 0; i < n; ++i) acc += (double)gbar[i] * (double)gbar[i];
  return acc;
}

// Clip coefficient: f32(min(max_norm / (sqrt(total_sq) + 1e-6), 1)); 1 when max_norm <= 0.
float oracle_clip_coef(double total_sq, double max_norm) {
  if (!(max_norm > 0)) return 1.0f;
  const double c = max_norm / (std::sqrt(total_sq) + 1e-6);
  return (float)(c < 1.0 ? c : 1.0);
}

// Pass 2: the update on g_i * coef; out_fmt 0 = bf16 working copy, 1 = fp16.
// Returns 2 (and changes nothing) when skip_nonfinite and total_sq is not finite.
int oracle_adam_from_gbar(const float* gbar, int64_t n, float* P, float* M, float* V, uint16_t* B, int32_t out_fmt,
                          const oracle_hp* hp, int64_t t, double total_sq, double max_norm, int32_t skip_nonfinite,
                          int32_t threads) {
  if (n < 0 || t < 1) return 1;
  if (skip_nonfinite && !std::isfinite(total_sq)) return 2;
  const Folded f = fold(*hp, t);
  const float k = oracle_clip_coef(total_sq, max_norm);
  parallel_ranges(n, threads, [&](int64_t lo, int64_t hi) {
    for (int64_t i = lo; i < hi; ++i) {
      const float g = gbar[i] * k;
      float m1 = f.b1 * M[i] + f.c1 * g;
      float v1 = f.b2 * V[i] + f.c2 * (g * g);
      float d = std::sqrt(v1) * f.rb + f.e;
      float u = m1 / d;
      float p1 = f.dk * P[i] - f.ss * u;
      P[i] = p1;
      M[i] = m1;
      V[i] = v1;
      B[i] = out_fmt ? to_f16(p1) : to_bf16(p1);
    }
  });
  return 0;
}

// Dynamic loss scale (fp16 training).  state: {scale, overflows since the
// budget was last restored (counted up to `hysteresis`), clean steps since the
// last overflow or growth}.  Returns 1 if the step is taken.
typedef struct oracle_scaler {
  double scale, min_scale;
  int64_t window, hysteresis, overflows, clean;
} oracle_scaler;

int oracle_scaler_update(oracle_scaler* s, int32_t overflow) {
  if (overflow) {
    s->clean = 0;
    if (s->overflows < s->hysteresis) s->overflows += 1;
    if (s->overflows >= s->hysteresis) {
      s->scale = s->scale / 2.0 < s->min_scale ? s->min_scale : s->scale / 2.0;
    }
    return 0;
  }
  s->clean += 1;
  if (s->clean >= s->window) {
    s->scale *= 2.0;
    s->clean = 0;
    s->overflows = 0;  // growth restores the budget
  }
  return 1;
}

int64_t oracle_state_bytes_per_param(void) { return 4 + 2 + 2 + 4 + 4; }

// Per-device model-state bytes when all of it is sharded over ndp ranks
// (Distributed-training chapter, §6).
double oracle_sharded_state_bytes(double psi, int32_t ndp) {
  return (double)oracle_state_bytes_per_param() * psi / (double)ndp;
}

// Bytes one step moves through memory for n parameters and N replicas: N bf16
// grads read, master/momentum/variance read and written, bf16 copy written.
int64_t oracle_step_traffic_bytes(int32_t N, int64_t n) { return (2 * (int64_t)N + 3 * 4 + 3 * 4 + 2) * n; }

}  // extern "C"
