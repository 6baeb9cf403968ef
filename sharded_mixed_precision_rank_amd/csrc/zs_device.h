// Device helpers shared by the libzshard kernels: vector types, addressing
// in the SGPR-base + 32-bit-offset form, bf16/fp16 conversions, the lane
// layout of a tile, and the per-parameter AdamW update.
#pragma once

#include <atomic>
#include <type_traits>

#include "zs_internal.h"

namespace zs {

// Workgroups of `kernel` (launched with `block` threads) that fit on the
// current device at once: compute units x resident workgroups per unit, the
// grid of a persistent kernel.  Cached per device in `cache` (kMaxDevices
// slots, one array per kernel instance).  0 when the runtime gives no figure;
// the callers then launch their one-tile-per-workgroup kernel instead.
template <class K>
int resident_grid(K kernel, int block, std::atomic<int>* cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int g = cache[dev].load(std::memory_order_relaxed);
  if (g > 0) return g;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess) return 0;
  g = cus * per_cu;
  if (g > 0) cache[dev].store(g, std::memory_order_relaxed);
  return g;
}

namespace dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kBatch = 8;  // replica loads in flight per thread per batch


#define GLB __attribute__((address_space(1)))

// A tile's base pointer: wave-uniform, in the global address space, pinned in
// SGPRs and opaque to the optimizer.  Adding a lane's 32-bit byte offset then
// stays the SGPR-base + VGPR-offset addressing form (one offset register for
// every array) instead of being folded into a 64-bit per-lane address.
template <class T>
__device__ __forceinline__ GLB T* tile_base(T* p) {
  GLB T* q = (GLB T*)p;
  asm volatile("" : "+s"(q));
  return q;
}
// A lane's 32-bit offset re-materialised in the current basic block:
// instruction selection only recognises base + zero-extended 32-bit offset
// when the extension is visible in the block of the access, and the loop
// optimisers would otherwise hoist it out of the tile loop.
__device__ __forceinline__ uint32_t here(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
template <class T>
__device__ __forceinline__ GLB T* at(GLB T* base, uint32_t bytes) {
  return (GLB T*)((GLB char*)base + bytes);
}
template <class T>
__device__ __forceinline__ T ld_g(const GLB T* p) {
  return __builtin_nontemporal_load(p);
}
template <class T>
__device__ __forceinline__ void st_g(GLB T* p, T x) {
  __builtin_nontemporal_store(x, p);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf_one(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2 h = __builtin_convertvector((f32x2){a, b}, bf16x2);  // round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ uint16_t to_bf16(float a) { return __builtin_bit_cast(uint16_t, (__bf16)a); }

// s / N.  For the replica counts the kernels are specialised on (powers of
// two) this is a multiply by the exact reciprocal, the same correctly rounded
// result; otherwise a correctly rounded divide.
template <int NT>
__device__ __forceinline__ float mean_of(float s, const Scalars& c) {
  if constexpr (NT > 0 && (NT & (NT - 1)) == 0)
    return s * (1.0f / (float)NT);
  else
    return s / (float)c.n_rep;
}

// The per-parameter AdamW update; every path calls this one function.
__device__ __forceinline__ void adam(float g, float& p, float& m, float& v, const Scalars& c) {
  const float m1 = c.b1 * m + c.c1 * g;
  const float v1 = c.b2 * v + c.c2 * (g * g);
  const float d = __builtin_sqrtf(v1) * c.rb + c.e;
  const float u = m1 / d;
  p = c.dk * p - c.ss * u;
  m = m1;
  v = v1;
}

// The launch's scalars: the host-folded ones, or the device table's row for
// the device step.  False when that step is outside the table: the launch
// then updates nothing (every workgroup reads the same step), and one thread
// records it in *status.
__device__ __forceinline__ bool step_scalars(const StepRef& r, Scalars& c) {
  if (!r.table) return true;
  const int64_t t = *r.step;
  if (t < r.t0 || t - r.t0 >= r.count) {
    if (r.status && blockIdx.x == 0 && threadIdx.x == 0) *r.status = 1;
    return false;
  }
  const zs_folded f = r.table[t - r.t0];
  c.b1 = f.b1;
  c.c1 = f.c1;
  c.b2 = f.b2;
  c.c2 = f.c2;
  c.e = f.eps;
  c.ss = f.ss;
  c.rb = f.rb;
  c.dk = f.dk;
  return true;
}

// 16-bit storage formats of gradients and of the working copy.
constexpr int kBF16 = 0;
constexpr int kFP16 = 1;

__device__ __forceinline__ float fp16_one(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// Exact widening of the low / high 16-bit half of a packed word.
template <int FMT>
__device__ __forceinline__ float h_lo(uint32_t w) {
  if constexpr (FMT == kBF16) return bf_lo(w);
  else return fp16_one((uint16_t)(w & 0xFFFFu));
}
template <int FMT>
__device__ __forceinline__ float h_hi(uint32_t w) {
  if constexpr (FMT == kBF16) return bf_hi(w);
  else return fp16_one((uint16_t)(w >> 16));
}
template <int FMT>
__device__ __forceinline__ float h_one(uint16_t h) {
  if constexpr (FMT == kBF16) return bf_one(h);
  else return fp16_one(h);
}

// Round to nearest even into the 16-bit format; two values packed low, high.
template <int FMT>
__device__ __forceinline__ uint32_t pack_half(float a, float b) {
  if constexpr (FMT == kBF16) {
    return pack_bf16(a, b);
  } else {
    const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)a);
    const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)b);
    return lo | (hi << 16);
  }
}
template <int FMT>
__device__ __forceinline__ uint16_t to_half(float a) {
  if constexpr (FMT == kBF16) return to_bf16(a);
  else return __builtin_bit_cast(uint16_t, (_Float16)a);
}

template <int FMT = kBF16>
__device__ __forceinline__ void accumulate(float (&acc)[8], const u32x4 w) {
  acc[0] = acc[0] + h_lo<FMT>(w.x);
  acc[1] = acc[1] + h_hi<FMT>(w.x);
  acc[2] = acc[2] + h_lo<FMT>(w.y);
  acc[3] = acc[3] + h_hi<FMT>(w.y);
  acc[4] = acc[4] + h_lo<FMT>(w.z);
  acc[5] = acc[5] + h_hi<FMT>(w.z);
  acc[6] = acc[6] + h_lo<FMT>(w.w);
  acc[7] = acc[7] + h_hi<FMT>(w.w);
}

// acc = the 8 values of replica 0's group (the first term of the rank-ordered sum).
template <int FMT>
__device__ __forceinline__ void widen_first(float (&acc)[8], const u32x4 w) {
  acc[0] = h_lo<FMT>(w.x);
  acc[1] = h_hi<FMT>(w.x);
  acc[2] = h_lo<FMT>(w.y);
  acc[3] = h_hi<FMT>(w.y);
  acc[4] = h_lo<FMT>(w.z);
  acc[5] = h_hi<FMT>(w.z);
  acc[6] = h_lo<FMT>(w.w);
  acc[7] = h_hi<FMT>(w.w);
}

// A value every lane of the wave holds, moved to scalar registers.  The
// compiler computes some wave-uniform values (64-bit divisions, loads through
// a vector index) in vector registers; where one feeds an SGPR-pinned tile
// base it must be read back into scalar registers first.
__device__ __forceinline__ const uint16_t* uniform_ptr(const uint16_t* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const uint16_t*>(((uint64_t)hi << 32) | lo);
}

template <class T>
__device__ __forceinline__ T* uniform_fptr(T* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t uniform_i64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Lane layout of a wave tile (one 8-parameter group per thread): lane l of
// wave q owns the quads at tile elements 512q + 4l and 512q + 256 + 4l.  Every
// access instruction of a wave then covers whole contiguous lines: 1 KiB per
// fp32 access, 512 B per bf16 access (8 bytes per lane).  Writes in particular
// go out as full lines.  A partial tile keeps the layout, with a predicate per
// quad (partial_step).
struct Layout {
  static __device__ __forceinline__ uint32_t first() { return 512u * (threadIdx.x >> 6) + 4u * (threadIdx.x & 63u); }
  static constexpr uint32_t kSecond = 256u;  // element distance to the 2nd quad
};


// Replica r's 8 gradient values (bf16 or fp16 bits) of this lane's group.  G(r) is replica r's
// gradient pointer advanced to the tile (wave-uniform, SGPRs); `e` is the
// lane's first element in the tile.
template <class GP>
__device__ __forceinline__ u32x4 ld_grad(GP G, int r, uint32_t e) {
  const GLB u32x2* a = (const GLB u32x2*)at(G(r), here(e) * 2u);
  const u32x2 x = ld_g(a), y = ld_g(a + Layout::kSecond / 4);
  return (u32x4){x.x, x.y, y.x, y.y};
}

template <class GP>
__device__ __forceinline__ void load_batch(GP G, int r, int N, uint32_t e, u32x4 (&w)[kBatch]) {
#pragma unroll
  for (int j = 0; j < kBatch; ++j)
    if (r + j < N) w[j] = ld_grad(G, r + j, e);
}

// Adds a batch, then pins the accumulators: the sums must be formed here, not
// sunk towards their use after the last batch (which would keep every loaded
// batch live at once).
template <int FMT>
__device__ __forceinline__ void add_batch(float (&acc)[8], const u32x4 (&w)[kBatch], int r, int N) {
#pragma unroll
  for (int j = 0; j < kBatch; ++j)
    if (r + j < N) accumulate<FMT>(acc, w[j]);
#pragma unroll
  for (int k = 0; k < 8; ++k) asm volatile("" : "+v"(acc[k]));
}

// acc[k] = sum over replicas r = 0..N-1, in that order, of element k of the
// lane's group.  Replicas 1..N-1 stream in batches of kBatch loads; the next
// batch is in flight while the current one is added (two register buffers),
// and scheduling barriers stop the compiler from hoisting later batches,
// which would buy nothing but registers.
template <int NT, int FMT = kBF16, class GP>
__device__ __forceinline__ void reduce_replicas(GP G, int N, uint32_t e, float (&acc)[8]) {
  widen_first<FMT>(acc, ld_grad(G, 0, e));
  if constexpr (NT > 0) {
    constexpr int NB = (NT - 1 + kBatch - 1) / kBatch;
    u32x4 w[2][kBatch];
    if constexpr (NB > 0) load_batch(G, 1, NT, e, w[0]);
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (k + 1 < NB) load_batch(G, 1 + (k + 1) * kBatch, NT, e, w[(k + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      add_batch<FMT>(acc, w[k & 1], 1 + k * kBatch, NT);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    u32x4 wa[kBatch], wb[kBatch];
    if (N > 1) load_batch(G, 1, N, e, wa);
#pragma unroll 1
    for (int r0 = 1; r0 < N; r0 += 2 * kBatch) {
      const int r1 = r0 + kBatch, r2 = r1 + kBatch;
      if (r1 < N) load_batch(G, r1, N, e, wb);
      __builtin_amdgcn_sched_barrier(0);
      add_batch<FMT>(acc, wa, r0, N);
      __builtin_amdgcn_sched_barrier(0);
      if (r2 < N) load_batch(G, r2, N, e, wa);
      __builtin_amdgcn_sched_barrier(0);
      if (r1 < N) add_batch<FMT>(acc, wb, r1, N);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ---------------------------------------------------------------- write windows
// The finished outputs of one full tile in the split lane layout, and the
// two-slot hold of the windowed flat step (see flat_window_kernel).
struct TileOut {
  f32x4 p0, p1, m0, m1, v0, v1;
  u32x2 b0, b1;
};

__device__ __forceinline__ TileOut tile_outputs(const float (&p)[8], const float (&m)[8], const float (&v)[8]) {
  TileOut h;
  h.p0 = (f32x4){p[0], p[1], p[2], p[3]};
  h.p1 = (f32x4){p[4], p[5], p[6], p[7]};
  h.m0 = (f32x4){m[0], m[1], m[2], m[3]};
  h.m1 = (f32x4){m[4], m[5], m[6], m[7]};
  h.v0 = (f32x4){v[0], v[1], v[2], v[3]};
  h.v1 = (f32x4){v[4], v[5], v[6], v[7]};
  h.b0 = (u32x2){pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
  h.b1 = (u32x2){pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])};
  return h;
}

// Stores a full tile's outputs at tile element e0 (split layout).
__device__ __forceinline__ void store_tile(const FlatShape& s, int64_t e0, const TileOut& h) {
  constexpr uint32_t q2 = Layout::kSecond / 4;
  const uint32_t e = Layout::first();
  const uint32_t o = here(e) * 4u;
  GLB f32x4* P4 = (GLB f32x4*)at(tile_base(s.p + e0), o);
  GLB f32x4* M4 = (GLB f32x4*)at(tile_base(s.m + e0), o);
  GLB f32x4* V4 = (GLB f32x4*)at(tile_base(s.v + e0), o);
  st_g(P4, h.p0);
  st_g(P4 + q2, h.p1);
  st_g(M4, h.m0);
  st_g(M4 + q2, h.m1);
  st_g(V4, h.v0);
  st_g(V4 + q2, h.v1);
  GLB u32x2* B2 = (GLB u32x2*)at(tile_base(s.b + e0), here(e) * 2u);
  st_g(B2, h.b0);
  st_g(B2 + Layout::kSecond / 4, h.b1);
}

// The device's 100 MHz real-time counter, one clock for the whole chip.
__device__ __forceinline__ uint64_t device_clock() { return __builtin_amdgcn_s_memrealtime(); }

// If the write window is open: flush(), then sleep until the window's end.
// That end is an absolute clock value, so the wait ends once the clock passes
// it whatever the clock's resolution, and it is capped at kWindowMaxSleeps
// sleeps (more than the longest window) in any case.
template <class FLUSH>
__device__ __forceinline__ void window_wait(const WriteWindow& w, FLUSH&& flush) {
  const uint64_t now = device_clock();
  const uint64_t phase = now & w.period_mask;
  if (phase < w.open_ticks) {
    flush();
    const uint64_t end = now - phase + w.open_ticks;
    for (int k = 0; k < kWindowMaxSleeps && device_clock() < end; ++k) __builtin_amdgcn_s_sleep(2);
  }
}

// Up to two finished tiles held in registers (`a` is the older when both are
// used).  push() stores the older tile at once when both slots are full;
// check() stores everything held when the window is open and then sleeps
// until the window's end (window_wait).
struct HeldTiles {
  int n = 0;
  int64_t ea = 0, eb = 0;
  TileOut a, b;

  __device__ __forceinline__ void flush(const FlatShape& s) {
    if (n >= 1) store_tile(s, ea, a);
    if (n == 2) store_tile(s, eb, b);
    n = 0;
  }
  __device__ __forceinline__ void push(const FlatShape& s, int64_t e0, const TileOut& h) {
    if (n == 2) {
      store_tile(s, ea, a);
      a = b;
      ea = eb;
      b = h;
      eb = e0;
    } else if (n == 1) {
      b = h;
      eb = e0;
      n = 2;
    } else {
      a = h;
      ea = e0;
      n = 1;
    }
  }
  __device__ __forceinline__ void check(const FlatShape& s, const WriteWindow& w) {
    window_wait(w, [&]() { flush(s); });
  }
};

// Pass 1 of the two-pass form: the fp32 mean gradients of up to K finished
// full tiles (8 per lane, split layout) held in registers; push() stores the
// oldest at once when all K slots are used.
template <int K>
struct HeldMeans {
  int n = 0;
  int64_t e[K];
  f32x4 g0[K], g1[K];

  __device__ __forceinline__ static void store(float* gbar, int64_t e0, f32x4 a, f32x4 b) {
    const uint32_t o = here(Layout::first()) * 4u;
    GLB f32x4* O = (GLB f32x4*)at(tile_base(gbar + e0), o);
    st_g(O, a);
    st_g(O + Layout::kSecond / 4, b);
  }
  __device__ __forceinline__ void flush(float* gbar) {
#pragma unroll
    for (int i = 0; i < K; ++i)
      if (i < n) store(gbar, e[i], g0[i], g1[i]);
    n = 0;
  }
  __device__ __forceinline__ void push(float* gbar, int64_t e0, f32x4 a, f32x4 b) {
    if (n == K) {
      store(gbar, e[0], g0[0], g1[0]);
#pragma unroll
      for (int i = 0; i + 1 < K; ++i) {
        e[i] = e[i + 1];
        g0[i] = g0[i + 1];
        g1[i] = g1[i + 1];
      }
      n = K - 1;
    }
#pragma unroll
    for (int i = 0; i < K; ++i)
      if (i == n) {
        e[i] = e0;
        g0[i] = a;
        g1[i] = b;
      }
    n = n + 1;
  }
  __device__ __forceinline__ void check(float* gbar, const WriteWindow& w) {
    window_wait(w, [&]() { flush(gbar); });
  }
};

// reduce_replicas for a templated replica count on a full tile (split layout),
// calling hook() after every kBatch / CHK replica loads of the stream, at
// wave-uniform points between loads.  The windowed kernels (the flat step and
// pass 1 of the two-pass form) check the device clock there.  Same loads, same rank-ordered adds as reduce_replicas.
template <int NT, int CHK, int FMT = kBF16, class GP, class HOOK>
__device__ __forceinline__ void reduce_replicas_hooked(GP G, uint32_t e, float (&acc)[8], HOOK&& hook) {
  static_assert(NT > 0 && kBatch % CHK == 0, "templated replica count, CHK divides the batch");
  widen_first<FMT>(acc, ld_grad(G, 0, e));
  constexpr int NB = (NT - 1 + kBatch - 1) / kBatch;
  if constexpr (NB == 0) {
    hook();
  } else {
    u32x4 w[2][kBatch];
    load_batch(G, 1, NT, e, w[0]);
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (k + 1 < NB) {
        const int r0 = 1 + (k + 1) * kBatch;
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          if (r0 + j < NT) w[(k + 1) & 1][j] = ld_grad(G, r0 + j, e);
          if (CHK > 1 && (j + 1) % (kBatch / CHK) == 0 && j + 1 < kBatch) {
            __builtin_amdgcn_sched_barrier(0);
            hook();
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      hook();
      __builtin_amdgcn_sched_barrier(0);
      add_batch<FMT>(acc, w[k & 1], 1 + k * kBatch, NT);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The same for a replica count known only at run time (1 <= N): replicas
// 1..N-1 stream in double-buffered batches of kBatch as in reduce_replicas,
// with hook() after each batch's loads are issued.
template <int FMT = kBF16, class GP, class HOOK>
__device__ __forceinline__ void reduce_replicas_hooked_rt(GP G, int N, uint32_t e, float (&acc)[8], HOOK&& hook) {
  widen_first<FMT>(acc, ld_grad(G, 0, e));
  u32x4 wa[kBatch], wb[kBatch];
  if (N > 1) load_batch(G, 1, N, e, wa);
  hook();
#pragma unroll 1
  for (int r0 = 1; r0 < N; r0 += 2 * kBatch) {
    const int r1 = r0 + kBatch, r2 = r1 + kBatch;
    if (r1 < N) load_batch(G, r1, N, e, wb);
    __builtin_amdgcn_sched_barrier(0);
    hook();
    __builtin_amdgcn_sched_barrier(0);
    add_batch<FMT>(acc, wa, r0, N);
    __builtin_amdgcn_sched_barrier(0);
    if (r2 < N) load_batch(G, r2, N, e, wa);
    __builtin_amdgcn_sched_barrier(0);
    hook();
    __builtin_amdgcn_sched_barrier(0);
    if (r1 < N) add_batch<FMT>(acc, wb, r1, N);
    __builtin_amdgcn_sched_barrier(0);
  }
}

}  // namespace dev
}  // namespace zs
