// Two-pass form of the shard step, for the features that need a whole-model
// quantity before any state may change: global-norm gradient clipping and
// fp16 dynamic loss scaling (the gradient_clipping and fp16 settings of the
// DeepSpeed config in "Почему training 70B модели требует optimizer sharding
// (ZeRO-3)?", §8).
//
//  pass 1 (reduce_kernel)   g = (rank-ordered sum / N) * (1 / loss scale), from
//          bf16 or fp16 replicas; g is written to an fp32 workspace and its
//          squared norm is summed in double, one partial per 2048-parameter
//          tile, then the partials in a fixed two-stage order
//          (finalize_partial_kernel, finalize_kernel).  The result does not
//          depend on the launch size.
//  pass 2 (gbar_kernel)     reads the global squared norm from device memory:
//          if it is not finite the step is skipped (nothing is written);
//          otherwise k = f32(min(1, max_norm / (sqrt(norm^2) + 1e-6))) (k = 1
//          without clipping) and the AdamW update runs on g * k, writing the
//          working copy as bf16 or fp16.
//
// Bytes per parameter: pass 1 reads 2N and writes 4; pass 2 reads 4 + 12 and
// writes 12 + 2: (2N + 34) in all, against (2N + 26) for the fused step.
#include <atomic>

#include "zs_device.h"
#include "zs_phased.h"
#include "zs_twopass.h"

namespace zs {
namespace {

using namespace dev;

constexpr int kTile = kBlock * 8;  // parameters per tile

// Fixed-order block sum of one double per thread: butterfly within each wave,
// then the waves' sums in wave order.  Every thread gets the result.
__device__ __forceinline__ double block_sum(double x, double* lds4) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  if ((threadIdx.x & 63) == 0) lds4[threadIdx.x >> 6] = x;
  __syncthreads();
  const double r = (lds4[0] + lds4[1]) + (lds4[2] + lds4[3]);
  __syncthreads();
  return r;
}

template <int NT>
struct ReduceArgs {
  const uint16_t* g[NT > 0 ? NT : ZS_MAX_REPLICAS];
  float* gbar;
  double* partials;  // ntiles + 1 slots; the last one holds the head elements
  int64_t n;
  int64_t head;      // elements before the first tile (alignment peel)
  int64_t ntiles;    // tiles of kTile parameters starting at `head` (the last may be partial)
  int32_t scalar_only;
  int32_t n_rep;
  float inv_scale;   // f32(1 / loss scale)
  const double* scale_dev;  // if set: the loss scale in device memory (inv_scale is then unused)
  // reduce_kernel's tiles in this launch, [t_lo, t_hi); head = 1 when it also
  // takes the head elements (the windowed kernel covers every tile)
  int64_t t_lo, t_hi;
  int32_t head_here;
};

// f32(1 / loss scale): from the kernel argument, or from device memory (the
// same double divide, rounded once, as the host form).
template <int NT>
__device__ __forceinline__ float unscale_factor(const ReduceArgs<NT>& a) {
  return a.scale_dev ? (float)(1.0 / *a.scale_dev) : a.inv_scale;
}

// g of element i through the per-element path.
template <int FMT, class GP>
__device__ __forceinline__ float elem_mean(GP G, int N, int64_t i, float inv) {
  float acc = h_one<FMT>(G(0)[i]);
  for (int r = 1; r < N; ++r) acc = acc + h_one<FMT>(G(r)[i]);
  return (acc / (float)N) * inv;
}

// The tile at e0 element by element (a partial tile, or a shard without a
// common alignment): thread t takes elements e0 + 8t .. e0 + 8t + 7; returns
// the thread's sum of squares.
template <int FMT, class GP>
__device__ __forceinline__ double elem_tile(GP G0, int N, int64_t e0, int64_t n, float inv, float* gbar) {
  double sq = 0.0;
  const int64_t lo = e0 + 8 * (int64_t)threadIdx.x;
  for (int k = 0; k < 8; ++k) {
    const int64_t i = lo + k;
    if (i < n && i < e0 + kTile) {
      const float g = elem_mean<FMT>(G0, N, i, inv);
      gbar[i] = g;
      sq += (double)g * (double)g;
    }
  }
  return sq;
}

// The head elements (before the first tile) and their partial, slot ntiles.
template <int NT, int FMT, class GP>
__device__ __forceinline__ void head_partial(const ReduceArgs<NT>& a, GP G0, int N, float inv, double* lds4) {
  double sq = 0.0;
  if (threadIdx.x < a.head) {
    const float g = elem_mean<FMT>(G0, N, threadIdx.x, inv);
    a.gbar[threadIdx.x] = g;
    sq = (double)g * (double)g;
  }
  sq = block_sum(sq, lds4);
  if (threadIdx.x == 0) a.partials[a.ntiles] = sq;
}

template <int NT, int FMT>
__global__ __launch_bounds__(kBlock) void reduce_kernel(const ReduceArgs<NT> a) {
  __shared__ double lds4[4];
  const int N = NT > 0 ? NT : a.n_rep;
  Scalars c{};
  c.n_rep = N;
  const float inv = unscale_factor(a);
  auto G0 = [&](int r) { return a.g[r]; };
  for (int64_t t = a.t_lo + blockIdx.x; t < a.t_hi; t += gridDim.x) {
    const int64_t e0 = a.head + t * kTile;
    double sq = 0.0;
    if (!a.scalar_only && e0 + kTile <= a.n) {
      // full tile, whole-line layout
      auto G = [&](int r) { return tile_base(G0(r) + e0); };
      const uint32_t e = Layout::first();
      float acc[8];
      reduce_replicas<NT, FMT>(G, N, e, acc);
      float g[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) g[k] = mean_of<NT>(acc[k], c) * inv;
      GLB f32x4* O = (GLB f32x4*)at(tile_base(a.gbar + e0), here(e) * 4u);
      st_g(O, (f32x4){g[0], g[1], g[2], g[3]});
      st_g(O + Layout::kSecond / 4, (f32x4){g[4], g[5], g[6], g[7]});
#pragma unroll
      for (int k = 0; k < 8; ++k) sq += (double)g[k] * (double)g[k];
    } else {
      // partial tile, or a shard without a common alignment: element by element
      sq = elem_tile<FMT>(G0, N, e0, a.n, inv, a.gbar);
    }
    sq = block_sum(sq, lds4);
    if (threadIdx.x == 0) a.partials[t] = sq;
  }
  if (a.head_here && blockIdx.x == 0) head_partial<NT, FMT>(a, G0, N, inv, lds4);
}

// Pass 1 with its mean-gradient writes grouped in device-clock windows, as
// the windowed flat step groups its write-back (see flat_window_kernel):
// persistent workgroups hold the means of up to kHeldMeans finished tiles
// per wave and store them while the window is open, issuing no loads then.
// The norm partials are the same per-tile fixed-order sums as reduce_kernel's
// (written as each tile finishes: 8 bytes per 2048 parameters), so the
// norm, like the means, is the same bits.  Full tiles only in the loop; the
// partial tile and the head follow, unwindowed.
template <int NT, int FMT>
__global__ __launch_bounds__(kBlock) void reduce_window_kernel(const ReduceArgs<NT> a, const WriteWindow w) {
  __shared__ double lds4[4];
  const int N = NT > 0 ? NT : a.n_rep;
  Scalars c{};
  c.n_rep = N;
  const float inv = unscale_factor(a);
  auto G0 = [&](int r) { return a.g[r]; };
  const int64_t full = (a.n - a.head) / kTile;  // whole tiles (the shard has a common alignment)
  const uint32_t e = Layout::first();
  HeldMeans<kHeldMeans> held;
  auto check = [&]() { held.check(a.gbar, w); };
  for (int64_t t = blockIdx.x; t < full; t += gridDim.x) {
    const int64_t e0 = a.head + t * kTile;
    auto G = [&](int r) { return tile_base(G0(r) + e0); };
    float acc[8];
    if constexpr (NT > 0)
      reduce_replicas_hooked<NT, kWindowChecks, FMT>(G, e, acc, check);
    else
      reduce_replicas_hooked_rt<FMT>(G, N, e, acc, check);
    float g[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) g[k] = mean_of<NT>(acc[k], c) * inv;
    double sq = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) sq += (double)g[k] * (double)g[k];
    held.push(a.gbar, e0, (f32x4){g[0], g[1], g[2], g[3]}, (f32x4){g[4], g[5], g[6], g[7]});
    sq = block_sum(sq, lds4);
    if (threadIdx.x == 0) a.partials[t] = sq;
  }
  held.flush(a.gbar);
  if (blockIdx.x == gridDim.x - 1) {
    for (int64_t t = full; t < a.ntiles; ++t) {
      double sq = elem_tile<FMT>(G0, N, a.head + t * kTile, a.n, inv, a.gbar);
      sq = block_sum(sq, lds4);
      if (threadIdx.x == 0) a.partials[t] = sq;
    }
  }
  if (blockIdx.x == 0) head_partial<NT, FMT>(a, G0, N, inv, lds4);
}

// One super-chunk of pass 1 on the phased schedule: slot k of the wave is
// wave tile t0 + k*nw + gw (with PART, slots 0..kk-1); `c` numbers the grid
// barrier.
template <int NT, int FMT, bool PART>
__device__ __forceinline__ void reduce_super_chunk(const ReduceArgs<NT>& a, int N, const Scalars& c, float inv,
                                                   int64_t t0, int64_t nw, int64_t gw, int wave, uint32_t e,
                                                   uint32_t* counter, int64_t cnum, int32_t max_polls,
                                                   double (&wsum)[kReducePhasedTiles][kPhasedWaves], int kk,
                                                   f32x4 (*la)[2][64]) {
  constexpr int KR = kReduceRegTiles, KL = kReduceLdsTiles, K = KR + KL;
  constexpr int kQuarters = kTile / (8 * kFlatBlock);   // wave tiles per norm tile
  constexpr int kNormTiles = kPhasedWaves / kQuarters;  // per slot per workgroup
  auto gp = [&](int r) { return a.g[r]; };
  int64_t es[K];
#pragma unroll
  for (int k = 0; k < K; ++k) es[k] = a.head + 8 * kFlatBlock * (t0 + k * nw + gw);
  float acc[KR][8];
  phased_accumulate<NT, FMT, KR, KL, PART>(gp, N, es, e, acc, la, true, kk);
  phased_grid_barrier(counter, (uint32_t)cnum * gridDim.x + phased_quorum(gridDim.x), max_polls);
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (PART && k >= kk) continue;
    float g[8];
    phased_sums<KR, KL>(acc, la, k, g);
#pragma unroll
    for (int j = 0; j < 8; ++j) g[j] = mean_of<NT>(g[j], c) * inv;
    GLB f32x4* O = (GLB f32x4*)at(tile_base(a.gbar + es[k]), here(e) * 4u);
    st_g(O, (f32x4){g[0], g[1], g[2], g[3]});
    st_g(O + Layout::kSecond / 4, (f32x4){g[4], g[5], g[6], g[7]});
    double sq = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) sq += (double)g[j] * (double)g[j];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sq += __shfl_xor(sq, off, 64);
    if ((threadIdx.x & 63) == 0) wsum[k][wave] = sq;
  }
  __syncthreads();
  if (threadIdx.x < (PART ? kk : K) * kNormTiles) {
    const int k = threadIdx.x / kNormTiles, i = threadIdx.x % kNormTiles;
    const double* q = &wsum[k][kQuarters * i];
    const int64_t w0 = t0 + k * nw + (int64_t)blockIdx.x * kPhasedWaves + kQuarters * i;
    a.partials[w0 / kQuarters] = (q[0] + q[1]) + (q[2] + q[3]);
  }
  __syncthreads();
}

// Pass 1 on the phased schedule of the flat step (flat_phased_kernel): one
// workgroup of kPhasedWaves waves per compute unit; for each of `nsup` whole
// super-chunks of wave tiles (512 parameters from `head`, kReducePhasedTiles
// per wave, slot k of wave w at tile sc*per + k*waves + w), and then a part
// super-chunk of `kk` tiles per wave when kk > 0, phase A streams the
// replicas in rank order into fp32 accumulators (phased_accumulate, the flat
// step's own code; kReduceRegTiles tiles in registers, kReduceLdsTiles in the
// wave's own LDS region), the grid barrier follows, and phase B writes the
// means and the norm partials.  Pass 1's phase B writes only its 4-byte
// means, so its super-chunks pay for more of their fixed cost than the flat
// step's: the LDS tiles' longer super-chunks measured 1% faster here and no
// faster (0.4% slower) on the flat step.  A 2048-parameter norm tile is four
// consecutive wave tiles, held by four consecutive waves of one workgroup in
// the same slot: each wave forms its sum of squares as reduce_kernel's wave
// does for that quarter (per thread in element order, then the same
// butterfly), and the four are added in reduce_kernel's order, so the
// partials, and the norm, are the same bits.  reduce_kernel takes the norm
// tiles after the super-chunks and the head elements.
template <int NT, int FMT>
__global__ __launch_bounds__(kFlatBlock* kPhasedWaves) void reduce_phased_kernel(const ReduceArgs<NT> a,
                                                                                 const PhasedCtl ctl, int64_t nsup,
                                                                                 int32_t kk) {
  constexpr int kQuarters = kTile / (8 * kFlatBlock);  // wave tiles per norm tile
  static_assert(kQuarters == 4 && kPhasedWaves % kQuarters == 0, "norm tiles of whole waves of one workgroup");
  __shared__ double wsum[kReducePhasedTiles][kPhasedWaves];
  __shared__ f32x4 lds[kPhasedWaves][kReduceLdsTiles][2][64];  // the waves' accumulator tiles beyond registers
  const int N = NT > 0 ? NT : a.n_rep;
  Scalars c{};
  c.n_rep = N;
  const float inv = unscale_factor(a);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t e = 4u * (threadIdx.x & 63u);
  const int64_t nw = (int64_t)gridDim.x * kPhasedWaves;
  const int64_t gw = (int64_t)blockIdx.x * kPhasedWaves + wave;
  const int64_t per = nw * kReducePhasedTiles;
  uint32_t* counter = &g_phased_counters[32 * ctl.slot];
  for (int64_t sc = 0; sc < nsup; ++sc)
    reduce_super_chunk<NT, FMT, false>(a, N, c, inv, sc * per, nw, gw, wave, e, counter, sc, ctl.max_polls, wsum,
                                       kReducePhasedTiles, lds[wave]);
  if (kk > 0)
    reduce_super_chunk<NT, FMT, true>(a, N, c, inv, nsup * per, nw, gw, wave, e, counter, nsup, ctl.max_polls, wsum,
                                      kk, lds[wave]);
}

// First stage of the norm: workgroup b takes partials [b*kFinalSeg,
// (b+1)*kFinalSeg); thread t sums its 16 of them (t, t+256, ...) in order,
// then the fixed-order block sum.  The loads are issued together, so the
// stage costs one memory latency instead of one per partial.
__global__ __launch_bounds__(kBlock) void finalize_partial_kernel(const double* __restrict__ partials, int64_t count,
                                                                  double* __restrict__ out) {
  static_assert(kFinalSeg % kBlock == 0, "segment = whole rows of the workgroup");
  constexpr int kPer = (int)(kFinalSeg / kBlock);
  __shared__ double lds4[4];
  const int64_t lo = (int64_t)blockIdx.x * kFinalSeg + threadIdx.x;
  double v[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int64_t i = lo + (int64_t)k * kBlock;
    v[k] = i < count ? partials[i] : 0.0;
  }
  double x = 0.0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) x += v[k];
  x = block_sum(x, lds4);
  if (threadIdx.x == 0) out[blockIdx.x] = x;
}

// One workgroup: thread t sums values t, t+256, ... in order, then the
// fixed-order block sum.
__global__ __launch_bounds__(kBlock) void finalize_kernel(const double* __restrict__ partials, int64_t count,
                                                          double* __restrict__ out) {
  __shared__ double lds4[4];
  double x = 0.0;
  for (int64_t i = threadIdx.x; i < count; i += kBlock) x += partials[i];
  x = block_sum(x, lds4);
  if (threadIdx.x == 0) *out = x;
}

struct GbarArgs {
  const float* gbar;
  FlatShape s;  // master / m / v / working copy, with the common peel over all five arrays
  Scalars c;
  const double* total_sq;
  double max_norm;
  int32_t skip_nonfinite;
  StepRef r;  // table == NULL: the step of `c`
  // this launch's tiles, [t_lo, t_hi); edges = 1 when it also takes the head
  // and tail elements of a vector-path shard
  int64_t t_lo, t_hi;
  int32_t edges;
};

__device__ __forceinline__ float clip_factor(double total_sq, double max_norm) {
  if (!(max_norm > 0)) return 1.0f;
  const double q = max_norm / (__builtin_sqrt(total_sq) + 1e-6);
  return (float)(q < 1.0 ? q : 1.0);
}

template <int OFMT>
__device__ __forceinline__ void gbar_elem(const GbarArgs& a, const Scalars& c, int64_t i, float k) {
  float p = a.s.p[i], m = a.s.m[i], v = a.s.v[i];
  adam(a.gbar[i] * k, p, m, v, c);
  a.s.p[i] = p;
  a.s.m[i] = m;
  a.s.v[i] = v;
  a.s.b[i] = to_half<OFMT>(p);
}

template <int OFMT, int BLK>
__global__ __launch_bounds__(BLK) void gbar_kernel(const GbarArgs a) {
  constexpr int64_t kT = 8 * BLK;  // parameters per tile
  Scalars c = a.c;
  if (!step_scalars(a.r, c)) return;
  const double tsq = *a.total_sq;
  if (a.skip_nonfinite && !__builtin_isfinite(tsq)) return;  // overflow: the step is skipped everywhere
  const float k = clip_factor(tsq, a.max_norm);
  const FlatShape& s = a.s;
  for (int64_t t = a.t_lo + blockIdx.x; t < a.t_hi; t += gridDim.x) {
    if (!s.scalar_only && (t + 1) * BLK <= s.nvec) {
      const int64_t e0 = s.head + t * kT;
      const uint32_t e = Layout::first();
      constexpr uint32_t q2 = Layout::kSecond / 4;
      const uint32_t o = here(e) * 4u;
      const GLB f32x4* G4 = (const GLB f32x4*)at(tile_base(a.gbar + e0), o);
      const GLB f32x4* P4 = (const GLB f32x4*)at(tile_base(s.p + e0), o);
      const GLB f32x4* M4 = (const GLB f32x4*)at(tile_base(s.m + e0), o);
      const GLB f32x4* V4 = (const GLB f32x4*)at(tile_base(s.v + e0), o);
      const f32x4 ga = ld_g(G4), gb = ld_g(G4 + q2);
      const f32x4 pa = ld_g(P4), pb = ld_g(P4 + q2);
      const f32x4 ma = ld_g(M4), mb = ld_g(M4 + q2);
      const f32x4 va = ld_g(V4), vb = ld_g(V4 + q2);
      float g[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
      float p[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
      float m[8] = {ma.x, ma.y, ma.z, ma.w, mb.x, mb.y, mb.z, mb.w};
      float v[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) adam(g[j] * k, p[j], m[j], v[j], c);
      const uint32_t o2 = here(e) * 4u;
      GLB f32x4* Po = (GLB f32x4*)at(tile_base(s.p + e0), o2);
      GLB f32x4* Mo = (GLB f32x4*)at(tile_base(s.m + e0), o2);
      GLB f32x4* Vo = (GLB f32x4*)at(tile_base(s.v + e0), o2);
      st_g(Po, (f32x4){p[0], p[1], p[2], p[3]});
      st_g(Po + q2, (f32x4){p[4], p[5], p[6], p[7]});
      st_g(Mo, (f32x4){m[0], m[1], m[2], m[3]});
      st_g(Mo + q2, (f32x4){m[4], m[5], m[6], m[7]});
      st_g(Vo, (f32x4){v[0], v[1], v[2], v[3]});
      st_g(Vo + q2, (f32x4){v[4], v[5], v[6], v[7]});
      GLB u32x2* B2 = (GLB u32x2*)at(tile_base(s.b + e0), here(e) * 2u);
      st_g(B2, (u32x2){pack_half<OFMT>(p[0], p[1]), pack_half<OFMT>(p[2], p[3])});
      st_g(B2 + Layout::kSecond / 4, (u32x2){pack_half<OFMT>(p[4], p[5]), pack_half<OFMT>(p[6], p[7])});
    } else {
      // partial tile (vector shards) or any tile of a shard without common alignment
      const int64_t e0 = s.scalar_only ? t * kT : s.head + t * kT;
      const int64_t end = s.scalar_only ? s.n : s.head + 8 * s.nvec;
      const int64_t lo = e0 + 8 * (int64_t)threadIdx.x;
      for (int j = 0; j < 8; ++j)
        if (lo + j < end && lo + j < e0 + kT) gbar_elem<OFMT>(a, c, lo + j, k);
    }
  }
  if (a.edges && blockIdx.x == 0 && !s.scalar_only) {  // head and tail elements
    const int64_t tail = s.n - s.head - 8 * s.nvec;
    for (int64_t t = threadIdx.x; t < s.head + tail; t += BLK)
      gbar_elem<OFMT>(a, c, t < s.head ? t : s.head + 8 * s.nvec + (t - s.head), k);
  }
}

template <int NT, int FMT>
hipError_t go_reduce(const uint16_t* const* grads, const TwoPassShape& sh, int blocks, hipStream_t stream) {
  (void)hipGetLastError();
  if (sh.ntiles < 0) {  // empty shard: write a zero norm
    finalize_kernel<<<dim3(1), dim3(kBlock), 0, stream>>>(nullptr, 0, sh.sqnorm);
    return hipGetLastError();
  }
  ReduceArgs<NT> a;
  for (int r = 0; r < sh.n_rep; ++r) a.g[r] = grads[r];
  a.gbar = sh.gbar;
  a.partials = sh.partials;
  a.n = sh.n;
  a.head = sh.head;
  a.ntiles = sh.ntiles;
  a.scalar_only = sh.scalar_only;
  a.n_rep = sh.n_rep;
  a.inv_scale = sh.inv_scale;
  a.scale_dev = sh.scale_dev;
  a.t_lo = 0;
  a.t_hi = sh.ntiles;
  a.head_here = 1;
  bool windowed = false;
  int64_t t_first = 0;  // the first norm tile left to the one-tile kernel
  // phased: the whole super-chunks of wave tiles, when the grid fits the device (templated for 64
  // replicas; other counts take the run-time instance)
  if (sh.phased && !sh.scalar_only) {
    static std::atomic<int> cache[kMaxDevices];
    const bool t64 = NT == 64;
    int grid = t64 ? resident_grid(reduce_phased_kernel<64, FMT>, kFlatBlock * kPhasedWaves, cache)
                   : resident_grid(reduce_phased_kernel<0, FMT>, kFlatBlock * kPhasedWaves, cache);
    if (grid > 0) {
      if (blocks < grid) grid = blocks;
      const int64_t nw = (int64_t)grid * kPhasedWaves;
      const int64_t per = nw * kReducePhasedTiles;  // wave tiles per super-chunk
      const int64_t full = (sh.n - sh.head) / (8 * kFlatBlock);
      const int64_t nsup = full / per;
      const int32_t kk = phased_part_tiles(full - nsup * per, nw, kReducePhasedTiles);
      if (nsup > 0 || kk > 0) {
        (void)hipGetLastError();
        phased_clear_kernel<<<dim3(1), dim3(64), 0, stream>>>(sh.ctl.slot);
        if constexpr (NT == 64) {
          reduce_phased_kernel<64, FMT><<<dim3(grid), dim3(kFlatBlock * kPhasedWaves), 0, stream>>>(a, sh.ctl, nsup, kk);
        } else {
          ReduceArgs<0> b;
          for (int r = 0; r < sh.n_rep; ++r) b.g[r] = grads[r];
          b.gbar = a.gbar;
          b.partials = a.partials;
          b.n = a.n;
          b.head = a.head;
          b.ntiles = a.ntiles;
          b.scalar_only = a.scalar_only;
          b.n_rep = a.n_rep;
          b.inv_scale = a.inv_scale;
          b.scale_dev = a.scale_dev;
          b.t_lo = a.t_lo;
          b.t_hi = a.t_hi;
          b.head_here = a.head_here;
          reduce_phased_kernel<0, FMT><<<dim3(grid), dim3(kFlatBlock * kPhasedWaves), 0, stream>>>(b, sh.ctl, nsup, kk);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        t_first = (nsup * per + kk * nw) / 4;  // four wave tiles per norm tile
      }
    } else {
      (void)hipGetLastError();  // no occupancy figure: the one-tile kernel takes the shard
    }
  }
  // windowed: shards of many whole tiles, when a window is set
  if (!sh.phased && sh.window.period_mask != 0 && !sh.scalar_only &&
      (sh.n - sh.head) / kTile >= kReduceWindowMinTiles) {
    static std::atomic<int> cache[kMaxDevices];
    int grid = resident_grid(reduce_window_kernel<NT, FMT>, kBlock, cache);
    if (grid > 0) {
      if (blocks < grid) grid = blocks;
      (void)hipGetLastError();
      reduce_window_kernel<NT, FMT><<<dim3(grid), dim3(kBlock), 0, stream>>>(a, sh.window);
      windowed = true;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!windowed) {
    // consecutive launches of at most launch_bytes() each (2N + 4 bytes per
    // parameter); the first also takes the head elements
    const int64_t per = units_per_launch((2 * (int64_t)sh.n_rep + 4) * kTile, 1);
    int64_t lo = t_first;
    do {
      const int64_t hi = sh.ntiles - lo > per ? lo + per : sh.ntiles;
      a.t_lo = lo;
      a.t_hi = hi;
      a.head_here = lo == t_first;
      int grid = (int)(hi - lo < blocks ? hi - lo : blocks);
      if (grid < 1) grid = 1;
      (void)hipGetLastError();
      reduce_kernel<NT, FMT><<<dim3(grid), dim3(kBlock), 0, stream>>>(a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      lo = hi;
    } while (lo < sh.ntiles);
  }
  // the norm: tile partials -> one sum per kFinalSeg of them -> the total, in a fixed order
  const int64_t count = sh.ntiles + 1;
  const int64_t nb1 = (count + kFinalSeg - 1) / kFinalSeg;
  finalize_partial_kernel<<<dim3((unsigned)nb1), dim3(kBlock), 0, stream>>>(sh.partials, count, sh.partials2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  finalize_kernel<<<dim3(1), dim3(kBlock), 0, stream>>>(sh.partials2, nb1, sh.sqnorm);
  return hipGetLastError();
}

template <int FMT>
hipError_t dispatch_reduce(const uint16_t* const* grads, const TwoPassShape& sh, int blocks, hipStream_t stream) {
  switch (sh.n_rep) {
    case 1: return go_reduce<1, FMT>(grads, sh, blocks, stream);
    case 2: return go_reduce<2, FMT>(grads, sh, blocks, stream);
    case 4: return go_reduce<4, FMT>(grads, sh, blocks, stream);
    case 8: return go_reduce<8, FMT>(grads, sh, blocks, stream);
    case 16: return go_reduce<16, FMT>(grads, sh, blocks, stream);
    case 32: return go_reduce<32, FMT>(grads, sh, blocks, stream);
    case 64: return go_reduce<64, FMT>(grads, sh, blocks, stream);
    default: return go_reduce<0, FMT>(grads, sh, blocks, stream);
  }
}

}  // namespace

hipError_t launch_reduce(const uint16_t* const* grads, const TwoPassShape& sh, int grad_format, int blocks,
                         hipStream_t stream) {
  return grad_format == 1 ? dispatch_reduce<kFP16>(grads, sh, blocks, stream)
                          : dispatch_reduce<kBF16>(grads, sh, blocks, stream);
}

namespace {

// The loss-scale update of zs_loss_scaler_update, on one device thread, so an
// fp16 step needs no round trip to the host: the overflow is a non-finite
// global squared norm (the same test pass 2 uses to skip the step).
__global__ void scaler_update_kernel(zs_loss_scaler* __restrict__ s, const double* __restrict__ total_sq,
                                     int32_t* __restrict__ taken) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  const bool overflow = !__builtin_isfinite(*total_sq);
  int64_t overflows = s->overflows, clean = s->clean;
  double scale = s->scale;
  if (overflow) {
    clean = 0;
    if (overflows < s->hysteresis) ++overflows;
    if (overflows >= s->hysteresis) {
      const double half = scale / 2.0;
      scale = half < s->min_scale ? s->min_scale : half;
    }
  } else if (++clean >= s->window) {
    scale *= 2.0;
    clean = 0;
    overflows = 0;
  }
  s->scale = scale;
  s->overflows = overflows;
  s->clean = clean;
  if (taken) *taken = overflow ? 0 : 1;
}

}  // namespace

hipError_t launch_scaler_update(zs_loss_scaler* state, const double* total_sq, int32_t* taken, hipStream_t stream) {
  (void)hipGetLastError();
  scaler_update_kernel<<<dim3(1), dim3(64), 0, stream>>>(state, total_sq, taken);
  return hipGetLastError();
}

hipError_t launch_gbar(const float* gbar, const FlatShape& s, const Scalars& c, const StepRef& ref,
                       const double* total_sq, double max_norm, int skip_nonfinite, int param_format, int blocks,
                       hipStream_t stream) {
  GbarArgs a;
  a.gbar = gbar;
  a.s = s;
  a.c = c;
  a.r = ref;
  a.total_sq = total_sq;
  a.max_norm = max_norm;
  a.skip_nonfinite = skip_nonfinite;
  // one wave per workgroup, one 512-parameter tile each, as the fused step
  // (two runs in separate processes: 5.72 / 5.20 ms against 5.95 / 5.29 ms
  // for four-wave 2048-parameter tiles on the 70B/64 shard)
  constexpr int BLK = kFlatBlock;
  constexpr int64_t kT = 8 * BLK;
  const int64_t ntiles = s.scalar_only ? (s.n + kT - 1) / kT : (s.nvec + BLK - 1) / BLK;
  // consecutive launches of at most launch_bytes() each (30 bytes per
  // parameter; 1 GB unless set, kPass2LaunchBytes); the first also takes the
  // head and tail elements
  const int64_t per = units_per_launch(30 * kT, 1, kPass2LaunchBytes);
  int64_t lo = 0;
  do {
    const int64_t hi = ntiles - lo > per ? lo + per : ntiles;
    a.t_lo = lo;
    a.t_hi = hi;
    a.edges = lo == 0;
    int grid = (int)(hi - lo < blocks ? hi - lo : blocks);
    if (grid < 1) grid = 1;
    (void)hipGetLastError();
    if (param_format == 1)
      gbar_kernel<kFP16, BLK><<<dim3(grid), dim3(BLK), 0, stream>>>(a);
    else
      gbar_kernel<kBF16, BLK><<<dim3(grid), dim3(BLK), 0, stream>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    lo = hi;
  } while (lo < ntiles);
  return hipSuccess;
}

}  // namespace zs
