// The phased schedule's super-chunk loop (see flat_phased_kernel in
// zs_kernels.hip), shared by the library's kernel and the benchmark's
// access-pattern probe, which replays it with its arithmetic taken out: one
// copy of the code, so the probe's pattern is the kernel's.
#pragma once

#include "zs_device.h"

namespace zs {
namespace dev {
namespace {  // each including source file (the library's, the probe's) gets its own counters

// Grid-barrier counters, one per slot, each in its own 128-byte line; a
// launch clears its slot on its stream before the kernel starts.
__device__ __align__(128) uint32_t g_phased_counters[kPhasedSlots * 32];

__global__ void phased_clear_kernel(int32_t slot) {
  if (blockIdx.x == 0 && threadIdx.x == 0)
    __hip_atomic_store(&g_phased_counters[32 * slot], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every workgroup adds one to the counter and waits (bounded) until it reads
// at least `target`.
__device__ __forceinline__ void phased_grid_barrier(uint32_t* counter, uint32_t target, int32_t max_polls) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int32_t k = 0; k < max_polls; ++k) {
      if (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) break;
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

// Workgroups whose arrival releases a grid barrier: kPhasedQuorum of the grid (all of a grid of up to 19).
__device__ __forceinline__ uint32_t phased_quorum(uint32_t grid) {
  return (grid * kPhasedQuorumPct + 99u) / 100u;
}

// Phase A of a super-chunk: replicas 0..N-1 (rank order) of a wave's
// K = KR + KL tiles (tile k from element es[k], wave-uniform; the split lane
// layout, lane offset e) into fp32 accumulators, tiles 0..KR-1 in registers
// (acc) and tiles KR..K-1 in the wave's own LDS region `la` (tile l at la[l],
// lane t's quads at la[l][0][t] and la[l][1][t]; each replica's values read,
// added in the same fp32 order and written back, so the sums are the same
// bits), one replica's K tiles in flight per wave, the workgroup's waves
// meeting at a workgroup barrier after every replica so that they read the
// same replica at about the same time.  gp(r) is replica r's gradient
// pointer (bf16 or fp16 bits per FMT).  A second
// replica buffer (replica r + 1 requested before r is added) measured no
// faster with 12 waves per compute unit; its registers go to more tiles per
// super-chunk instead.  A barrier after every replica measured 0.2-0.4%
// faster than after every two, and after every four 0.1% slower.
//  A wave with `active` false (wave-uniform) issues no loads and leaves acc
// undefined, but meets every workgroup barrier with the others.  With PART,
// only tiles 0..kk-1 (kk wave-uniform) are read; the others' accumulators are
// left undefined.  The tile loops skip the others with `continue` (the same
// tiles as a `break`): with `break` this compiler turned a tile base into a
// vector value and failed ("illegal VGPR to SGPR copy").  UNROLL unrolls the
// replica loop of a fixed replica count.
template <int NT, int FMT, int KR, int KL, bool PART = false, int UNROLL = 1, class GP>
__device__ __forceinline__ void phased_accumulate(GP gp, int N, const int64_t (&es)[KR + KL], uint32_t e,
                                                  float (&acc)[KR][8], f32x4 (*la)[2][64], bool active = true,
                                                  int kk = KR + KL) {
  constexpr int K = KR + KL;
  constexpr uint32_t q2 = Layout::kSecond / 4;
  const uint32_t lane = threadIdx.x & 63u;
  u32x2 w[K][2];
  auto load = [&](int r) {
    if (!active) return;
    const uint16_t* g = gp(r);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (PART && k >= kk) continue;
      const GLB u32x2* q = (const GLB u32x2*)at(tile_base(g + es[k]), here(e) * 2u);
      w[k][0] = ld_g(q);
      w[k][1] = ld_g(q + q2);  // the second quad: 256 elements on (64 u32x2)
    }
  };
  auto widen = [&](int k, float (&x)[8]) {
    x[0] = h_lo<FMT>(w[k][0].x);
    x[1] = h_hi<FMT>(w[k][0].x);
    x[2] = h_lo<FMT>(w[k][0].y);
    x[3] = h_hi<FMT>(w[k][0].y);
    x[4] = h_lo<FMT>(w[k][1].x);
    x[5] = h_hi<FMT>(w[k][1].x);
    x[6] = h_lo<FMT>(w[k][1].y);
    x[7] = h_hi<FMT>(w[k][1].y);
  };
  auto add = [&](bool first) {
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      if (PART && k >= kk) continue;
      float x[8];
      widen(k, x);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[k][j] = first ? x[j] : acc[k][j] + x[j];
    }
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      if (PART && k >= kk) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(acc[k][j]));
    }
    // the tiles kept in LDS: the wave's own region, so no other wave reads or writes it
#pragma unroll
    for (int l = 0; l < KL; ++l) {
      if (PART && KR + l >= kk) continue;
      float x[8];
      widen(KR + l, x);
      f32x4 a0, a1;
      if (first) {
        a0 = (f32x4){x[0], x[1], x[2], x[3]};
        a1 = (f32x4){x[4], x[5], x[6], x[7]};
      } else {
        a0 = la[l][0][lane];
        a1 = la[l][1][lane];
        a0.x = a0.x + x[0];
        a0.y = a0.y + x[1];
        a0.z = a0.z + x[2];
        a0.w = a0.w + x[3];
        a1.x = a1.x + x[4];
        a1.y = a1.y + x[5];
        a1.z = a1.z + x[6];
        a1.w = a1.w + x[7];
      }
      la[l][0][lane] = a0;
      la[l][1][lane] = a1;
    }
  };
  // replica 0 initialises the accumulators; replicas 1..N-1 are added in rank order
  load(0);
  __builtin_amdgcn_sched_barrier(0);
  add(true);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();  // keep the workgroup's waves on the same replica
  auto step = [&](int r) {
    load(r);
    __builtin_amdgcn_sched_barrier(0);
    add(false);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  };
  if constexpr (NT > 0) {
#pragma unroll UNROLL
    for (int r = 1; r < NT; ++r) step(r);
  } else {
#pragma unroll 1
    for (int r = 1; r < N; ++r) step(r);
  }
}

// Tile k's 8 rank-ordered sums of a lane after phase A: from the registers
// (k < KR) or from the wave's LDS tiles.
template <int KR, int KL>
__device__ __forceinline__ void phased_sums(const float (&acc)[KR][8], f32x4 (*la)[2][64], int k, float (&g)[8]) {
  if (k < KR) {
#pragma unroll
    for (int j = 0; j < 8; ++j) g[j] = acc[k < KR ? k : 0][j];
  } else {
    const uint32_t lane = threadIdx.x & 63u;
    const int l = k >= KR ? k - KR : 0;
    const f32x4 a0 = la[l][0][lane], a1 = la[l][1][lane];
    g[0] = a0.x;
    g[1] = a0.y;
    g[2] = a0.z;
    g[3] = a0.w;
    g[4] = a1.x;
    g[5] = a1.y;
    g[6] = a1.z;
    g[7] = a1.w;
  }
}

// Phase B's state loads of a wave's tile k: master, m and v at element es[k].
template <int K>
__device__ __forceinline__ void phased_state_load(const FlatShape& s, const int64_t (&es)[K], int k, uint32_t e,
                                                  f32x4 (&q)[6]) {
  constexpr uint32_t q2 = Layout::kSecond / 4;
  const uint32_t o = here(e) * 4u;
  const GLB f32x4* P4 = (const GLB f32x4*)at(tile_base(s.p + es[k]), o);
  const GLB f32x4* M4 = (const GLB f32x4*)at(tile_base(s.m + es[k]), o);
  const GLB f32x4* V4 = (const GLB f32x4*)at(tile_base(s.v + es[k]), o);
  q[0] = ld_g(P4);
  q[1] = ld_g(P4 + q2);
  q[2] = ld_g(M4);
  q[3] = ld_g(M4 + q2);
  q[4] = ld_g(V4);
  q[5] = ld_g(V4 + q2);
}

// Phase B after the grid barrier, tile by tile with the next tile's state in
// flight (tile 0's state already requested into st[0]): upd(acc, p, m, v)
// turns a lane's 8 rank-ordered replica sums and its 8 master, m and v values
// into the new master, m and v, and the four outputs are stored.  With PART,
// tiles 0..kk-1 only.
template <int KR, int KL, bool PART = false, class UPD>
__device__ __forceinline__ void phased_update(const FlatShape& s, const int64_t (&es)[KR + KL], uint32_t e,
                                              float (&acc)[KR][8], f32x4 (*la)[2][64], f32x4 (&st)[2][6],
                                              UPD&& upd, int kk = KR + KL) {
  constexpr int K = KR + KL;
  constexpr uint32_t q2 = Layout::kSecond / 4;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (PART && k >= kk) continue;
    if (k + 1 < K && (!PART || k + 1 < kk)) phased_state_load(s, es, k + 1, e, st[(k + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
    const f32x4* q = st[k & 1];
    float p[8] = {q[0].x, q[0].y, q[0].z, q[0].w, q[1].x, q[1].y, q[1].z, q[1].w};
    float m[8] = {q[2].x, q[2].y, q[2].z, q[2].w, q[3].x, q[3].y, q[3].z, q[3].w};
    float v[8] = {q[4].x, q[4].y, q[4].z, q[4].w, q[5].x, q[5].y, q[5].z, q[5].w};
    float g[8];
    phased_sums<KR, KL>(acc, la, k, g);
    upd(g, p, m, v);
    const TileOut h = tile_outputs(p, m, v);
    const uint32_t o = here(e) * 4u;
    GLB f32x4* P4 = (GLB f32x4*)at(tile_base(s.p + es[k]), o);
    GLB f32x4* M4 = (GLB f32x4*)at(tile_base(s.m + es[k]), o);
    GLB f32x4* V4 = (GLB f32x4*)at(tile_base(s.v + es[k]), o);
    st_g(P4, h.p0);
    st_g(P4 + q2, h.p1);
    st_g(M4, h.m0);
    st_g(M4 + q2, h.m1);
    st_g(V4, h.v0);
    st_g(V4 + q2, h.v1);
    GLB u32x2* B2 = (GLB u32x2*)at(tile_base(s.b + es[k]), here(e) * 2u);
    st_g(B2, h.b0);
    st_g(B2 + q2, h.b1);
  }
}

// Tiles per wave of the part super-chunk after the whole ones (of `tiles`
// tiles per wave), out of `rest` tiles left: the part runs phased only with at
// least half a super-chunk's tiles per wave (fewer keep too few loads in
// flight per compute unit; they go one tile per wave); 0 otherwise.
__device__ __host__ inline int phased_part_tiles(int64_t rest, int64_t waves, int tiles = kPhasedTiles) {
  const int64_t kk = rest / waves;
  return 2 * kk >= tiles ? (int)(kk < tiles ? kk : tiles - 1) : 0;
}

// One super-chunk of a flat shard: phase A, the grid barrier (release number
// `c` of the slot's counter), phase B.  Slot k of the wave is tile t0 + k*nw +
// gw (nw waves in the grid, gw the wave's index); with PART, slots 0..kk-1.
template <int NT, bool PART, class GP, class UPD>
__device__ __forceinline__ void phased_super_chunk(GP gp, int N, const FlatShape& s, int64_t t0, int64_t nw,
                                                   int64_t gw, uint32_t e, uint32_t* counter, int64_t c,
                                                   int32_t max_polls, UPD&& upd, int kk) {
  constexpr int KR = kPhasedTiles, KL = 0, K = KR;
  f32x4(*la)[2][64] = nullptr;  // every accumulator in registers
  int64_t es[K];
#pragma unroll
  for (int k = 0; k < K; ++k) es[k] = s.head + 8 * kFlatBlock * (t0 + k * nw + gw);
  // ---- phase A: the replicas, in rank order, into the accumulators
  float acc[KR][8];
  phased_accumulate<NT, kBF16, KR, KL, PART, 2>(gp, N, es, e, acc, la, true, kk);
  // ---- phase B: state, AdamW, outputs, tile by tile (the next tile's state in flight).  The first
  // tile's state is requested before the barrier: reads, like the stragglers' replica reads.
  f32x4 st[2][6];
  phased_state_load(s, es, 0, e, st[0]);
  // the grid barrier lets the workgroups go once kPhasedQuorum of them have arrived: waiting for the
  // last few costs more than their reads overlapping the others' writes
  phased_grid_barrier(counter, (uint32_t)c * gridDim.x + phased_quorum(gridDim.x), max_polls);
  phased_update<KR, KL, PART>(s, es, e, acc, la, st, upd, kk);
}

// The super-chunks of a flat shard (tiles of 512 parameters from element
// s.head; s.nvec 8-element groups on the vector path): the whole ones, then
// the part-super-chunk of phased_part_tiles tiles per wave.  gp(r) is
// replica r's gradient pointer (the shard's element 0); upd(acc, p, m, v)
// turns the 8 rank-ordered replica sums of a lane and its 8 master, m and v
// values into the new master, m and v.  Returns the number of whole tiles
// covered; the caller takes the rest.  Launched as one workgroup of
// kPhasedWaves waves per compute unit.
template <int NT, class GP, class UPD>
__device__ __forceinline__ int64_t phased_super_chunks(GP gp, int N, const FlatShape& s, int32_t slot,
                                                      int32_t max_polls, UPD&& upd) {
  constexpr int K = kPhasedTiles;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t e = 4u * (threadIdx.x & 63u);  // the split lane layout inside a tile
  const int64_t nw = (int64_t)gridDim.x * kPhasedWaves;
  const int64_t gw = (int64_t)blockIdx.x * kPhasedWaves + wave;
  const int64_t full = s.nvec / kFlatBlock;  // whole tiles
  const int64_t per = nw * K;                // tiles per super-chunk
  const int64_t nsup = uniform_i64(full / per);  // whole super-chunks
  uint32_t* counter = &g_phased_counters[32 * slot];
  for (int64_t c = 0; c < nsup; ++c)
    phased_super_chunk<NT, false>(gp, N, s, c * per, nw, gw, e, counter, c, max_polls, upd, K);
  const int kk = __builtin_amdgcn_readfirstlane(phased_part_tiles(full - nsup * per, nw));
  if (kk > 0) phased_super_chunk<NT, true>(gp, N, s, nsup * per, nw, gw, e, counter, nsup, max_polls, upd, kk);
  return nsup * per + kk * nw;
}

}  // namespace
}  // namespace dev
}  // namespace zs
