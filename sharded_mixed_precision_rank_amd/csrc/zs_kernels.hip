// Device kernels of libzshard: the fused reduce + AdamW + bf16 re-cast step.
//
// The step is a pure stream: per parameter it reads N bf16 gradients and the
// fp32 master/momentum/variance and writes those three back plus a bf16 copy,
// (2N + 26) bytes with no reuse, against a handful of ALU operations per byte.
// HBM bandwidth bounds it; there is no contraction, so no MFMA.  Design:
//
//  * One thread owns an 8-parameter group: one 16-byte load per replica
//    (8 bf16), two 16-byte loads/stores per fp32 array, one 16-byte bf16
//    store.  A wave touches 1 KiB contiguous per array per access, so every
//    cache line is fully used and writes never need the line's old contents.
//  * Replica pointers are wave-uniform.  For the flat call they sit in the
//    kernel-argument segment; for lists in the plan's device table.  Either
//    way they reach SGPRs through scalar loads, and each global load is SGPR
//    base + one shared VGPR offset.
//  * Replicas are accumulated in fp32 registers strictly in rank order
//    0..N-1; loads are issued in batches so that several are in flight per
//    thread without holding all N in registers.
//  * The master/momentum/variance loads are issued before the gradient
//    stream so their latency overlaps it.
//  * Every access is marked non-temporal: nothing is re-read, so nothing
//    should displace useful lines in L2 or the Infinity Cache.
//  * One wave per workgroup, one 512-parameter tile each, for flat shards and
//    list plans alike (a list plan's table names one tensor per wave tile).
//    The measurements behind this are noted at kFlatBlock.
//  * Tiles start where every array sits on a 128-byte line boundary when the
//    arrays allow it (else 64, 32 or 16 bytes), so each wave access covers
//    whole lines and no line is written in two halves by two tiles; and,
//    where the arrays allow, on a boundary of 512 of their own elements (a
//    flat shard whose arrays start elsewhere runs its first elements as a
//    shard of their own; a list tensor's groups before that point form a
//    partial tile of their own).
//  * Elements outside the aligned middle (at most 63 before it, 7 after) and
//    shards whose arrays share no common alignment go through a per-element
//    path with the identical operation sequence (same inline function), so
//    results do not depend on alignment, grid size or path.
//  * Large flat shards and list plans at N >= 48 run flat_window_kernel and
//    list_window_kernel instead: the same tiles and arithmetic, with the
//    write-back held in registers and stored in short device-clock windows,
//    so the memory system sees read-only and write-only phases instead of the
//    two interleaved (see "write windows" below).
//  * Without windows, a long shard runs as consecutive launches of at most
//    about 3 GB each (kLaunchBytes).
//
// Arithmetic: see include/zshard.h.  Built with -ffp-contract=off (no FMA
// contraction) and correctly rounded fp32 divide and sqrt; fp32 denormals are
// kept.  Division by N is a multiply by 1/N only when N is a power of two,
// where both are the same correctly rounded result.
#include <atomic>

#include "zs_device.h"
#include "zs_phased.h"

namespace zs {
namespace {

using namespace dev;

// One 8-parameter group of the whole wave tile starting at element e0
// (wave-uniform, 16-byte aligned in every array): the lane's quads at tile
// elements e and e + 256 (see Layout).  G(r) returns replica r's gradient
// pointer advanced to e0.
template <int NT, class GP>
__device__ __forceinline__ void group_step_at(GP G, int N, int64_t e0, uint32_t e, const FlatShape& s,
                                              const Scalars& c) {
  constexpr uint32_t q2 = Layout::kSecond / 4;  // second quad, in f32x4 units
  f32x4 pa, pb, ma, mb, va, vb;
  {
    const uint32_t o = here(e) * 4u;  // byte offset in fp32 arrays
    const GLB f32x4* P4 = (const GLB f32x4*)at(tile_base(s.p + e0), o);
    const GLB f32x4* M4 = (const GLB f32x4*)at(tile_base(s.m + e0), o);
    const GLB f32x4* V4 = (const GLB f32x4*)at(tile_base(s.v + e0), o);
    pa = ld_g(P4);
    pb = ld_g(P4 + q2);
    ma = ld_g(M4);
    mb = ld_g(M4 + q2);
    va = ld_g(V4);
    vb = ld_g(V4 + q2);
  }

  float acc[8];
  reduce_replicas<NT>(G, N, e, acc);

  float p[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
  float m[8] = {ma.x, ma.y, ma.z, ma.w, mb.x, mb.y, mb.z, mb.w};
  float v[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
  for (int k = 0; k < 8; ++k) adam(mean_of<NT>(acc[k], c), p[k], m[k], v[k], c);

  // addresses recomputed here so they stay SGPR base + 32-bit lane offset
  const uint32_t o = here(e) * 4u;
  GLB f32x4* P4 = (GLB f32x4*)at(tile_base(s.p + e0), o);
  GLB f32x4* M4 = (GLB f32x4*)at(tile_base(s.m + e0), o);
  GLB f32x4* V4 = (GLB f32x4*)at(tile_base(s.v + e0), o);
  st_g(P4, (f32x4){p[0], p[1], p[2], p[3]});
  st_g(P4 + q2, (f32x4){p[4], p[5], p[6], p[7]});
  st_g(M4, (f32x4){m[0], m[1], m[2], m[3]});
  st_g(M4 + q2, (f32x4){m[4], m[5], m[6], m[7]});
  st_g(V4, (f32x4){v[0], v[1], v[2], v[3]});
  st_g(V4 + q2, (f32x4){v[4], v[5], v[6], v[7]});
  GLB u32x2* B2 = (GLB u32x2*)at(tile_base(s.b + e0), here(e) * 2u);
  st_g(B2, (u32x2){pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])});
  st_g(B2 + Layout::kSecond / 4, (u32x2){pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])});
}

// The same with the lane's offset in the tile taken from the workgroup's
// layout (one tile per workgroup).
template <int NT, class GP>
__device__ __forceinline__ void group_step(GP G, int N, int64_t e0, const FlatShape& s, const Scalars& c) {
  group_step_at<NT>(G, N, e0, Layout::first(), s, c);
}

// A partial wave tile: `groups` (1..63) 8-groups from element e0, in the split
// lane layout of a whole tile (lane t holds the quads at tile elements 4t and
// 256 + 4t).  A quad past the tile's end is neither loaded nor stored (its
// lane computes on zeros there).  The loads, the rank-ordered sums and the
// update are those of group_step, so every element gets the same bits as on
// a whole tile; and each store instruction writes whole 128-byte lines except
// at the tile's end.  The contiguous layout, where two store instructions
// write alternate 16-byte pieces of every line, made each partial tile cost
// several whole ones: lists whose tensors each ended in a partial tile ran
// 1.6-2.0% behind a flat call over the same arena.
template <int NT, class GP>
__device__ __forceinline__ void partial_step(GP G, int N, int64_t e0, int64_t groups, const FlatShape& s,
                                             const Scalars& c) {
  constexpr uint32_t q2 = Layout::kSecond / 4;  // second quad, in f32x4 units
  const uint32_t t = threadIdx.x & 63u;
  const uint32_t e = 4u * t;
  const bool qa = (int64_t)t < 2 * groups, qb = (int64_t)t + 64 < 2 * groups;
  auto ldq = [&](int r) {
    const GLB u32x2* a = (const GLB u32x2*)at(G(r), here(e) * 2u);
    u32x2 x = {0u, 0u}, y = {0u, 0u};
    if (qa) x = ld_g(a);
    if (qb) y = ld_g(a + q2);
    return (u32x4){x.x, x.y, y.x, y.y};
  };
  const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
  f32x4 pa = z, pb = z, ma = z, mb = z, va = z, vb = z;
  {
    const uint32_t o = here(e) * 4u;
    const GLB f32x4* P4 = (const GLB f32x4*)at(tile_base(s.p + e0), o);
    const GLB f32x4* M4 = (const GLB f32x4*)at(tile_base(s.m + e0), o);
    const GLB f32x4* V4 = (const GLB f32x4*)at(tile_base(s.v + e0), o);
    if (qa) {
      pa = ld_g(P4);
      ma = ld_g(M4);
      va = ld_g(V4);
    }
    if (qb) {
      pb = ld_g(P4 + q2);
      mb = ld_g(M4 + q2);
      vb = ld_g(V4 + q2);
    }
  }
  float acc[8];
  widen_first<kBF16>(acc, ldq(0));
  for (int r = 1; r < N; r += kBatch) {
    u32x4 w[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (r + j < N) w[j] = ldq(r + j);
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (r + j < N) accumulate<kBF16>(acc, w[j]);
  }
  float p[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
  float m[8] = {ma.x, ma.y, ma.z, ma.w, mb.x, mb.y, mb.z, mb.w};
  float v[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
  for (int k = 0; k < 8; ++k) adam(mean_of<NT>(acc[k], c), p[k], m[k], v[k], c);
  const TileOut h = tile_outputs(p, m, v);
  const uint32_t o = here(e) * 4u;
  GLB f32x4* P4 = (GLB f32x4*)at(tile_base(s.p + e0), o);
  GLB f32x4* M4 = (GLB f32x4*)at(tile_base(s.m + e0), o);
  GLB f32x4* V4 = (GLB f32x4*)at(tile_base(s.v + e0), o);
  GLB u32x2* B2 = (GLB u32x2*)at(tile_base(s.b + e0), here(e) * 2u);
  if (qa) {
    st_g(P4, h.p0);
    st_g(M4, h.m0);
    st_g(V4, h.v0);
    st_g(B2, h.b0);
  }
  if (qb) {
    st_g(P4 + q2, h.p1);
    st_g(M4 + q2, h.m1);
    st_g(V4 + q2, h.v1);
    st_g(B2 + q2, h.b1);
  }
}

// Groups [g_begin, g_end) of a vector-path shard, one workgroup-wide tile of
// BLOCK groups at a time starting at tile index `tile0` and stepping by
// `tstep` tiles.  G0(r) returns replica r's unadvanced base pointer.  Every
// tile uses the split layout (the last, partial one through partial_step).
template <int NT, int BLOCK, class GP0>
__device__ __forceinline__ void tiles(GP0 G0, int N, int64_t g_begin, int64_t g_end, int64_t tile0, int64_t tstep,
                                      const FlatShape& s, const Scalars& c) {
  for (int64_t t = tile0;; t += tstep) {
    const int64_t gt = g_begin + t * BLOCK;  // first group of the tile
    if (gt >= g_end) break;
    const int64_t e0 = s.head + 8 * gt;
    auto G = [&](int r) { return tile_base(G0(r) + e0); };
    if (gt + BLOCK <= g_end)
      group_step<NT>(G, N, e0, s, c);
    else
      partial_step<NT>(G, N, e0, g_end - gt, s, c);
  }
}

// One element, any alignment: the same operations as group_step.
template <class GP>
__device__ __forceinline__ void elem_step(GP G, int N, int64_t i, const FlatShape& s, const Scalars& c) {
  float acc = bf_one(G(0)[i]);
  for (int r = 1; r < N; ++r) acc = acc + bf_one(G(r)[i]);
  float p = s.p[i], m = s.m[i], v = s.v[i];
  adam(mean_of<0>(acc, c), p, m, v, c);
  s.p[i] = p;
  s.m[i] = m;
  s.v[i] = v;
  s.b[i] = to_bf16(p);
}

// Head and tail elements of a vector-path shard (at most 63 + 7), spread
// over the workgroup's BLOCK threads.
template <int BLOCK, class GP>
__device__ __forceinline__ void edge_step(GP G, int N, const FlatShape& s, const Scalars& c) {
  const int64_t tail = s.n - s.head - 8 * s.nvec;
  for (int64_t t = threadIdx.x; t < s.head + tail; t += BLOCK)
    elem_step(G, N, t < s.head ? t : s.head + 8 * s.nvec + (t - s.head), s, c);
}

template <int NT>
struct FlatArgs {
  const uint16_t* g[NT > 0 ? NT : ZS_MAX_REPLICAS];
  FlatShape s;
  Scalars c;
  StepRef r;  // table == NULL: the step of `c`
  // flat_kernel's share of the shard in this launch: 8-element groups
  // [lo, hi) on the vector path (lo a multiple of a tile), elements [lo, hi)
  // on the per-element path; edges = 1 when it also takes the head and tail
  // elements.  The windowed kernel covers the whole shard and ignores them.
  int64_t lo, hi;
  int32_t edges;
};

template <int NT>
__global__ __launch_bounds__(kFlatBlock) void flat_kernel(const FlatArgs<NT> a) {
  Scalars c = a.c;
  if (!step_scalars(a.r, c)) return;
  const int N = NT > 0 ? NT : c.n_rep;
  if (!a.s.scalar_only) {
    auto G0 = [&](int r) { return a.g[r]; };
    tiles<NT, kFlatBlock>(G0, N, a.lo, a.hi, blockIdx.x, gridDim.x, a.s, c);
    auto G = [&](int r) { return a.g[r]; };
    if (a.edges && blockIdx.x == gridDim.x - 1) edge_step<kFlatBlock>(G, N, a.s, c);
  } else {
    auto G = [&](int r) { return a.g[r]; };
    const int64_t stride = (int64_t)gridDim.x * kFlatBlock;
    for (int64_t i = a.lo + (int64_t)blockIdx.x * kFlatBlock + threadIdx.x; i < a.hi; i += stride)
      elem_step(G, N, i, a.s, c);
  }
}

// ---------------------------------------------------------------- write windows
// The step's 14 bytes per parameter of write-back cost far more when they
// trickle out beside the replica read streams than when the same bytes are
// written on their own.  The windowed kernel therefore groups them in time:
// persistent one-wave workgroups keep the finished outputs of up to two tiles
// in registers and store them only while the device's 100 MHz real-time
// counter (s_memrealtime, one clock for the whole chip) is inside a short
// window that opens once per period.  While the window is open every wave
// issues no loads: it stores what it holds and sleeps until the window closes,
// so the memory system sees alternating read-only and write-only phases.  A
// wave whose two slots are full stores the older tile at once.  Which tile is
// stored when changes nothing in the results: each tile's outputs are formed
// exactly as in flat_kernel and written to its own addresses.

template <int NT>
__global__ __launch_bounds__(kFlatBlock) void flat_window_kernel(const FlatArgs<NT> a, const WriteWindow w) {
  Scalars c = a.c;
  if (!step_scalars(a.r, c)) return;
  const int N = NT > 0 ? NT : c.n_rep;
  const FlatShape& s = a.s;
  constexpr uint32_t q2 = Layout::kSecond / 4;
  const uint32_t e = Layout::first();
  const int64_t full = s.nvec / kFlatBlock;  // whole tiles
  HeldTiles held;
  auto check = [&]() { held.check(s, w); };
  for (int64_t t = blockIdx.x; t < full; t += gridDim.x) {
    const int64_t e0 = s.head + 8 * kFlatBlock * t;
    f32x4 pa, pb, ma, mb, va, vb;
    {
      const uint32_t o = here(e) * 4u;
      const GLB f32x4* P4 = (const GLB f32x4*)at(tile_base(s.p + e0), o);
      const GLB f32x4* M4 = (const GLB f32x4*)at(tile_base(s.m + e0), o);
      const GLB f32x4* V4 = (const GLB f32x4*)at(tile_base(s.v + e0), o);
      pa = ld_g(P4);
      pb = ld_g(P4 + q2);
      ma = ld_g(M4);
      mb = ld_g(M4 + q2);
      va = ld_g(V4);
      vb = ld_g(V4 + q2);
    }
    auto G = [&](int r) { return tile_base(a.g[r] + e0); };
    float acc[8];
    if constexpr (NT > 0)
      reduce_replicas_hooked<NT, kWindowChecks>(G, e, acc, check);
    else
      reduce_replicas_hooked_rt(G, N, e, acc, check);
    float p[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
    float m[8] = {ma.x, ma.y, ma.z, ma.w, mb.x, mb.y, mb.z, mb.w};
    float v[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) adam(mean_of<NT>(acc[k], c), p[k], m[k], v[k], c);
    held.push(s, e0, tile_outputs(p, m, v));
  }
  held.flush(s);
  // the one partial tile and the head and tail elements, unwindowed
  if (blockIdx.x == gridDim.x - 1) {
    const int64_t gt = full * kFlatBlock;
    const int64_t e0 = s.head + 8 * gt;
    if (gt < s.nvec) {
      auto G = [&](int r) { return tile_base(a.g[r] + e0); };
      partial_step<NT>(G, N, e0, s.nvec - gt, s, c);
    }
    auto G1 = [&](int r) { return a.g[r]; };
    edge_step<kFlatBlock>(G1, N, s, c);
  }
}

// ---------------------------------------------------------------- phased schedule
// The flat step in super-chunks of (workgroups x kPhasedWaves x kPhasedTiles)
// whole tiles.  Phase A: every wave streams replicas 0..N-1 (rank order) of
// its kPhasedTiles tiles into fp32 register accumulators, one replica's tiles
// in flight at a time; the waves of a workgroup meet at a workgroup barrier
// after every replica, and all workgroups start the phase together, so at any
// moment the chip reads one or two replica streams, each over one contiguous
// region, instead of all N interleaved (on this memory system reading 2
// streams at once runs about 9% faster than reading 64).  The workgroups then
// meet at a grid barrier, which lets them go once kPhasedQuorumPct percent of
// them have arrived.  Each super-chunk costs about 8 us beyond its bytes (the
// barrier and the phases' ramps), so the super-chunk is as large as the
// registers allow: 12 tiles per wave, 18.9M parameters on 256 compute units.
// Slot k of the grid's W waves is tiles k*W .. k*W + W - 1 in workgroup
// order, so consecutive workgroups (which the dispatcher spreads round-robin
// over the 8 XCDs) take consecutive tiles; giving each XCD a contiguous
// eighth of the slot instead ran 4.3% slower.
// Phase B: each wave reads its tiles' master, m and v, applies AdamW and
// writes master, m, v and the bf16 copy, so the super-chunk's 14 bytes per
// parameter of writes go out together instead of trickling out beside the
// replica reads.  Slot k of wave w in super-chunk c is tile
// c*T + k*W + w (T tiles per super-chunk, W waves in the grid): in phase B
// the grid walks each array in one contiguous front.  After the whole
// super-chunks, a part super-chunk of fewer tiles per wave runs phased when at
// least half a super-chunk's tiles are left (phased_part_tiles); the whole
// tiles after that go one per wave, stored as each is done, and the last
// workgroup's first wave takes the partial tile and the head and tail
// elements.
//
// The barriers only shape the timing.  Every tile's outputs are formed by the
// same operations as in flat_kernel and stored to its own addresses, so the
// results are the same bits whatever the barriers do; a workgroup waits at
// most ctl.max_polls polls at the grid barrier and then goes on, so the kernel
// ends even when not every workgroup is resident (other work on the device).

template <int NT>
__global__ __launch_bounds__(kFlatBlock* kPhasedWaves) void flat_phased_kernel(const FlatArgs<NT> a,
                                                                                const PhasedCtl ctl) {
  Scalars c = a.c;
  if (!step_scalars(a.r, c)) return;  // the same decision in every workgroup
  const int N = NT > 0 ? NT : c.n_rep;
  const FlatShape& s = a.s;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t e = 4u * (threadIdx.x & 63u);
  const int64_t nw = (int64_t)gridDim.x * kPhasedWaves;
  const int64_t gw = (int64_t)blockIdx.x * kPhasedWaves + wave;
  const int64_t full = s.nvec / kFlatBlock;  // whole tiles
  auto G0 = [&](int r) { return a.g[r]; };
  const int64_t covered = phased_super_chunks<NT>(
      G0, N, s, ctl.slot, ctl.max_polls, [&](const float(&acc)[8], float(&p)[8], float(&m)[8], float(&v)[8]) {
#pragma unroll
        for (int j = 0; j < 8; ++j) adam(mean_of<NT>(acc[j], c), p[j], m[j], v[j], c);
      });
  // the whole tiles after the last super-chunk, one at a time per wave, stored as each is done
  for (int64_t t = covered + gw; t < full; t += nw) {
    const int64_t e0 = s.head + 8 * kFlatBlock * t;
    auto G = [&](int r) { return tile_base(a.g[r] + e0); };
    group_step_at<NT>(G, N, e0, e, s, c);
  }
  // the one partial tile and the head and tail elements: the last workgroup's first wave
  if (blockIdx.x == gridDim.x - 1 && wave == 0) {
    const int64_t gt = full * kFlatBlock;
    const int64_t e1 = s.head + 8 * gt;
    if (gt < s.nvec) {
      auto G = [&](int r) { return tile_base(a.g[r] + e1); };
      partial_step<NT>(G, N, e1, s.nvec - gt, s, c);
    }
    auto G1 = [&](int r) { return a.g[r]; };
    edge_step<kFlatBlock>(G1, N, s, c);
  }
}

__global__ void step_advance_kernel(int64_t* step) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *step = *step + 1;
}

// NG sets of folded scalars: one for every tensor (NG = 1), or one per
// hyperparameter group, the group of a tensor being its descriptor's `group`.
template <int NG>
struct ListScalars {
  Scalars c[NG];
};

// A list plan's work item: one wave tile (or part of one) of one tensor.
struct ListWork {
  FlatShape s;                // the tensor (wave-uniform)
  const uint16_t* const* gp;  // its N replica pointers in the plan's table
  int64_t lo, hi;             // vector tensor: 8-groups [lo, hi); scalar-only: elements [lo, hi)
  int32_t grp;                // hyperparameter group
  bool first;                 // the tensor's first item, which also takes its head and tail elements
};

// Item i0 + it of the plan, whose tensor index is items[it]: the tensor's
// descriptor and its share of it (see ListTensor), by scalar loads.
__device__ __forceinline__ ListWork list_work(const int32_t* __restrict__ items, int64_t it, int64_t i0,
                                              const ListTensor* __restrict__ tensors,
                                              const uint16_t* const* __restrict__ gptrs, int N) {
  constexpr int64_t kGroups = kTileElemsWave / 8;
  const int32_t t = items[it];
  const ListTensor& T = tensors[t];
  ListWork w;
  w.s.p = uniform_fptr(T.p);
  w.s.m = uniform_fptr(T.m);
  w.s.v = uniform_fptr(T.v);
  w.s.b = uniform_fptr(T.b);
  w.s.n = uniform_i64(T.n);
  const int32_t hl = T.head_lead;
  w.s.head = hl & 0xFF;
  w.s.nvec = uniform_i64(T.nvec);
  w.s.scalar_only = T.scalar_only;
  w.grp = T.group;
  w.gp = gptrs + (int64_t)t * N;
  const int64_t k = i0 + it - T.item0;  // the item's place in its tensor
  w.first = k == 0;
  if (w.s.scalar_only) {
    w.lo = k * kTileElemsWave;
    w.hi = w.lo + kTileElemsWave < w.s.n ? w.lo + kTileElemsWave : w.s.n;
  } else {
    const int32_t lead = hl >> 8;
    const int64_t g = (lead > 0 ? lead - kGroups : 0) + k * kGroups;
    w.lo = g > 0 ? g : 0;
    w.hi = g + kGroups < w.s.nvec ? g + kGroups : w.s.nvec;
  }
  return w;
}

// One work item of a list plan (see list_work), by one wave of any workgroup:
// a whole tile (the split layout), a partial tile, or 512 elements of a
// scalar-only tensor, and for a tensor's first item its head and tail elements.
template <int NT>
__device__ __forceinline__ void list_item_step(const ListWork& w, int N, const Scalars& c) {
  const uint32_t lane = threadIdx.x & 63u;
  const FlatShape& s = w.s;
  auto G0 = [&](int r) { return uniform_ptr(w.gp[r]); };
  if (s.scalar_only) {
    for (int64_t i = w.lo + lane; i < w.hi; i += kFlatBlock) elem_step(G0, N, i, s, c);
    return;
  }
  const int64_t e0 = s.head + 8 * w.lo;
  auto G = [&](int r) { return tile_base(G0(r) + e0); };
  if (w.hi - w.lo == kFlatBlock)
    group_step_at<NT>(G, N, e0, 4u * lane, s, c);
  else
    partial_step<NT>(G, N, e0, w.hi - w.lo, s, c);
  if (w.first) {
    const int64_t tail = s.n - s.head - 8 * s.nvec;
    for (int64_t t = lane; t < s.head + tail; t += kFlatBlock)
      elem_step(G0, N, t < s.head ? t : s.head + 8 * s.nvec + (t - s.head), s, c);
  }
}

// The ragged-list step: one-wave workgroups, one work item each, as
// flat_kernel takes one tile: the plan's table holds one entry per wave tile
// of every tensor (its tensor's index), tensor by tensor, so every workgroup
// has work.  A vector tensor's tiles start at its tile grid's anchor, the
// groups before it forming a partial tile of their own.  The tensor's
// descriptor and replica pointers come by scalar loads from the table, so no
// LDS staging and no barrier sit between a workgroup's start and its first
// gradient load.  A scalar-only tensor's items take 512 elements each, element
// by element; a vector tensor's first item also takes its head and tail
// elements.  Every element goes through the same operations as in flat_kernel.
template <int NT, int NG>
__global__ __launch_bounds__(kFlatBlock) void list_kernel(const int32_t* __restrict__ items, int32_t n_items,
                                                           int64_t i0, const ListTensor* __restrict__ tensors,
                                                           const uint16_t* const* __restrict__ gptrs,
                                                           const ListScalars<NG> sc, const StepRef ref) {
  const int N = NT > 0 ? NT : sc.c[0].n_rep;
  Scalars one = sc.c[0];
  if constexpr (NG == 1) {
    if (!step_scalars(ref, one)) return;
  }
  for (int64_t it = blockIdx.x; it < n_items; it += gridDim.x) {
    const ListWork w = list_work(items, it, i0, tensors, gptrs, N);
    list_item_step<NT>(w, N, NG == 1 ? one : sc.c[w.grp]);
  }
}

// The list step with its write-back in device-clock windows, as
// flat_window_kernel does for a flat shard.  Persistent one-wave workgroups
// take the plan's work items (one wave tile of one tensor each; see
// list_kernel) in turn; each item's tensor descriptor and replica pointers
// come by scalar loads from the plan's table.  A full tile is held (with its
// tensor's arrays) and stored in a window; a partial tile, a tensor's head and
// tail elements and scalar-only tensors are stored at once.  Every element
// goes through the same operations as in list_kernel.
struct HeldListTiles {
  int n = 0;
  FlatShape sa, sb;  // the held tiles' tensors (arrays only)
  int64_t ea = 0, eb = 0;
  TileOut a, b;

  __device__ __forceinline__ static FlatShape arrays(const FlatShape& s) {
    FlatShape u{};
    u.p = uniform_fptr(s.p);
    u.m = uniform_fptr(s.m);
    u.v = uniform_fptr(s.v);
    u.b = uniform_fptr(s.b);
    return u;
  }
  __device__ __forceinline__ void flush() {
    if (n >= 1) store_tile(arrays(sa), uniform_i64(ea), a);
    if (n == 2) store_tile(arrays(sb), uniform_i64(eb), b);
    n = 0;
  }
  __device__ __forceinline__ void push(const FlatShape& s, int64_t e0, const TileOut& h) {
    if (n == 2) {
      store_tile(arrays(sa), uniform_i64(ea), a);
      sa = sb;
      ea = eb;
      a = b;
      sb = s;
      eb = e0;
      b = h;
    } else if (n == 1) {
      sb = s;
      eb = e0;
      b = h;
      n = 2;
    } else {
      sa = s;
      ea = e0;
      a = h;
      n = 1;
    }
  }
  __device__ __forceinline__ void check(const WriteWindow& w) {
    window_wait(w, [&]() { flush(); });
  }
};

template <int NT, int NG>
__global__ __launch_bounds__(kFlatBlock) void list_window_kernel(const int32_t* __restrict__ items, int32_t n_items,
                                                             const ListTensor* __restrict__ tensors,
                                                             const uint16_t* const* __restrict__ gptrs,
                                                             const ListScalars<NG> sc, const StepRef ref,
                                                             const WriteWindow w) {
  constexpr uint32_t q2 = Layout::kSecond / 4;
  const int N = NT > 0 ? NT : sc.c[0].n_rep;
  Scalars one = sc.c[0];
  if constexpr (NG == 1) {
    if (!step_scalars(ref, one)) return;
  }
  const uint32_t e = Layout::first();
  HeldListTiles held;
  auto check = [&]() { held.check(w); };
  for (int64_t it = blockIdx.x; it < n_items; it += gridDim.x) {
    const ListWork wk = list_work(items, it, 0, tensors, gptrs, N);
    const FlatShape& s = wk.s;
    const Scalars& c = NG == 1 ? one : sc.c[wk.grp];
    auto G0 = [&](int r) { return uniform_ptr(wk.gp[r]); };
    if (s.scalar_only) {
      for (int64_t i = wk.lo + threadIdx.x; i < wk.hi; i += kFlatBlock) elem_step(G0, N, i, s, c);
      continue;
    }
    const int64_t e0 = s.head + 8 * wk.lo;
    if (wk.hi - wk.lo == kFlatBlock) {
      f32x4 pa, pb, ma, mb, va, vb;
      {
        const uint32_t o = here(e) * 4u;
        const GLB f32x4* P4 = (const GLB f32x4*)at(tile_base(s.p + e0), o);
        const GLB f32x4* M4 = (const GLB f32x4*)at(tile_base(s.m + e0), o);
        const GLB f32x4* V4 = (const GLB f32x4*)at(tile_base(s.v + e0), o);
        pa = ld_g(P4);
        pb = ld_g(P4 + q2);
        ma = ld_g(M4);
        mb = ld_g(M4 + q2);
        va = ld_g(V4);
        vb = ld_g(V4 + q2);
      }
      auto G = [&](int r) { return tile_base(G0(r) + e0); };
      float acc[8];
      if constexpr (NT > 0)
        reduce_replicas_hooked<NT, kWindowChecks>(G, e, acc, check);
      else
        reduce_replicas_hooked_rt(G, N, e, acc, check);
      float p[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
      float m[8] = {ma.x, ma.y, ma.z, ma.w, mb.x, mb.y, mb.z, mb.w};
      float v[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) adam(mean_of<NT>(acc[k], c), p[k], m[k], v[k], c);
      held.push(s, e0, tile_outputs(p, m, v));
    } else {
      // a partial wave tile (a tensor's last, or the groups before its tile grid's anchor), stored at once
      auto G = [&](int r) { return tile_base(G0(r) + e0); };
      partial_step<NT>(G, N, e0, wk.hi - wk.lo, s, c);
    }
    if (wk.first) edge_step<kFlatBlock>(G0, N, s, c);
  }
  held.flush();
}

// List plans on the phased schedule (see flat_phased_kernel): one workgroup of
// kPhasedWaves waves per compute unit; super-chunk c gives wave w the
// kListPhasedTiles (10) consecutive items from (c*W + w)*10 (W waves in the
// grid; the per-wave descriptor leaves registers for 10 accumulator tiles,
// not the flat step's 12).  When they are whole tiles of one tensor (all but
// a few waves in a list of large tensors), the wave streams their replicas
// into its accumulators in phase A (the flat step's own code; the tensor's
// replica pointers come from the plan's table, one per lane for up to 64
// replicas, else one scalar load per replica) and updates them in phase B
// after the grid barrier.  Otherwise the wave reads
// nothing in phase A, meets the same barriers, and takes its items one at a
// time in phase B.  Items after the last whole super-chunk go one per wave.
// Every element goes through the same operations as in list_kernel.
template <int NT, int NG>
__global__ __launch_bounds__(kFlatBlock* kPhasedWaves) void list_phased_kernel(
    const int32_t* __restrict__ items, int32_t n_items, const ListTensor* __restrict__ tensors,
    const uint16_t* const* __restrict__ gptrs, const ListScalars<NG> sc, const StepRef ref, const PhasedCtl ctl) {
  constexpr int K = kListPhasedTiles;
  constexpr int64_t kGroups = kTileElemsWave / 8;
  const int N = NT > 0 ? NT : sc.c[0].n_rep;
  Scalars one = sc.c[0];
  if constexpr (NG == 1) {
    if (!step_scalars(ref, one)) return;  // the same decision in every workgroup
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t e = 4u * lane;
  const int64_t nw = (int64_t)gridDim.x * kPhasedWaves;
  const int64_t gw = (int64_t)blockIdx.x * kPhasedWaves + wave;
  const int64_t per = nw * K;
  const int64_t nsup = n_items / per;
  uint32_t* counter = &g_phased_counters[32 * ctl.slot];
  // the wave's K items of super-chunk c: their tensor, its descriptor as a shard, the first item's
  // place in it and first 8-group, and whether all K are whole tiles of that tensor
  struct Span {
    int32_t t;
    FlatShape s;
    int64_t k0, g0;
    bool whole;
  };
  auto span = [&](int64_t c) {
    Span o;
    const int64_t it0 = (c * nw + gw) * K;
    o.t = items[it0];
    const ListTensor& T = tensors[o.t];
    o.s.p = uniform_fptr(T.p);
    o.s.m = uniform_fptr(T.m);
    o.s.v = uniform_fptr(T.v);
    o.s.b = uniform_fptr(T.b);
    o.s.n = uniform_i64(T.n);
    const int32_t hl = T.head_lead;
    const int32_t lead = hl >> 8;
    o.s.head = hl & 0xFF;
    o.s.nvec = uniform_i64(T.nvec);
    o.s.scalar_only = T.scalar_only;
    o.k0 = it0 - T.item0;
    o.g0 = (lead > 0 ? lead - kGroups : 0) + o.k0 * kGroups;
    o.whole = !o.s.scalar_only && items[it0 + K - 1] == o.t && o.g0 >= 0 && o.g0 + K * kGroups <= o.s.nvec;
    return o;
  };
  for (int64_t c = 0; c < nsup; ++c) {
    const Span o = span(c);
    const FlatShape& s = o.s;
    int64_t es[K];
#pragma unroll
    for (int k = 0; k < K; ++k) es[k] = s.head + 8 * (o.g0 + k * kGroups);
    const uint16_t* const* gpt = gptrs + (int64_t)o.t * N;
    // up to 64 replicas: lane r holds replica r's pointer, one vector load per span, and each replica
    // step takes its pointer by v_readlane instead of a scalar load that its gradient loads wait on
    // (0.2-0.4% faster on the llama70b/64 list)
    uint32_t plo = 0u, phi = 0u;
    if constexpr (NT > 0 && NT <= 64) {
      if ((int)lane < N) {
        const uint64_t u = reinterpret_cast<uint64_t>(gpt[lane]);
        plo = (uint32_t)u;
        phi = (uint32_t)(u >> 32);
      }
    }
    auto gp = [&](int r) {
      if constexpr (NT > 0 && NT <= 64) {
        const uint32_t lo = __builtin_amdgcn_readlane(plo, r), hi = __builtin_amdgcn_readlane(phi, r);
        return reinterpret_cast<const uint16_t*>(((uint64_t)hi << 32) | lo);
      } else {
        return uniform_ptr(gpt[r]);
      }
    };
    float acc[K][8];
    phased_accumulate<NT, kBF16, K, 0>(gp, N, es, e, acc, nullptr, o.whole);
    f32x4 st[2][6];
    if (o.whole) phased_state_load(s, es, 0, e, st[0]);
    phased_grid_barrier(counter, (uint32_t)c * gridDim.x + phased_quorum(gridDim.x), ctl.max_polls);
    if (o.whole) {
      const Scalars& cs = NG == 1 ? one : sc.c[tensors[o.t].group];
      phased_update<K, 0>(s, es, e, acc, nullptr, st, [&](const float(&a)[8], float(&p)[8], float(&m)[8], float(&v)[8]) {
#pragma unroll
        for (int j = 0; j < 8; ++j) adam(mean_of<NT>(a[j], cs), p[j], m[j], v[j], cs);
      });
    }
  }
  // after the super-chunks: the items of the wave's spans that were not whole tiles of one tensor, one
  // at a time; the head and tail elements of a tensor whose first item led a whole span; then the items
  // after the last whole super-chunk, one per wave
  for (int64_t c = 0; c < nsup; ++c) {
    const Span o = span(c);
    if (o.whole) {
      if (o.k0 == 0) {
        const FlatShape& s = o.s;
        const uint16_t* const* gpt = gptrs + (int64_t)o.t * N;
        auto gp = [&](int r) { return uniform_ptr(gpt[r]); };
        const Scalars& cs = NG == 1 ? one : sc.c[tensors[o.t].group];
        const int64_t tail = s.n - s.head - 8 * s.nvec;
        for (int64_t i = lane; i < s.head + tail; i += kFlatBlock)
          elem_step(gp, N, i < s.head ? i : s.head + 8 * s.nvec + (i - s.head), s, cs);
      }
    } else {
      const int64_t it0 = (c * nw + gw) * K;
      for (int k = 0; k < K; ++k) {
        const ListWork w = list_work(items, it0 + k, 0, tensors, gptrs, N);
        list_item_step<NT>(w, N, NG == 1 ? one : sc.c[w.grp]);
      }
    }
  }
  for (int64_t it = nsup * per + gw; it < n_items; it += nw) {
    // the index is the wave's own (wave-uniform): say so, or the descriptor's pointers land in vector registers
    const ListWork w = list_work(items, uniform_i64(it), 0, tensors, gptrs, N);
    list_item_step<NT>(w, N, NG == 1 ? one : sc.c[w.grp]);
  }
}

// Flat-kernel grid: `blocks`, but no more workgroups than tiles.
int clamp_grid(int blocks, int64_t work) {
  int64_t need = (work + kFlatBlock - 1) / kFlatBlock;
  if (need < 1) need = 1;
  return (int)(blocks < need ? blocks : need);
}

template <int NT>
hipError_t go_phased(const uint16_t* const* grads, const FlatShape& s, const Scalars& c, const StepRef& ref,
                     int blocks, const PhasedCtl& ctl, hipStream_t stream, bool* launched) {
  static std::atomic<int> cache[kMaxDevices];
  *launched = false;
  int grid = resident_grid(flat_phased_kernel<NT>, kFlatBlock * kPhasedWaves, cache);
  if (grid <= 0) {
    (void)hipGetLastError();  // no occupancy figure: the caller takes the one-tile kernel
    return hipSuccess;
  }
  if (blocks < grid) grid = blocks;
  FlatArgs<NT> a;
  for (int r = 0; r < c.n_rep; ++r) a.g[r] = grads[r];
  a.s = s;
  a.c = c;
  a.r = ref;
  a.lo = 0;
  a.hi = s.nvec;
  a.edges = 1;
  (void)hipGetLastError();
  phased_clear_kernel<<<dim3(1), dim3(64), 0, stream>>>(ctl.slot);
  flat_phased_kernel<NT><<<dim3(grid), dim3(kFlatBlock * kPhasedWaves), 0, stream>>>(a, ctl);
  *launched = true;
  return hipGetLastError();
}

template <int NT>
hipError_t go_flat(const uint16_t* const* grads, const FlatShape& s, const Scalars& c, const StepRef& ref,
                   int blocks, FlatSchedule sched, const WriteWindow& win, const PhasedCtl& ctl,
                   hipStream_t stream) {
  FlatArgs<NT> a;
  for (int r = 0; r < c.n_rep; ++r) a.g[r] = grads[r];
  a.s = s;
  a.c = c;
  a.r = ref;
  const int64_t work = s.scalar_only ? s.n : s.nvec;  // elements, or 8-element groups
  a.lo = 0;
  a.hi = work;
  a.edges = 1;
  // phased: shards of at least one whole tile, when the grid fits the device (templated for 64
  // replicas; other counts take the run-time instance)
  if (sched == FlatSchedule::kPhased && !s.scalar_only && s.nvec / kFlatBlock >= 1) {
    bool launched = false;
    const hipError_t e = NT == 64 ? go_phased<64>(grads, s, c, ref, blocks, ctl, stream, &launched)
                                  : go_phased<0>(grads, s, c, ref, blocks, ctl, stream, &launched);
    if (launched || e != hipSuccess) return e;
  }
  // windowed: shards of many whole tiles, when a window is set
  if (sched == FlatSchedule::kWindowed && win.period_mask != 0 && !s.scalar_only &&
      s.nvec / kFlatBlock >= kWindowMinTiles) {
    static std::atomic<int> cache[kMaxDevices];
    int grid = resident_grid(flat_window_kernel<NT>, kFlatBlock, cache);
    if (grid > 0) {
      if (blocks < grid) grid = blocks;
      (void)hipGetLastError();
      flat_window_kernel<NT><<<dim3(grid), dim3(kFlatBlock), 0, stream>>>(a, win);
      return hipGetLastError();
    }
    (void)hipGetLastError();  // no occupancy figure: take the one-tile kernel
  }
  // consecutive launches of at most launch_bytes() each, whole tiles apart
  // from the last; the last also takes the head and tail elements
  const int64_t bpp = 2 * (int64_t)c.n_rep + 26;
  const int64_t per = s.scalar_only ? units_per_launch(bpp, kFlatBlock) : units_per_launch(8 * bpp, kFlatBlock);
  int64_t lo = 0;
  do {
    const int64_t hi = work - lo > per ? lo + per : work;
    a.lo = lo;
    a.hi = hi;
    a.edges = hi == work;
    (void)hipGetLastError();
    flat_kernel<NT><<<dim3(clamp_grid(blocks, hi - lo)), dim3(kFlatBlock), 0, stream>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    lo = hi;
  } while (lo < work);
  return hipSuccess;
}

template <int NT, int NG>
hipError_t go_list_window(const int32_t* items, int32_t n_items, const ListTensor* tensors,
                          const uint16_t* const* gptrs, const ListScalars<NG>& sc, const StepRef& ref, int blocks,
                          const WriteWindow& win, hipStream_t stream, bool* launched) {
  static std::atomic<int> cache[kMaxDevices];
  *launched = false;
  int grid = resident_grid(list_window_kernel<NT, NG>, kFlatBlock, cache);
  if (grid <= 0) {
    (void)hipGetLastError();  // no occupancy figure: take the one-tile kernel
    return hipSuccess;
  }
  if (blocks < grid) grid = blocks;
  (void)hipGetLastError();
  list_window_kernel<NT, NG><<<dim3(grid), dim3(kFlatBlock), 0, stream>>>(items, n_items, tensors, gptrs, sc, ref,
                                                                           win);
  *launched = true;
  return hipGetLastError();
}

template <int NT, int NG>
hipError_t go_list_phased(const int32_t* items, int32_t n_items, const ListTensor* tensors,
                          const uint16_t* const* gptrs, const ListScalars<NG>& sc, const StepRef& ref, int blocks,
                          const PhasedCtl& ctl, hipStream_t stream, bool* launched) {
  // templated for 64 replicas; other counts take the run-time instance
  constexpr int KT = NT == 64 ? 64 : 0;
  static std::atomic<int> cache[kMaxDevices];
  *launched = false;
  int grid = resident_grid(list_phased_kernel<KT, NG>, kFlatBlock * kPhasedWaves, cache);
  if (grid <= 0) {
    (void)hipGetLastError();  // no occupancy figure: the caller takes the one-tile kernel
    return hipSuccess;
  }
  if (blocks < grid) grid = blocks;
  (void)hipGetLastError();
  phased_clear_kernel<<<dim3(1), dim3(64), 0, stream>>>(ctl.slot);
  list_phased_kernel<KT, NG><<<dim3(grid), dim3(kFlatBlock * kPhasedWaves), 0, stream>>>(items, n_items, tensors,
                                                                                        gptrs, sc, ref, ctl);
  *launched = true;
  return hipGetLastError();
}

template <int NT>
hipError_t go_list(const int32_t* items, int32_t n_items, const ListTensor* tensors,
                   const uint16_t* const* gptrs, const Scalars* cs, int n_sets, const StepRef& ref, int blocks,
                   FlatSchedule sched, const WriteWindow& win, const PhasedCtl& ctl, hipStream_t stream) {
  ListScalars<1> sc1;
  ListScalars<kMaxGroups> scg;
  sc1.c[0] = cs[0];
  for (int k = 0; k < kMaxGroups; ++k) scg.c[k] = cs[k < n_sets ? k : 0];
  if (sched == FlatSchedule::kPhased) {
    bool launched = false;
    const hipError_t e =
        n_sets <= 1 ? go_list_phased<NT, 1>(items, n_items, tensors, gptrs, sc1, ref, blocks, ctl, stream, &launched)
                    : go_list_phased<NT, kMaxGroups>(items, n_items, tensors, gptrs, scg, ref, blocks, ctl, stream,
                                                     &launched);
    if (launched || e != hipSuccess) return e;
  }
  if (sched == FlatSchedule::kWindowed && win.period_mask != 0) {
    bool launched = false;
    const hipError_t e =
        n_sets <= 1
            ? go_list_window<NT, 1>(items, n_items, tensors, gptrs, sc1, ref, blocks, win, stream, &launched)
            : go_list_window<NT, kMaxGroups>(items, n_items, tensors, gptrs, scg, ref, blocks, win, stream, &launched);
    if (launched || e != hipSuccess) return e;
  }
  // consecutive launches over the item table, each at most launch_bytes()
  // (an item is at most one wave tile; every item is complete in itself, its
  // tensor's head and tail included)
  const int64_t per = units_per_launch(kTileElemsWave * (2 * (int64_t)cs[0].n_rep + 26), 1);
  for (int64_t i0 = 0; i0 < n_items; i0 += per) {
    const int32_t cnt = (int32_t)(n_items - i0 > per ? per : n_items - i0);
    const int grid = blocks < cnt ? blocks : cnt;
    (void)hipGetLastError();
    if (n_sets <= 1)
      list_kernel<NT, 1><<<dim3(grid), dim3(kFlatBlock), 0, stream>>>(items + i0, cnt, i0, tensors, gptrs, sc1, ref);
    else
      list_kernel<NT, kMaxGroups><<<dim3(grid), dim3(kFlatBlock), 0, stream>>>(items + i0, cnt, i0, tensors, gptrs,
                                                                               scg, ref);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_flat(const uint16_t* const* grads, const FlatShape& s, const Scalars& c, const StepRef& ref,
                       int blocks, FlatSchedule sched, const WriteWindow& win, const PhasedCtl& ctl,
                       hipStream_t stream) {
  switch (c.n_rep) {
    case 1: return go_flat<1>(grads, s, c, ref, blocks, sched, win, ctl, stream);
    case 2: return go_flat<2>(grads, s, c, ref, blocks, sched, win, ctl, stream);
    case 4: return go_flat<4>(grads, s, c, ref, blocks, sched, win, ctl, stream);
    case 8: return go_flat<8>(grads, s, c, ref, blocks, sched, win, ctl, stream);
    case 16: return go_flat<16>(grads, s, c, ref, blocks, sched, win, ctl, stream);
    case 32: return go_flat<32>(grads, s, c, ref, blocks, sched, win, ctl, stream);
    case 64: return go_flat<64>(grads, s, c, ref, blocks, sched, win, ctl, stream);
    default: return go_flat<0>(grads, s, c, ref, blocks, sched, win, ctl, stream);
  }
}

hipError_t launch_step_advance(int64_t* step, hipStream_t stream) {
  (void)hipGetLastError();
  step_advance_kernel<<<dim3(1), dim3(64), 0, stream>>>(step);
  return hipGetLastError();
}

hipError_t launch_list(const int32_t* items, int32_t n_items, const ListTensor* tensors,
                       const uint16_t* const* gptrs, const Scalars* cs, int n_sets, const StepRef& ref, int blocks,
                       FlatSchedule sched, const WriteWindow& win, const PhasedCtl& ctl, hipStream_t stream) {
  switch (cs[0].n_rep) {
    case 1: return go_list<1>(items, n_items, tensors, gptrs, cs, n_sets, ref, blocks, sched, win, ctl, stream);
    case 2: return go_list<2>(items, n_items, tensors, gptrs, cs, n_sets, ref, blocks, sched, win, ctl, stream);
    case 4: return go_list<4>(items, n_items, tensors, gptrs, cs, n_sets, ref, blocks, sched, win, ctl, stream);
    case 8: return go_list<8>(items, n_items, tensors, gptrs, cs, n_sets, ref, blocks, sched, win, ctl, stream);
    case 16: return go_list<16>(items, n_items, tensors, gptrs, cs, n_sets, ref, blocks, sched, win, ctl, stream);
    case 32: return go_list<32>(items, n_items, tensors, gptrs, cs, n_sets, ref, blocks, sched, win, ctl, stream);
    case 64: return go_list<64>(items, n_items, tensors, gptrs, cs, n_sets, ref, blocks, sched, win, ctl, stream);
    default: return go_list<0>(items, n_items, tensors, gptrs, cs, n_sets, ref, blocks, sched, win, ctl, stream);
  }
}

}  // namespace zs
