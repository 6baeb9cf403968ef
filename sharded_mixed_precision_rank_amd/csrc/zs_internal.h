// Internal interface between the C-ABI front end (zs_api.cpp) and the device
// kernels of the fused step (zs_kernels.hip).  Not installed; not part of the
// ABI.  The two-pass form's interface is in zs_twopass.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/zshard.h"

namespace zs {

// Scalars of one step, folded on the host (double -> fp32 once).
struct Scalars {
  float b1, c1, b2, c2, e, ss, rb, dk;
  float inv_n;      // exactly 1/N when N is a power of two
  int32_t n_rep;    // N
  int32_t pow2;     // N is a power of two: s * inv_n is bit-identical to s / N
};

// Where a launch takes its step's folded scalars from: the host-folded
// Scalars (table == NULL), or row *step - t0 of a device table (the step
// index in device memory; a step outside the table skips the launch and sets
// *status when status is not NULL).
struct StepRef {
  const zs_folded* table;
  const int64_t* step;
  int32_t* status;
  int64_t t0;
  int64_t count;
};

// Flat shard, as the kernel sees it.  Elements [0, head) and
// [head + 8*nvec, n) go through the per-element path; the 8-element groups in
// between through vector accesses (16-byte aligned at least, 128-byte when the
// arrays allow).  scalar_only = 1 means no common
// alignment offset exists and every element takes the per-element path.
struct FlatShape {
  float* p;
  float* m;
  float* v;
  uint16_t* b;
  int64_t n;
  int64_t head;
  int64_t nvec;
  int32_t scalar_only;
};

// One tensor of a list plan (64 bytes, device table).  Its work items are
// items [item0, item0 + count) of the plan, one wave tile each: for a vector
// tensor, item item0 + k takes 8-groups [max(0, gofs + 64k), gofs + 64k + 64)
// (clipped to nvec), with gofs = lead - 64 when lead > 0 (the groups before the
// tensor's tile grid anchor, a partial tile of their own) and 0 otherwise, and
// its first item also the head and tail elements; for a scalar-only tensor,
// item item0 + k takes elements [512k, 512k + 512), element by element.
struct ListTensor {
  float* p;
  float* m;
  float* v;
  uint16_t* b;
  int64_t n;
  int64_t nvec;
  int32_t item0;
  int32_t group;  // hyperparameter group (list plans with groups; else 0)
  // head | lead << 8: the elements before the first 8-group (< 64) and the
  // 8-groups before the tile grid anchor (< 64), in one word for one scalar load
  int32_t head_lead;
  int32_t scalar_only;
};

static_assert(sizeof(ListTensor) == 64, "ListTensor layout");

// Common alignment peel: the smallest h such that every pointer advanced by h
// elements sits on a 128-byte line boundary (h < 64); failing that, a 64-,
// 32- or 16-byte boundary; -1 if not even a 16-byte one exists.
int64_t common_peel(const float* p, const float* m, const float* v, const uint16_t* b,
                    const uint16_t* const* g, int32_t N);

// The same peel over (pointer, element size) pairs.
int64_t common_peel_sized(const void* const* ptrs, const int* elem_bytes, int count);

// Elements in a wave tile, and the anchor of the tile grid: the smallest a in
// [0, kTileElemsWave) such that every pointer advanced by a elements sits on a
// boundary of kTileElemsWave of its own elements (2 KiB of fp32, 1 KiB of
// bf16), or -1 if the arrays reach such boundaries at different elements.
constexpr int64_t kTileElemsWave = 512;
int64_t tile_anchor_sized(const void* const* ptrs, const int* elem_bytes, int count);
int64_t tile_anchor(const float* p, const float* m, const float* v, const uint16_t* b, const uint16_t* const* g,
                    int32_t N);

// Write windows of the flat step (see flat_window_kernel): stores go out while
// (device real-time counter & period_mask) < open_ticks.  period_mask == 0:
// no windows (one tile per workgroup, stores as soon as a tile is done).
struct WriteWindow {
  uint64_t period_mask;  // period - 1, the period a power of two of 100 MHz ticks
  uint64_t open_ticks;   // window length, 1 .. period - 1
};

// How the flat step schedules its reads and writes (zs_set_flat_schedule):
//  kStream:   one tile per workgroup, each tile's stores issued as it finishes;
//  kWindowed: persistent waves holding finished tiles in registers, storing
//             them in device-clock write windows (flat_window_kernel);
//  kPhased:   persistent workgroups that read every replica of a super-chunk
//             into register accumulators (all waves on about the same replica
//             at once), meet at a grid barrier, then read the state and write
//             the outputs of that super-chunk (flat_phased_kernel).
enum class FlatSchedule : int32_t { kStream = 1, kWindowed = 2, kPhased = 3 };

// The phased kernel's control: its barrier counter (one of kPhasedSlots in
// device memory, picked per launch) and the longest a workgroup waits at a
// barrier, in polls of about 50 ns.
struct PhasedCtl {
  int32_t slot;
  int32_t max_polls;
};

// Launches (host side, defined with the kernels).
hipError_t launch_flat(const uint16_t* const* grads, const FlatShape& s, const Scalars& c, const StepRef& ref,
                       int blocks, FlatSchedule sched, const WriteWindow& win, const PhasedCtl& ctl,
                       hipStream_t stream);
// One device thread: *step += 1.
hipError_t launch_step_advance(int64_t* step, hipStream_t stream);
// cs: n_sets folded scalar sets, one per hyperparameter group (1 <= n_sets <=
// kMaxGroups); with a device step (ref.table set) n_sets is 1 and the table
// supplies the folded scalars.
// sched: the schedule (list_phased_kernel, list_window_kernel with `win`, or
// list_kernel), as for a flat shard of the plan's size.
// items: n_items tensor indices, one per work item (a wave tile), tensor by
// tensor in order.
hipError_t launch_list(const int32_t* items, int32_t n_items, const ListTensor* tensors,
                       const uint16_t* const* gptrs, const Scalars* cs, int n_sets, const StepRef& ref, int blocks,
                       FlatSchedule sched, const WriteWindow& win, const PhasedCtl& ctl, hipStream_t stream);

// Threads per workgroup of the fused step's kernels; each thread owns one
// 8-parameter group, so a tile is 8x this many parameters.  One wave: a
// 512-parameter tile dispatched and retired on its own.  Measured on the same
// buffers against 256-thread workgroups: 1-4% faster for flat shards (70B/64
// shard +1.2%, 124M-parameter N=8 shard +4.4%); for list plans, one wave per
// tile with scalar descriptor loads ran 0-1.6% faster than a four-wave
// workgroup per 4096-parameter chunk that staged its descriptor through LDS.
constexpr int kFlatBlock = 64;
static_assert(kTileElemsWave == 8 * kFlatBlock, "a wave tile: one 8-group per thread");
// Threads per workgroup of pass 1 of the two-pass form (four waves; its norm
// partials are reduced across the waves through LDS).  Pass 2 runs one wave
// per workgroup, as the fused step.
constexpr int kBlock = 256;
// Hyperparameter groups a list plan can carry (their scalars travel as kernel arguments).
constexpr int kMaxGroups = ZS_MAX_GROUPS;
// Windowed flat step: clock checks per batch of replica loads, the fewest
// whole tiles for which a shard takes the windowed kernel, and the most
// devices whose resident-grid figure is cached.
constexpr int kWindowChecks = 4;
constexpr int64_t kWindowMinTiles = 65536;
constexpr int kMaxDevices = 64;
// Phased schedule: 512-parameter tiles per wave in one super-chunk of the
// flat step (their fp32 accumulators take 96 VGPRs, one replica's loads in
// flight 48 more), of pass 1 (10 in registers and 4 in LDS, 96 KB per
// workgroup) and of a list plan (10: its per-wave descriptor takes registers
// of its own), waves per workgroup (one workgroup
// per compute unit at 3 waves per SIMD), barrier counter slots and the
// default longest wait at one barrier (polls of about 50 ns: about 3 ms).
// When the automatic schedule takes the phased kernel is a host decision
// (zs_api.cpp, with its measurements).
constexpr int kPhasedTiles = 12;
constexpr int kReduceRegTiles = 10;
constexpr int kReduceLdsTiles = 4;
constexpr int kReducePhasedTiles = kReduceRegTiles + kReduceLdsTiles;
constexpr int kListPhasedTiles = 10;
constexpr int kPhasedWaves = 12;
constexpr int kPhasedSlots = 16;
constexpr int32_t kPhasedMaxPolls = 1 << 16;
// The share of the grid, in percent, whose arrival at a grid barrier releases it.  On the 70B/64 shard
// the workgroups reach the barrier over about 26 us of a 297 us super-chunk; releasing at 92-96% was
// 0.6-1% faster than waiting for all (releasing at 88% let stragglers fall a super-chunk behind).
constexpr uint32_t kPhasedQuorumPct = 95;
// Write-window bounds, in ticks of the 100 MHz device clock: the period a
// power of two in [kWindowMinPeriod, kWindowMaxPeriod], the open part at most
// kWindowMaxOpen; a wave's wait in a window is capped at kWindowMaxSleeps
// sleeps of 128 cycles (about 0.2 ms at 2.4 GHz, past any allowed window).
constexpr int32_t kWindowMinPeriod = 64;
constexpr int32_t kWindowMaxPeriod = 1 << 20;
constexpr int32_t kWindowMaxOpen = 1 << 14;
constexpr int kWindowMaxSleeps = 4096;
// The one-tile-per-workgroup kernels (the flat step without windows, list
// plans without windows, both passes of the two-pass form without windows)
// cover a shard in consecutive launches of at most about kLaunchBytes
// algorithmic bytes each.  Measured on one shard, one long launch ran up to
// 13% slower than the same work cut into launches of 1.3-5 GB; the persistent
// windowed kernels run as one launch and showed no such loss.  Results do not
// depend on the cut: every element is computed the same way in any launch.
constexpr int64_t kLaunchBytes = 3000000000LL;
// Pass 2 of the two-pass form (16 bytes read and 14 written per parameter)
// runs best in shorter launches: on the 70B/64 shard 5.69-5.71 ms at 0.75-1 GB
// per launch, against 5.83-5.86 ms at 3 GB, 5.74-5.75 at 0.5 GB and 6.0 at
// 0.25 GB.
constexpr int64_t kPass2LaunchBytes = 1000000000LL;
// The current limit (zs_set_launch_bytes; `fallback` unless set).
int64_t launch_bytes(int64_t fallback = kLaunchBytes);
// Units of `bytes_per_unit` algorithmic bytes per launch under that limit: a
// multiple of `align` units, and at least `align`.
inline int64_t units_per_launch(int64_t bytes_per_unit, int64_t align, int64_t fallback = kLaunchBytes) {
  const int64_t u = launch_bytes(fallback) / bytes_per_unit / align * align;
  return u < align ? align : u;
}

}  // namespace zs
