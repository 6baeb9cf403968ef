// C-ABI front end of libzshard: argument checks, scalar folding, list plans,
// launches and error reporting.  The arithmetic contract is in include/zshard.h.
#include <algorithm>
#include <atomic>
#include <cstddef>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "zs_cpu_adam.h"
#include "zs_internal.h"
#include "zs_twopass.h"

namespace {

thread_local std::string g_last_error;
std::atomic<int32_t> g_grid_blocks{0};
std::atomic<int64_t> g_launch_bytes{0};  // zs_set_launch_bytes; 0 = zs::kLaunchBytes
// zs_set_write_window: (period << 32) | open, one word so a reader never pairs
// one call's period with another's open length; period 0 = automatic, 1 = no
// windows
std::atomic<uint64_t> g_window{0};
// zs_set_flat_schedule (0 = automatic) and zs_set_phased_max_polls (0 = default)
std::atomic<int32_t> g_flat_schedule{0};
std::atomic<int32_t> g_phased_max_polls{0};
// the phased kernel's barrier-counter slot of the next launch (round robin)
std::atomic<uint32_t> g_phased_slot{0};

zs_status fail(zs_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

zs_status hip_fail(hipError_t e, const char* what) {
  return fail(ZS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool sync_mode() {
  static const bool on = [] {
    const char* s = std::getenv("ZS_SYNC");
    return s && s[0] && std::strcmp(s, "0") != 0;
  }();
  return on;
}

zs_status check_hp(const zs_adam_hp* hp, int64_t step) {
  if (!hp) return fail(ZS_ERR_NULL, "hp is NULL");
  const double xs[5] = {hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay};
  for (double x : xs)
    if (!std::isfinite(x)) return fail(ZS_ERR_RANGE, "hyperparameters must be finite");
  if (hp->lr < 0) return fail(ZS_ERR_RANGE, "lr must be >= 0 (got %g)", hp->lr);
  if (!(hp->beta1 >= 0 && hp->beta1 < 1)) return fail(ZS_ERR_RANGE, "beta1 must be in [0, 1) (got %g)", hp->beta1);
  if (!(hp->beta2 >= 0 && hp->beta2 < 1)) return fail(ZS_ERR_RANGE, "beta2 must be in [0, 1) (got %g)", hp->beta2);
  if (!(hp->eps > 0)) return fail(ZS_ERR_RANGE, "eps must be > 0 (got %g)", hp->eps);
  if (hp->weight_decay < 0) return fail(ZS_ERR_RANGE, "weight_decay must be >= 0 (got %g)", hp->weight_decay);
  if (step < 1) return fail(ZS_ERR_RANGE, "step must be >= 1 (got %lld)", (long long)step);
  return ZS_OK;
}

void fold_scalars(const zs_adam_hp& hp, int64_t step, zs_folded* f) {
  const double t = (double)step;
  f->b1 = (float)hp.beta1;
  f->c1 = (float)(1.0 - hp.beta1);
  f->b2 = (float)hp.beta2;
  f->c2 = (float)(1.0 - hp.beta2);
  f->eps = (float)hp.eps;
  f->ss = (float)(hp.lr / (1.0 - std::pow(hp.beta1, t)));
  f->rb = (float)(1.0 / std::sqrt(1.0 - std::pow(hp.beta2, t)));
  f->dk = (float)(1.0 - hp.lr * hp.weight_decay);
}

zs::Scalars make_scalars(const zs_adam_hp& hp, int64_t step, int32_t N) {
  zs_folded f;
  fold_scalars(hp, step, &f);
  zs::Scalars c;
  c.b1 = f.b1;
  c.c1 = f.c1;
  c.b2 = f.b2;
  c.c2 = f.c2;
  c.e = f.eps;
  c.ss = f.ss;
  c.rb = f.rb;
  c.dk = f.dk;
  c.n_rep = N;
  c.pow2 = (N & (N - 1)) == 0;
  c.inv_n = (float)(1.0 / (double)N);
  return c;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
  int kind;          // 0 = output, 1 = gradient
  int64_t owner;
};

// Outputs pairwise disjoint; no gradient range overlaps an output.
zs_status check_alias(std::vector<Range>& rs) {
  std::vector<Range> outs, grads;
  for (const Range& r : rs)
    if (r.hi > r.lo) (r.kind == 0 ? outs : grads).push_back(r);
  std::sort(outs.begin(), outs.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t k = 1; k < outs.size(); ++k)
    if (outs[k].lo < outs[k - 1].hi)
      return fail(ZS_ERR_ALIAS, "output arrays overlap (tensors %lld and %lld)", (long long)outs[k - 1].owner,
                  (long long)outs[k].owner);
  // Sorted disjoint outputs also have sorted ends, so of the outputs that start
  // below a gradient range's end, only the last can reach past its start.
  for (const Range& g : grads) {
    auto it = std::lower_bound(outs.begin(), outs.end(), g.hi, [](const Range& o, uintptr_t x) { return o.lo < x; });
    if (it != outs.begin()) {
      const Range& o = *(it - 1);
      if (o.hi > g.lo)
        return fail(ZS_ERR_ALIAS, "a gradient chunk overlaps an output array (tensor %lld)", (long long)g.owner);
    }
  }
  return ZS_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Per-tensor checks shared by the flat call and the list plans; appends the
// tensor's address ranges to `rs`.
zs_status check_tensor(const uint16_t* const* g, int32_t N, int64_t n, const float* p, const float* m,
                       const float* v, const uint16_t* b, int64_t owner, std::vector<Range>& rs) {
  if (n < 0) return fail(ZS_ERR_RANGE, "n must be >= 0 (tensor %lld)", (long long)owner);
  if (n > (int64_t(1) << 56)) return fail(ZS_ERR_RANGE, "n too large (tensor %lld)", (long long)owner);
  if (n == 0) return ZS_OK;
  if (!g) return fail(ZS_ERR_NULL, "grad_chunks is NULL (tensor %lld)", (long long)owner);
  if (!p || !m || !v || !b) return fail(ZS_ERR_NULL, "master/m/v/param_bf16 is NULL (tensor %lld)", (long long)owner);
  for (int32_t r = 0; r < N; ++r) {
    if (!g[r]) return fail(ZS_ERR_NULL, "grad_chunks[%d] is NULL (tensor %lld)", r, (long long)owner);
    if (!aligned(g[r], 2)) return fail(ZS_ERR_ALIGN, "grad_chunks[%d] not 2-byte aligned", r);
  }
  if (!aligned(p, 4) || !aligned(m, 4) || !aligned(v, 4))
    return fail(ZS_ERR_ALIGN, "fp32 arrays must be 4-byte aligned (tensor %lld)", (long long)owner);
  if (!aligned(b, 2)) return fail(ZS_ERR_ALIGN, "param_bf16 must be 2-byte aligned (tensor %lld)", (long long)owner);
  const uintptr_t n4 = (uintptr_t)n * 4, n2 = (uintptr_t)n * 2;
  rs.push_back({(uintptr_t)p, (uintptr_t)p + n4, 0, owner});
  rs.push_back({(uintptr_t)m, (uintptr_t)m + n4, 0, owner});
  rs.push_back({(uintptr_t)v, (uintptr_t)v + n4, 0, owner});
  rs.push_back({(uintptr_t)b, (uintptr_t)b + n2, 0, owner});
  for (int32_t r = 0; r < N; ++r) rs.push_back({(uintptr_t)g[r], (uintptr_t)g[r] + n2, 1, owner});
  return ZS_OK;
}

zs::FlatShape shape_of(const uint16_t* const* g, int32_t N, int64_t n, float* p, float* m, float* v,
                       uint16_t* b) {
  zs::FlatShape s;
  s.p = p;
  s.m = m;
  s.v = v;
  s.b = b;
  s.n = n;
  const int64_t h = zs::common_peel(p, m, v, b, g, N);
  if (h < 0 || n < h + 8) {
    s.head = 0;
    s.nvec = 0;
    s.scalar_only = 1;
  } else {
    s.head = h;
    s.nvec = (n - h) / 8;
    s.scalar_only = 0;
  }
  return s;
}

// Workgroups per launch: one per tile (measured best; each launch clamps this
// to its tile count, and the tile loops cover shards of more than 2^30 tiles),
// unless zs_set_grid_blocks fixed a count.
int auto_blocks() {
  const int32_t forced = g_grid_blocks.load(std::memory_order_relaxed);
  return forced > 0 ? forced : 1 << 30;
}

// When the automatic schedule takes the phased kernel: for N replicas on n
// parameters, when some rule {replicas, params} has N >= replicas and
// n >= params.  The rules follow the crossings measured against per-tile
// stores (one process per point, % of 8 TB/s by the byte model, phased /
// per-tile):
//  - the flat step: from 2^25 parameters at N >= 40 (N = 40: 73% / 70% at
//    2^25; 48: 72% / 68%; 64: 74% / 70.5%), from 2^27 at N = 24-39 (N = 24:
//    67% / 70% at 2^25, 72.5% / 71.6% at 2^27, 77.5% / 74% at 2^30; N = 32:
//    70% / 71.6% at 2^25, 74% / 70% at 2^27).  Below 24 replicas it gains at
//    most 1.4% on 2^29-2^30 parameters and loses on smaller shards (N = 18:
//    67% / 72% at 2^25, 73% / 72% at 2^30; N = 8: 66% / 74% at 2^30);
//  - list plans (spans of 10 consecutive items, per-span descriptors), on
//    lists of large tensors (the llama7b shapes scaled to 2^25-2^29.6
//    parameters, 1-4% of items outside whole spans): from 2^26 at N >= 64
//    (74% / 70.6%; 71% / 71% at 2^25), from 2^27 at N = 40-63 (71% / 66.4%;
//    69% / 69.3% at 2^26), from 2^28 at N = 32-39 (72% / 67.8%; 69.7% /
//    69.6% at 2^27); per-tile stores won at N = 18 and 24 on 2^29.6.  Items
//    outside whole spans go one at a time after the super-chunks: the ragged
//    list of 20,000 tensors lost phased at every N from 32 to 64 when scaled
//    to 2^25-2^27 parameters (33-76% of its items loose; 48-62% / 65-70%),
//    lost at N = 32 and 40 on 2^28 (20% loose; 63% / 66-69%), and won at
//    N = 24 and 32 on 2^31 (3.5% loose; 73.6% / 71.2%).  So lists take it
//    from 1.5x the power of two where it first won (3 * 2^24 at N >= 64,
//    3 * 2^25 at N >= 40, 3 * 2^26 at N >= 32: halfway to the tie below in
//    log terms) with at most 1 item in 20 outside whole spans;
//  - pass 1 of the two-pass form, whose write phase is its 4-byte means
//    alone: phased wins or ties from N = 12 on 2^25 parameters and more
//    (N = 12: 65.5% / 65.1% at 2^25, 74% / 71% at 2^27; N = 16: 66% / 66.6%
//    at 2^25, 73.6% / 69.6% at 2^26, 77% / 72% at 2^30; N = 8: 74.7% / 75.4%
//    at 2^30).
struct PhasedRule {
  int32_t replicas;
  int64_t params;
};
constexpr PhasedRule kFlatPhased[] = {{40, (int64_t)1 << 25}, {24, (int64_t)1 << 27}};
constexpr PhasedRule kListPhased[] = {{64, (int64_t)3 << 24}, {40, (int64_t)3 << 25}, {32, (int64_t)3 << 26}};
// ... and list plans only when at most 1/20 of their items lie outside whole spans (kLooseShareMax)
constexpr int64_t kLooseShareMax = 20;
constexpr PhasedRule kReducePhased[] = {{12, (int64_t)1 << 25}};

template <size_t R>
bool phased_by_rule(const PhasedRule (&rules)[R], int32_t N, int64_t n) {
  for (const PhasedRule& r : rules)
    if (N >= r.replicas && n >= r.params) return true;
  return false;
}

// The flat step's schedule for N replicas on a shard of n parameters (and a
// list plan's, for n parameters in all, with `list_items` >= 0: its items, of
// which `loose_items` lie outside whole spans), and the write window it takes
// (period_mask 0 unless windowed).  An explicit zs_set_flat_schedule
// wins; otherwise an explicit zs_set_write_window decides (no windows:
// per-tile stores; a window: the windowed kernel); otherwise the phased
// kernel where its rules say (above), and per-tile stores elsewhere.  The
// windowed kernel's default window is a 4096-tick (41 us) period with 640
// ticks open for N < 64, 512 up to 128 and 384 above: the writes' share of
// the bytes shrinks as N grows.
zs::FlatSchedule flat_schedule(int32_t N, int64_t n, zs::WriteWindow* win, int64_t list_items = -1,
                               int64_t loose_items = 0) {
  const bool list = list_items >= 0;
  const int32_t forced = g_flat_schedule.load(std::memory_order_relaxed);
  const uint64_t word = g_window.load(std::memory_order_relaxed);
  const int32_t period = (int32_t)(word >> 32);
  zs::FlatSchedule sched;
  if (forced != 0)
    sched = (zs::FlatSchedule)forced;
  else if (period == 1)
    sched = zs::FlatSchedule::kStream;
  else if (period > 1)
    sched = zs::FlatSchedule::kWindowed;
  else
    sched = (list ? phased_by_rule(kListPhased, N, n) && loose_items * kLooseShareMax <= list_items
                  : phased_by_rule(kFlatPhased, N, n))
                ? zs::FlatSchedule::kPhased
                : zs::FlatSchedule::kStream;
  zs::WriteWindow w{0, 0};
  if (sched == zs::FlatSchedule::kWindowed) {
    // an explicit window, none when windows were switched off, else the default for N (any N)
    const int32_t open = (int32_t)(word & 0xFFFFFFFFu);
    if (period > 1)
      w = zs::WriteWindow{(uint64_t)period - 1, (uint64_t)open};
    else if (period == 0)
      w = zs::WriteWindow{4096 - 1, N < 64 ? 640u : N <= 128 ? 512u : 384u};
  }
  if (win) *win = w;
  return sched;
}

zs::PhasedCtl phased_ctl() {
  const int32_t polls = g_phased_max_polls.load(std::memory_order_relaxed);
  return zs::PhasedCtl{(int32_t)(g_phased_slot.fetch_add(1, std::memory_order_relaxed) % zs::kPhasedSlots),
                       polls > 0 ? polls : zs::kPhasedMaxPolls};
}

// Pass 1 of the two-pass form (2N bytes read and 4 written per parameter)
// follows the same setting: an explicit schedule, else an explicit window
// (1: none, > 1: windowed), else phased where its rules say (above), else
// one tile per workgroup.  Its windowed default is 4096 / 256.
zs::FlatSchedule reduce_schedule(int32_t N, int64_t n, zs::WriteWindow* win) {
  const int32_t forced = g_flat_schedule.load(std::memory_order_relaxed);
  const uint64_t word = g_window.load(std::memory_order_relaxed);
  const int32_t period = (int32_t)(word >> 32), open = (int32_t)(word & 0xFFFFFFFFu);
  zs::FlatSchedule sched;
  if (forced != 0)
    sched = (zs::FlatSchedule)forced;
  else if (period == 1)
    sched = zs::FlatSchedule::kStream;
  else if (period > 1)
    sched = zs::FlatSchedule::kWindowed;
  else
    sched = phased_by_rule(kReducePhased, N, n) ? zs::FlatSchedule::kPhased : zs::FlatSchedule::kStream;
  zs::WriteWindow w{0, 0};
  if (sched == zs::FlatSchedule::kWindowed) {
    if (period > 1)
      w = zs::WriteWindow{(uint64_t)period - 1, (uint64_t)open};
    else if (period == 0)
      w = zs::WriteWindow{4096 - 1, 256};
  }
  if (win) *win = w;
  return sched;
}

zs_status after_launch(hipError_t e, hipStream_t stream, const char* what) {
  if (e != hipSuccess) return hip_fail(e, what);
  if (sync_mode()) {
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, what);
  }
  return ZS_OK;
}

// A device step source: checked, its ranges appended to `rs` (the table and
// the step are read, the status word is written), and turned into the
// kernels' StepRef.
zs_status step_ref_of(const zs_step_source* src, std::vector<Range>& rs, zs::StepRef* ref) {
  if (!src) return fail(ZS_ERR_NULL, "src is NULL");
  if (!src->table || !src->step) return fail(ZS_ERR_NULL, "src->table and src->step must not be NULL");
  if (src->t0 < 1 || src->count < 1 || src->count > (int64_t(1) << 40))
    return fail(ZS_ERR_RANGE, "src->t0 must be >= 1 and src->count in [1, 2^40]");
  if (!aligned(src->table, 4) || !aligned(src->step, 8) || (src->status && !aligned(src->status, 4)))
    return fail(ZS_ERR_ALIGN, "the table must be 4-byte, the step 8-byte and the status 4-byte aligned");
  const uintptr_t tb = (uintptr_t)src->table, te = tb + sizeof(zs_folded) * (uintptr_t)src->count;
  const uintptr_t sp = (uintptr_t)src->step;
  if (src->status) {  // the one output among these: it must not lie inside the table or the step
    const uintptr_t st = (uintptr_t)src->status;
    if ((st < te && tb < st + 4) || (st < sp + 8 && sp < st + 4))
      return fail(ZS_ERR_ALIAS, "src->status overlaps the table or the step");
    rs.push_back({st, st + 4, 0, -1});
  }
  rs.push_back({tb, te, 1, -1});
  rs.push_back({sp, sp + 8, 1, -1});
  *ref = zs::StepRef{src->table, src->step, src->status, src->t0, src->count};
  return ZS_OK;
}

}  // namespace

namespace zs {

int64_t launch_bytes(int64_t fallback) {
  const int64_t b = g_launch_bytes.load(std::memory_order_relaxed);
  return b > 0 ? b : fallback;
}

// Tiles that start on a cache-line boundary in every array keep every wave
// access on whole 128-byte lines; a tile grid that straddles lines turns each
// line at a tile edge into two partial writes (measured 7-9% slower).  So the
// peel first looks for a common 128-byte boundary, then 64, 32 and finally the
// 16 bytes the vector accesses need.
int64_t common_peel_sized(const void* const* ptrs, const int* elem_bytes, int count) {
  for (int64_t align : {128, 64, 32, 16}) {
    for (int64_t h = 0; h < align / 2; ++h) {  // bf16 needs up to align/2 - 1 elements
      bool ok = true;
      for (int k = 0; ok && k < count; ++k)
        ok = aligned(static_cast<const char*>(ptrs[k]) + h * elem_bytes[k], align);
      if (ok) return h;
    }
  }
  return -1;
}

// Tiles that also start on a boundary of 512 of their own elements run
// faster again: the same flat shard with every array starting 64 to 448
// elements past such a boundary took 2.6-4.1% longer than from the boundary
// (a ragged list, whose tensors start at every phase, lost about as much).
int64_t tile_anchor_sized(const void* const* ptrs, const int* elem_bytes, int count) {
  int64_t phase = -1;
  for (int k = 0; k < count; ++k) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(ptrs[k]);
    if (a % (uintptr_t)elem_bytes[k] != 0) return -1;
    const int64_t ph = (int64_t)((a / (uintptr_t)elem_bytes[k]) % (uintptr_t)kTileElemsWave);
    if (phase >= 0 && ph != phase) return -1;
    phase = ph;
  }
  return phase <= 0 ? 0 : kTileElemsWave - phase;
}

int64_t tile_anchor(const float* p, const float* m, const float* v, const uint16_t* b, const uint16_t* const* g,
                    int32_t N) {
  std::vector<const void*> ptrs{p, m, v, b};
  std::vector<int> sizes{4, 4, 4, 2};
  for (int32_t r = 0; r < N; ++r) {
    ptrs.push_back(g[r]);
    sizes.push_back(2);
  }
  return tile_anchor_sized(ptrs.data(), sizes.data(), (int)ptrs.size());
}

int64_t common_peel(const float* p, const float* m, const float* v, const uint16_t* b, const uint16_t* const* g,
                    int32_t N) {
  std::vector<const void*> ptrs{p, m, v, b};
  std::vector<int> sizes{4, 4, 4, 2};
  for (int32_t r = 0; r < N; ++r) {
    ptrs.push_back(g[r]);
    sizes.push_back(2);
  }
  return common_peel_sized(ptrs.data(), sizes.data(), (int)ptrs.size());
}

}  // namespace zs

namespace {

constexpr int64_t kTileElems = (int64_t)zs::kBlock * 8;

struct WorkspaceLayout {
  float* gbar;
  double* partials;
  double* partials2;
  size_t need;  // bytes from the workspace start
};

// Norm slots for n parameters: one per tile plus the head slot (at most
// n / kTileElems + 2), and one first-stage sum per kFinalSeg of those.
size_t partial_slots(int64_t n) { return (size_t)(n / kTileElems + 2); }
size_t partial2_slots(int64_t n) { return partial_slots(n) / (size_t)zs::kFinalSeg + 1; }

// fp32 gradient at the first 256-byte boundary, then the per-tile norm
// partials, then their first-stage sums.
WorkspaceLayout layout_of(const void* ws, int64_t n) {
  WorkspaceLayout L;
  const uintptr_t base = reinterpret_cast<uintptr_t>(ws);
  const uintptr_t g = (base + 255) & ~(uintptr_t)255;
  const uintptr_t p = g + (((uintptr_t)n * 4 + 255) & ~(uintptr_t)255);
  const uintptr_t p2 = p + 8 * partial_slots(n);
  L.gbar = reinterpret_cast<float*>(g);
  L.partials = reinterpret_cast<double*>(p);
  L.partials2 = reinterpret_cast<double*>(p2);
  L.need = (size_t)(p2 - base) + 8 * partial2_slots(n);
  return L;
}

// Pass-1 shape for n parameters of replicas `g` and workspace `ws` (the
// workspace must already be known to be large enough).
void reduce_shape(const uint16_t* const* g, int32_t N, int64_t n, void* ws, double* sq, float inv_scale,
                  zs::TwoPassShape* sh) {
  *sh = zs::TwoPassShape{};
  sh->sqnorm = sq;
  sh->n = n;
  sh->n_rep = N;
  sh->inv_scale = inv_scale;
  const WorkspaceLayout L = layout_of(ws, n);
  sh->gbar = L.gbar;
  sh->partials = L.partials;
  sh->partials2 = L.partials2;
  std::vector<const void*> ptrs(g, g + N);
  std::vector<int> sizes(N, 2);
  ptrs.push_back(L.gbar);
  sizes.push_back(4);
  const int64_t h = zs::common_peel_sized(ptrs.data(), sizes.data(), (int)ptrs.size());
  if (h < 0) {
    sh->scalar_only = 1;
    sh->head = 0;
  } else {
    sh->scalar_only = 0;
    sh->head = h < n ? h : n;
  }
  sh->ntiles = (n - sh->head + kTileElems - 1) / kTileElems;
}

}  // namespace

namespace zs {

zs_status offload_fail(zs_status st, const char* msg) { return fail(st, "%s", msg); }

bool offload_fold(const zs_adam_hp* hp, int64_t step, HostScalars* out) {
  g_last_error.clear();
  if (check_hp(hp, step) != ZS_OK) return false;
  zs_folded f;
  fold_scalars(*hp, step, &f);
  *out = HostScalars{f.b1, f.c1, f.b2, f.c2, f.eps, f.ss, f.rb, f.dk, 1.0f};
  return true;
}

bool offload_reduce_shape(const uint16_t* const* grads, int32_t N, int64_t n, void* ws, double* sq,
                          TwoPassShape* sh) {
  if (n <= 0) return false;
  reduce_shape(grads, N, n, ws, sq, 1.0f, sh);
  return true;
}

int offload_blocks() { return auto_blocks(); }

}  // namespace zs

namespace {

// A list plan's device table, laid out on the host: items | tensors | grad
// pointers, in one byte image ready to upload.
struct ListTable {
  std::vector<unsigned char> bytes;
  size_t off_tensors = 0, off_gptrs = 0;
  int32_t n_items = 0;
  int32_t loose_items = 0;  // items outside whole spans of the phased list kernel
  int64_t n_params = 0;
};

// Checks the tensors (as zs_list_plan_create documents) and lays out their
// table: one work item per wave tile, tensor by tensor.  A vector tensor's
// tiles start at its tile grid's anchor (the groups before it, if any, a
// partial tile of their own); a scalar-only tensor's items take 512 elements
// each.  Every item is a whole or partial tile of one tensor, so no workgroup
// is launched for nothing.
zs_status build_list_table(const zs_tensor* tensors, int32_t T, int32_t N, ListTable& out) {
  if (T < 0) return fail(ZS_ERR_RANGE, "T must be >= 0 (got %d)", T);
  if (T > 0 && !tensors) return fail(ZS_ERR_NULL, "tensors is NULL");
  if (N < 1 || N > ZS_MAX_REPLICAS) return fail(ZS_ERR_RANGE, "N must be in [1, %d] (got %d)", ZS_MAX_REPLICAS, N);
  std::vector<Range> rs;
  int64_t total = 0;
  for (int32_t t = 0; t < T; ++t) {
    const zs_tensor& x = tensors[t];
    zs_status st = check_tensor(x.grad_chunks, N, x.n, x.master, x.m, x.v, x.param_bf16, t, rs);
    if (st) return st;
    total += x.n;
  }
  zs_status st = check_alias(rs);
  if (st) return st;

  constexpr int64_t kGroupsPerTile = zs::kTileElemsWave / 8;
  constexpr int64_t K = zs::kListPhasedTiles;
  int64_t whole = 0;  // items in whole spans: K consecutive items from a multiple of K, all whole tiles of one tensor
  std::vector<zs::ListTensor> ht;
  std::vector<int32_t> hi;
  std::vector<const uint16_t*> hg;
  ht.reserve(T);
  hg.reserve((size_t)T * N);
  for (int32_t t = 0; t < T; ++t) {
    const zs_tensor& x = tensors[t];
    if ((int64_t)hi.size() > (int64_t)INT32_MAX) return fail(ZS_ERR_RANGE, "too many work items");
    zs::ListTensor d{};
    d.item0 = (int32_t)hi.size();
    int64_t items = 0;
    if (x.n == 0) {
      d.scalar_only = 1;
    } else {
      const zs::FlatShape s = shape_of(x.grad_chunks, N, x.n, x.master, x.m, x.v, x.param_bf16);
      d.p = s.p;
      d.m = s.m;
      d.v = s.v;
      d.b = s.b;
      d.n = s.n;
      d.head_lead = (int32_t)s.head;
      d.nvec = s.nvec;
      d.scalar_only = s.scalar_only;
      if (!s.scalar_only) {
        // the groups before the tile grid's anchor form a partial tile of their own, so that every
        // later tile starts on a 512-element boundary of every array
        const int64_t a = zs::tile_anchor(x.master, x.m, x.v, x.param_bf16, x.grad_chunks, N);
        const int64_t lead = a > s.head ? std::min(s.nvec, (a - s.head) / 8) : 0;
        d.head_lead |= (int32_t)lead << 8;
        const int64_t gofs = lead > 0 ? lead - kGroupsPerTile : 0;
        items = (s.nvec - gofs + kGroupsPerTile - 1) / kGroupsPerTile;
        const int64_t i0 = (int64_t)hi.size();
        for (int64_t j = (i0 + K - 1) / K; (j + 1) * K <= i0 + items; ++j) {
          const int64_t g0 = gofs + (j * K - i0) * kGroupsPerTile;
          if (g0 >= 0 && g0 + K * kGroupsPerTile <= s.nvec) whole += K;
        }
      } else {
        items = (s.n + zs::kTileElemsWave - 1) / zs::kTileElemsWave;
      }
    }
    if ((int64_t)hi.size() + items > (int64_t)INT32_MAX) return fail(ZS_ERR_RANGE, "too many work items");
    hi.insert(hi.end(), (size_t)items, t);
    ht.push_back(d);
    for (int32_t r = 0; r < N; ++r) hg.push_back(x.n ? x.grad_chunks[r] : nullptr);
  }
  // the tensor descriptors start on a 64-byte boundary after the item indices
  const size_t bi = (hi.size() * sizeof(int32_t) + 63) / 64 * 64, bt = ht.size() * sizeof(zs::ListTensor),
               bg = hg.size() * sizeof(void*);
  out.bytes.assign(bi + bt + bg, 0);
  if (!hi.empty()) std::memcpy(out.bytes.data(), hi.data(), hi.size() * sizeof(int32_t));
  if (bt) std::memcpy(out.bytes.data() + bi, ht.data(), bt);
  if (bg) std::memcpy(out.bytes.data() + bi + bt, hg.data(), bg);
  out.off_tensors = bi;
  out.off_gptrs = bi + bt;
  out.n_items = (int32_t)hi.size();
  out.loose_items = (int32_t)((int64_t)hi.size() - whole);
  out.n_params = total;
  return ZS_OK;
}

}  // namespace

struct zs_list_plan {
  int device;
  int32_t N;
  int32_t T;
  int32_t n_items;
  int32_t loose_items;  // items outside whole spans (the automatic schedule's list rule)
  int64_t n_params;
  int32_t n_groups;  // hyperparameter groups set by zs_list_plan_set_groups (1 until then)
  void* table;  // device: items | tensors | grad pointers
  int32_t* items;
  zs::ListTensor* tensors;
  const uint16_t** gptrs;
};

namespace {

// zs_reduce_adam_flat with the step from the host (src == NULL) or the device.
zs_status flat_step(const uint16_t* const* grad_chunks, int32_t N, int64_t n, float* master, float* m, float* v,
                    uint16_t* param_bf16, const zs_adam_hp* hp, int64_t step, const zs_step_source* src,
                    zs_stream stream, const char* what) {
  try {
    g_last_error.clear();
    if (!src) {
      zs_status st = check_hp(hp, step);
      if (st) return st;
    }
    if (N < 1 || N > ZS_MAX_REPLICAS) return fail(ZS_ERR_RANGE, "N must be in [1, %d] (got %d)", ZS_MAX_REPLICAS, N);
    std::vector<Range> rs;
    zs_status st = check_tensor(grad_chunks, N, n, master, m, v, param_bf16, 0, rs);
    if (st) return st;
    zs::StepRef ref{};
    if (src) {
      st = step_ref_of(src, rs, &ref);
      if (st) return st;
    }
    if (n == 0) return ZS_OK;
    st = check_alias(rs);
    if (st) return st;
    const zs::FlatShape s = shape_of(grad_chunks, N, n, master, m, v, param_bf16);
    // with a device step the table supplies the folded scalars; only N's fields are used from these
    const zs_adam_hp placeholder = {0.0, 0.0, 0.0, 1.0, 0.0};
    const zs::Scalars c = make_scalars(src ? placeholder : *hp, src ? 1 : step, N);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    zs::WriteWindow win{};
    const int64_t a = s.scalar_only ? 0 : zs::tile_anchor(master, m, v, param_bf16, grad_chunks, N);
    if (a > 0 && a < n) {
      // the elements before the tile grid's anchor as a shard of their own (one-tile kernel), then the
      // rest from the anchor, whose tiles start on a 512-element boundary of every array
      const zs::FlatShape f = shape_of(grad_chunks, N, a, master, m, v, param_bf16);
      const hipError_t e = zs::launch_flat(grad_chunks, f, c, ref, auto_blocks(), zs::FlatSchedule::kStream,
                                           zs::WriteWindow{}, phased_ctl(), hs);
      if (e != hipSuccess) return after_launch(e, hs, what);
      std::vector<const uint16_t*> ga(grad_chunks, grad_chunks + N);
      for (auto& q : ga) q += a;
      const zs::FlatShape r = shape_of(ga.data(), N, n - a, master + a, m + a, v + a, param_bf16 + a);
      const zs::FlatSchedule sched = flat_schedule(N, n - a, &win);
      return after_launch(zs::launch_flat(ga.data(), r, c, ref, auto_blocks(), sched, win, phased_ctl(), hs), hs,
                          what);
    }
    const zs::FlatSchedule sched = flat_schedule(N, n, &win);
    return after_launch(zs::launch_flat(grad_chunks, s, c, ref, auto_blocks(), sched, win, phased_ctl(), hs), hs,
                        what);
  } catch (const std::bad_alloc&) {
    return fail(ZS_ERR_NOMEM, "host allocation failed");
  } catch (...) {
    return fail(ZS_ERR_HIP, "unexpected exception");
  }
}

}  // namespace

extern "C" {

int zs_abi_version(void) { return ZS_ABI_VERSION; }

const char* zs_status_string(int status) {
  switch (status) {
    case ZS_OK: return "ZS_OK";
    case ZS_ERR_NULL: return "ZS_ERR_NULL";
    case ZS_ERR_RANGE: return "ZS_ERR_RANGE";
    case ZS_ERR_ALIAS: return "ZS_ERR_ALIAS";
    case ZS_ERR_ALIGN: return "ZS_ERR_ALIGN";
    case ZS_ERR_HIP: return "ZS_ERR_HIP";
    case ZS_ERR_NOMEM: return "ZS_ERR_NOMEM";
    default: return "ZS_ERR_UNKNOWN";
  }
}

const char* zs_last_error(void) { return g_last_error.c_str(); }

zs_status zs_fold(const zs_adam_hp* hp, int64_t step, zs_folded* out) {
  g_last_error.clear();
  if (!out) return fail(ZS_ERR_NULL, "out is NULL");
  zs_status st = check_hp(hp, step);
  if (st) return st;
  fold_scalars(*hp, step, out);
  return ZS_OK;
}

zs_status zs_set_grid_blocks(int32_t blocks) {
  if (blocks < 0 || blocks > (1 << 24)) return fail(ZS_ERR_RANGE, "blocks must be in [0, 2^24]");
  g_grid_blocks.store(blocks, std::memory_order_relaxed);
  return ZS_OK;
}

zs_status zs_set_launch_bytes(int64_t bytes) {
  g_last_error.clear();
  if (bytes < 0) return fail(ZS_ERR_RANGE, "bytes must be >= 0 (got %lld)", (long long)bytes);
  g_launch_bytes.store(bytes, std::memory_order_relaxed);
  return ZS_OK;
}

int64_t zs_launch_bytes(void) { return zs::launch_bytes(); }

zs_status zs_set_write_window(int32_t period_ticks, int32_t open_ticks) {
  g_last_error.clear();
  if (period_ticks == 0 || period_ticks == 1) {
    g_window.store((uint64_t)period_ticks << 32, std::memory_order_relaxed);
    return ZS_OK;
  }
  if (period_ticks < zs::kWindowMinPeriod || period_ticks > zs::kWindowMaxPeriod ||
      (period_ticks & (period_ticks - 1)) != 0)
    return fail(ZS_ERR_RANGE, "period_ticks must be 0, 1 or a power of two in [%d, %d] (got %d)",
                zs::kWindowMinPeriod, zs::kWindowMaxPeriod, period_ticks);
  if (open_ticks < 1 || open_ticks >= period_ticks || open_ticks > zs::kWindowMaxOpen)
    return fail(ZS_ERR_RANGE, "open_ticks must be in [1, min(period_ticks - 1, %d)] (got %d)", zs::kWindowMaxOpen,
                open_ticks);
  g_window.store(((uint64_t)period_ticks << 32) | (uint32_t)open_ticks, std::memory_order_relaxed);
  return ZS_OK;
}

zs_status zs_write_window(int32_t kernel, int32_t N, int64_t n, int32_t* period_ticks, int32_t* open_ticks) {
  g_last_error.clear();
  if (!period_ticks || !open_ticks) return fail(ZS_ERR_NULL, "period_ticks or open_ticks is NULL");
  if (kernel != ZS_WINDOW_FLAT_STEP && kernel != ZS_WINDOW_REDUCE_PASS && kernel != ZS_WINDOW_LIST_PLAN)
    return fail(ZS_ERR_RANGE, "kernel must be ZS_WINDOW_FLAT_STEP, _REDUCE_PASS or _LIST_PLAN (got %d)", kernel);
  if (N < 1 || N > ZS_MAX_REPLICAS) return fail(ZS_ERR_RANGE, "N must be in [1, %d] (got %d)", ZS_MAX_REPLICAS, N);
  if (n < 0) return fail(ZS_ERR_RANGE, "n must be >= 0");
  const bool flat = kernel != ZS_WINDOW_REDUCE_PASS;  // the flat step and list plans: 512-parameter tiles
  zs::WriteWindow w{};
  if (kernel == ZS_WINDOW_REDUCE_PASS)
    (void)reduce_schedule(N, n, &w);
  else if (kernel == ZS_WINDOW_LIST_PLAN)  // a flat shard's schedule for the plan's size, by the list rules
    (void)flat_schedule(N, n, &w, 0);
  else
    (void)flat_schedule(N, n, &w);
  const bool big = flat ? n / 8 / zs::kFlatBlock >= zs::kWindowMinTiles
                        : n / kTileElems >= zs::kReduceWindowMinTiles;
  const bool used = w.period_mask != 0 && big;
  *period_ticks = used ? (int32_t)(w.period_mask + 1) : 0;
  *open_ticks = used ? (int32_t)w.open_ticks : 0;
  return ZS_OK;
}

zs_status zs_set_flat_schedule(int32_t schedule) {
  g_last_error.clear();
  if (schedule < 0 || schedule > ZS_SCHEDULE_PHASED)
    return fail(ZS_ERR_RANGE, "schedule must be ZS_SCHEDULE_AUTO, _STREAM, _WINDOWED or _PHASED (got %d)", schedule);
  g_flat_schedule.store(schedule, std::memory_order_relaxed);
  return ZS_OK;
}

zs_status zs_reduce_schedule(int32_t N, int64_t n, int32_t* schedule) {
  g_last_error.clear();
  if (!schedule) return fail(ZS_ERR_NULL, "schedule is NULL");
  if (N < 1 || N > ZS_MAX_REPLICAS) return fail(ZS_ERR_RANGE, "N must be in [1, %d] (got %d)", ZS_MAX_REPLICAS, N);
  if (n < 0) return fail(ZS_ERR_RANGE, "n must be >= 0");
  zs::WriteWindow w{};
  zs::FlatSchedule sched = reduce_schedule(N, n, &w);
  // the kernels' own size conditions (a shard on a common 128-byte line phase)
  if (sched == zs::FlatSchedule::kWindowed && (w.period_mask == 0 || n / kTileElems < zs::kReduceWindowMinTiles))
    sched = zs::FlatSchedule::kStream;
  if (sched == zs::FlatSchedule::kPhased && n / (8 * zs::kFlatBlock) < 1) sched = zs::FlatSchedule::kStream;
  *schedule = (int32_t)sched;
  return ZS_OK;
}

zs_status zs_flat_schedule(int32_t N, int64_t n, int32_t* schedule) {
  g_last_error.clear();
  if (!schedule) return fail(ZS_ERR_NULL, "schedule is NULL");
  if (N < 1 || N > ZS_MAX_REPLICAS) return fail(ZS_ERR_RANGE, "N must be in [1, %d] (got %d)", ZS_MAX_REPLICAS, N);
  if (n < 0) return fail(ZS_ERR_RANGE, "n must be >= 0");
  zs::WriteWindow w{};
  zs::FlatSchedule sched = flat_schedule(N, n, &w);
  const int64_t tiles = n / 8 / zs::kFlatBlock;
  // the kernels' own size conditions (a shard on a common 128-byte line phase)
  if (sched == zs::FlatSchedule::kWindowed && (w.period_mask == 0 || tiles < zs::kWindowMinTiles))
    sched = zs::FlatSchedule::kStream;
  if (sched == zs::FlatSchedule::kPhased && tiles < 1) sched = zs::FlatSchedule::kStream;
  *schedule = (int32_t)sched;
  return ZS_OK;
}

zs_status zs_list_schedule(const zs_tensor* tensors, int32_t T, int32_t N, int32_t* schedule) {
  try {
    g_last_error.clear();
    if (!schedule) return fail(ZS_ERR_NULL, "schedule is NULL");
    ListTable tab;
    zs_status st = build_list_table(tensors, T, N, tab);
    if (st) return st;
    zs::WriteWindow w{};
    zs::FlatSchedule sched = flat_schedule(N, tab.n_params, &w, tab.n_items, tab.loose_items);
    // the windowed list kernel's size condition
    if (sched == zs::FlatSchedule::kWindowed &&
        (w.period_mask == 0 || tab.n_params < ((int64_t)zs::kWindowMinTiles << 9)))
      sched = zs::FlatSchedule::kStream;
    *schedule = (int32_t)sched;
    return ZS_OK;
  } catch (const std::bad_alloc&) {
    return fail(ZS_ERR_NOMEM, "host allocation failed");
  }
}

zs_status zs_set_phased_max_polls(int32_t polls) {
  g_last_error.clear();
  if (polls < 0) return fail(ZS_ERR_RANGE, "polls must be >= 0 (got %d)", polls);
  g_phased_max_polls.store(polls, std::memory_order_relaxed);
  return ZS_OK;
}

zs_status zs_reduce_adam_flat(const uint16_t* const* grad_chunks, int32_t N, int64_t n, float* master, float* m,
                              float* v, uint16_t* param_bf16, const zs_adam_hp* hp, int64_t step,
                              zs_stream stream) {
  return flat_step(grad_chunks, N, n, master, m, v, param_bf16, hp, step, nullptr, stream,
                   "zs_reduce_adam_flat launch");
}

zs_status zs_reduce_adam_flat_devstep(const uint16_t* const* grad_chunks, int32_t N, int64_t n, float* master,
                                      float* m, float* v, uint16_t* param_bf16, const zs_step_source* src,
                                      zs_stream stream) {
  if (!src) return fail(ZS_ERR_NULL, "src is NULL");
  return flat_step(grad_chunks, N, n, master, m, v, param_bf16, nullptr, 0, src, stream,
                   "zs_reduce_adam_flat_devstep launch");
}

zs_status zs_fold_table(const zs_adam_hp* hp, int64_t t0, int64_t count, zs_folded* out) {
  g_last_error.clear();
  if (!out) return fail(ZS_ERR_NULL, "out is NULL");
  if (count < 1 || count > (int64_t(1) << 40)) return fail(ZS_ERR_RANGE, "count must be in [1, 2^40]");
  zs_status st = check_hp(hp, t0);
  if (st) return st;
  for (int64_t k = 0; k < count; ++k) fold_scalars(*hp, t0 + k, out + k);
  return ZS_OK;
}

zs_status zs_step_advance(int64_t* step, zs_stream stream) {
  g_last_error.clear();
  if (!step) return fail(ZS_ERR_NULL, "step is NULL");
  if (!aligned(step, 8)) return fail(ZS_ERR_ALIGN, "step must be 8-byte aligned");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  return after_launch(zs::launch_step_advance(step, hs), hs, "zs_step_advance");
}

zs_status zs_list_plan_create(const zs_tensor* tensors, int32_t T, int32_t N, zs_stream stream,
                              zs_list_plan_t* out) {
  try {
    g_last_error.clear();
    if (!out) return fail(ZS_ERR_NULL, "out is NULL");
    *out = nullptr;
    ListTable tab;
    zs_status st = build_list_table(tensors, T, N, tab);
    if (st) return st;
    zs_list_plan* plan = new zs_list_plan();
    plan->N = N;
    plan->T = T;
    plan->n_items = tab.n_items;
    plan->loose_items = tab.loose_items;
    plan->n_params = tab.n_params;
    plan->n_groups = 1;
    plan->table = nullptr;
    if (hipGetDevice(&plan->device) != hipSuccess) plan->device = 0;
    const size_t bytes = tab.bytes.size();
    if (bytes > 0) {
      hipError_t e = hipMalloc(&plan->table, bytes);
      if (e != hipSuccess) {
        delete plan;
        (void)hipGetLastError();
        return fail(ZS_ERR_NOMEM, "plan table of %zu bytes: %s", bytes, hipGetErrorString(e));
      }
      hipStream_t hs = static_cast<hipStream_t>(stream);
      e = hipMemcpyAsync(plan->table, tab.bytes.data(), bytes, hipMemcpyHostToDevice, hs);
      if (e == hipSuccess) e = hipStreamSynchronize(hs);
      if (e != hipSuccess) {
        (void)hipFree(plan->table);
        delete plan;
        return hip_fail(e, "plan table upload");
      }
    }
    unsigned char* base = static_cast<unsigned char*>(plan->table);
    plan->items = reinterpret_cast<int32_t*>(base);
    plan->tensors = reinterpret_cast<zs::ListTensor*>(base + tab.off_tensors);
    plan->gptrs = reinterpret_cast<const uint16_t**>(base + tab.off_gptrs);
    *out = plan;
    return ZS_OK;
  } catch (const std::bad_alloc&) {
    return fail(ZS_ERR_NOMEM, "host allocation failed");
  } catch (...) {
    return fail(ZS_ERR_HIP, "unexpected exception");
  }
}

}  // extern "C"

namespace {

zs_status plan_on_current_device(zs_list_plan_t plan) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (cur != plan->device)  // the table lives in the other device's memory
    return fail(ZS_ERR_RANGE, "the plan was built on device %d, device %d is current", plan->device, cur);
  return ZS_OK;
}

// The list step over a device table (a plan's, or the fixed array of zs_reduce_adam_list_static).
zs_status launch_list_table(const int32_t* items, int32_t n_items, int32_t loose_items,
                            const zs::ListTensor* tensors, const uint16_t* const* gptrs, int32_t N, int64_t n_params,
                            const zs::Scalars* cs, int32_t n_sets, const zs::StepRef& ref, zs_stream stream) {
  hipStream_t hs = static_cast<hipStream_t>(stream);
  // the flat step's schedule for a shard of the plan's size, by the list rules; windows for plans of at
  // least 2^25 parameters
  zs::WriteWindow win{};
  const zs::FlatSchedule sched = flat_schedule(N, n_params, &win, n_items, loose_items);
  if (n_params < ((int64_t)zs::kWindowMinTiles << 9)) win = zs::WriteWindow{0, 0};
  return after_launch(zs::launch_list(items, n_items, tensors, gptrs, cs, n_sets, ref, auto_blocks(), sched, win,
                                      phased_ctl(), hs),
                      hs, "zs_reduce_adam_list launch");
}

// The step with `n` hyperparameter sets (one for every tensor, n == 1, or one
// per group), or with the device step of `src` (hps == NULL, n == 1).
zs_status run_plan(zs_list_plan_t plan, const zs_adam_hp* hps, int32_t n, int64_t step, const zs_step_source* src,
                   zs_stream stream) {
  zs::StepRef ref{};
  zs::Scalars cs[zs::kMaxGroups];
  if (src) {
    std::vector<Range> rs;
    zs_status st = step_ref_of(src, rs, &ref);
    if (st) return st;
    const zs_adam_hp placeholder = {0.0, 0.0, 0.0, 1.0, 0.0};  // the table supplies the folded scalars
    cs[0] = make_scalars(placeholder, 1, plan->N);
  } else {
    for (int32_t k = 0; k < n; ++k) {
      zs_status st = check_hp(hps + k, step);
      if (st) return st;
    }
    for (int32_t k = 0; k < n; ++k) cs[k] = make_scalars(hps[k], step, plan->N);
  }
  if (plan->n_items == 0) return ZS_OK;
  zs_status st = plan_on_current_device(plan);
  if (st) return st;
  return launch_list_table(plan->items, plan->n_items, plan->loose_items, plan->tensors, plan->gptrs, plan->N,
                           plan->n_params, cs, n, ref, stream);
}

}  // namespace

extern "C" {

zs_status zs_reduce_adam_list_plan(zs_list_plan_t plan, const zs_adam_hp* hp, int64_t step, zs_stream stream) {
  g_last_error.clear();
  if (!plan) return fail(ZS_ERR_NULL, "plan is NULL");
  return run_plan(plan, hp, 1, step, nullptr, stream);
}

zs_status zs_reduce_adam_list_plan_devstep(zs_list_plan_t plan, const zs_step_source* src, zs_stream stream) {
  g_last_error.clear();
  if (!plan) return fail(ZS_ERR_NULL, "plan is NULL");
  if (!src) return fail(ZS_ERR_NULL, "src is NULL");
  return run_plan(plan, nullptr, 1, 0, src, stream);
}

zs_status zs_list_plan_set_groups(zs_list_plan_t plan, const int32_t* group, int32_t n_groups, zs_stream stream) {
  g_last_error.clear();
  if (!plan) return fail(ZS_ERR_NULL, "plan is NULL");
  if (n_groups < 1 || n_groups > ZS_MAX_GROUPS)
    return fail(ZS_ERR_RANGE, "n_groups must be in [1, %d] (got %d)", ZS_MAX_GROUPS, n_groups);
  if (plan->T > 0 && !group) return fail(ZS_ERR_NULL, "group is NULL");
  for (int32_t t = 0; t < plan->T; ++t)
    if (group[t] < 0 || group[t] >= n_groups)
      return fail(ZS_ERR_RANGE, "group[%d] = %d is not in [0, %d)", t, group[t], n_groups);
  if (plan->T > 0) {
    zs_status st = plan_on_current_device(plan);
    if (st) return st;
    // each tensor descriptor's `group` field, one int32 every sizeof(ListTensor) bytes
    hipStream_t hs = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpy2DAsync(reinterpret_cast<char*>(plan->tensors) + offsetof(zs::ListTensor, group),
                                    sizeof(zs::ListTensor), group, sizeof(int32_t), sizeof(int32_t), (size_t)plan->T,
                                    hipMemcpyHostToDevice, hs);
    if (e == hipSuccess) e = hipStreamSynchronize(hs);  // `group` may be freed on return
    if (e != hipSuccess) return hip_fail(e, "group upload");
  }
  plan->n_groups = n_groups;
  return ZS_OK;
}

zs_status zs_reduce_adam_list_plan_groups(zs_list_plan_t plan, const zs_adam_hp* hps, int32_t n_groups,
                                          int64_t step, zs_stream stream) {
  g_last_error.clear();
  if (!plan) return fail(ZS_ERR_NULL, "plan is NULL");
  if (!hps) return fail(ZS_ERR_NULL, "hps is NULL");
  if (n_groups != plan->n_groups)
    return fail(ZS_ERR_RANGE, "the plan has %d groups, %d hyperparameter sets were given", plan->n_groups, n_groups);
  return run_plan(plan, hps, n_groups, step, nullptr, stream);
}

}  // extern "C"

namespace {

// Frees a plan; with wait_device, first waits for every stream of its device
// (the plan may have been launched on any of them).
void free_plan(zs_list_plan_t plan, bool wait_device) {
  if (!plan) return;
  if (plan->table) {
    int cur = 0;
    (void)hipGetDevice(&cur);
    (void)hipSetDevice(plan->device);
    if (wait_device) (void)hipDeviceSynchronize();
    (void)hipFree(plan->table);
    (void)hipSetDevice(cur);
  }
  delete plan;
}

}  // namespace

extern "C" {

void zs_list_plan_destroy(zs_list_plan_t plan) { free_plan(plan, true); }

zs_status zs_reduce_adam_list(const zs_tensor* tensors, int32_t T, int32_t N, const zs_adam_hp* hp, int64_t step,
                              zs_stream stream) {
  zs_status st = check_hp(hp, step);
  if (st) return st;
  zs_list_plan_t plan = nullptr;
  st = zs_list_plan_create(tensors, T, N, stream, &plan);
  if (st) return st;
  st = zs_reduce_adam_list_plan(plan, hp, step, stream);
  // the plan's only launch is on `stream`: once the stream is idle the table is free
  const hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (st == ZS_OK && e != hipSuccess) st = hip_fail(e, "zs_reduce_adam_list");
  free_plan(plan, e != hipSuccess);
  return st;
}

}  // extern "C"

// ---------------------------------------------------------------- no allocation
// The table of zs_reduce_adam_list_static lives here: device memory held by
// the library on each device it runs on, for the life of the process.  Host
// code never names this array as an address: it takes the device's address
// from hipGetSymbolAddress (scratch_address) and uses that.
constexpr size_t kStaticTableBytes = (size_t)ZS_STATIC_TABLE_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticTableBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[zs::kMaxDevices];  // per device: scratch's device address there

// scratch's address on the current device, looked up once per device with
// that device current.
zs_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= zs::kMaxDevices) return fail(ZS_ERR_RANGE, "device %d is beyond the library's %d", dev,
                                                     zs::kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ZS_OK;
}

}  // namespace

extern "C" {

zs_status zs_reduce_adam_list_static(const zs_tensor* tensors, int32_t T, int32_t N, const zs_adam_hp* hp,
                                     int64_t step, zs_stream stream) {
  try {
    g_last_error.clear();
    zs_status st = check_hp(hp, step);
    if (st) return st;
    // the host image of the table, kept per thread so that repeated calls reuse its memory
    thread_local ListTable tab;
    st = build_list_table(tensors, T, N, tab);
    if (st) return st;
    if (tab.bytes.size() > kStaticTableBytes)
      return fail(ZS_ERR_RANGE,
                  "the list's table needs %zu bytes (%d work items of up to %lld parameters, %d tensors, %d "
                  "replicas); zs_reduce_adam_list_static holds at most %zu: use zs_reduce_adam_list or a plan",
                  tab.bytes.size(), tab.n_items, (long long)zs::kTileElemsWave, T, N, kStaticTableBytes);
    if (tab.n_items == 0) return ZS_OK;
    void* base = nullptr;
    st = scratch_address(&base);
    if (st) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(base, tab.bytes.data(), tab.bytes.size(), hipMemcpyHostToDevice, hs);
    if (e != hipSuccess) return hip_fail(e, "table upload");
    unsigned char* b = static_cast<unsigned char*>(base);
    const zs::Scalars c = make_scalars(*hp, step, N);
    st = launch_list_table(reinterpret_cast<const int32_t*>(b), tab.n_items, tab.loose_items,
                           reinterpret_cast<const zs::ListTensor*>(b + tab.off_tensors),
                           reinterpret_cast<const uint16_t* const*>(b + tab.off_gptrs), N, tab.n_params, &c, 1,
                           zs::StepRef{}, stream);
    // the next call on this device rewrites the table, and the host image is reused: wait for this step
    e = hipStreamSynchronize(hs);
    if (st == ZS_OK && e != hipSuccess) st = hip_fail(e, "zs_reduce_adam_list_static");
    return st;
  } catch (const std::bad_alloc&) {
    return fail(ZS_ERR_NOMEM, "host allocation failed");
  } catch (...) {
    return fail(ZS_ERR_HIP, "unexpected exception");
  }
}

size_t zs_two_pass_workspace_bytes(int64_t n) {
  if (n < 0) return 0;
  return 255 + (((size_t)n * 4 + 255) & ~(size_t)255) + 8 * (partial_slots(n) + partial2_slots(n));
}

}  // extern "C"

namespace {

// Pass 1 with the loss scale given on the host (scale_state == NULL) or read
// on the device from scale_state->scale.
zs_status reduce_grads(const uint16_t* const* grad_chunks, int32_t N, int64_t n, int32_t grad_format,
                       double loss_scale, const zs_loss_scaler* scale_state, void* workspace,
                       size_t workspace_bytes, double* sqnorm, zs_stream stream, const char* what) {
  try {
    g_last_error.clear();
    if (N < 1 || N > ZS_MAX_REPLICAS) return fail(ZS_ERR_RANGE, "N must be in [1, %d] (got %d)", ZS_MAX_REPLICAS, N);
    if (n < 0 || n > (int64_t(1) << 56)) return fail(ZS_ERR_RANGE, "n out of range");
    if (grad_format != ZS_FORMAT_BF16 && grad_format != ZS_FORMAT_FP16)
      return fail(ZS_ERR_RANGE, "grad_format must be ZS_FORMAT_BF16 or ZS_FORMAT_FP16");
    if (!scale_state && (!(loss_scale > 0) || !std::isfinite(loss_scale)))
      return fail(ZS_ERR_RANGE, "loss_scale must be finite and > 0");
    if (scale_state && !aligned(scale_state, 8)) return fail(ZS_ERR_ALIGN, "the scaler state must be 8-byte aligned");
    if (!sqnorm) return fail(ZS_ERR_NULL, "sqnorm is NULL");
    if (!aligned(sqnorm, 8)) return fail(ZS_ERR_ALIGN, "sqnorm must be 8-byte aligned");
    if (n > 0 && !workspace) return fail(ZS_ERR_NULL, "workspace is NULL");
    std::vector<Range> rs;
    if (n > 0) {
      if (!grad_chunks) return fail(ZS_ERR_NULL, "grad_chunks is NULL");
      for (int32_t r = 0; r < N; ++r) {
        if (!grad_chunks[r]) return fail(ZS_ERR_NULL, "grad_chunks[%d] is NULL", r);
        if (!aligned(grad_chunks[r], 2)) return fail(ZS_ERR_ALIGN, "grad_chunks[%d] not 2-byte aligned", r);
        rs.push_back({(uintptr_t)grad_chunks[r], (uintptr_t)grad_chunks[r] + 2 * (uintptr_t)n, 1, 0});
      }
    }
    if (scale_state)  // read by the kernels: it must not overlap what they write
      rs.push_back({(uintptr_t)scale_state, (uintptr_t)scale_state + sizeof(zs_loss_scaler), 1, 0});
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const double host_scale = scale_state ? 1.0 : loss_scale;
    zs::TwoPassShape sh{};
    sh.sqnorm = sqnorm;
    sh.n = n;
    sh.n_rep = N;
    sh.inv_scale = (float)(1.0 / host_scale);
    if (n == 0) {  // an empty shard: only the (zero) norm is written
      sh.partials = nullptr;
      sh.ntiles = -1;
      rs.push_back({(uintptr_t)sqnorm, (uintptr_t)sqnorm + 8, 0, 1});
      zs_status st = check_alias(rs);
      if (st) return st;
    } else {
      const WorkspaceLayout L = layout_of(workspace, n);
      if (workspace_bytes < L.need)
        return fail(ZS_ERR_RANGE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, L.need);
      rs.push_back({(uintptr_t)workspace, (uintptr_t)workspace + L.need, 0, 0});
      rs.push_back({(uintptr_t)sqnorm, (uintptr_t)sqnorm + 8, 0, 1});
      zs_status st = check_alias(rs);
      if (st) return st;
      reduce_shape(grad_chunks, N, n, workspace, sqnorm, (float)(1.0 / host_scale), &sh);
    }
    sh.scale_dev = scale_state ? &scale_state->scale : nullptr;
    zs::WriteWindow w{};
    const zs::FlatSchedule sched = reduce_schedule(N, n, &w);
    sh.window = w;
    sh.phased = sched == zs::FlatSchedule::kPhased ? 1 : 0;
    sh.ctl = phased_ctl();
    return after_launch(zs::launch_reduce(grad_chunks, sh, grad_format, auto_blocks(), hs), hs, what);
  } catch (const std::bad_alloc&) {
    return fail(ZS_ERR_NOMEM, "host allocation failed");
  } catch (...) {
    return fail(ZS_ERR_HIP, "unexpected exception");
  }
}

}  // namespace

extern "C" {

zs_status zs_reduce_grads_flat(const uint16_t* const* grad_chunks, int32_t N, int64_t n, int32_t grad_format,
                               double loss_scale, void* workspace, size_t workspace_bytes, double* sqnorm,
                               zs_stream stream) {
  return reduce_grads(grad_chunks, N, n, grad_format, loss_scale, nullptr, workspace, workspace_bytes, sqnorm,
                      stream, "zs_reduce_grads_flat launch");
}

zs_status zs_reduce_grads_flat_device_scale(const uint16_t* const* grad_chunks, int32_t N, int64_t n,
                                            int32_t grad_format, const zs_loss_scaler* scale_state,
                                            void* workspace, size_t workspace_bytes, double* sqnorm,
                                            zs_stream stream) {
  if (!scale_state) return fail(ZS_ERR_NULL, "scale_state is NULL");
  return reduce_grads(grad_chunks, N, n, grad_format, 1.0, scale_state, workspace, workspace_bytes, sqnorm,
                      stream, "zs_reduce_grads_flat_device_scale launch");
}

zs_status zs_loss_scaler_update_device(zs_loss_scaler* state, const double* total_sq, int32_t* taken,
                                       zs_stream stream) {
  g_last_error.clear();
  if (!state || !total_sq) return fail(ZS_ERR_NULL, "state and total_sq must not be NULL");
  if (!aligned(state, 8) || !aligned(total_sq, 8) || (taken && !aligned(taken, 4)))
    return fail(ZS_ERR_ALIGN, "state and total_sq must be 8-byte aligned, taken 4-byte aligned");
  const uintptr_t s0 = (uintptr_t)state, s1 = s0 + sizeof(zs_loss_scaler);
  if (((uintptr_t)total_sq < s1 && s0 < (uintptr_t)total_sq + 8) ||
      (taken && (uintptr_t)taken < s1 && s0 < (uintptr_t)taken + 4))
    return fail(ZS_ERR_ALIAS, "total_sq or taken overlaps the scaler state");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  return after_launch(zs::launch_scaler_update(state, total_sq, taken, hs), hs, "zs_loss_scaler_update_device");
}

}  // extern "C"

namespace {

// Pass 2 with the step from the host (src == NULL) or the device.
zs_status gbar_step(const void* workspace, size_t workspace_bytes, int64_t n, float* master, float* m, float* v,
                    uint16_t* param_half, int32_t param_format, const zs_adam_hp* hp, int64_t step,
                    const zs_step_source* src, const double* total_sq, double max_norm, int32_t skip_nonfinite,
                    zs_stream stream, const char* what) {
  try {
    g_last_error.clear();
    zs_status st = ZS_OK;
    if (!src) {
      st = check_hp(hp, step);
      if (st) return st;
    }
    if (n < 0 || n > (int64_t(1) << 56)) return fail(ZS_ERR_RANGE, "n out of range");
    if (param_format != ZS_FORMAT_BF16 && param_format != ZS_FORMAT_FP16)
      return fail(ZS_ERR_RANGE, "param_format must be ZS_FORMAT_BF16 or ZS_FORMAT_FP16");
    if (!std::isfinite(max_norm)) return fail(ZS_ERR_RANGE, "max_norm must be finite (<= 0: no clipping)");
    if (n == 0) return ZS_OK;
    if (!workspace || !total_sq || !master || !m || !v || !param_half)
      return fail(ZS_ERR_NULL, "workspace, total_sq, master, m, v and param_half must be non-NULL");
    if (!aligned(total_sq, 8)) return fail(ZS_ERR_ALIGN, "total_sq must be 8-byte aligned");
    if (!aligned(master, 4) || !aligned(m, 4) || !aligned(v, 4) || !aligned(param_half, 2))
      return fail(ZS_ERR_ALIGN, "master/m/v must be 4-byte and param_half 2-byte aligned");
    const WorkspaceLayout L = layout_of(workspace, n);
    if (workspace_bytes < L.need)
      return fail(ZS_ERR_RANGE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, L.need);
    const uintptr_t n4 = (uintptr_t)n * 4, n2 = (uintptr_t)n * 2;
    std::vector<Range> rs = {{(uintptr_t)master, (uintptr_t)master + n4, 0, 0},
                             {(uintptr_t)m, (uintptr_t)m + n4, 0, 0},
                             {(uintptr_t)v, (uintptr_t)v + n4, 0, 0},
                             {(uintptr_t)param_half, (uintptr_t)param_half + n2, 0, 0},
                             {(uintptr_t)workspace, (uintptr_t)workspace + L.need, 1, 0},
                             {(uintptr_t)total_sq, (uintptr_t)total_sq + 8, 1, 0}};
    zs::StepRef ref{};
    if (src) {
      st = step_ref_of(src, rs, &ref);
      if (st) return st;
    }
    st = check_alias(rs);
    if (st) return st;
    zs::FlatShape s;
    s.p = master;
    s.m = m;
    s.v = v;
    s.b = param_half;
    s.n = n;
    const void* ptrs[5] = {L.gbar, master, m, v, param_half};
    const int sizes[5] = {4, 4, 4, 4, 2};
    const int64_t h = zs::common_peel_sized(ptrs, sizes, 5);
    if (h < 0 || n < h + 8) {
      s.head = 0;
      s.nvec = 0;
      s.scalar_only = 1;
    } else {
      s.head = h;
      s.nvec = (n - h) / 8;
      s.scalar_only = 0;
    }
    const zs_adam_hp placeholder = {0.0, 0.0, 0.0, 1.0, 0.0};  // a device step: the table supplies the scalars
    const zs::Scalars c = make_scalars(src ? placeholder : *hp, src ? 1 : step, 1);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    return after_launch(zs::launch_gbar(L.gbar, s, c, ref, total_sq, max_norm, skip_nonfinite, param_format,
                                        auto_blocks(), hs),
                        hs, what);
  } catch (const std::bad_alloc&) {
    return fail(ZS_ERR_NOMEM, "host allocation failed");
  } catch (...) {
    return fail(ZS_ERR_HIP, "unexpected exception");
  }
}

}  // namespace

extern "C" {

zs_status zs_adam_from_grads_flat(const void* workspace, size_t workspace_bytes, int64_t n, float* master, float* m,
                                  float* v, uint16_t* param_half, int32_t param_format, const zs_adam_hp* hp,
                                  int64_t step, const double* total_sq, double max_norm, int32_t skip_nonfinite,
                                  zs_stream stream) {
  return gbar_step(workspace, workspace_bytes, n, master, m, v, param_half, param_format, hp, step, nullptr,
                   total_sq, max_norm, skip_nonfinite, stream, "zs_adam_from_grads_flat launch");
}

zs_status zs_adam_from_grads_flat_devstep(const void* workspace, size_t workspace_bytes, int64_t n, float* master,
                                          float* m, float* v, uint16_t* param_half, int32_t param_format,
                                          const zs_step_source* src, const double* total_sq, double max_norm,
                                          int32_t skip_nonfinite, zs_stream stream) {
  if (!src) return fail(ZS_ERR_NULL, "src is NULL");
  return gbar_step(workspace, workspace_bytes, n, master, m, v, param_half, param_format, nullptr, 0, src,
                   total_sq, max_norm, skip_nonfinite, stream, "zs_adam_from_grads_flat_devstep launch");
}

zs_status zs_loss_scaler_init(zs_loss_scaler* s, double initial_scale, double min_scale, int64_t window,
                              int64_t hysteresis) {
  g_last_error.clear();
  if (!s) return fail(ZS_ERR_NULL, "scaler is NULL");
  if (!(min_scale > 0) || !(initial_scale >= min_scale) || !std::isfinite(initial_scale) || window < 1 ||
      hysteresis < 1)
    return fail(ZS_ERR_RANGE, "need 0 < min_scale <= initial_scale (finite), window >= 1, hysteresis >= 1");
  s->scale = initial_scale;
  s->min_scale = min_scale;
  s->window = window;
  s->hysteresis = hysteresis;
  s->overflows = 0;
  s->clean = 0;
  return ZS_OK;
}

int32_t zs_loss_scaler_update(zs_loss_scaler* s, int32_t overflow) {
  if (!s) return 0;
  if (overflow) {
    s->clean = 0;
    // the budget is spent by overflows and restored only by growth
    if (s->overflows < s->hysteresis) ++s->overflows;
    if (s->overflows >= s->hysteresis) {
      const double half = s->scale / 2.0;
      s->scale = half < s->min_scale ? s->min_scale : half;
    }
    return 0;
  }
  if (++s->clean >= s->window) {
    s->scale *= 2.0;
    s->clean = 0;
    s->overflows = 0;
  }
  return 1;
}

zs_status zs_list_plan_info(zs_list_plan_t plan, int64_t* n_params, int32_t* n_tensors, int32_t* n_items) {
  if (!plan) return fail(ZS_ERR_NULL, "plan is NULL");
  if (n_params) *n_params = plan->n_params;
  if (n_tensors) *n_tensors = plan->T;
  if (n_items) *n_items = plan->n_items;
  return ZS_OK;
}

}  // extern "C"
