// Measurement probe for the benchmark (libzshard_probe.so; not part of the
// library or its ABI).  Two instruments:
//
// 1. The fused step's exact HBM access pattern with the AdamW arithmetic taken
//    out, to measure what the memory system delivers for this mix of streams
//    on the box at hand.  Each workgroup takes one full 512-parameter tile (one
//    wave), as the flat kernel's workgroups do, with the same whole-line lane
//    layout, SGPR-base addressing, non-temporal accesses,
//    state-before-replicas load order and batched rank-ordered replica stream.
//    Then:
//      write = 0: nothing is stored: the read streams alone, (2N + 12) bytes
//                 per parameter.  Every loaded value feeds one sum that an
//                 empty asm statement consumes, so no load can be dropped or
//                 moved behind a branch;
//      write = 1: master, m, v and the 16-bit copy are written back with
//                 values that need one add per element: the full (2N + 26)
//                 bytes per parameter of the step;
//      windowed:  (zs_probe_pattern_windowed) the writes of write = 1 grouped
//                 in device-clock windows, as the windowed flat step writes.
//    Only full tiles are processed; the caller passes arrays that start on a
//    128-byte boundary.  The values written are meaningless: run the probe on
//    scratch state or after the state is no longer needed.
//
// 2. A copy (zs_probe_copy): the box's rate for an even read/write stream,
//    built the way the step's kernels are: one wave per 512-element fp32 tile,
//    the whole-line lane layout (every access instruction covers whole 128-byte
//    lines), SGPR-base addressing, non-temporal loads and stores, and
//    consecutive launches of at most 3e9 bytes each.
#include "zs_device.h"
#include "zs_phased.h"

namespace zs {
namespace {

using namespace dev;

template <int NT>
struct ProbeArgs {
  const uint16_t* g[NT];
  float* p;
  float* m;
  float* v;
  uint16_t* b;
};

template <int NT, bool WRITE>
__global__ __launch_bounds__(kFlatBlock) void pattern_kernel(const ProbeArgs<NT> a) {
  constexpr uint32_t q2 = Layout::kSecond / 4;
  const int64_t e0 = (int64_t)blockIdx.x * (kFlatBlock * 8);
  const uint32_t e = Layout::first();
  f32x4 pa, pb, ma, mb, va, vb;
  {
    const uint32_t o = here(e) * 4u;
    const GLB f32x4* P4 = (const GLB f32x4*)at(tile_base(a.p + e0), o);
    const GLB f32x4* M4 = (const GLB f32x4*)at(tile_base(a.m + e0), o);
    const GLB f32x4* V4 = (const GLB f32x4*)at(tile_base(a.v + e0), o);
    pa = ld_g(P4);
    pb = ld_g(P4 + q2);
    ma = ld_g(M4);
    mb = ld_g(M4 + q2);
    va = ld_g(V4);
    vb = ld_g(V4 + q2);
  }
  auto G = [&](int r) { return tile_base(a.g[r] + e0); };
  float acc[8];
  reduce_replicas<NT>(G, NT, e, acc);
  float p[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
  float m[8] = {ma.x, ma.y, ma.z, ma.w, mb.x, mb.y, mb.z, mb.w};
  float v[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
  if constexpr (WRITE) {
#pragma unroll
    for (int k = 0; k < 8; ++k) p[k] = p[k] + acc[k];
    const uint32_t o = here(e) * 4u;
    GLB f32x4* P4 = (GLB f32x4*)at(tile_base(a.p + e0), o);
    GLB f32x4* M4 = (GLB f32x4*)at(tile_base(a.m + e0), o);
    GLB f32x4* V4 = (GLB f32x4*)at(tile_base(a.v + e0), o);
    st_g(P4, (f32x4){p[0], p[1], p[2], p[3]});
    st_g(P4 + q2, (f32x4){p[4], p[5], p[6], p[7]});
    st_g(M4, (f32x4){acc[0], acc[1], acc[2], acc[3]});
    st_g(M4 + q2, (f32x4){acc[4], acc[5], acc[6], acc[7]});
    st_g(V4, (f32x4){v[0] + m[0], v[1] + m[1], v[2] + m[2], v[3] + m[3]});
    st_g(V4 + q2, (f32x4){v[4] + m[4], v[5] + m[5], v[6] + m[6], v[7] + m[7]});
    GLB u32x2* B2 = (GLB u32x2*)at(tile_base(a.b + e0), here(e) * 2u);
    st_g(B2, (u32x2){pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])});
    st_g(B2 + Layout::kSecond / 4, (u32x2){pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])});
  } else {
    float x = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) x = x + acc[k] + p[k] + m[k] + v[k];
    asm volatile("" ::"v"(x));
  }
}

// write = 2: the writes of write = 1, grouped in device-clock windows as the
// windowed flat step groups them (persistent one-wave workgroups, up to two
// finished tiles held, the same clock checks in the replica stream and the
// same pauses of all loads while a window is open).
template <int NT>
__global__ __launch_bounds__(kFlatBlock) void pattern_window_kernel(const ProbeArgs<NT> a, int64_t tiles,
                                                                    const WriteWindow w) {
  constexpr uint32_t q2 = Layout::kSecond / 4;
  const uint32_t e = Layout::first();
  FlatShape s{};
  s.p = a.p;
  s.m = a.m;
  s.v = a.v;
  s.b = a.b;
  HeldTiles held;
  auto check = [&]() { held.check(s, w); };
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int64_t e0 = t * (kFlatBlock * 8);
    f32x4 pa, pb, ma, mb, va, vb;
    {
      const uint32_t o = here(e) * 4u;
      const GLB f32x4* P4 = (const GLB f32x4*)at(tile_base(a.p + e0), o);
      const GLB f32x4* M4 = (const GLB f32x4*)at(tile_base(a.m + e0), o);
      const GLB f32x4* V4 = (const GLB f32x4*)at(tile_base(a.v + e0), o);
      pa = ld_g(P4);
      pb = ld_g(P4 + q2);
      ma = ld_g(M4);
      mb = ld_g(M4 + q2);
      va = ld_g(V4);
      vb = ld_g(V4 + q2);
    }
    auto G = [&](int r) { return tile_base(a.g[r] + e0); };
    float acc[8];
    reduce_replicas_hooked<NT, kWindowChecks>(G, e, acc, check);
    float p[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
    float m[8] = {ma.x, ma.y, ma.z, ma.w, mb.x, mb.y, mb.z, mb.w};
    float v[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      p[k] = p[k] + acc[k];
      v[k] = v[k] + m[k];
      m[k] = acc[k];
    }
    held.push(s, e0, tile_outputs(p, m, v));
  }
  held.flush(s);
}

template <int NT>
hipError_t go_window(const uint16_t* const* g, int64_t tiles, float* p, float* m, float* v, uint16_t* b,
                     const WriteWindow& w, hipStream_t stream) {
  ProbeArgs<NT> a;
  for (int r = 0; r < NT; ++r) a.g[r] = g[r];
  a.p = p;
  a.m = m;
  a.v = v;
  a.b = b;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, pattern_window_kernel<NT>, kFlatBlock, 0) != hipSuccess ||
      cus * per_cu < 1)
    return hipErrorInvalidValue;
  const int64_t grid = (int64_t)cus * per_cu < tiles ? (int64_t)cus * per_cu : tiles;
  (void)hipGetLastError();
  pattern_window_kernel<NT><<<dim3((unsigned)grid), dim3(kFlatBlock), 0, stream>>>(a, tiles, w);
  return hipGetLastError();
}

template <int NT>
hipError_t go(const uint16_t* const* g, int64_t tiles, float* p, float* m, float* v, uint16_t* b, int write,
              hipStream_t stream) {
  ProbeArgs<NT> a;
  for (int r = 0; r < NT; ++r) a.g[r] = g[r];
  a.p = p;
  a.m = m;
  a.v = v;
  a.b = b;
  (void)hipGetLastError();
  if (write)
    pattern_kernel<NT, true><<<dim3((unsigned)tiles), dim3(kFlatBlock), 0, stream>>>(a);
  else
    pattern_kernel<NT, false><<<dim3((unsigned)tiles), dim3(kFlatBlock), 0, stream>>>(a);
  return hipGetLastError();
}

// One 512-element fp32 tile per one-wave workgroup, tiles [t0, t0 + gridDim.x);
// the workgroup holding the last tile also copies the tail elements.
__global__ __launch_bounds__(kFlatBlock) void copy_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                          int64_t t0, int64_t n) {
  constexpr uint32_t q2 = Layout::kSecond / 4;
  const int64_t t = t0 + blockIdx.x;
  const int64_t e0 = t * (kFlatBlock * 8);
  if (e0 + kFlatBlock * 8 <= n) {
    const uint32_t o = here(Layout::first()) * 4u;
    const GLB f32x4* S = (const GLB f32x4*)at(tile_base(src + e0), o);
    GLB f32x4* D = (GLB f32x4*)at(tile_base(dst + e0), o);
    const f32x4 x = ld_g(S), y = ld_g(S + q2);
    st_g(D, x);
    st_g(D + q2, y);
  } else {
    for (int64_t i = e0 + threadIdx.x; i < n; i += kFlatBlock) dst[i] = src[i];
  }
}

// The phased schedule's pattern (zs_probe_pattern_phased): the library's own
// super-chunk loop (zs_phased.h), its AdamW replaced by the write = 1 values.
template <int NT>
__global__ __launch_bounds__(kFlatBlock* kPhasedWaves) void pattern_phased_kernel(const ProbeArgs<NT> a, int64_t n,
                                                                                   int32_t slot, int64_t* covered) {
  FlatShape s{};
  s.p = a.p;
  s.m = a.m;
  s.v = a.v;
  s.b = a.b;
  s.n = n;
  s.head = 0;
  s.nvec = n / 8;
  auto G = [&](int r) { return a.g[r]; };
  const int64_t t = phased_super_chunks<NT>(G, NT, s, slot, kPhasedMaxPolls,
                                            [](const float(&acc)[8], float(&p)[8], float(&m)[8], float(&v)[8]) {
#pragma unroll
                                              for (int k = 0; k < 8; ++k) {
                                                p[k] = p[k] + acc[k];
                                                v[k] = v[k] + m[k];
                                                m[k] = acc[k];
                                              }
                                            });
  if (blockIdx.x == 0 && threadIdx.x == 0) *covered = t * (kFlatBlock * 8);
}

bool line_aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 127) == 0; }

}  // namespace
}  // namespace zs

// Runs the windowed write pattern (write = 2 above) over the n / 512 full
// tiles, with the write window period_ticks / open_ticks (ticks of the 100 MHz
// device clock; the period a power of two in [64, 2^20], 1 <= open_ticks <
// period, open_ticks <= 2^14).  Returns as zs_probe_pattern.
extern "C" __attribute__((visibility("default"))) int zs_probe_pattern_windowed(
    const uint16_t* const* g, int32_t N, int64_t n, float* p, float* m, float* v, uint16_t* b, int32_t period_ticks,
    int32_t open_ticks, void* stream) {
  using namespace zs;
  const int64_t tiles = n / (kFlatBlock * 8);
  if (tiles < 1 || !g || !p || !m || !v || !b) return 1;
  if (period_ticks < kWindowMinPeriod || period_ticks > kWindowMaxPeriod || (period_ticks & (period_ticks - 1)) ||
      open_ticks < 1 || open_ticks >= period_ticks || open_ticks > kWindowMaxOpen)
    return 1;
  if (!line_aligned(p) || !line_aligned(m) || !line_aligned(v) || !line_aligned(b)) return 1;
  for (int32_t r = 0; r < N; ++r)
    if (!g[r] || !line_aligned(g[r])) return 1;
  const WriteWindow w{(uint64_t)period_ticks - 1, (uint64_t)open_ticks};
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (N) {
    case 2: e = go_window<2>(g, tiles, p, m, v, b, w, s); break;
    case 8: e = go_window<8>(g, tiles, p, m, v, b, w, s); break;
    case 16: e = go_window<16>(g, tiles, p, m, v, b, w, s); break;
    case 64: e = go_window<64>(g, tiles, p, m, v, b, w, s); break;
    default: return 1;
  }
  return e == hipSuccess ? 0 : 2;
}

// Runs the probe over the n / 512 full tiles of the shard on `stream`.
// Returns 0 on success, 1 for unsupported arguments (N not 2, 8, 16 or 64,
// fewer than 512 parameters, an array not on a 128-byte boundary), 2 for a
// launch error.
extern "C" __attribute__((visibility("default"))) int zs_probe_pattern(const uint16_t* const* g, int32_t N,
                                                                       int64_t n, float* p, float* m, float* v,
                                                                       uint16_t* b, int32_t write, void* stream) {
  using namespace zs;
  const int64_t tiles = n / (kFlatBlock * 8);
  if (tiles < 1 || tiles > 0x7FFFFFFF || !g || !p || !m || !v || !b) return 1;
  if (!line_aligned(p) || !line_aligned(m) || !line_aligned(v) || !line_aligned(b)) return 1;
  for (int32_t r = 0; r < N; ++r)
    if (!g[r] || !line_aligned(g[r])) return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (N) {
    case 2: e = go<2>(g, tiles, p, m, v, b, write, s); break;
    case 8: e = go<8>(g, tiles, p, m, v, b, write, s); break;
    case 16: e = go<16>(g, tiles, p, m, v, b, write, s); break;
    case 64: e = go<64>(g, tiles, p, m, v, b, write, s); break;
    default: return 1;
  }
  return e == hipSuccess ? 0 : 2;
}

// Copies n fp32 values src -> dst on `stream` (the arrays must not overlap and
// must be 16-byte aligned).  Returns 0 on success, 1 for bad arguments, 2 for
// a launch error.
extern "C" __attribute__((visibility("default"))) int zs_probe_copy(const float* src, float* dst, int64_t n,
                                                                    void* stream) {
  using namespace zs;
  if (n < 0 || (n > 0 && (!src || !dst))) return 1;
  if (((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u) != 0) return 1;
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  if (n > 0 && s0 < d0 + 4 * (uintptr_t)n && d0 < s0 + 4 * (uintptr_t)n) return 1;
  constexpr int64_t kTile = kFlatBlock * 8;
  const int64_t tiles = (n + kTile - 1) / kTile;
  const int64_t per = kLaunchBytes / (8 * kTile);  // tiles per launch: 8 bytes per element
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int64_t t0 = 0; t0 < tiles; t0 += per) {
    const int64_t cnt = tiles - t0 < per ? tiles - t0 : per;
    (void)hipGetLastError();
    copy_kernel<<<dim3((unsigned)cnt), dim3(kFlatBlock), 0, s>>>(src, dst, t0, n);
    if (hipGetLastError() != hipSuccess) return 2;
  }
  return 0;
}

// The phased pattern over the whole super-chunks of the n-parameter arrays (N =
// 64 only), one workgroup of 12 waves per compute unit; *covered (device
// int64) receives the number of parameters it covered.  Returns as
// zs_probe_pattern.
extern "C" __attribute__((visibility("default"))) int zs_probe_pattern_phased(
    const uint16_t* const* g, int32_t N, int64_t n, float* p, float* m, float* v, uint16_t* b, int64_t* covered,
    void* stream) {
  using namespace zs;
  if (N != 64 || n < kFlatBlock * 8 || !g || !p || !m || !v || !b || !covered) return 1;
  if (!line_aligned(p) || !line_aligned(m) || !line_aligned(v) || !line_aligned(b)) return 1;
  for (int32_t r = 0; r < N; ++r)
    if (!g[r] || !line_aligned(g[r])) return 1;
  ProbeArgs<64> a;
  for (int r = 0; r < 64; ++r) a.g[r] = g[r];
  a.p = p;
  a.m = m;
  a.v = v;
  a.b = b;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, pattern_phased_kernel<64>, kFlatBlock * kPhasedWaves,
                                                   0) != hipSuccess ||
      cus * per_cu < 1)
    return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  phased_clear_kernel<<<dim3(1), dim3(64), 0, s>>>(0);
  pattern_phased_kernel<64><<<dim3(cus * per_cu), dim3(kFlatBlock * kPhasedWaves), 0, s>>>(a, n, 0, covered);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
