// Optimizer-offload path: the rank's fp32 master, momentum and variance live
// in host memory (ZeRO-Offload, "Почему training 70B модели требует optimizer
// sharding (ZeRO-3)?", §6-§8: offload_optimizer to the CPU, pinned memory).
//
// Per chunk of the shard, pipelined two chunks deep:
//   GPU    reduce the N replicas into an fp32 gradient (the two-pass form's
//          pass 1 kernel) on the caller's stream;
//   PCIe   copy it into a pinned host buffer (4 B/param down);
//   CPU    AdamW on the host state, bf16 copy into a pinned buffer;
//   PCIe   copy the bf16 copy to the device working copy (2 B/param up), on the
//          context's own stream.
// While the CPU updates chunk k, the GPU reduces and copies chunk k+1 (and
// k+2 is queued).  Results are bit-identical to the fused device step.
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "zs_cpu_adam.h"
#include "zs_internal.h"
#include "zs_twopass.h"

namespace zs {
zs_status offload_fail(zs_status st, const char* msg);
bool offload_fold(const zs_adam_hp* hp, int64_t step, HostScalars* out);
bool offload_reduce_shape(const uint16_t* const* grads, int32_t N, int64_t n, void* ws, double* sq, TwoPassShape* sh);
int offload_blocks();
}  // namespace zs

struct zs_offload {
  int device = -1;
  int64_t chunk = 0;
  int threads = 1;
  size_t ws_bytes = 0;
  void* ws[2] = {nullptr, nullptr};        // device: pass-1 workspaces
  double* sq = nullptr;                    // device: unused norm slot
  float* hg[2] = {nullptr, nullptr};       // pinned: gradient chunks
  uint16_t* hb[2] = {nullptr, nullptr};    // pinned: bf16 chunks
  hipStream_t up = nullptr;                // host-to-device copies
  hipEvent_t ev_down[2] = {nullptr, nullptr}, ev_up[2] = {nullptr, nullptr}, ev_done = nullptr;
  hipEvent_t ev_start = nullptr;           // orders the copy stream after the caller's stream
};

namespace {

// Frees every buffer, stream and event the context holds (on its device).
void free_resources(zs_offload* c) {
  if (c->device >= 0) {
    int cur = 0;
    (void)hipGetDevice(&cur);
    (void)hipSetDevice(c->device);
    if (c->up) (void)hipStreamSynchronize(c->up);
    for (int s = 0; s < 2; ++s) {
      if (c->ws[s]) (void)hipFree(c->ws[s]);
      if (c->hg[s]) (void)hipHostFree(c->hg[s]);
      if (c->hb[s]) (void)hipHostFree(c->hb[s]);
      if (c->ev_down[s]) (void)hipEventDestroy(c->ev_down[s]);
      if (c->ev_up[s]) (void)hipEventDestroy(c->ev_up[s]);
    }
    if (c->sq) (void)hipFree(c->sq);
    if (c->ev_done) (void)hipEventDestroy(c->ev_done);
    if (c->ev_start) (void)hipEventDestroy(c->ev_start);
    if (c->up) (void)hipStreamDestroy(c->up);
    (void)hipSetDevice(cur);
  }
  const int64_t chunk = c->chunk;
  const int threads = c->threads;
  *c = zs_offload{};
  c->chunk = chunk;
  c->threads = threads;
}

void release(zs_offload* c) {
  if (!c) return;
  free_resources(c);
  delete c;
}

// Allocates the buffers on the current device at the first step.
hipError_t ensure(zs_offload* c) {
  if (c->device >= 0) return hipSuccess;
  hipError_t e = hipGetDevice(&c->device);
  if (e != hipSuccess) return e;
  c->ws_bytes = zs_two_pass_workspace_bytes(c->chunk);
  for (int s = 0; s < 2 && e == hipSuccess; ++s) {
    e = hipMalloc(&c->ws[s], c->ws_bytes);
    if (e == hipSuccess) e = hipHostMalloc((void**)&c->hg[s], 4 * (size_t)c->chunk, hipHostMallocDefault);
    if (e == hipSuccess) e = hipHostMalloc((void**)&c->hb[s], 2 * (size_t)c->chunk, hipHostMallocDefault);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_down[s], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_up[s], hipEventDisableTiming);
  }
  if (e == hipSuccess) e = hipMalloc((void**)&c->sq, 8);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_done, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_start, hipEventDisableTiming);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&c->up, hipStreamNonBlocking);
  if (e != hipSuccess) free_resources(c);  // the next step starts from scratch
  return e;
}

zs_status run_step(zs_offload* ctx, const uint16_t* const* grad_chunks, int32_t N, int64_t n, float* master,
                   float* m, float* v, uint16_t* param_dev, const zs::HostScalars& c, hipStream_t hs);

}  // namespace

extern "C" {

zs_status zs_offload_create(int64_t chunk_elems, int32_t threads, zs_offload_t* out) {
  if (!out) return zs::offload_fail(ZS_ERR_NULL, "out is NULL");
  *out = nullptr;
  if (chunk_elems < 2048 || chunk_elems > (int64_t(1) << 32))
    return zs::offload_fail(ZS_ERR_RANGE, "chunk_elems must be in [2048, 2^32]");
  if (threads < 1 || threads > 1024) return zs::offload_fail(ZS_ERR_RANGE, "threads must be in [1, 1024]");
  zs_offload* c = new (std::nothrow) zs_offload();
  if (!c) return zs::offload_fail(ZS_ERR_NOMEM, "host allocation failed");
  c->chunk = (chunk_elems + 7) & ~int64_t(7);
  c->threads = threads;
  *out = c;
  return ZS_OK;
}

void zs_offload_destroy(zs_offload_t ctx) { release(ctx); }

zs_status zs_cpu_adam(const float* gbar, int64_t n, float* master, float* m, float* v, uint16_t* param_bf16,
                      const zs_adam_hp* hp, int64_t step, int32_t threads) {
  zs::HostScalars c;
  if (!zs::offload_fold(hp, step, &c)) return ZS_ERR_RANGE;  // detail already set
  if (n < 0) return zs::offload_fail(ZS_ERR_RANGE, "n must be >= 0");
  if (n == 0) return ZS_OK;
  if (!gbar || !master || !m || !v || !param_bf16) return zs::offload_fail(ZS_ERR_NULL, "NULL array");
  if (threads < 1) threads = 1;
  try {
    zs::cpu_adam(gbar, n, master, m, v, param_bf16, c, threads);
  } catch (...) {
    return zs::offload_fail(ZS_ERR_HIP, "host error (thread creation)");
  }
  return ZS_OK;
}

zs_status zs_offload_step_flat(zs_offload_t ctx, const uint16_t* const* grad_chunks, int32_t N, int64_t n,
                               float* master, float* m, float* v, uint16_t* param_dev, const zs_adam_hp* hp,
                               int64_t step, zs_stream stream) {
  if (!ctx) return zs::offload_fail(ZS_ERR_NULL, "ctx is NULL");
  zs::HostScalars c;
  if (!zs::offload_fold(hp, step, &c)) return ZS_ERR_RANGE;
  if (N < 1 || N > ZS_MAX_REPLICAS) return zs::offload_fail(ZS_ERR_RANGE, "N out of range");
  if (n < 0) return zs::offload_fail(ZS_ERR_RANGE, "n must be >= 0");
  if (n == 0) return ZS_OK;
  if (!grad_chunks || !master || !m || !v || !param_dev) return zs::offload_fail(ZS_ERR_NULL, "NULL array");
  for (int32_t r = 0; r < N; ++r)
    if (!grad_chunks[r]) return zs::offload_fail(ZS_ERR_NULL, "grad_chunks[r] is NULL");
  if (((uintptr_t)param_dev & 1) || ((uintptr_t)master & 3) || ((uintptr_t)m & 3) || ((uintptr_t)v & 3))
    return zs::offload_fail(ZS_ERR_ALIGN, "misaligned array");
  {
    const uintptr_t a[3] = {(uintptr_t)master, (uintptr_t)m, (uintptr_t)v};
    const uintptr_t len = 4 * (uintptr_t)n;
    for (int i = 0; i < 3; ++i)
      for (int j = i + 1; j < 3; ++j)
        if (a[i] < a[j] + len && a[j] < a[i] + len)
          return zs::offload_fail(ZS_ERR_ALIAS, "host master/m/v overlap");
    for (int32_t r = 0; r < N; ++r) {
      const uintptr_t g0 = (uintptr_t)grad_chunks[r], g1 = g0 + 2 * (uintptr_t)n;
      if ((uintptr_t)param_dev < g1 && g0 < (uintptr_t)param_dev + 2 * (uintptr_t)n)
        return zs::offload_fail(ZS_ERR_ALIAS, "param overlaps a gradient chunk");
    }
  }
  try {
    return run_step(ctx, grad_chunks, N, n, master, m, v, param_dev, c, static_cast<hipStream_t>(stream));
  } catch (const std::bad_alloc&) {
    return zs::offload_fail(ZS_ERR_NOMEM, "host allocation failed");
  } catch (...) {
    return zs::offload_fail(ZS_ERR_HIP, "host error (thread creation)");
  }
}

}  // extern "C"

namespace {

zs_status run_step(zs_offload* ctx, const uint16_t* const* grad_chunks, int32_t N, int64_t n, float* master,
                   float* m, float* v, uint16_t* param_dev, const zs::HostScalars& c, hipStream_t hs) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return zs::offload_fail(ZS_ERR_HIP, hipGetErrorString(e));
  if (ctx->device >= 0 && cur != ctx->device)
    return zs::offload_fail(ZS_ERR_RANGE, "the context belongs to another device than the current one");
  e = ensure(ctx);
  if (e != hipSuccess) return zs::offload_fail(ZS_ERR_HIP, hipGetErrorString(e));
  // the uploads run on the context's stream: order them after everything already on the caller's stream
  e = hipEventRecord(ctx->ev_start, hs);
  if (e == hipSuccess) e = hipStreamWaitEvent(ctx->up, ctx->ev_start, 0);
  if (e != hipSuccess) return zs::offload_fail(ZS_ERR_HIP, hipGetErrorString(e));
  const int64_t C = ctx->chunk;
  const int64_t K = (n + C - 1) / C;
  std::vector<const uint16_t*> g(N);

  auto enqueue_down = [&](int64_t k) -> hipError_t {
    const int s = (int)(k & 1);
    const int64_t lo = k * C, len = n - lo < C ? n - lo : C;
    for (int32_t r = 0; r < N; ++r) g[r] = grad_chunks[r] + lo;
    zs::TwoPassShape sh;
    if (!zs::offload_reduce_shape(g.data(), N, len, ctx->ws[s], ctx->sq, &sh)) return hipErrorInvalidValue;
    hipError_t er = zs::launch_reduce(g.data(), sh, 0, zs::offload_blocks(), hs);
    if (er == hipSuccess) er = hipMemcpyAsync(ctx->hg[s], sh.gbar, 4 * (size_t)len, hipMemcpyDeviceToHost, hs);
    if (er == hipSuccess) er = hipEventRecord(ctx->ev_down[s], hs);
    return er;
  };

  e = enqueue_down(0);
  if (e == hipSuccess && K > 1) e = enqueue_down(1);
  // A host exception (thread creation) inside the loop must not leave copies in flight
  // into buffers the caller may free: drain both streams before passing it on.
  try {
    for (int64_t k = 0; k < K && e == hipSuccess; ++k) {
      const int s = (int)(k & 1);
      const int64_t lo = k * C, len = n - lo < C ? n - lo : C;
      e = hipEventSynchronize(ctx->ev_down[s]);
      if (e == hipSuccess && k >= 2) e = hipEventSynchronize(ctx->ev_up[s]);  // its bf16 buffer is free
      if (e != hipSuccess) break;
      zs::cpu_adam(ctx->hg[s], len, master + lo, m + lo, v + lo, ctx->hb[s], c, ctx->threads);
      e = hipMemcpyAsync(param_dev + lo, ctx->hb[s], 2 * (size_t)len, hipMemcpyHostToDevice, ctx->up);
      if (e == hipSuccess) e = hipEventRecord(ctx->ev_up[s], ctx->up);
      if (e == hipSuccess && k + 2 < K) e = enqueue_down(k + 2);
    }
  } catch (...) {
    (void)hipStreamSynchronize(hs);
    (void)hipStreamSynchronize(ctx->up);
    throw;
  }
  if (e == hipSuccess) e = hipEventRecord(ctx->ev_done, ctx->up);
  if (e == hipSuccess) e = hipStreamWaitEvent(hs, ctx->ev_done, 0);  // later work on `stream` sees the copy
  if (e == hipSuccess) e = hipStreamSynchronize(ctx->up);
  if (e != hipSuccess) {
    (void)hipStreamSynchronize(hs);
    (void)hipStreamSynchronize(ctx->up);
    return zs::offload_fail(ZS_ERR_HIP, hipGetErrorString(e));
  }
  return ZS_OK;
}

}  // namespace
