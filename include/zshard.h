/*
 * libzshard — one ZeRO rank's optimizer-side step on one MI355X (gfx950) GPU.
 *
 * The step, per parameter of the rank's shard (all arithmetic IEEE binary32,
 * round to nearest even, one rounding per operation, no fused multiply-add, in
 * exactly this order):
 *
 *   reduce   s = G_0[i]; s = s + G_r[i] for r = 1..N-1;  g = s / N
 *            The reduce half of the gradient reduce-scatter: the rank keeps the
 *            average of the N data-parallel replicas' gradients for the
 *            parameters it owns ("Почему training 70B модели требует optimizer
 *            sharding (ZeRO-3)?", §5, ZeRO-3 step algorithm, steps 2-3; the
 *            average is the gradient-synchronisation equation of "Data
 *            Parallelism 数据并行（二）", section 数据并行训练（DP）, read as N
 *            terms).  Floating-point addition is not associative (same
 *            section), so the order is fixed: rank 0 first, up to N-1.
 *   update   m1 = b1*M + c1*g;  v1 = b2*V + c2*(g*g);  d = sqrt(v1)*rb + e
 *            p1 = dk*P - ss*(m1/d)
 *            Mixed-precision AdamW on the 16-byte-per-parameter state of the
 *            Data Parallelism page's appendix (fp32 master, fp32 momentum, fp32
 *            variance, bf16 working copy, bf16 gradient).  The pages print no
 *            update equations: these are Kingma & Ba's Adam (Algorithm 1,
 *            bias-corrected, eps after the square root) with Loshchilov &
 *            Hutter's decoupled weight decay scaled by lr.  Scalars are folded
 *            on the host in double and rounded once to fp32:
 *              b1 = beta1, c1 = 1-beta1, b2 = beta2, c2 = 1-beta2, e = eps,
 *              ss = lr/(1-beta1^t), rb = 1/sqrt(1-beta2^t), dk = 1-lr*weight_decay
 *   re-cast  B = bf16_rne(p1): the working copy the next parameter all-gather
 *            ships (ZeRO-3 page, §5).  NaN stays NaN (payload unspecified).
 *
 * Non-finite gradients propagate (no skipping, no clipping).
 *
 * Memory: every buffer is caller-owned device memory.  The library allocates
 * device memory only for list-plan tables.  Host arrays passed in (grad_chunks,
 * tensors) are read during the call and may be freed when it returns.
 *
 * Asynchrony: the step calls enqueue their kernel on `stream` and return (one
 * launch, or consecutive launches of a few GB each on long shards: see
 * zs_set_launch_bytes); the caller keeps the buffers alive until the stream
 * reaches the work.  Faults
 * during execution surface at the caller's next synchronisation.  Setting the
 * environment variable ZS_SYNC=1 makes every step call synchronise the stream
 * and report kernel errors itself.
 *
 * Errors: arguments are checked before anything is enqueued; on failure nothing
 * is launched, a status is returned and zs_last_error() gives a thread-local
 * description.  No C++ exception crosses this interface.
 */
#ifndef ZSHARD_H
#define ZSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define ZS_API __attribute__((visibility("default")))
#else
#define ZS_API
#endif

#define ZS_ABI_VERSION 1
/* Largest replica count N one call accepts (the N chunk pointers travel as
   kernel arguments). */
#define ZS_MAX_REPLICAS 256
/* Hyperparameter groups a list plan can carry (zs_list_plan_set_groups). */
#define ZS_MAX_GROUPS 8

/* A hipStream_t, passed as an opaque pointer; NULL is the null stream. */
typedef void* zs_stream;

/* Adam/AdamW hyperparameters, as doubles.  Valid: all finite, lr >= 0,
   0 <= beta1 < 1, 0 <= beta2 < 1, eps > 0, weight_decay >= 0 (decoupled,
   applied as p *= 1 - lr*weight_decay). */
typedef struct zs_adam_hp {
  double lr, beta1, beta2, eps, weight_decay;
} zs_adam_hp;

typedef enum zs_status {
  ZS_OK = 0,
  ZS_ERR_NULL = 1,  /* a required pointer is NULL */
  ZS_ERR_RANGE = 2, /* N, n, T, step or a hyperparameter out of range */
  ZS_ERR_ALIAS = 3, /* an output overlaps another output or a gradient */
  ZS_ERR_ALIGN = 4, /* a pointer is not naturally aligned (4 B fp32, 2 B bf16) */
  ZS_ERR_HIP = 5,   /* the HIP runtime reported an error */
  ZS_ERR_NOMEM = 6  /* a plan table could not be allocated */
} zs_status;

/* The fp32 scalars one step uses, as folded on the host. */
typedef struct zs_folded {
  float b1, c1, b2, c2, eps, ss, rb, dk;
} zs_folded;

/* ABI version of the loaded library (ZS_ABI_VERSION it was built with). */
ZS_API int zs_abi_version(void);

/* Static name of a status value. */
ZS_API const char* zs_status_string(int status);

/* Thread-local description of the last failure on this thread ("" if none). */
ZS_API const char* zs_last_error(void);

/* Folds the step's scalars exactly as the step calls do (host only, no GPU).
   step is the 1-based index of the update.  Errors: ZS_ERR_NULL, ZS_ERR_RANGE. */
ZS_API zs_status zs_fold(const zs_adam_hp* hp, int64_t step, zs_folded* out);

/* The step on one flat shard of n parameters.
     grad_chunks  host array of N device pointers; grad_chunks[r] holds replica
                  r's n bf16 gradients (raw bf16 bits).  Read only; the same
                  pointer may appear more than once.
     N            replicas, 1..ZS_MAX_REPLICAS
     n            parameters in the shard, >= 0 (0 is a no-op)
     master, m, v device fp32 arrays of n, updated in place
     param_bf16   device bf16 array of n, written (never read)
     hp, step     hyperparameters; step >= 1 is the 1-based index of this
                  update (the library keeps no state and never increments it)
     stream       the stream the kernel is enqueued on
   Layout: any natural alignment works; when every array can be brought to
   16-byte alignment by the same element offset, the kernel uses vector
   accesses for all but at most 70 elements.  It prefers an offset that puts
   every array on a 128-byte line boundary (arrays whose addresses agree
   modulo 128 bytes, in elements, run fastest).
   Errors: ZS_ERR_NULL, ZS_ERR_RANGE, ZS_ERR_ALIGN, ZS_ERR_ALIAS (outputs must
   be pairwise disjoint and disjoint from every gradient range), ZS_ERR_HIP. */
ZS_API zs_status zs_reduce_adam_flat(const uint16_t* const* grad_chunks, int32_t N, int64_t n, float* master,
                                     float* m, float* v, uint16_t* param_bf16, const zs_adam_hp* hp, int64_t step,
                                     zs_stream stream);

/* One tensor of a ragged per-layer list (the per-layer parameter lists a
   model's layers hand to the gradient hooks and the optimizer, "Data
   Parallelism 数据并行（二）", section on integrating data parallelism into
   backpropagation).  Same meaning as the flat call's arguments. */
typedef struct zs_tensor {
  int64_t n;
  float* master;
  float* m;
  float* v;
  uint16_t* param_bf16;
  const uint16_t* const* grad_chunks; /* host array of N device pointers */
} zs_tensor;

/* A device-resident work table for a fixed list of tensors (one entry per
   512-parameter wave tile, naming its tensor): built once, then one kernel
   per step covers every tensor.  Tensors that lie back to back in every array
   (one arena per array, no gaps) with one hyperparameter set are also one flat
   shard: zs_reduce_adam_flat over the arenas computes the same bits and ran
   about 2% faster than a plan on a list of 720 such tensors (N = 64). */
typedef struct zs_list_plan* zs_list_plan_t;

/* Validates the list (as the flat call, per tensor, plus: outputs of all
   tensors pairwise disjoint and disjoint from every gradient range), splits
   every tensor into wave tiles, and uploads the table on `stream`; returns after
   the upload has completed.  T >= 0 tensors, 1 <= N <= ZS_MAX_REPLICAS.
   Errors: ZS_ERR_NULL, ZS_ERR_RANGE, ZS_ERR_ALIGN, ZS_ERR_ALIAS, ZS_ERR_NOMEM,
   ZS_ERR_HIP. */
ZS_API zs_status zs_list_plan_create(const zs_tensor* tensors, int32_t T, int32_t N, zs_stream stream,
                                     zs_list_plan_t* out);

/* The step on every tensor of the plan: one kernel on `stream` (one launch,
   or consecutive launches over the work table, zs_set_launch_bytes).  The
   plan's table lives on the device that was current at creation; calling with
   another device current fails with ZS_ERR_RANGE. */
ZS_API zs_status zs_reduce_adam_list_plan(zs_list_plan_t plan, const zs_adam_hp* hp, int64_t step,
                                          zs_stream stream);

/* Hyperparameter groups for a plan's tensors: AdamW setups commonly give norms
   and biases no weight decay, as separate parameter groups (the pages use a
   single setting, which a plan without groups keeps).  group: host array of
   the plan's T group indices, each in [0, n_groups), copied into the plan's
   table on `stream` before the call returns; 1 <= n_groups <= ZS_MAX_GROUPS.
   Until groups are set every tensor is in group 0.  Errors: ZS_ERR_NULL,
   ZS_ERR_RANGE (bad count or index, or another device current), ZS_ERR_HIP. */
ZS_API zs_status zs_list_plan_set_groups(zs_list_plan_t plan, const int32_t* group, int32_t n_groups,
                                         zs_stream stream);

/* The step with one hyperparameter set per group: hps is a host array of the
   n_groups sets (n_groups as set on the plan); tensor t uses hps[group[t]].
   One kernel launch; the same arithmetic per tensor as the single-set call
   with that tensor's set.  zs_reduce_adam_list_plan still applies its one hp
   to every tensor, whatever the groups.  Errors as zs_reduce_adam_list_plan,
   and ZS_ERR_RANGE if n_groups differs from the plan's. */
ZS_API zs_status zs_reduce_adam_list_plan_groups(zs_list_plan_t plan, const zs_adam_hp* hps, int32_t n_groups,
                                                 int64_t step, zs_stream stream);

/* One-shot form: create a plan, run it, wait for the step to finish on
   `stream`, destroy the plan.  Blocks the calling thread. */
ZS_API zs_status zs_reduce_adam_list(const zs_tensor* tensors, int32_t T, int32_t N, const zs_adam_hp* hp,
                                     int64_t step, zs_stream stream);

/* For callers that cannot allocate device memory (code that must not call
   hipMalloc, such as tight serving loops or harnesses that forbid it): the
   one-shot list step of zs_reduce_adam_list, with the same arguments,
   checks, kernels and results, whose work table goes into a fixed array of
   ZS_STATIC_TABLE_BYTES (32 MiB) of device memory that the library holds on
   each device it runs on until the process ends, instead of a plan allocated
   and freed per call.  The call uploads the table on `stream`, runs the step
   there and waits for it (it blocks the calling thread), and calls no
   hipMalloc or hipFree.  The table takes 4 bytes per work item (a wave tile:
   512 parameters of a tensor, or fewer at either end), 64 per tensor and 8 per
   tensor per replica: a list whose table needs more returns ZS_ERR_RANGE
   (about 4 billion parameters in all for 1,000 tensors and N = 64).  Every call on
   a device shares that device's array and rewrites it: calls that overlap on
   one device (from other threads, or on other streams) race and must be
   serialised by the caller.  Errors as zs_reduce_adam_list, and ZS_ERR_RANGE
   for a table beyond the array. */
#define ZS_STATIC_TABLE_BYTES (32u << 20)
ZS_API zs_status zs_reduce_adam_list_static(const zs_tensor* tensors, int32_t T, int32_t N, const zs_adam_hp* hp,
                                            int64_t step, zs_stream stream);

/* ---------------------------------------------------------------------------
 * Device-resident step index, for training steps captured once in a HIP graph
 * and replayed: the step index (and with it the bias corrections) must then
 * change on every replay without host work.  The folded scalars of a range of
 * steps are computed on the host once (zs_fold_table, the same values zs_fold
 * gives) and kept in device memory; the kernels read the row of the current
 * step, *step, and zs_step_advance increments it on the device.
 * ------------------------------------------------------------------------- */
typedef struct zs_step_source {
  const zs_folded* table; /* device: the folded scalars of steps t0 .. t0 + count - 1, in order */
  int64_t t0;             /* the step of table[0], >= 1 */
  int64_t count;          /* rows in the table, >= 1 */
  const int64_t* step;    /* device: the step index the kernels use, read when they run */
  int32_t* status;        /* device, optional: set to 1 by a kernel that found *step outside the table */
} zs_step_source;

/* The folded scalars of steps t0 .. t0 + count - 1 into the host array out
   (count rows).  Errors: ZS_ERR_NULL, ZS_ERR_RANGE (as zs_fold, or count < 1). */
ZS_API zs_status zs_fold_table(const zs_adam_hp* hp, int64_t t0, int64_t count, zs_folded* out);

/* zs_reduce_adam_flat with the step taken from src on the device.  A step
   outside the table updates nothing (the whole launch skips) and sets
   *src->status to 1 if status is given.  src itself is read during the call
   (its pointers are device addresses, 8-byte aligned; status 4-byte).  Other
   arguments and errors as zs_reduce_adam_flat; ZS_ERR_ALIAS if the table,
   step or status overlap an output or each other. */
ZS_API zs_status zs_reduce_adam_flat_devstep(const uint16_t* const* grad_chunks, int32_t N, int64_t n,
                                             float* master, float* m, float* v, uint16_t* param_bf16,
                                             const zs_step_source* src, zs_stream stream);

/* *step += 1 on the device (one thread), enqueued on `stream`.  Errors:
   ZS_ERR_NULL, ZS_ERR_ALIGN, ZS_ERR_HIP. */
ZS_API zs_status zs_step_advance(int64_t* step, zs_stream stream);

/* The plan's step with the step index taken from src on the device (see
   zs_step_source; one hyperparameter set for every tensor, the table's).  The
   plan keeps no copy of its tensors' address ranges, so this call checks src
   within itself only: src's buffers must not overlap the plan's tensors.
   Errors: ZS_ERR_NULL, ZS_ERR_RANGE, ZS_ERR_ALIGN, ZS_ERR_ALIAS (within src),
   ZS_ERR_HIP. */
ZS_API zs_status zs_reduce_adam_list_plan_devstep(zs_list_plan_t plan, const zs_step_source* src, zs_stream stream);

/* Waits for the device to go idle, then frees the plan's table.  NULL is a no-op. */
ZS_API void zs_list_plan_destroy(zs_list_plan_t plan);

/* Shape of a plan: total parameters, tensors and work items (wave tiles, one
   workgroup each; any output may be NULL). */
ZS_API zs_status zs_list_plan_info(zs_list_plan_t plan, int64_t* n_params, int32_t* n_tensors, int32_t* n_items);

/* ---------------------------------------------------------------------------
 * Two-pass form: global-norm gradient clipping and fp16 loss scaling.
 *
 * Both need a quantity over the whole model (the gradient norm, or whether
 * any gradient overflowed) before any state may change: the gradient_clipping
 * and dynamic fp16 loss-scale settings of the DeepSpeed config in "Почему
 * training 70B модели требует optimizer sharding (ZeRO-3)?", §8.  Pass 1
 * reduces the replicas into an fp32 gradient (in a caller-provided workspace)
 * and this shard's squared norm; the caller sums the shards' squared norms
 * over ranks (one scalar; on one GPU it is this shard's own); pass 2 applies
 * AdamW with the clip coefficient, or skips the step on overflow.  Without
 * clipping or loss scaling the two passes give exactly the fused step.
 * ------------------------------------------------------------------------- */

/* Storage format of 16-bit gradients and working copies. */
#define ZS_FORMAT_BF16 0
#define ZS_FORMAT_FP16 1

/* Bytes of workspace the two passes need for a shard of n parameters (the
   fp32 gradient, one double per 2048-parameter tile and one per 4096 tiles
   for the norm, and alignment slack). */
ZS_API size_t zs_two_pass_workspace_bytes(int64_t n);

/* Pass 1.  g[i] = (s_i / N) * f32(1/loss_scale), s_i the rank-ordered sum of
   the replicas (bf16 or fp16 bits per grad_format), written into `workspace`;
   *sqnorm (device double) = sum of g[i]^2 in double, reduced per 2048-parameter
   tile and then over tiles in a fixed order (independent of the launch size).
   loss_scale > 0 (1 = no scaling).  Enqueues two kernels on `stream`.
   Errors: ZS_ERR_NULL, ZS_ERR_RANGE (also: workspace too small),
   ZS_ERR_ALIGN, ZS_ERR_ALIAS (workspace or sqnorm overlapping a gradient), ZS_ERR_HIP. */
ZS_API zs_status zs_reduce_grads_flat(const uint16_t* const* grad_chunks, int32_t N, int64_t n, int32_t grad_format,
                                      double loss_scale, void* workspace, size_t workspace_bytes, double* sqnorm,
                                      zs_stream stream);

/* Pass 2.  Reads *total_sq (device double, the global squared norm) when the
   kernel runs: if skip_nonfinite and it is not finite, nothing is written (the
   step is skipped, e.g. an fp16 overflow).  Otherwise, with
   k = f32(min(1, max_norm / (sqrt(total_sq) + 1e-6))) (k = 1 when max_norm <= 0),
   applies the update to g[i]*k from `workspace` (as written by pass 1 for the
   same n), updating master/m/v in place and writing param_half in
   param_format.  Errors: ZS_ERR_NULL, ZS_ERR_RANGE, ZS_ERR_ALIGN, ZS_ERR_ALIAS,
   ZS_ERR_HIP. */
ZS_API zs_status zs_adam_from_grads_flat(const void* workspace, size_t workspace_bytes, int64_t n, float* master,
                                         float* m, float* v, uint16_t* param_half, int32_t param_format,
                                         const zs_adam_hp* hp, int64_t step, const double* total_sq,
                                         double max_norm, int32_t skip_nonfinite, zs_stream stream);

/* zs_adam_from_grads_flat with the step taken from src on the device (see
   zs_step_source); a step outside the table updates nothing and sets
   *src->status.  Other arguments and errors as zs_adam_from_grads_flat. */
ZS_API zs_status zs_adam_from_grads_flat_devstep(const void* workspace, size_t workspace_bytes, int64_t n,
                                                 float* master, float* m, float* v, uint16_t* param_half,
                                                 int32_t param_format, const zs_step_source* src,
                                                 const double* total_sq, double max_norm, int32_t skip_nonfinite,
                                                 zs_stream stream);

/* Dynamic loss scale for fp16 training (the DeepSpeed fp16 block's
   loss_scale 0 = dynamic, initial_scale_power, loss_scale_window, hysteresis,
   min_loss_scale, in "Почему training 70B модели требует optimizer sharding
   (ZeRO-3)?", §8).  The state lives in host memory for zs_loss_scaler_update,
   or in device memory (a copy of an initialised host state) for
   zs_loss_scaler_update_device and zs_reduce_grads_flat_device_scale. */
typedef struct zs_loss_scaler {
  double scale, min_scale;
  int64_t window, hysteresis, overflows, clean;
} zs_loss_scaler;

/* scale = initial_scale; window >= 1; hysteresis >= 1; 0 < min_scale <= initial_scale. */
ZS_API zs_status zs_loss_scaler_init(zs_loss_scaler* s, double initial_scale, double min_scale, int64_t window,
                                     int64_t hysteresis);

/* Records one step's outcome and returns 1 if the step was taken.  On
   overflow the step is skipped, and the scale halves (not below min_scale) on
   every overflow from the `hysteresis`-th one counted since the budget was
   last restored.  After `window` consecutive clean steps the scale doubles,
   and only that growth restores the budget: a halving does not, nor does a
   clean step short of the window (DeepSpeed's default reading of the fp16
   block's hysteresis, which the page sets without defining it).
   state.overflows counts overflows since the last restore, up to hysteresis;
   state.clean counts clean steps since the last overflow or growth. */
ZS_API int32_t zs_loss_scaler_update(zs_loss_scaler* s, int32_t overflow);

/* The same update, on the device, enqueued on `stream` after the work that
   writes the global squared norm: a non-finite *total_sq is an overflow (the
   test pass 2 uses to skip the step).  state: device zs_loss_scaler, 8-byte
   aligned, read and written; total_sq: device double, read; taken: optional
   device int32, set to 1 if the step was taken and 0 if it was skipped.  No
   host synchronisation.  Errors: ZS_ERR_NULL, ZS_ERR_ALIGN, ZS_ERR_ALIAS
   (total_sq or taken inside the state), ZS_ERR_HIP. */
ZS_API zs_status zs_loss_scaler_update_device(zs_loss_scaler* state, const double* total_sq, int32_t* taken,
                                              zs_stream stream);

/* Pass 1 with the loss scale read on the device from scale_state->scale
   (device memory; the unscale factor is f32(1/scale), as in
   zs_reduce_grads_flat).  With zs_loss_scaler_update_device this keeps an fp16
   step free of host round trips.  Other arguments and errors as
   zs_reduce_grads_flat; the state must not overlap the workspace or sqnorm
   (ZS_ERR_ALIAS). */
ZS_API zs_status zs_reduce_grads_flat_device_scale(const uint16_t* const* grad_chunks, int32_t N, int64_t n,
                                                   int32_t grad_format, const zs_loss_scaler* scale_state,
                                                   void* workspace, size_t workspace_bytes, double* sqnorm,
                                                   zs_stream stream);

/* ---------------------------------------------------------------------------
 * Optimizer offload (ZeRO-Offload, "Почему training 70B модели требует
 * optimizer sharding (ZeRO-3)?", §6-§8): the rank's fp32 master, momentum and
 * variance stay in host memory and the update runs on the CPU.  The GPU
 * reduces the replicas chunk by chunk; each fp32 gradient chunk crosses PCIe
 * (4 B/param), the CPU updates the host state, and the bf16 working copy
 * returns to the device (2 B/param).  Chunks are pipelined so the GPU reduce,
 * both copies and the CPU update overlap.  Results equal the fused device
 * step bit for bit.
 * ------------------------------------------------------------------------- */
typedef struct zs_offload* zs_offload_t;

/* A context holding two pipeline slots of chunk_elems parameters (device
   workspaces, pinned host buffers, a copy stream); buffers are allocated on
   the current device at the first step.  2048 <= chunk_elems <= 2^32;
   threads = CPU threads for the update.  Errors: ZS_ERR_NULL, ZS_ERR_RANGE,
   ZS_ERR_NOMEM. */
ZS_API zs_status zs_offload_create(int64_t chunk_elems, int32_t threads, zs_offload_t* out);

/* One step with host-resident state.  grad_chunks: host array of N device
   pointers (bf16); master, m, v: HOST fp32 arrays of n, updated in place
   before the call returns; param_dev: DEVICE bf16 array of n.  The reduce
   kernels run on `stream`; the copies into param_dev run on the context's
   stream after all work already enqueued on `stream`, and work enqueued on
   `stream` after the call sees the new param_dev.  Blocks until the host
   state is updated.  A context is bound to the device current at its first
   step; calling it with another device current fails with ZS_ERR_RANGE.
   Errors: ZS_ERR_NULL, ZS_ERR_RANGE, ZS_ERR_ALIGN, ZS_ERR_ALIAS, ZS_ERR_NOMEM,
   ZS_ERR_HIP (after ZS_ERR_HIP or ZS_ERR_NOMEM the host state may be partly
   updated). */
ZS_API zs_status zs_offload_step_flat(zs_offload_t ctx, const uint16_t* const* grad_chunks, int32_t N, int64_t n,
                                      float* master, float* m, float* v, uint16_t* param_dev, const zs_adam_hp* hp,
                                      int64_t step, zs_stream stream);

/* Waits for the context's copies, frees its buffers.  NULL is a no-op. */
ZS_API void zs_offload_destroy(zs_offload_t ctx);

/* The host AdamW on its own (no GPU): master/m/v updated from gbar, bf16
   copy into param_bf16; all host arrays of n.  Errors: ZS_ERR_NULL, ZS_ERR_RANGE. */
ZS_API zs_status zs_cpu_adam(const float* gbar, int64_t n, float* master, float* m, float* v, uint16_t* param_bf16,
                             const zs_adam_hp* hp, int64_t step, int32_t threads);

/* Workgroups per launch for all later step calls in this process: 0 picks
   automatically from the device's compute-unit count.  Results do not depend
   on it (every element is computed by one thread with the same operations). */
ZS_API zs_status zs_set_grid_blocks(int32_t blocks);

/* The most algorithmic bytes one launch of a one-tile-per-workgroup kernel
   moves, for all later calls in this process: the flat step and list plans
   when they take no write windows, and both passes of the two-pass form
   (pass 1 when it takes none).  Such a call covers its shard in consecutive
   launches on its stream, each of whole tiles (whole work items for list plans)
   and at most this many bytes by the step's byte model, and always at least
   one tile.  On this memory system one long launch lost up to 13% against
   the same work cut into launches of 1.3-5 GB.  The windowed kernels are
   persistent and always one launch.  Results do not depend on the setting.
     bytes = 0: the defaults: 3e9, and 1e9 for pass 2 of the two-pass form
                (zs_adam_from_grads_flat and its device-step form), which ran
                2.5% faster at 0.75-1 GB than at 3 GB;
     bytes > 0: that limit (a value below one tile's bytes gives one tile per
                launch; INT64_MAX gives one launch per call).
   Errors: ZS_ERR_RANGE (bytes < 0). */
ZS_API zs_status zs_set_launch_bytes(int64_t bytes);
/* The limit in force (3e9 when none was set; pass 2 then takes 1e9). */
ZS_API int64_t zs_launch_bytes(void);

/* Write windows of the flat step (zs_reduce_adam_flat and its device-step
   form), of list plans (every list step call; a plan counts its total
   parameters) and of pass 1 of the two-pass form (zs_reduce_grads_flat and its
   device-scale form), for all later calls in this process.  The flat step
   writes 14 bytes per parameter back beside 2N + 12 read, pass 1 writes 4
   beside 2N; on this memory system the writes cost far less when grouped in
   time than when they trickle out beside the read streams.  On shards of at
   least 2^25 parameters, the kernel then runs as persistent workgroups that
   hold finished tiles in registers and store them while the device's 100 MHz
   real-time counter, taken modulo period_ticks, is below open_ticks; no loads
   are issued in that window.  Results do not depend on the setting: each tile's outputs are
   computed identically and written to their own addresses (pass 1's norm
   partials too).
     period_ticks = 0: the library's measured default (the default;
                       open_ticks is ignored): windows only on the windowed
                       schedule (zs_set_flat_schedule): a 4096-tick period
                       with 640 (N < 64), 512 (N <= 128) or 384 ticks open
                       for the flat step and list plans, 4096 / 256 for
                       pass 1;
     period_ticks = 1: no windows (tiles stored as they finish);
     otherwise a power of two in [64, 2^20], with 1 <= open_ticks < period_ticks
     and open_ticks <= 2^14.
   A wave waits at most the window's length, and never more than about 0.2 ms
   (a fixed number of sleeps), whatever the clock does.  Other work running on
   the device at the same time is not paused: the windows then group only this
   kernel's writes.
   Errors: ZS_ERR_RANGE. */
ZS_API zs_status zs_set_write_window(int32_t period_ticks, int32_t open_ticks);

/* The write window a kernel takes, under the current settings, for N
   replicas on a shard of n parameters whose arrays share a 128-byte line
   phase:
     kernel = ZS_WINDOW_FLAT_STEP:   the flat step (zs_reduce_adam_flat): only
                                     on the windowed schedule
                                     (zs_set_flat_schedule), on shards of at
                                     least 2^25 parameters;
     kernel = ZS_WINDOW_REDUCE_PASS: pass 1 of the two-pass form
                                     (zs_reduce_grads_flat): only on the
                                     windowed schedule (zs_reduce_schedule),
                                     on shards of at least 2^25 parameters;
     kernel = ZS_WINDOW_LIST_PLAN:   a list plan of n parameters in all: as the
                                     flat step on a shard of that size.
   *period_ticks = *open_ticks = 0 when it takes no windows.  No GPU call.
   Errors: ZS_ERR_NULL, ZS_ERR_RANGE. */
#define ZS_WINDOW_FLAT_STEP 0
#define ZS_WINDOW_REDUCE_PASS 1
#define ZS_WINDOW_LIST_PLAN 2
ZS_API zs_status zs_write_window(int32_t kernel, int32_t N, int64_t n, int32_t* period_ticks, int32_t* open_ticks);

/* The schedule of the flat step (zs_reduce_adam_flat and its device-step
   form), of list plans (every zs_reduce_adam_list* call, taking the schedule
   of a flat shard of the plan's total size by the list rules of
   ZS_SCHEDULE_AUTO below: zs_list_schedule) and of pass 1 of the two-pass
   form (zs_reduce_grads_flat and its device-scale form), for all later calls
   in this process.  Every schedule
   computes every parameter by the same operations in the same order, and
   pass 1's norm partials in the same order, so results do not depend on it;
   only when the bytes move does.  For pass 1 the phased schedule writes the
   mean gradient and the norm partials after the grid barrier, and its
   windowed default is 4096 / 256 ticks.  A list plan on the phased schedule
   gives each wave 10 consecutive wave tiles per super-chunk; when they are not
   whole tiles of one tensor (near a tensor's ends) the wave takes them one at
   a time after the barrier.
     ZS_SCHEDULE_AUTO:     the default.  An explicit zs_set_write_window
                           decides when one was made (no windows:
                           ZS_SCHEDULE_STREAM; a window: ZS_SCHEDULE_WINDOWED);
                           otherwise ZS_SCHEDULE_PHASED for N >= 40 replicas on
                           shards of at least 2^25 parameters and for N >= 24
                           on at least 2^27, and ZS_SCHEDULE_STREAM elsewhere
                           (where per-tile stores measured faster).  List
                           plans: zs_list_schedule; pass 1: N >= 12 on 2^25.
     ZS_SCHEDULE_STREAM:   one 512-parameter tile per workgroup, its outputs
                           stored as soon as it is done; consecutive launches
                           of at most zs_launch_bytes() each.
     ZS_SCHEDULE_WINDOWED: persistent waves that hold up to two finished tiles
                           and store them in device-clock write windows
                           (zs_set_write_window; the default window when none
                           was set), on shards of at least 2^25 parameters
                           (ZS_SCHEDULE_STREAM below).
     ZS_SCHEDULE_PHASED:   one persistent workgroup of 12 waves per compute
                           unit; the shard goes in super-chunks of 12 tiles
                           per wave (pass 1: 10), then a part super-chunk of
                           fewer tiles per wave when at least half a
                           super-chunk's tiles are left, the rest one tile per
                           wave.  First every wave reads all N replicas of its
                           tiles into register accumulators, the workgroup's
                           waves kept on the same replicas, so the device
                           reads one replica stream at a time over one
                           contiguous region; then, after a grid barrier
                           (released once 95% of the workgroups have
                           arrived), it reads master, m and v and writes the
                           four outputs of the super-chunk.  Any shard of at least
                           one whole tile.  The barrier counter lives in the
                           library's device memory (16 slots, one per launch in
                           turn): phased calls that run at the same time on one
                           device may meet at each other's barriers, which
                           changes their timing only.  A workgroup waits at a
                           barrier at most zs_set_phased_max_polls() polls.
   When the device cannot hold the persistent grid of the windowed or phased
   kernel, the call takes ZS_SCHEDULE_STREAM.  Errors: ZS_ERR_RANGE. */
#define ZS_SCHEDULE_AUTO 0
#define ZS_SCHEDULE_STREAM 1
#define ZS_SCHEDULE_WINDOWED 2
#define ZS_SCHEDULE_PHASED 3
ZS_API zs_status zs_set_flat_schedule(int32_t schedule);

/* The schedule a flat step for N replicas on a shard of n parameters (arrays
   on a common 128-byte line phase) takes under the current settings
   (ZS_SCHEDULE_STREAM, _WINDOWED or _PHASED).  No GPU call.
   Errors: ZS_ERR_NULL, ZS_ERR_RANGE. */
ZS_API zs_status zs_flat_schedule(int32_t N, int64_t n, int32_t* schedule);

/* The same for pass 1 of the two-pass form (zs_reduce_grads_flat) on a shard
   of n parameters whose replicas and fp32 workspace share a 128-byte line
   phase.  No GPU call.  Errors: ZS_ERR_NULL, ZS_ERR_RANGE. */
ZS_API zs_status zs_reduce_schedule(int32_t N, int64_t n, int32_t* schedule);

/* The schedule a list plan of these T tensors over N replicas
   (zs_list_plan_create's arguments, validated as there) takes under the
   current settings.  By the list rules of ZS_SCHEDULE_AUTO: the phased kernel
   needs N >= 64 on 3 * 2^24 parameters in all, N >= 40 on 3 * 2^25 or
   N >= 32 on 3 * 2^26, and at most 1 in 20 of the plan's wave tiles outside
   whole spans (10
   consecutive tiles of one tensor, counted from the list's first tile); lists
   of many small tensors, whose tiles the phased kernel takes one at a time,
   keep per-tile stores.  The pointers are only read for their alignment.
   No GPU call.  Errors: ZS_ERR_NULL, ZS_ERR_RANGE, ZS_ERR_ALIGN, ZS_ERR_ALIAS,
   ZS_ERR_NOMEM. */
ZS_API zs_status zs_list_schedule(const zs_tensor* tensors, int32_t T, int32_t N, int32_t* schedule);

/* The longest a workgroup of the phased schedule waits at a grid barrier, in
   polls of about 50 ns (0: the default, 2^16, about 3 ms).  Past it the
   workgroup goes on; results do not change, only the timing.  A test knob for
   the bounded wait, and a guard for devices shared with other work.
   Errors: ZS_ERR_RANGE (polls < 0). */
ZS_API zs_status zs_set_phased_max_polls(int32_t polls);

#ifdef __cplusplus
}
#endif

#endif /* ZSHARD_H */
