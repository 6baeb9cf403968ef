// Internal interface of the two-pass form (zs_twopass.hip): pass 1 (mean,
// unscale, norm), the norm's finalize, pass 2 (AdamW from the mean) and the
// device-side loss-scale update.  Not installed; not part of the ABI.
#pragma once

#include "zs_internal.h"

namespace zs {

// Pass 1 of the two-pass form: tiles of kBlock*8 parameters start at `head`
// (the common alignment peel of the replicas and the fp32 gradient buffer);
// scalar_only = 1 when no common peel exists.
struct TwoPassShape {
  float* gbar;
  double* partials;  // ntiles + 1 slots
  double* partials2; // first-stage sums of the partials, one per kFinalSeg of them
  double* sqnorm;    // the shard's squared norm (device)
  int64_t n;
  int64_t head;
  int64_t ntiles;
  int32_t scalar_only;
  int32_t n_rep;
  float inv_scale;
  const double* scale_dev;  // if set, the loss scale is read here on the device and inv_scale is unused
  WriteWindow window;       // write windows of pass 1 (period_mask == 0: none)
  int32_t phased;           // pass 1 on the phased schedule (reduce_phased_kernel) where the shard allows
  PhasedCtl ctl;            // its barrier slot and wait bound
};

// Per-tile norm partials summed by one first-stage workgroup.
constexpr int64_t kFinalSeg = 4096;
// Windowed pass 1: finished tiles' means held per wave, and the fewest whole
// 2048-parameter tiles for which a shard takes it (2^25 parameters).
constexpr int kHeldMeans = 4;
constexpr int64_t kReduceWindowMinTiles = 16384;

hipError_t launch_reduce(const uint16_t* const* grads, const TwoPassShape& sh, int grad_format, int blocks,
                         hipStream_t stream);
// One device thread applies zs_loss_scaler_update to the state at `state`,
// taking a non-finite *total_sq as an overflow; writes 1 (taken) or 0 to
// *taken when taken is not NULL.
hipError_t launch_scaler_update(zs_loss_scaler* state, const double* total_sq, int32_t* taken, hipStream_t stream);

hipError_t launch_gbar(const float* gbar, const FlatShape& s, const Scalars& c, const StepRef& ref,
                       const double* total_sq, double max_norm, int skip_nonfinite, int param_format, int blocks,
                       hipStream_t stream);

}  // namespace zs
