// Internal declarations shared by the host planner and the device entry
// points of libzero_mi355x.
#pragma once

#include "zero.h"

namespace zero {

// Records a printf-style detail for zero_last_error() and returns s.
zero_status fail(zero_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// Domain checks of the AdamW hyper-parameters shared by the step entry points;
// inv_loss_scale is checked only when no device loss-scale state replaces it.
zero_status check_adamw(const zero_adamw &hp, bool host_inv_scale, const char *what);

// Domain checks of the dynamic loss-scaling parameters.
zero_status check_scaler(const zero_loss_scaler &cfg, const char *what);

// Enqueues the one-thread kernel that advances *d_state for one step from
// *d_stats (NULL: no clip, never skip) and the inverse loss scale (from
// *d_scale when not NULL, else hp.inv_loss_scale) on `stream` (a hipStream_t).
zero_status launch_adam_scalars(const zero_adamw &hp, const zero_grad_stats_t *d_stats,
                                const zero_loss_scale_t *d_scale, zero_adam_state_t *d_state,
                                void *stream);

}  // namespace zero
