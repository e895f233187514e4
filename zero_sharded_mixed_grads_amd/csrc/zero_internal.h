// Internal declarations shared by the host planner and the device entry
// points of libzero_mi355x.
#pragma once

#include "zero.h"

namespace zero {

// Records a printf-style detail for zero_last_error() and returns s.
zero_status fail(zero_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// Domain checks of the AdamW hyper-parameters shared by the step entry points.
zero_status check_adamw(const zero_adamw &hp, const char *what);

// Enqueues the one-thread kernel that advances *d_state for one step from
// *d_stats (NULL: no clip, never skip) on `stream` (a hipStream_t).
zero_status launch_adam_scalars(const zero_adamw &hp, const zero_grad_stats_t *d_stats,
                                zero_adam_state_t *d_state, void *stream);

}  // namespace zero
