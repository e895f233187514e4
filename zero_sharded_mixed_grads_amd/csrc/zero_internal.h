// Internal declarations shared by the host planner and the device entry
// points of libzero_mi355x.
#pragma once

#include "zero.h"

namespace zero {

// Records a printf-style detail for zero_last_error() and returns s.
zero_status fail(zero_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace zero
