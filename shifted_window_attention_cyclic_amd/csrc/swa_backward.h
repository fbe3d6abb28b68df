// Host queries of the backward pass beyond those in swa_geometry.h (swa_backward.hip).
#pragma once

#include "swa_geometry.h"

namespace swa {

// 0: the backward pass does not take the window; 1: one workgroup per
// (window, head) with the whole window in LDS; 2: the key-blocked bf16
// kernels for larger windows.
int backward_schedule(const Geometry& g, bool bf16);

} // namespace swa
