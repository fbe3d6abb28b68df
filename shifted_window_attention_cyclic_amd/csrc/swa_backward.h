// Host side of the backward pass (swa_backward.hip).
#pragma once

#include "swa_geometry.h"

namespace swa {

// Whether a kernel takes the window, the workspace it needs (bytes: per-unit shares of the table gradient and their
// per-chunk sums), kernel set-up, and the launch (attention gradients, then the
// two table-gradient sums).
bool backward_fits(const Geometry& g, bool bf16);
size_t backward_workspace_bytes(const Geometry& g);
hipError_t prepare_backward_kernels(int max_lds);
// Workgroups of the persistent small-window backward kernel for g (a multiple
// of the XCD count), of the persistent big-window key kernel (heads * key
// groups * runs of windows), or 0 where the one-shot kernels run; after
// prepare_backward_kernels, on the device the launches will use.
hipError_t backward_plan(const Geometry& g, bool bf16, int* blocks);
// blocks: backward_plan's.  With lse and o (the forward's statistics and
// output; both may be null) the big-window kernels take the softmax
// statistics from the forward pass.
hipError_t launch_backward(const Geometry& g, bool bf16, const void* q, const void* k, const void* v,
                           const float* table, const void* dout, void* dq, void* dk, void* dv, float* dtable,
                           void* workspace, const void* o, const float* lse, int blocks, hipStream_t s);
// The same gradients through a fixed scratch buffer of scratch_bytes, in
// passes over runs of window chunks (bitwise equal to launch_backward), and
// the least scratch that takes (one chunk of windows).
size_t backward_scratch_bytes(const Geometry& g, bool bf16);
hipError_t launch_backward_scratch(const Geometry& g, bool bf16, const void* q, const void* k, const void* v,
                                   const float* table, const void* dout, void* dq, void* dk, void* dv, float* dtable,
                                   void* scratch, size_t scratch_bytes, int blocks, hipStream_t s);

// 0: the backward pass does not take the window; 1: one workgroup per
// (window, head) with the whole window in LDS; 2: the key-blocked bf16
// kernels for larger windows.
int backward_schedule(const Geometry& g, bool bf16);

} // namespace swa
