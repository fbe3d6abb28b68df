// Host entry points of the linear projections (swa_projection.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

// out[m][n] = sum_k x[m][k] * w[n][k] + bias[n] for tokens m < M and features
// n < N, x [M][K], w [N][K]; column n is written to tensor n / split (d0, d1
// or d2) at [m][n % split].  The shapes the kernels take: N and split
// multiples of 8 with N <= 3 * split and N <= 2^15, K a multiple of 32 up to
// 2^16, M below 2^31.
bool projection_fits(int64_t M, int N, int K, int split);
hipError_t launch_projection(bool bf16, const void* x, const void* w, const float* bias, int64_t M, int N, int K,
                             int split, void* d0, void* d1, void* d2, hipStream_t s);

} // namespace swa
