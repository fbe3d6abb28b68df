// Host entry points of the fused projection-attention layer kernel (swa_layer.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "swa_geometry.h"

namespace swa {

// Whether the fused kernel takes the geometry (bf16 only; the caller checks
// the dtype): head_dim 32 or 64 with windows of up to 9 query tiles (144
// tokens), or head_dim 128 with up to 5; C = heads * head_dim a multiple of
// 32 of at least 96; the LDS layout within a compute unit's; row indices and
// the attention output within 31 bits.
bool layer_fused_fits(const Geometry& g);
hipError_t prepare_layer_kernels(int max_lds);
// o[token][h][d] = the window attention of q, k, v = x W_qkv^T + b_qkv, every
// real token; x [tokens][C], w_qkv [3C][C], b_qkv [3C] fp32, o [tokens][C].
hipError_t launch_layer_qkv_attention(const Geometry& g, const uint16_t* x, const uint16_t* w_qkv,
                                      const float* b_qkv, const float* table, uint16_t* o, hipStream_t s);

} // namespace swa
