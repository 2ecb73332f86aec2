// Host-side launcher of the teacher-forced block loss (block_loss.hip) for the
// ABI layer.  Not part of the public ABI.
#pragma once

#include "internal.h"

namespace dspark {

size_t block_loss_workspace(int64_t M, int64_t V);
// bf16, rank 256, 16-byte aligned W1, W2 and workspace
bool block_loss_shape_ok(int64_t r, const void* W1, const void* W2, const void* ws);
hipError_t block_loss_launch(int64_t N, int64_t gamma, int64_t V, int64_t H, const void* U, const void* t,
                             const void* h, const void* W1, const void* W2, const void* w_conf, float b_conf,
                             const int32_t* xp, const int32_t* y, const float* mask, float decay, float a_ce,
                             float a_l1, float a_conf, float* ce, float* l1, float* conf, float* bce, float* loss,
                             void* ws, hipStream_t stream);

}  // namespace dspark
