// Internal launcher interface of the small kernels of the streaming encoder
// step (Voxtral Realtime 2602 audio encoder, transcribe.cpp "Voxtral" family
// notes, Architecture: pre-norm RMSNorm layers over a causal two-convolution
// stem).  Arguments reaching these functions have already been validated.
#pragma once

#include "vx_launch.h"

namespace vx {

// y[m, :] = x[m, :] / sqrt(mean(x[m, :]^2) + eps) * g, x fp32 [M, dim], g and
// y bf16; dim a multiple of 8.
hipError_t launch_rmsnorm(const float* x, const bf16* g, bf16* y, int M, int dim, float eps,
                          hipStream_t st);

// Per stream s, frame slots lo and lo+1 of each convolution's input buffer
// move to slots 0 and 1: a [S, F_a, C_a] and b [S, F_b, C_b] (bf16, C a
// multiple of 8), lo_a = F_a - 2, lo_b = F_b - 2.
hipError_t launch_stem_shift(bf16* a, int Fa, int Ca, bf16* b, int Fb, int Cb, int S,
                             hipStream_t st);

}  // namespace vx
