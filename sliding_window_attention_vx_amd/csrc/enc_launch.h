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

// x[m, :] += P_0[m, :] + .. + P_{np-1}[m, :] + bias (fp32, the parts summed in
// order; parts [np, M, dim], bias bf16 [dim] or NULL), then, if g is not
// NULL, h[m, :] = rmsnorm(x[m, :]) * g as launch_rmsnorm computes it, bit for
// bit.  dim a multiple of 8, at most 64 * 8 * 8.
constexpr int kReduceMaxDim = 4096;
hipError_t launch_residual_reduce(float* x, const float* parts, int np, const bf16* bias,
                                  const bf16* g, bf16* h, int M, int dim, float eps,
                                  hipStream_t st);

// Per stream s, frame slots lo and lo+1 of each convolution's input buffer
// move to slots 0 and 1: a [S, F_a, C_a] and b [S, F_b, C_b] (bf16, C a
// multiple of 8), lo_a = F_a - 2, lo_b = F_b - 2.
hipError_t launch_stem_shift(bf16* a, int Fa, int Ca, bf16* b, int Fb, int Cb, int S,
                             hipStream_t st);

}  // namespace vx
