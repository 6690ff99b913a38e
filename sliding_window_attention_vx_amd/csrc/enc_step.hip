// Small kernels of the streaming encoder step: the RMSNorm in front of the
// attention and of the feed-forward block, and the move of each causal
// convolution's last two input frames to the front of its buffer, where the
// next step's frames find them (Voxtral Realtime 2602 audio encoder,
// transcribe.cpp "Voxtral" family notes, Architecture: RMSNorm pre-norm
// layers, a stem of two kernel-3 causal convolutions).
//
// Both are HBM-bound row sweeps: one wave per row, 16-byte accesses.
#include "enc_launch.h"

namespace vx {

namespace {

constexpr int kNormWaves = 4;

// One wave per row; each lane owns chunks of 8 floats (lane, lane+64, ...).
// With CPL > 0 every lane holds its at most CPL chunks (and their gains) in
// registers: all of the row's loads are issued at once and the normalised
// values come from the registers, one memory round trip per row.  CPL == 0
// (rows longer than 64 * 8 * 8 floats) reads the row twice instead.
template <int CPL>
__global__ __launch_bounds__(kNormWaves * 64) void rmsnorm_kernel(const float* __restrict__ x,
                                                                  const bf16* __restrict__ g,
                                                                  bf16* __restrict__ y, int M,
                                                                  int dim, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kNormWaves + (threadIdx.x >> 6);
  if (row >= M) return;
  const float* xr = x + row * dim;
  bf16* yr = y + row * dim;
  const int c8 = dim / 8;
  float ss = 0.f;
  if constexpr (CPL > 0) {
    float v[CPL][8], gv[CPL][8];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      if (c < c8) {
        load8(xr + 8 * c, v[j]);
        load8(g + 8 * c, gv[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j)
      if (lane + 64 * j < c8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(v[j][e], v[j][e], ss);
      }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    const float r = 1.0f / sqrtf(ss / (float)dim + eps);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      if (c < c8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[j][e] = v[j][e] * r * gv[j][e];
        store8(yr + 8 * c, v[j]);
      }
    }
  } else {
    for (int c = lane; c < c8; c += 64) {
      float v[8];
      load8(xr + 8 * c, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    const float r = 1.0f / sqrtf(ss / (float)dim + eps);
    for (int c = lane; c < c8; c += 64) {
      float v[8], gv[8];
      load8(xr + 8 * c, v);
      load8(g + 8 * c, gv);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = v[e] * r * gv[e];
      store8(yr + 8 * c, v);
    }
  }
}

// Block s handles stream s: 16-byte chunks of the two frames of both buffers.
__global__ __launch_bounds__(256) void stem_shift_kernel(bf16* __restrict__ a, int Fa, int Ca,
                                                         bf16* __restrict__ b, int Fb, int Cb) {
  const int64_t s = blockIdx.x;
  const int na = 2 * Ca / 8, nb = 2 * Cb / 8;
  for (int u = threadIdx.x; u < na + nb; u += blockDim.x) {
    const bool in_a = u < na;
    bf16* base = in_a ? a + s * Fa * Ca : b + s * Fb * Cb;
    const int F = in_a ? Fa : Fb, C = in_a ? Ca : Cb, c = in_a ? u : u - na;
    // chunk c covers elements 8c .. 8c+7 of the two-frame block
    const u32x4 v = *reinterpret_cast<const u32x4*>(base + (int64_t)(F - 2) * C + 8 * c);
    *reinterpret_cast<u32x4*>(base + 8 * c) = v;
  }
}

}  // namespace

hipError_t launch_rmsnorm(const float* x, const bf16* g, bf16* y, int M, int dim, float eps,
                          hipStream_t st) {
  const unsigned blocks = (unsigned)((M + kNormWaves - 1) / kNormWaves);
  const int cpl = (dim / 8 + 63) / 64;  // 16-byte chunk pairs per lane
  const dim3 grid(blocks), blk(kNormWaves * 64);
  if (cpl <= 1)
    hipLaunchKernelGGL(rmsnorm_kernel<1>, grid, blk, 0, st, x, g, y, M, dim, eps);
  else if (cpl <= 2)
    hipLaunchKernelGGL(rmsnorm_kernel<2>, grid, blk, 0, st, x, g, y, M, dim, eps);
  else if (cpl <= 4)
    hipLaunchKernelGGL(rmsnorm_kernel<4>, grid, blk, 0, st, x, g, y, M, dim, eps);
  else if (cpl <= 8)
    hipLaunchKernelGGL(rmsnorm_kernel<8>, grid, blk, 0, st, x, g, y, M, dim, eps);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<0>, grid, blk, 0, st, x, g, y, M, dim, eps);
  return hipGetLastError();
}

hipError_t launch_stem_shift(bf16* a, int Fa, int Ca, bf16* b, int Fb, int Cb, int S,
                             hipStream_t st) {
  hipLaunchKernelGGL(stem_shift_kernel, dim3((unsigned)S), dim3(256), 0, st, a, Fa, Ca, b, Fb, Cb);
  return hipGetLastError();
}

}  // namespace vx
