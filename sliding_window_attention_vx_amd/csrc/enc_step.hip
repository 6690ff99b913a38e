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

// The row's normalisation from the lane's chunks in registers (chunk j is
// elements 8 (lane + 64 j) ..): the sum of squares in chunk order, the wave
// reduction, then v * r * g stored as bf16.  The RMSNorm kernel and the
// residual reduction below both call it, so their normalised states agree bit
// for bit.
template <int CPL>
__device__ __forceinline__ void norm_row_store(float (&v)[CPL][8], const bf16* __restrict__ g,
                                               bf16* __restrict__ yr, int lane, int c8, int dim,
                                               float eps) {
  float gv[CPL][8];
#pragma unroll
  for (int j = 0; j < CPL; ++j)
    if (lane + 64 * j < c8) load8(g + 8 * (lane + 64 * j), gv[j]);
  float ss = 0.f;
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
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = v[j][e] * r * gv[j][e];
      store8(yr + 8 * c, o);
    }
  }
}

// One wave per row; each lane owns chunks of 8 floats (lane, lane+64, ...).
// With CPL > 0 every lane holds its at most CPL chunks in registers: all of
// the row's loads are issued at once and the normalised values come from the
// registers, one memory round trip per row.  CPL == 0 (rows longer than
// 64 * 8 * 8 floats) reads the row twice instead.
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
    float v[CPL][8];
#pragma unroll
    for (int j = 0; j < CPL; ++j)
      if (lane + 64 * j < c8) load8(xr + 8 * (lane + 64 * j), v[j]);
    norm_row_store<CPL>(v, g, yr, lane, c8, dim, eps);
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

// The end of a split product added into the residual stream, one wave per
// row: x = x + (P_0 + .. + P_{np-1} + bias) with the K parts' fp32 sums in
// order, then optionally h = rmsnorm(x) * g (bf16) for the next product.
// With NP > 0 (np == NP) every load of the row (parts, bias, x) is issued
// before the first add, so the row costs one memory round trip; NP == 0
// takes any np.
template <int CPL, bool NORM, int NP>
__global__ __launch_bounds__(kNormWaves * 64) void residual_reduce_kernel(
    float* __restrict__ x, const float* __restrict__ parts, int np, const bf16* __restrict__ bias,
    const bf16* __restrict__ g, bf16* __restrict__ h, int M, int dim, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kNormWaves + (threadIdx.x >> 6);
  if (row >= M) return;
  const int c8 = dim / 8;
  const size_t pstride = (size_t)M * dim;
  float* xr = x + row * dim;
  float v[CPL][8];
  if constexpr (NP > 0) {
    float pv[NP][CPL][8], bv[CPL][8];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      if (c >= c8) continue;
#pragma unroll
      for (int p = 0; p < NP; ++p) load8(parts + p * pstride + row * dim + 8 * c, pv[p][j]);
      if (bias) load8(bias + 8 * c, bv[j]);
      load8(xr + 8 * c, v[j]);
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      if (c >= c8) continue;
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = pv[0][j][e];
#pragma unroll
      for (int p = 1; p < NP; ++p)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += pv[p][j][e];
      if (bias) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += bv[j][e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = acc[e] + v[j][e];
      store8(xr + 8 * c, v[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      if (c >= c8) continue;
      float acc[8], t[8];
      load8(parts + row * dim + 8 * c, acc);
      for (int p = 1; p < np; ++p) {
        load8(parts + p * pstride + row * dim + 8 * c, t);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += t[e];
      }
      if (bias) {
        load8(bias + 8 * c, t);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += t[e];
      }
      load8(xr + 8 * c, t);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = acc[e] + t[e];
      store8(xr + 8 * c, v[j]);
    }
  }
  if constexpr (NORM) norm_row_store<CPL>(v, g, h + row * dim, lane, c8, dim, eps);
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

hipError_t launch_residual_reduce(float* x, const float* parts, int np, const bf16* bias,
                                  const bf16* g, bf16* h, int M, int dim, float eps,
                                  hipStream_t st) {
  const unsigned blocks = (unsigned)((M + kNormWaves - 1) / kNormWaves);
  const dim3 grid(blocks), blk(kNormWaves * 64);
  const int cpl = (dim / 8 + 63) / 64;
#define VX_RR3(C, P)                                                                          \
  if (g)                                                                                      \
    hipLaunchKernelGGL((residual_reduce_kernel<C, true, P>), grid, blk, 0, st, x, parts, np, bias, \
                       g, h, M, dim, eps);                                                    \
  else                                                                                        \
    hipLaunchKernelGGL((residual_reduce_kernel<C, false, P>), grid, blk, 0, st, x, parts, np,     \
                       bias, g, h, M, dim, eps);
#define VX_RR(C)                                                                              \
  if (np == 2) {                                                                              \
    VX_RR3(C, 2)                                                                              \
  } else if (np == 1) {                                                                       \
    VX_RR3(C, 1)                                                                              \
  } else {                                                                                    \
    VX_RR3(C, 0)                                                                              \
  }
  if (cpl <= 1) {
    VX_RR(1)
  } else if (cpl <= 2) {
    VX_RR(2)
  } else if (cpl <= 4) {
    VX_RR(4)
  } else {
    VX_RR3(8, 0)  // rows past 4 chunks per lane: loads in two rounds, fewer registers
  }
#undef VX_RR
#undef VX_RR3
  return hipGetLastError();
}

hipError_t launch_stem_shift(bf16* a, int Fa, int Ca, bf16* b, int Fb, int Cb, int S,
                             hipStream_t st) {
  hipLaunchKernelGGL(stem_shift_kernel, dim3((unsigned)S), dim3(256), 0, st, a, Fa, Ca, b, Fb, Cb);
  return hipGetLastError();
}

}  // namespace vx
