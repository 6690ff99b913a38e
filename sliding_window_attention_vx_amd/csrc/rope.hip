// RoPE kernels: the cos/sin table and the in-place rotation of q and k.
// Both are HBM-bound element-wise kernels; the angle is formed in float64 by
// rope_cs() so every path agrees bit for bit on rotated values.
#include "vx_launch.h"

namespace vx {

__global__ void rope_table_kernel(float* __restrict__ table, int64_t p_begin, int count,
                                  RopeFreqs fr) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)count * kHalf) return;
  const int64_t j = idx / kHalf;
  const int i = (int)(idx % kHalf);
  float c, s;
  rope_cs(p_begin + j, fr.f[i], &c, &s);
  table[j * kD + i] = c;
  table[j * kD + kHalf + i] = s;
}

// Rows b*T + t of a table for batch entries at their own positions:
// cos/sin of position pos0[b] + t (pos0 nullptr = 0).  Used as the prefill's
// cos/sin cache when the caller gives a workspace instead of a table.
__global__ void rope_table_batched_kernel(float* __restrict__ table,
                                          const int64_t* __restrict__ pos0, int T, int64_t rows,
                                          RopeFreqs fr) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * kHalf) return;
  const int64_t j = idx / kHalf;
  const int i = (int)(idx % kHalf);
  const int64_t b = j / T;
  const int64_t p = (pos0 ? pos0[b] : 0) + (j - b * T);
  float c, s;
  rope_cs(p, fr.f[i], &c, &s);
  table[j * kD + i] = c;
  table[j * kD + kHalf + i] = s;
}

// One workgroup per (b, t) row: the row's 32 cos/sin pairs go to LDS once and
// serve every head of q and k.  A thread rotates 8 pairs (two 8-element chunks).
// Frame t of batch entry b is at position pos0[b] + t; a negative pos0[b]
// is an invalid position and makes the entry's rows NaN (loud, not partial).
template <typename T>
__global__ __launch_bounds__(128) void rope_qk_kernel(T* __restrict__ q, T* __restrict__ k,
                                                      int T_, int H,
                                                      const int64_t* __restrict__ pos0,
                                                      RopeFreqs fr) {
  __shared__ float cs[2][kHalf];
  const int64_t row = blockIdx.x;  // b * T + t
  const int t = (int)(row % T_);
  const int64_t p0 = pos0 ? pos0[row / T_] : 0;
  if (threadIdx.x < kHalf) {
    float c, s;
    rope_cs(p0 + t, fr.f[threadIdx.x], &c, &s);
    if (p0 < 0) c = s = __builtin_nanf("");
    cs[0][threadIdx.x] = c;
    cs[1][threadIdx.x] = s;
  }
  __syncthreads();
  const int units = H * 4;  // (head, chunk) per tensor
  for (int u = threadIdx.x; u < 2 * units; u += blockDim.x) {
    T* base = (u < units) ? q : k;
    if (base == nullptr) continue;
    const int uu = u % units;
    const int h = uu >> 2, c = uu & 3;
    T* p = base + (row * H + h) * kD + 8 * c;
    float x[8], y[8];
    load8(p, x);
    load8(p + kHalf, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float xo, yo;
      rope_pair(x[e], y[e], cs[0][8 * c + e], cs[1][8 * c + e], &xo, &yo);
      x[e] = xo;
      y[e] = yo;
    }
    store8(p, x);
    store8(p + kHalf, y);
  }
}

hipError_t launch_rope_table(float* table, int64_t p_begin, int count, const RopeFreqs& fr,
                             hipStream_t st) {
  const int64_t total = (int64_t)count * kHalf;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(threads), 0, st, table,
                     p_begin, count, fr);
  return hipGetLastError();
}

hipError_t launch_rope_table_batched(float* table, const int64_t* pos0, int B, int T,
                                     const RopeFreqs& fr, hipStream_t st) {
  const int64_t rows = (int64_t)B * T;
  const int threads = 256;
  const int64_t blocks = (rows * kHalf + threads - 1) / threads;
  hipLaunchKernelGGL(rope_table_batched_kernel, dim3((unsigned)blocks), dim3(threads), 0, st,
                     table, pos0, T, rows, fr);
  return hipGetLastError();
}

hipError_t launch_rope_qk(void* q, void* k, int B, int T, int H, const int64_t* pos0, DT io,
                          const RopeFreqs& fr, hipStream_t st) {
  const unsigned blocks = (unsigned)((int64_t)B * T);
  if (io == DT::BF16)
    hipLaunchKernelGGL(rope_qk_kernel<bf16>, dim3(blocks), dim3(128), 0, st, (bf16*)q, (bf16*)k,
                       T, H, pos0, fr);
  else
    hipLaunchKernelGGL(rope_qk_kernel<float>, dim3(blocks), dim3(128), 0, st, (float*)q,
                       (float*)k, T, H, pos0, fr);
  return hipGetLastError();
}

}  // namespace vx
