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

// Keys rotated once, into a separate buffer, for a prefill that then stages
// them as they are: frame t of batch entry b takes the cos/sin row the
// prefill's own staging would read (row table_bstride*b + (table_pos ?
// pos0[b] : 0) + t + table_off), and the same rotation, so the prefill's
// results keep their bits.  One workgroup per (b, t) frame, its row of the
// table in LDS for all H heads.  Frames whose row lies outside the table, or
// whose entry has a negative position, are skipped: the prefill writes NaN
// over such an entry without reading its keys.
__global__ __launch_bounds__(128) void rope_k_table_kernel(
    const bf16* __restrict__ k, bf16* __restrict__ ko, int T_, int H,
    const int64_t* __restrict__ pos0, const float* __restrict__ table, int64_t table_off,
    int64_t table_bstride, bool table_pos, int64_t table_len) {
  __shared__ __attribute__((aligned(16))) float cs[kD];
  const int64_t row = blockIdx.x;  // b * T + t
  const int64_t b = row / T_;
  const int t = (int)(row - b * T_);
  const int64_t p0 = pos0 ? pos0[b] : 0;
  const int64_t tr = table_bstride * b + (table_pos ? p0 : 0) + table_off + t;
  if (p0 < 0 || tr < 0 || tr >= table_len) return;  // the same for the whole workgroup
  const int units = H * 4;  // (head, 8-pair chunk)
  // with one chunk per thread (H <= 32) its key loads go out before the
  // table row's, so the two memory latencies overlap
  const bool one = units <= (int)blockDim.x;
  float x[8], y[8];
  const size_t off1 = (size_t)row * H * kD + (size_t)(threadIdx.x >> 2) * kD + 8 * (threadIdx.x & 3);
  if (one && (int)threadIdx.x < units) {
    load8(k + off1, x);
    load8(k + off1 + kHalf, y);
  }
  if (threadIdx.x < kD / 4)
    reinterpret_cast<f32x4*>(cs)[threadIdx.x] =
        reinterpret_cast<const f32x4*>(table + tr * kD)[threadIdx.x];
  __syncthreads();
  auto rotate = [&](size_t off, int c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float xo, yo;
      rope_pair(x[e], y[e], cs[8 * c + e], cs[kHalf + 8 * c + e], &xo, &yo);
      x[e] = xo;
      y[e] = yo;
    }
    store8(ko + off, x);
    store8(ko + off + kHalf, y);
  };
  if (one) {
    if ((int)threadIdx.x < units) rotate(off1, threadIdx.x & 3);
    return;
  }
  for (int u = threadIdx.x; u < units; u += blockDim.x) {
    const size_t off = (size_t)(row * H + (u >> 2)) * kD + 8 * (u & 3);
    load8(k + off, x);
    load8(k + off + kHalf, y);
    rotate(off, u & 3);
  }
}

hipError_t launch_rope_k_table(const PrefillArgs& a, void* k_out, hipStream_t st) {
  const unsigned blocks = (unsigned)((int64_t)a.B * a.T);
  hipLaunchKernelGGL(rope_k_table_kernel, dim3(blocks), dim3(128), 0, st, (const bf16*)a.k,
                     (bf16*)k_out, a.T, a.H, a.pos0, a.table, a.table_off, a.table_bstride,
                     a.table_pos, a.table_len);
  return hipGetLastError();
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
