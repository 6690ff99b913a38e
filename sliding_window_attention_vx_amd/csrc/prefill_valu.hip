// Causal sliding-window prefill on the vector ALU, float32 arithmetic.
//
// This is the float32-I/O path (where bf16 matrix cores would lose the
// required precision) and a cross-check of the bf16 matrix-core kernel.  One
// wave per (batch, head, 64-query tile); lane = query.  Key/value tiles of 64
// rows are staged in LDS as float32, keys rotated (from the cos/sin table) and,
// for bf16 inputs, rounded back to bf16 exactly as the rotated tensor would be
// stored.  Online softmax in the log2 domain.
#include "vx_launch.h"

namespace vx {

namespace {

constexpr int kTile = 64;

// cos/sin of position p: the table row, or the same float64 angle computed
// here when there is no table (frequencies from LDS, fr_lds).
__device__ __forceinline__ void row_cs(const PrefillArgs& a, const double* fr_lds, int64_t trow,
                                       int64_t p, float cs[kD]) {
  if (a.table) {
#pragma unroll
    for (int i = 0; i < kD; i += 8) load8(a.table + trow * kD + i, cs + i);
  } else {
#pragma unroll
    for (int i = 0; i < kHalf; ++i) rope_cs(p, fr_lds[i], &cs[i], &cs[kHalf + i]);
  }
}

template <typename TI>
__device__ __forceinline__ void load_rot_row(const TI* __restrict__ src, const float* __restrict__ cs,
                                             bool rope, float out[kD]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float x[8], y[8];
    load8(src + 8 * c, x);
    load8(src + kHalf + 8 * c, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float xo = x[e], yo = y[e];
      if (rope) {
        rope_pair(x[e], y[e], cs[8 * c + e], cs[kHalf + 8 * c + e], &xo, &yo);
        xo = round_to<TI>(xo);
        yo = round_to<TI>(yo);
      }
      out[8 * c + e] = xo;
      out[kHalf + 8 * c + e] = yo;
    }
  }
}

template <typename TI, typename TO>
__global__ __launch_bounds__(64) void prefill_valu_kernel(PrefillArgs a) {
  __shared__ float Ks[kTile][kD + 1];
  __shared__ float Vs[kTile][kD + 1];
  const TI* __restrict__ q = (const TI*)a.q;
  const TI* __restrict__ k = (const TI*)a.k;
  const TI* __restrict__ v = (const TI*)a.v;
  TO* __restrict__ o = (TO*)a.o;
  const int T = a.T, H = a.H, W = a.W;
  const int b = blockIdx.z, h = blockIdx.y, q0 = blockIdx.x * kTile;
  const int lane = threadIdx.x;
  const int t = q0 + lane;
  const size_t rs = (size_t)H * kD;  // stride between frames
  const size_t base = (size_t)b * T * rs + (size_t)h * kD;
  // frame t at position p0 + t, its cos/sin at table row trow0 + t; invalid
  // positions or table rows make every output of the tile NaN
  const int64_t p0 = a.pos0 ? a.pos0[b] : 0;
  const int64_t trow0 = a.table_bstride * b + (a.table_pos ? p0 : 0) + a.table_off;
  if (p0 < 0 || (a.rope && a.table && (trow0 < 0 || trow0 + T > a.table_len))) {
    if (t < T) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = __builtin_nanf("");
#pragma unroll
      for (int c = 0; c < 8; ++c) store8(o + base + (size_t)t * rs + 8 * c, x);
    }
    return;
  }
  float cs[kD];
  // the frequencies, for cos/sin computed here (a table-less call): read
  // from LDS, not held in registers across the kernel
  __shared__ double fr_lds[kHalf];
  if (lane < kHalf) fr_lds[lane] = a.fr.f[lane];
  __syncthreads();

  float qr[kD];
  if (t < T) {
    if (a.rope) row_cs(a, fr_lds, trow0 + t, p0 + t, cs);
    load_rot_row<TI>(q + base + (size_t)t * rs, cs, a.rope, qr);
  } else {
#pragma unroll
    for (int d = 0; d < kD; ++d) qr[d] = 0.f;
  }
  float acc[kD];
#pragma unroll
  for (int d = 0; d < kD; ++d) acc[d] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int kbeg = max(0, q0 - W + 1);
  const int kend = min(T, q0 + kTile);  // exclusive
  for (int k0 = kbeg; k0 < kend; k0 += kTile) {
    const int key = k0 + lane;
    if (key < kend) {
      float row[kD];
      if (a.rope) row_cs(a, fr_lds, trow0 + key, p0 + key, cs);
      load_rot_row<TI>(k + base + (size_t)key * rs, cs, a.rope, row);
#pragma unroll
      for (int d = 0; d < kD; ++d) Ks[lane][d] = row[d];
      const TI* vp = v + base + (size_t)key * rs;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float x[8];
        load8(vp + 8 * c, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) Vs[lane][8 * c + e] = x[e];
      }
    }
    __syncthreads();
    const int nk = min(kTile, kend - k0);
    for (int j = 0; j < nk; ++j) {
      const int kk = k0 + j;
      if (kk > t || kk < t - W + 1) continue;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < kD; ++d) s = fmaf(qr[d], Ks[j][d], s);
      const float x = s * a.scale_log2;
      if (x > m) {
        const float alpha = exp2f(m - x);
        l *= alpha;
#pragma unroll
        for (int d = 0; d < kD; ++d) acc[d] *= alpha;
        m = x;
      }
      const float p = exp2f(x - m);
      l += p;
#pragma unroll
      for (int d = 0; d < kD; ++d) acc[d] = fmaf(p, Vs[j][d], acc[d]);
    }
    __syncthreads();
  }
  if (t < T) {
    const float inv = 1.f / l;
    TO* op = o + base + (size_t)t * rs;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = acc[8 * c + e] * inv;
      store8(op + 8 * c, x);
    }
  }
}

}  // namespace

hipError_t launch_prefill_valu(const PrefillArgs& a, DT io, DT out, hipStream_t st) {
  dim3 grid((a.T + kTile - 1) / kTile, a.H, a.B);
  if (io == DT::F32)
    hipLaunchKernelGGL((prefill_valu_kernel<float, float>), grid, dim3(64), 0, st, a);
  else if (out == DT::BF16)
    hipLaunchKernelGGL((prefill_valu_kernel<bf16, bf16>), grid, dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_valu_kernel<bf16, float>), grid, dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace vx
