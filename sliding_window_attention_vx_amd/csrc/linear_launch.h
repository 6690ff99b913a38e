// Internal launcher interface of the projection kernels around the encoder's
// attention (Voxtral Realtime 2602 audio encoder, transcribe.cpp "Voxtral"
// family notes, Architecture: q/k/v projections of the 1280-wide hidden state
// to 32 heads x 64 with no k_proj bias, and the output projection back).
// Arguments reaching these functions have already been validated.
#pragma once

#include "vx_launch.h"

namespace vx {

constexpr int kLinKStep = 128;  // K must be a multiple of this

struct LinearArgs {
  const bf16* x;  // rows of K contiguous elements (see the row map below)
  const bf16* w;  // [N, K] row-major: y = x w^T
  int M, N, K;
  // Row map: row m of x starts at element (m / rpg) * xgs + (m % rpg) * xrs, and
  // row m of y at (m / rpg) * ygs + (m % rpg) * yrs (rows may overlap: a causal
  // convolution reads k consecutive frames as one row).  x_bytes bounds x.
  int rpg = 1;
  int64_t xgs = 0, xrs = 0, ygs = 0, yrs = 0;
  int64_t x_bytes = 0;
  // plain / GELU / residual output: y, optional bias [N]; residual: y (fp32)
  // = res + x w^T + bias, res (fp32, same map as y) may equal y
  const bf16* bias = nullptr;
  void* y = nullptr;
  const float* res = nullptr;
  // SwiGLU: w holds the gate rows, w2 the up rows (both [F, K]); N = 2F and
  // y [M, F] = silu(x w^T) * (x w2^T), bf16
  const bf16* w2 = nullptr;
  // Partial: K is split in `splits` equal parts; part z writes its fp32 sum
  // x[:, zK/splits ..) w[:, zK/splits ..)^T to y + z*M*N (dense [M, N])
  int splits = 1;
  // q/k/v output (N = 3*HD): columns [0, HD) are q (+ b_q, rotated), [HD, 2HD)
  // k (rotated, no bias), [2HD, 3HD) v (+ b_v); row m sits at position
  // pos[m / n] + m % n; q, k, v are [M, HD] bf16.
  int HD = 0, n = 1;
  const int64_t* pos = nullptr;
  const bf16* b_q = nullptr;
  const bf16* b_v = nullptr;
  bf16* q = nullptr;
  bf16* k = nullptr;
  bf16* v = nullptr;
};

enum class LinEpi { Plain, Gelu, Residual, SwiGLU, Partial };

// Fills the row map of a dense [M, K] -> [M, N] product.
inline void dense_rows(LinearArgs& a) {
  a.rpg = a.M > 0 ? a.M : 1;
  a.xgs = 0;
  a.xrs = a.K;
  a.ygs = 0;
  a.yrs = a.N;
  a.x_bytes = (int64_t)a.M * a.K * 2;
}

hipError_t launch_linear(const LinearArgs& a, DT out, hipStream_t st, LinEpi epi = LinEpi::Plain);
hipError_t launch_qkv_rope(const LinearArgs& a, const RopeFreqs& fr, hipStream_t st);

}  // namespace vx
