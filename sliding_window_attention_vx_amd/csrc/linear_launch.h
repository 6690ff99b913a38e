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
  const bf16* x;  // [M, K] row-major
  const bf16* w;  // [N, K] row-major: y = x w^T
  int M, N, K;
  // plain output: y [M, N], optional bias [N]
  const bf16* bias = nullptr;
  void* y = nullptr;
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

hipError_t launch_linear(const LinearArgs& a, DT out, hipStream_t st);
hipError_t launch_qkv_rope(const LinearArgs& a, const RopeFreqs& fr, hipStream_t st);

}  // namespace vx
