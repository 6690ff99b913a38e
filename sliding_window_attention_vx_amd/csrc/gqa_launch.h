// Internal launcher interface of the grouped-query kernels (head_dim 128):
// the text decoder of Voxtral Realtime 2602 (transcribe.cpp "Voxtral" family
// notes, Architecture: 32 query heads over 8 key/value heads, head_dim 128,
// sliding window 8192, RoPE theta 1e6).  Query head h reads key/value head
// h / G with G = Hq / Hkv.  Arguments reaching these functions have already
// been validated by the C ABI.
#pragma once

#include "vx_launch.h"

namespace vx {

constexpr int kGD = 128;    // head_dim of the grouped-query kernels
constexpr int kGHalf = 64;  // rotation pairs per head vector: (i, i+64)

// Rotation frequencies f_i = theta^(-2i/128), computed on the host in float64.
struct RopeFreqs128 {
  double f[kGHalf];
};

struct GqaPrefillArgs {
  const bf16* q;  // [B,T,Hq,128]
  const bf16* k;  // [B,T,Hkv,128]
  const bf16* v;  // [B,T,Hkv,128]
  void* o;        // [B,T,Hq,128]
  int B, T, Hq, Hkv, W;
  bool rope;             // rotate q (and k unless rope_k is false) on load from the table
  bool rope_k = true;    // false: k holds rotated keys already (written by the rows kernel)
  const float* table;    // [.., 2, 64] cos/sin rows
  int64_t table_row0;    // table row of position pos0
  float scale_log2;      // softmax scale * log2(e)
  // Ring seeding (ring_k != nullptr): rotated keys and values of frames
  // t >= T - W go to slot t mod W of [B,Hkv,W,128] rings, pos_out[b] = T.
  bf16* ring_k = nullptr;
  bf16* ring_v = nullptr;
  int64_t* pos_out = nullptr;
};

struct GqaDecodeArgs {
  const bf16* q;  // [S,n,Hq,128]
  const bf16* k;  // [S,n,Hkv,128]
  const bf16* v;  // [S,n,Hkv,128]
  bf16* ring_k;   // [S,Hkv,W,128] rotated keys, slot = position mod W
  bf16* ring_v;
  const int64_t* pos_in;  // [S] position of the first new token
  int64_t* pos_out;       // [S] written: pos_in[s] + n (distinct from pos_in)
  void* o;                // [S,n,Hq,128]
  int S, n, Hq, Hkv, W;
  bool rope;
  float scale_log2;
};

constexpr int kGqaMaxCols = 16;  // n * Hq/Hkv query columns per decode workgroup

hipError_t launch_gqa_rope_table(float* table, int64_t p_begin, int count,
                                 const RopeFreqs128& fr, hipStream_t st);
hipError_t launch_gqa_prefill(const GqaPrefillArgs& a, DT out, hipStream_t st);
// k_rot[b,t,h] = k[b,t,h] rotated at position pos0 + t from the table (row
// table_row0 + t), rounded to bf16: the rotation the prefill's staging applies.
hipError_t launch_gqa_rope_rows(const bf16* k, bf16* k_rot, int B, int T, int Hkv,
                                const float* table, int64_t table_row0, hipStream_t st);
hipError_t launch_gqa_decode(const GqaDecodeArgs& a, DT out, const RopeFreqs128& fr,
                             hipStream_t st);

}  // namespace vx
