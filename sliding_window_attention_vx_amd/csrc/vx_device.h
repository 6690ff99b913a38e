// Device-side helpers shared by the vx kernels (gfx950 only).
//
// RoPE (half-split pairing, as in the transcribe.cpp "Voxtral" family notes,
// Architecture: RoPE with theta 1e6 and head_dim 64 in the Realtime encoder):
// pair (i, i+32) of a head vector at absolute position p turns by angle
// p * f_i with f_i = theta^(-2i/64).  The angle is formed and reduced in
// float64 and its cosine/sine rounded to float32 once, by rope_cs(); every
// kernel (table, in-place rotation, fused prefill, streaming, ring append)
// goes through rope_cs() and rope_pair(), so a rotated value is the same bit
// pattern whichever path produced it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vx {

constexpr int kD = 64;      // head_dim
constexpr int kHalf = 32;   // rotation pairs per head vector

// Rotation frequencies f_i, computed on the host in float64 and passed by value.
struct RopeFreqs {
  double f[kHalf];
};

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void rope_cs(int64_t p, double f, float* c, float* s) {
  double sd, cd;
  sincos((double)p * f, &sd, &cd);
  *c = (float)cd;
  *s = (float)sd;
}

// (x, y) = (d_i, d_{i+32}) -> rotated pair, float32.
__device__ __forceinline__ void rope_pair(float x, float y, float c, float s, float* xo,
                                          float* yo) {
  *xo = fmaf(x, c, -(y * s));
  *yo = fmaf(y, c, x * s);
}

__device__ __forceinline__ float bf16_round_f32(float x) { return (float)(bf16)x; }

// bf16 pairs packed in 32-bit words (element 2i in the low half).  Working on
// words avoids per-element access to bf16 vectors.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (bf16)lo;  // round to nearest even (v_cvt_pk_bf16_f32)
  r[1] = (bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}
// acc + lo(w) + hi(w) for a packed bf16 pair (v_dot2c_f32_bf16 against (1, 1)).
// The word is taken by value: bit-casting an element of a vector expression
// directly in the builtin's argument has been miscompiled (every element read
// as element 0), a copy into a scalar avoids that.
__device__ __forceinline__ float dot2_ones(uint32_t w, float acc) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  bf16x2 x;
  __builtin_memcpy(&x, &w, sizeof x);
  return __builtin_amdgcn_fdot2_f32_bf16(x, one, acc, false);
}

__device__ __forceinline__ void unpack8(const u32x4 w, float v[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16lo(w[i]);
    v[2 * i + 1] = bf16hi(w[i]);
  }
}
__device__ __forceinline__ u32x4 pack8(const float v[8]) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  return w;
}

// ---- 8-element vector load/store with conversion to/from float32 ---------

__device__ __forceinline__ void load8(const float* p, float v[8]) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}
__device__ __forceinline__ void load8(const bf16* p, float v[8]) {
  unpack8(*reinterpret_cast<const u32x4*>(p), v);
}
__device__ __forceinline__ void store8(float* p, const float v[8]) {
  f32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = v[i];
    b[i] = v[4 + i];
  }
  *reinterpret_cast<f32x4*>(p) = a;
  *reinterpret_cast<f32x4*>(p + 4) = b;
}
__device__ __forceinline__ void store8(bf16* p, const float v[8]) {
  *reinterpret_cast<u32x4*>(p) = pack8(v);
}

template <typename T>
__device__ __forceinline__ float round_to(float x);
template <>
__device__ __forceinline__ float round_to<float>(float x) {
  return x;
}
template <>
__device__ __forceinline__ float round_to<bf16>(float x) {
  return bf16_round_f32(x);
}

}  // namespace vx
