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

// cos and sin of the float64 angle a = p * f, each rounded to float32 once.
// Cody-Waite reduction by pi/2 with a two-term constant and fused
// multiply-adds (C1 = pi/2 rounded to float64, C2 = pi/2 - C1 rounded, both
// from a 60-digit pi): r = a - k pi/2 with |r| <= pi/4 to within k * 2^-106,
// then the Taylor series of sin and cos at 0 through r^21 and r^20 (the
// first omitted term is below 1e-21 on [-pi/4, pi/4]), and the quadrant k
// mod 4 picks and signs the pair.  About 30 float64 operations where a
// general-purpose sincos takes four times as many; over 12.8 million
// angles (positions 0 .. 2e5 and around 2e9, all 32 frequencies) the
// float32 results equal the correctly rounded ones of a quad-precision
// evaluation.
struct RopeCsCoef {
  double s[10];  // (-1)^(i+1) / (2i+3)!
  double c[10];  // (-1)^(i+1) / (2i+2)!
  constexpr RopeCsCoef() : s(), c() {
    double f = 1.0;
    for (int n = 1; n <= 21; ++n) {
      f *= n;
      const double sg = ((n / 2) % 2) ? -1.0 : 1.0;
      if (n % 2 == 1 && n >= 3) s[(n - 3) / 2] = sg / f;
      if (n % 2 == 0) c[(n - 2) / 2] = sg / f;
    }
  }
};

__device__ __forceinline__ void rope_cs(int64_t p, double f, float* c, float* s) {
  constexpr double kC1 = 0x1.921fb54442d18p+0, kC2 = 0x1.1a62633145c07p-54;
  constexpr double kTwoOverPi = 0x1.45f306dc9c883p-1;
  constexpr RopeCsCoef K;
  const double a = (double)p * f;
  const double k = rint(a * kTwoOverPi);
  const double r = fma(-k, kC2, fma(-k, kC1, a));
  const double z = r * r;
  double sp = K.s[9], cp = K.c[9];
#pragma unroll
  for (int i = 8; i >= 0; --i) {
    sp = fma(sp, z, K.s[i]);
    cp = fma(cp, z, K.c[i]);
  }
  const double sn = fma(r * z, sp, r);
  const double cs = fma(z, cp, 1.0);
  const int q = (int)((int64_t)k & 3);
  const double so = (q & 1) ? cs : sn, co = (q & 1) ? sn : cs;
  *s = (float)((q & 2) ? -so : so);
  *c = (float)(((q + 1) & 2) ? -co : co);
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
