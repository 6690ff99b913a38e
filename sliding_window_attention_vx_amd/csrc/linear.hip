// Projections around the encoder's attention on bf16 matrix cores (gfx950):
// y = x w^T with x [M, K] and w [N, K] both K-contiguous, the layout of a
// hidden state and of a linear layer's weight (Voxtral Realtime 2602 audio
// encoder: 1280 -> 3 x 32 x 64 for q, k, v and 32 x 64 -> 1280 for the output
// projection; transcribe.cpp "Voxtral" family notes, Architecture).
//
// One workgroup computes an MT x NC tile of y with (MT/32) x (NC/32) waves,
// one 32 x 32 block per wave (v_mfma_f32_32x32x16_bf16: A = 32 rows of x,
// B = 32 rows of w, 16 k per step).  K advances in stages of 128: each stage's
// x and w rows go global -> registers -> LDS (rows padded to 272 bytes so the
// 16-byte operand reads of 16 consecutive rows hit distinct banks), with the
// next two stages' loads in flight in two register sets while the current
// stage computes (buffer loads with loop-invariant per-lane offsets, all
// unconditional, so the compiler keeps both stages in flight).  The epilogue
// parks the fp32 tile in LDS and writes whole 16-byte chunks: either
// y + bias (bf16 or fp32), or, for the fused q/k/v projection, q + b_q and k
// rotated at each row's position (RoPE pairs d and d+32 of a head lie in the
// same 64-column tile), v + b_v, all rounded to bf16.
#include "linear_launch.h"

namespace vx {

namespace {

constexpr int kKS = kLinKStep;       // k per stage
constexpr int kRowB = kKS * 2 + 16;  // LDS bytes per staged row

template <int MT, int NC>
struct Tile {
  static constexpr int WM = MT / 32, WN = NC / 32, NW = WM * WN, NTH = NW * 64;
  static constexpr int CH = kKS / 8;               // 16-byte chunks per staged row
  static constexpr int PX = MT * CH / NTH;         // x chunks per thread per stage
  static constexpr int PW = NC * CH / NTH;         // w chunks per thread per stage
  static constexpr int STAGE = (MT + NC) * kRowB;  // LDS bytes per stage
  static constexpr int TP = NC + 4;                // fp32 epilogue tile pitch (floats)
  static_assert(PX * NTH == MT * CH && PW * NTH == NC * CH, "stage chunks must divide evenly");
  static_assert(MT * TP * 4 <= 2 * STAGE, "epilogue tile must fit in the staging LDS");
};

enum class Epi { Plain, Gelu, Residual, SwiGLU, QkvRope };

template <int MT, int NC, Epi E, typename TO>
__global__ __launch_bounds__((MT / 32) * (NC / 32) * 64) void linear_kernel(LinearArgs a, RopeFreqs fr) {
  using TL = Tile<MT, NC>;
  __shared__ __attribute__((aligned(16))) char lds[2 * TL::STAGE];
  const int n0 = blockIdx.x * NC, m0 = blockIdx.y * MT;
  const int M = a.M, K = a.K;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % TL::WM, wn = wave / TL::WM;
  const int l32 = lane & 31, hh = lane >> 5;
  const bf16* __restrict__ x = a.x;
  const bf16* __restrict__ w = a.w;

  struct Stage {
    u32x4 x[TL::PX];
    u32x4 w[TL::PW];
  };
  // chunk u of a stage: row u / CH, 16-byte chunk u % CH (16 consecutive lanes
  // read one contiguous 256-byte row segment); rows past M repeat row M-1.
  // Buffer loads: each thread's byte offsets within the tile's rows stay in
  // VGPRs for the whole K loop and a stage adds its k offset as a scalar, so
  // no address registers are rebuilt per stage (rebuilt 64-bit addresses land
  // in registers of loads still in flight and force waits for them).  Each
  // resource covers the tile's rows exactly.
  // x rows follow the row map (the host keeps x below 2^30 bytes); w rows of
  // the tile are rows n0 .. n0+NC-1, or for SwiGLU gate rows n0/2 .. in the
  // first half of the tile and up rows n0/2 .. in the second.  A stage-load
  // slot j covers NTH/16 whole rows, so the halves fall on whole slots.
  uint32_t xo[TL::PX], wo[TL::PW];
#pragma unroll
  for (int j = 0; j < TL::PX; ++j) {
    const int u = tid + j * TL::NTH, r = u / TL::CH, c = u % TL::CH;
    const int mm = min(m0 + r, M - 1);
    xo[j] = (uint32_t)(((int64_t)(mm / a.rpg) * a.xgs + (int64_t)(mm % a.rpg) * a.xrs + 8 * c) * 2);
  }
  constexpr bool GLU = (E == Epi::SwiGLU);
#pragma unroll
  for (int j = 0; j < TL::PW; ++j) {
    const int u = tid + j * TL::NTH, r = u / TL::CH, c = u % TL::CH;
    const int rr = (GLU && j >= TL::PW / 2) ? r - NC / 2 : r;
    wo[j] = (uint32_t)(rr * K + 8 * c) * 2u;
  }
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16*>(x), (short)0, (int)a.x_bytes, 0x00020000);
  const int wrow0 = GLU ? n0 / 2 : n0, wrows = GLU ? NC / 2 : NC;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16*>(w + (size_t)wrow0 * K), (short)0, wrows * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t wr2 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16*>((GLU ? a.w2 : w) + (size_t)wrow0 * K), (short)0, wrows * K * 2, 0x00020000);
  auto load = [&](int s, Stage& R) {
    const int ko = s * kKS * 2;  // uniform byte offset of the stage
#pragma unroll
    for (int j = 0; j < TL::PX; ++j)
      R.x[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, (int)xo[j], ko, 0));
#pragma unroll
    for (int j = 0; j < TL::PW; ++j)
      R.w[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             (GLU && j >= TL::PW / 2) ? wr2 : wr, (int)wo[j], ko, 0));
  };
  auto commit = [&](const Stage& R, int b) {
    char* base = lds + b * TL::STAGE;
#pragma unroll
    for (int j = 0; j < TL::PX; ++j) {
      const int u = tid + j * TL::NTH, r = u / TL::CH, c = u % TL::CH;
      *reinterpret_cast<u32x4*>(base + r * kRowB + 16 * c) = R.x[j];
    }
#pragma unroll
    for (int j = 0; j < TL::PW; ++j) {
      const int u = tid + j * TL::NTH, r = u / TL::CH, c = u % TL::CH;
      *reinterpret_cast<u32x4*>(base + (MT + r) * kRowB + 16 * c) = R.w[j];
    }
  };
  f32x16 acc = f32x16{};
  // lane (l32, hh) holds row l32 of its 32-row block, k 8hh .. 8hh+7 of each 16-k step
  auto compute = [&](int b) {
    const char* base = lds + b * TL::STAGE;
    const char* pa = base + (32 * wm + l32) * kRowB + 16 * hh;
    const char* pb = base + (MT + 32 * wn + l32) * kRowB + 16 * hh;
#pragma unroll
    for (int kk = 0; kk < kKS / 16; ++kk) {
      const bf16x8 A = *reinterpret_cast<const bf16x8*>(pa + 32 * kk);
      const bf16x8 B = *reinterpret_cast<const bf16x8*>(pb + 32 * kk);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc, 0, 0, 0);
    }
  };

  // Every load is unconditional (past the last stage it repeats the last
  // stage, which the caches hold): with conditional loads the compiler cannot
  // count the loads in flight across the branch and waits for all of them
  // before each commit, which leaves one stage in flight instead of two.
  const int nk = K / kKS, last = nk - 1;
  Stage R0, R1;
  load(0, R0);
  load(min(1, last), R1);
  commit(R0, 0);
  __syncthreads();
  for (int s = 0; s < nk; s += 2) {
    load(min(s + 2, last), R0);
    compute(0);
    commit(R1, 1);
    __syncthreads();
    if (s + 1 >= nk) break;
    load(min(s + 3, last), R1);
    compute(1);
    commit(R0, 0);
    __syncthreads();
  }

  // ---- epilogue: the fp32 tile through LDS (the last loop step ended with a barrier)
  float* tile = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = 8 * (r >> 2) + 4 * hh + (r & 3);
    tile[(32 * wm + i) * TL::TP + 32 * wn + l32] = acc[r];
  }
  __syncthreads();

  if constexpr (E == Epi::Plain || E == Epi::Gelu || E == Epi::Residual) {
    constexpr int C8 = NC / 8;
    for (int u = tid; u < MT * C8; u += TL::NTH) {
      const int r = u / C8, c8 = u % C8, m = m0 + r;
      if (m >= M) continue;
      float v8[8];
      load8(tile + r * TL::TP + 8 * c8, v8);
      if (a.bias) {
        float b8[8];
        load8(a.bias + n0 + 8 * c8, b8);
#pragma unroll
        for (int e = 0; e < 8; ++e) v8[e] += b8[e];
      }
      const size_t yo = (size_t)((int64_t)(m / a.rpg) * a.ygs + (int64_t)(m % a.rpg) * a.yrs) + n0 + 8 * c8;
      if constexpr (E == Epi::Gelu) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v8[e] = 0.5f * v8[e] * (1.0f + erff(v8[e] * 0.70710678118654752f));
      }
      if constexpr (E == Epi::Residual) {
        float r8[8];
        load8(a.res + yo, r8);
#pragma unroll
        for (int e = 0; e < 8; ++e) v8[e] += r8[e];
      }
      store8((TO*)a.y + yo, v8);
    }
  } else if constexpr (E == Epi::SwiGLU) {
    // tile columns 0 .. NC/2-1 are gate features n0/2 .., NC/2 .. NC-1 the same up features
    constexpr int C8 = NC / 16;
    const int F = a.N / 2;
    for (int u = tid; u < MT * C8; u += TL::NTH) {
      const int r = u / C8, c8 = u % C8, m = m0 + r;
      if (m >= M) continue;
      float g8[8], u8[8];
      load8(tile + r * TL::TP + 8 * c8, g8);
      load8(tile + r * TL::TP + NC / 2 + 8 * c8, u8);
#pragma unroll
      for (int e = 0; e < 8; ++e) g8[e] = g8[e] / (1.0f + __expf(-g8[e])) * u8[e];
      store8((bf16*)a.y + (size_t)m * F + n0 / 2 + 8 * c8, g8);
    }
  } else {
    static_assert(NC == 64, "the q/k/v epilogue works on one head (64 columns) per tile");
    const int HD = a.HD;
    const int part = n0 / HD, nb = n0 - part * HD;  // 0: q, 1: k, 2: v; column of the head
    const bf16* bias = part == 0 ? a.b_q : (part == 2 ? a.b_v : nullptr);
    bf16* dst = part == 0 ? a.q : (part == 1 ? a.k : a.v);
    for (int u = tid; u < MT * 4; u += TL::NTH) {
      const int r = u >> 2, pc = u & 3, m = m0 + r;
      if (m >= M) continue;
      float xs[8], ys[8];  // dims 8pc .. 8pc+7 and their partners 32+8pc ..
      load8(tile + r * TL::TP + 8 * pc, xs);
      load8(tile + r * TL::TP + 32 + 8 * pc, ys);
      if (bias) {
        float bx[8], by[8];
        load8(bias + nb + 8 * pc, bx);
        load8(bias + nb + 32 + 8 * pc, by);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xs[e] += bx[e];
          ys[e] += by[e];
        }
      }
      if (part < 2) {
        const int64_t p = a.pos[m / a.n] + (m % a.n);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float c, s, xo, yo;
          rope_cs(p, fr.f[8 * pc + e], &c, &s);
          rope_pair(xs[e], ys[e], c, s, &xo, &yo);
          xs[e] = xo;
          ys[e] = yo;
        }
      }
      bf16* op = dst + (size_t)m * HD + nb + 8 * pc;
      store8(op, xs);
      store8(op + 32, ys);
    }
  }
}

template <int MT, int NC, Epi E, typename TO>
hipError_t launch_tile(const LinearArgs& a, const RopeFreqs& fr, hipStream_t st) {
  const dim3 grid((unsigned)(a.N / NC), (unsigned)((a.M + MT - 1) / MT));
  hipLaunchKernelGGL((linear_kernel<MT, NC, E, TO>), grid, dim3(Tile<MT, NC>::NTH), 0, st, a, fr);
  return hipGetLastError();
}

}  // namespace

template <Epi E, typename TO>
hipError_t launch_epi(const LinearArgs& a, hipStream_t st) {
  const RopeFreqs fr{};
  // 64 x 64 tiles when they alone give every CU a workgroup, else 64 x 32
  const bool wide = a.N % 64 == 0 && (int64_t)(a.N / 64) * ((a.M + 63) / 64) >= 256;
  return wide ? launch_tile<64, 64, E, TO>(a, fr, st) : launch_tile<64, 32, E, TO>(a, fr, st);
}

hipError_t launch_linear(const LinearArgs& a, DT out, hipStream_t st, LinEpi epi) {
  const bool b16 = out == DT::BF16;
  switch (epi) {
    case LinEpi::Plain:
      return b16 ? launch_epi<Epi::Plain, bf16>(a, st) : launch_epi<Epi::Plain, float>(a, st);
    case LinEpi::Gelu:
      return b16 ? launch_epi<Epi::Gelu, bf16>(a, st) : launch_epi<Epi::Gelu, float>(a, st);
    case LinEpi::Residual:
      return launch_epi<Epi::Residual, float>(a, st);
    case LinEpi::SwiGLU:
      return launch_epi<Epi::SwiGLU, bf16>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_qkv_rope(const LinearArgs& a, const RopeFreqs& fr, hipStream_t st) {
  return launch_tile<64, 64, Epi::QkvRope, bf16>(a, fr, st);
}

}  // namespace vx
