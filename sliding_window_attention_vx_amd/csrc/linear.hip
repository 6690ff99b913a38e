// Projections around the encoder's attention on bf16 matrix cores (gfx950):
// y = x w^T with x [M, K] and w [N, K] both K-contiguous, the layout of a
// hidden state and of a linear layer's weight (Voxtral Realtime 2602 audio
// encoder: 1280 -> 3 x 32 x 64 for q, k, v and 32 x 64 -> 1280 for the output
// projection; transcribe.cpp "Voxtral" family notes, Architecture).
//
// The same kernel runs the streaming encoder step's other products: the two
// causal convolutions of the stem (a row map reads each output frame's
// window of input frames as one K-contiguous row), the gate/up projection
// with SwiGLU, and the output and down projections added into the float32
// residual stream.
//
// One workgroup computes an MT x NC tile of y with (MT/32) x (NC/32) waves,
// one 32 x 32 block per wave (v_mfma_f32_32x32x16_bf16: A = 32 rows of x,
// B = 32 rows of w, 16 k per step).  K advances in stages of 64 (64 x 64
// tiles) or 128 (64 x 32 tiles); each stage's x and w rows go straight from
// global memory into LDS, three stages deep, and the operand reads come back
// through a chunk swizzle that keeps them free of bank conflicts.  The
// epilogue parks the fp32 tile in LDS and writes whole 16-byte chunks: y +
// bias (bf16 or fp32), GELU(y + bias), res + y + bias (fp32), silu(gate) * up
// (bf16), or for the fused q/k/v projection q + b_q and k rotated at each
// row's position (RoPE pairs d and d+32 of a head lie in the same 64-column
// tile), v + b_v, all rounded to bf16.
#include "linear_launch.h"

namespace vx {

namespace {

enum class Epi { Plain, Gelu, Residual, SwiGLU, Partial, QkvRope };

// Epilogue from the fp32 tile parked in LDS (pitch TP floats): whole 16-byte
// chunks of y, or of q, k, v for the fused projection.
template <int MT, int NC, Epi E, typename TO, int TP>
__device__ __forceinline__ void epilogue(const LinearArgs& a, const RopeFreqs& fr, const float* tile,
                                         int n0, int m0, int tid, int NTH) {
  const int M = a.M;
  if constexpr (E == Epi::Partial) {
    // this K part's fp32 sums, dense [M, N] at part blockIdx.z
    constexpr int C8 = NC / 8;
    float* yz = (float*)a.y + (size_t)blockIdx.z * M * a.N;
    for (int u = tid; u < MT * C8; u += NTH) {
      const int r = u / C8, c8 = u % C8, m = m0 + r;
      if (m >= M) continue;
      float v8[8];
      load8(tile + r * TP + 8 * c8, v8);
      store8(yz + (size_t)m * a.N + n0 + 8 * c8, v8);
    }
  } else if constexpr (E == Epi::Plain || E == Epi::Gelu || E == Epi::Residual) {
    constexpr int C8 = NC / 8;
    for (int u = tid; u < MT * C8; u += NTH) {
      const int r = u / C8, c8 = u % C8, m = m0 + r;
      if (m >= M) continue;
      float v8[8];
      load8(tile + r * TP + 8 * c8, v8);
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
    for (int u = tid; u < MT * C8; u += NTH) {
      const int r = u / C8, c8 = u % C8, m = m0 + r;
      if (m >= M) continue;
      float g8[8], u8[8];
      load8(tile + r * TP + 8 * c8, g8);
      load8(tile + r * TP + NC / 2 + 8 * c8, u8);
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
    for (int u = tid; u < MT * 4; u += NTH) {
      const int r = u >> 2, pc = u & 3, m = m0 + r;
      if (m >= M) continue;
      float xs[8], ys[8];  // dims 8pc .. 8pc+7 and their partners 32+8pc ..
      load8(tile + r * TP + 8 * pc, xs);
      load8(tile + r * TP + 32 + 8 * pc, ys);
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

// ---- main loop ---------------------------------------------------------------
// Stage loads go straight from global memory into LDS (buffer_load ... lds:
// lane i of a load writes 16 bytes at the wave's LDS base + 16 i): no staging
// registers and no LDS write instructions.  Three stages live in LDS, two in
// flight while one is computed.
//
// Stage layout: rows 0 .. MT-1 are x rows, MT .. MT+NC-1 w rows, KS k each
// (CH = KS/8 chunks of 16 bytes), unpadded.  Load j of wave w fills the RPI =
// 64/CH rows RPI (j NW + w) .. +RPI-1; its lane l fills row RPI (j NW + w) +
// l/CH, slot l%CH with the row's chunk (l%CH) ^ swz(row).  The MFMA operand
// reads (16 consecutive rows, one chunk) then hit distinct banks, with the
// LDS serving 16 lanes per cycle from 64 banks or 8 lanes from 32:
//   CH 8  (128-byte rows): swz(r) = (r ^ r/8) % 8, distinct (r%2, slot) over
//         16 consecutive rows and distinct slots over 8;
//   CH 16 (256-byte rows): swz(r) = r % 16, distinct slots over 16 rows and
//         distinct slots mod 8 over 8.
constexpr int kDStages = 3;

template <int CH>
__device__ __forceinline__ int dl_swz(int r) {
  if constexpr (CH == 8)
    return (r ^ (r >> 3)) & 7;
  else
    return r & 15;
}

template <int MT, int NC, int KS, int WB = 1>
struct Tile {
  // waves WM x WN, each WB 32 x 32 blocks side by side (32 x 32*WB outputs)
  static constexpr int WM = MT / 32, WN = NC / (32 * WB), NW = WM * WN, NTH = NW * 64;
  static constexpr int CH = KS / 8, RPI = 64 / CH, ROWB = KS * 2;
  static constexpr int ROWS = MT + NC;
  static constexpr int STAGE = ROWS * ROWB;
  static constexpr int NLD = ROWS * CH / NTH;  // 16-byte loads per thread per stage
  static constexpr int XLD = MT * CH / NTH;    // the first XLD of them are x rows
  static constexpr int TP = NC + 4;
  static_assert(CH == 8 || CH == 16, "stages of 64 or 128 k");
  static_assert(NLD * NTH == ROWS * CH && XLD * NTH == MT * CH, "row groups must divide evenly");
  static_assert((MT + NC / 2) % (RPI * NW) == 0, "each load takes x, gate or up rows only");
  static_assert(MT * TP * 4 <= kDStages * STAGE, "epilogue tile must fit in the staging LDS");
};

typedef __attribute__((address_space(3))) void lds_void_t;

// 16 bytes per lane from a buffer into LDS at dst + 16 * lane.  (Called from
// the kernel's lambdas through this device function: written in a lambda the
// builtin stops the host pass from emitting the kernel's launch stub.)
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, char* dst, uint32_t voff,
                                           int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 16, voff, soff, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // vmcnt N, expcnt and lgkmcnt left at their maxima (no wait)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int MT, int NC, int KS, int WB, Epi E, typename TO>
__global__ __launch_bounds__((MT / 32) * (NC / 32 / WB) * 64) void linear_kernel(LinearArgs a, RopeFreqs fr) {
  using TL = Tile<MT, NC, KS, WB>;
  constexpr int CH = TL::CH, RPI = TL::RPI;
  __shared__ __attribute__((aligned(16))) char lds[kDStages * TL::STAGE];
  const int n0 = blockIdx.x * NC, m0 = blockIdx.y * MT;
  const int M = a.M, K = a.K;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % TL::WM, wn = wave / TL::WM;
  const int l32 = lane & 31, hh = lane >> 5;
  constexpr bool GLU = (E == Epi::SwiGLU);

  // per-load source byte offsets (loop-invariant); rows past M repeat row M-1
  uint32_t vo[TL::NLD];
#pragma unroll
  for (int j = 0; j < TL::NLD; ++j) {
    const int r = RPI * (j * TL::NW + wave) + lane / CH;
    const int c = (lane % CH) ^ dl_swz<CH>(r);
    if (j < TL::XLD) {
      const int mm = min(m0 + r, M - 1);
      vo[j] = (uint32_t)(((int64_t)(mm / a.rpg) * a.xgs + (int64_t)(mm % a.rpg) * a.xrs + 8 * c) * 2);
    } else {
      const int rw = r - MT;
      const int rr = (GLU && rw >= NC / 2) ? rw - NC / 2 : rw;
      vo[j] = (uint32_t)(rr * K + 8 * c) * 2u;
    }
  }
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16*>(a.x), (short)0, (int)a.x_bytes, 0x00020000);
  const int wrow0 = GLU ? n0 / 2 : n0, wrows = GLU ? NC / 2 : NC;
  // K part of this workgroup (Partial: gridDim.z parts of nk stages each)
  const int nk = K / KS / (int)gridDim.z, kz0 = (int)blockIdx.z * nk;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16*>(a.w + (size_t)wrow0 * K), (short)0, wrows * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t wr2 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16*>((GLU ? a.w2 : a.w) + (size_t)wrow0 * K), (short)0, wrows * K * 2, 0x00020000);

  auto issue = [&](int s, int b) {
    const int ko = (s + kz0) * KS * 2;  // uniform byte offset of the stage
    char* base = lds + b * TL::STAGE;
#pragma unroll
    for (int j = 0; j < TL::NLD; ++j) {
      char* dst = base + 1024 * (j * TL::NW + wave);
      if (j < TL::XLD)
        lds_load16(xr, dst, vo[j], ko);
      else if (GLU && RPI * (j * TL::NW) >= MT + NC / 2)
        lds_load16(wr2, dst, vo[j], ko);
      else
        lds_load16(wr, dst, vo[j], ko);
    }
  };
  f32x16 acc[WB];
#pragma unroll
  for (int nb = 0; nb < WB; ++nb) acc[nb] = f32x16{};
  auto compute = [&](int b) {
    const char* base = lds + b * TL::STAGE;
    const int ra = 32 * wm + l32;
    const char* pa = base + ra * TL::ROWB;
    const int sa = dl_swz<CH>(ra);
#pragma unroll
    for (int kk = 0; kk < KS / 16; ++kk) {
      const int ch = 2 * kk + hh;
      const bf16x8 A = *reinterpret_cast<const bf16x8*>(pa + 16 * (ch ^ sa));
#pragma unroll
      for (int nb = 0; nb < WB; ++nb) {
        const int rb = MT + 32 * (WB * wn + nb) + l32;
        const bf16x8 B =
            *reinterpret_cast<const bf16x8*>(base + rb * TL::ROWB + 16 * (ch ^ dl_swz<CH>(rb)));
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc[nb], 0, 0, 0);
      }
    }
  };

  issue(0, 0);
  if (nk > 1) issue(1, 1);
  for (int s = 0; s < nk; ++s) {
    // stage s landed for this wave (stage s+1 may still be in flight), then
    // for every wave; the barrier also ends every wave's reads of stage s-1,
    // whose buffer the loads of stage s+2 reuse
    if (s + 1 < nk)
      wait_vmcnt<TL::NLD>();
    else
      wait_vmcnt<0>();
    // A plain barrier: __syncthreads() also orders this wave's memory
    // operations, which makes the compiler wait for every load in flight,
    // including the next stage's.  The wait above covers what the barrier
    // must publish; the asm statement keeps the compiler's LDS accesses on
    // their side of it.
    __asm__ volatile("s_barrier" ::: "memory");
    if (s + 2 < nk) issue(s + 2, (s + 2) % kDStages);
    compute(s % kDStages);
  }
  __syncthreads();  // every wave is done reading the stages

  float* tile = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int nb = 0; nb < WB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 8 * (r >> 2) + 4 * hh + (r & 3);
      tile[(32 * wm + i) * TL::TP + 32 * (WB * wn + nb) + l32] = acc[nb][r];
    }
  __syncthreads();
  epilogue<MT, NC, E, TO, TL::TP>(a, fr, tile, n0, m0, tid, TL::NTH);
}

template <int MT, int NC, Epi E, typename TO, int WB = 1>
hipError_t launch_tile(const LinearArgs& a, const RopeFreqs& fr, hipStream_t st) {
  const unsigned parts = E == Epi::Partial ? (unsigned)a.splits : 1u;
  const dim3 grid((unsigned)(a.N / NC), (unsigned)((a.M + MT - 1) / MT), parts);
  // 64-wide stages keep three 64 x 64 stages at 48 KB; the two-wave 64 x 32
  // tiles take 128-wide stages (half the barriers) at 72 KB
  constexpr int KS = NC >= 64 ? 64 : 128;
  hipLaunchKernelGGL((linear_kernel<MT, NC, KS, WB, E, TO>), grid, dim3(Tile<MT, NC, KS, WB>::NTH), 0,
                     st, a, fr);
  return hipGetLastError();
}

}  // namespace

template <Epi E, typename TO>
hipError_t launch_epi(const LinearArgs& a, hipStream_t st) {
  const RopeFreqs fr{};
  // 64 x 64 tiles when they alone give every CU a workgroup, else 64 x 32
  const bool wide = a.N % 64 == 0 && (int64_t)(a.N / 64) * ((a.M + 63) / 64) >= 256;
  // gate/up + SwiGLU over many columns: 64 x 128 tiles, each wave 32 x 64 (an
  // A-operand read feeds two MFMAs, and half as many tiles re-read x)
  if constexpr (E == Epi::SwiGLU) {
    if (a.N % 128 == 0 && (int64_t)(a.N / 128) * ((a.M + 63) / 64) >= 256)
      return launch_tile<64, 128, E, TO, 2>(a, fr, st);
  }
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
    case LinEpi::Partial:
      return launch_epi<Epi::Partial, float>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_qkv_rope(const LinearArgs& a, const RopeFreqs& fr, hipStream_t st) {
  return launch_tile<64, 64, Epi::QkvRope, bf16>(a, fr, st);
}

}  // namespace vx
