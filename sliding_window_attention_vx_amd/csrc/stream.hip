// Streaming step over a W-slot KV ring, and the ring append.
//
// Schedule from the transcribe.cpp "Voxtral" family notes (Streaming
// schedule): each step brings 4 encoder frames per stream.  A step is HBM
// bound: every (stream, head) reads its whole ring of rotated keys and
// values once (2 x W x 128 B in bf16) for only a handful of queries.
//
// stream_step_kernel: one workgroup (4 waves) per (stream, head, group of up
// to 4 new queries).  The keys of the group form one list: ring frames at
// positions lo .. P-1 (slot = position mod W) followed by new frames
// 0 .. i1-1 (rotated into LDS first).  The list is processed in blocks of
// 256 keys, each in two passes so K and V are read exactly once:
//   scores : 8 lanes per 128-byte key row (one 16-byte load each, fully
//            coalesced: a wave reads 8 consecutive rows per instruction);
//            partial dot products for the 4 queries are summed across the
//            8 lanes with DPP moves; masked scores become -inf; the scores
//            go to LDS;
//   softmax: one key per thread, block max/sum per query by wave shuffles,
//            running max/sum rescale (float32, log2 domain);
//   P V    : same lane layout over the value rows, p read from LDS.
// The 8-dim partial outputs are reduced across lanes and waves at the end.
//
// ring_append_kernel: one workgroup per stream; rotates the new keys (cos/sin
// per position computed once into LDS), writes keys and values to slot
// (pos+i) mod W, then advances pos after a workgroup barrier so that every
// thread has read the old value.
#include "vx_launch.h"

namespace vx {

namespace {

constexpr int kQC = 4;    // queries per workgroup
constexpr int kKB = 256;  // keys per block (one per thread in the softmax pass)

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL,
                                                            0xF, 0xF, false));
}

// Sum over each aligned group of 8 lanes; every lane of the group gets the sum.
__device__ __forceinline__ float sum8(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__host__ __device__ constexpr size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// NaN over the outputs of new queries i0 .. i1-1 of one (stream, head).
template <typename TO>
__device__ void poison_queries(TO* o, size_t frs, int i0, int i1) {
  for (int u = threadIdx.x; u < (i1 - i0) * 8; u += blockDim.x) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = __builtin_nanf("");
    store8(o + (size_t)(i0 + u / 8) * frs + 8 * (u % 8), x);
  }
}

// Dynamic LDS layout of stream_step_kernel for i1 new keys.
struct StepLds {
  size_t cs, knew, qs, sc, red, total;
  __host__ __device__ StepLds(int i1, size_t elem) {
    cs = 0;                                                // [i1][2][32] float
    knew = align16(cs + (size_t)i1 * kD * sizeof(float));  // [i1][64] TI
    qs = align16(knew + (size_t)i1 * kD * elem);           // [kQC][64] float
    sc = align16(qs + (size_t)kQC * kD * sizeof(float));   // [kKB][kQC] float
    red = align16(sc + (size_t)kKB * kQC * sizeof(float)); // [2][4 waves][kQC] float
    total = align16(red + 2 * 4 * kQC * sizeof(float));
  }
};

template <typename TI, typename TO>
__global__ __launch_bounds__(256) void stream_step_kernel(StreamArgs a, RopeFreqs fr) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int H = a.H, W = a.W, n = a.n;
  const int s = blockIdx.x / H, h = blockIdx.x % H;
  const int i0 = blockIdx.y * kQC;
  const int i1 = min(n, i0 + kQC);
  const int nq = i1 - i0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 7;  // 8-dim chunk handled by this lane

  const StepLds L(i1, sizeof(TI));
  float* cs = (float*)(smem + L.cs);
  TI* knew = (TI*)(smem + L.knew);
  float* qs = (float*)(smem + L.qs);
  float* sc = (float*)(smem + L.sc);
  float* red = (float*)(smem + L.red);

  const int64_t P = a.pos[s];
  const size_t frs = (size_t)H * kD;
  const size_t fbase = (size_t)s * n * frs + (size_t)h * kD;
  if (P < 0) {
    // an invalid position: the stream's outputs are NaN (loud, not partial)
    poison_queries<TO>((TO*)a.o + fbase, frs, i0, i1);
    return;
  }
  const int64_t lo = max((int64_t)0, P + i0 - W + 1);
  const int nring = (int)max((int64_t)0, P - lo);  // ring keys at positions lo .. P-1
  const int nk = nring + i1;
  const int lo_slot = (int)(lo % W);  // ring key kk sits at slot lo_slot + kk (mod W), kk < W
  const TI* __restrict__ qn = (const TI*)a.q + fbase;
  const TI* __restrict__ kn = (const TI*)a.k + fbase;
  const TI* __restrict__ vn = (const TI*)a.v + fbase;
  const size_t rbase = ((size_t)s * H + h) * (size_t)W * kD;
  const TI* __restrict__ rk = (const TI*)a.ring_k + rbase;
  const TI* __restrict__ rv = (const TI*)a.ring_v + rbase;

  // ---- prologue: rotate new keys 0..i1-1 into LDS, queries i0..i1-1 into qs
  if (a.rope) {
    for (int u = tid; u < i1 * kHalf; u += blockDim.x) {
      const int j = u / kHalf, i = u % kHalf;
      float cc, ss;
      rope_cs(P + j, fr.f[i], &cc, &ss);
      cs[j * kD + i] = cc;
      cs[j * kD + kHalf + i] = ss;
    }
    __syncthreads();
  }
  for (int u = tid; u < (i1 + kQC) * 4; u += blockDim.x) {
    const int row = u >> 2, cp = u & 3;
    const bool isq = row >= i1;
    const int qi = row - i1;  // query slot when isq
    if (isq && qi >= nq) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qs[qi * kD + 8 * cp + e] = 0.f;
        qs[qi * kD + kHalf + 8 * cp + e] = 0.f;
      }
      continue;
    }
    const int j = isq ? i0 + qi : row;  // new-frame index
    const TI* src = (isq ? qn : kn) + (size_t)j * frs + 8 * cp;
    float x[8], y[8];
    load8(src, x);
    load8(src + kHalf, y);
    if (a.rope) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float xo, yo;
        rope_pair(x[e], y[e], cs[j * kD + 8 * cp + e], cs[j * kD + kHalf + 8 * cp + e], &xo, &yo);
        x[e] = round_to<TI>(xo);
        y[e] = round_to<TI>(yo);
      }
    }
    if (isq) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qs[qi * kD + 8 * cp + e] = x[e];
        qs[qi * kD + kHalf + 8 * cp + e] = y[e];
      }
    } else {
      store8(knew + (size_t)j * kD + 8 * cp, x);
      store8(knew + (size_t)j * kD + kHalf + 8 * cp, y);
    }
  }
  __syncthreads();

  float qreg[kQC][8];
#pragma unroll
  for (int i = 0; i < kQC; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) qreg[i][e] = qs[i * kD + 8 * c + e];

  float m_i[kQC], l_i[kQC], op[kQC][8];
#pragma unroll
  for (int i = 0; i < kQC; ++i) {
    m_i[i] = -INFINITY;
    l_i[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) op[i][e] = 0.f;
  }
  const float c2 = a.scale_log2;
  const int sub = wave * 8 + (lane >> 3);  // row within a 32-row slab

  for (int kb0 = 0; kb0 < nk; kb0 += kKB) {
    const int nkb = min(kKB, nk - kb0);
    // -- scores
    for (int r0 = 0; r0 < nkb; r0 += 32) {
      const int kr = r0 + sub;  // key within block
      const int kk = kb0 + kr;  // key within list
      float part[kQC];
#pragma unroll
      for (int i = 0; i < kQC; ++i) part[i] = 0.f;
      if (kr < nkb) {
        float kv[8];
        if (kk < nring) {
          int slot = lo_slot + kk;
          if (slot >= W) slot -= W;
          load8(rk + (size_t)slot * kD + 8 * c, kv);
        } else {
          load8(knew + (size_t)(kk - nring) * kD + 8 * c, kv);
        }
#pragma unroll
        for (int i = 0; i < kQC; ++i)
#pragma unroll
          for (int e = 0; e < 8; ++e) part[i] = fmaf(qreg[i][e], kv[e], part[i]);
      }
#pragma unroll
      for (int i = 0; i < kQC; ++i) part[i] = sum8(part[i]);
      if (c == 0 && kr < nkb) {
        const int64_t p = lo + kk;  // absolute position of this key
        f32x4 w;
#pragma unroll
        for (int i = 0; i < kQC; ++i) {
          const int64_t pq = P + i0 + i;
          const bool ok = (i < nq) && (p <= pq) && (p >= pq - W + 1);
          w[i] = ok ? part[i] * c2 : -INFINITY;
        }
        *reinterpret_cast<f32x4*>(sc + kr * kQC) = w;
      }
    }
    __syncthreads();
    // -- block softmax statistics (thread = key)
    f32x4 xv;
    if (tid < nkb) {
      xv = *reinterpret_cast<const f32x4*>(sc + tid * kQC);
    } else {
#pragma unroll
      for (int i = 0; i < kQC; ++i) xv[i] = -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < kQC; ++i) {
      const float bm = wave_max(xv[i]);
      if (lane == 0) red[wave * kQC + i] = bm;
    }
    __syncthreads();
    float alpha[kQC], mu[kQC];
#pragma unroll
    for (int i = 0; i < kQC; ++i) {
      float bm = red[i];
#pragma unroll
      for (int w = 1; w < 4; ++w) bm = fmaxf(bm, red[w * kQC + i]);
      const float mn = fmaxf(m_i[i], bm);
      alpha[i] = (mn == -INFINITY) ? 1.f : exp2f(m_i[i] - mn);
      mu[i] = (mn == -INFINITY) ? 0.f : mn;
      m_i[i] = mn;
    }
    f32x4 pv;
#pragma unroll
    for (int i = 0; i < kQC; ++i) pv[i] = exp2f(xv[i] - mu[i]);
    if (tid < nkb) *reinterpret_cast<f32x4*>(sc + tid * kQC) = pv;
#pragma unroll
    for (int i = 0; i < kQC; ++i) {
      const float bs = wave_sum(pv[i]);
      if (lane == 0) red[4 * kQC + wave * kQC + i] = bs;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kQC; ++i) {
      float bs = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) bs += red[4 * kQC + w * kQC + i];
      l_i[i] = l_i[i] * alpha[i] + bs;
#pragma unroll
      for (int e = 0; e < 8; ++e) op[i][e] *= alpha[i];
    }
    // -- P V
    for (int r0 = 0; r0 < nkb; r0 += 32) {
      const int kr = r0 + sub;
      const int kk = kb0 + kr;
      if (kr < nkb) {
        float vv[8];
        if (kk < nring) {
          int slot = lo_slot + kk;
          if (slot >= W) slot -= W;
          load8(rv + (size_t)slot * kD + 8 * c, vv);
        } else {
          load8(vn + (size_t)(kk - nring) * frs + 8 * c, vv);
        }
        const f32x4 pp = *reinterpret_cast<const f32x4*>(sc + kr * kQC);
#pragma unroll
        for (int i = 0; i < kQC; ++i)
#pragma unroll
          for (int e = 0; e < 8; ++e) op[i][e] = fmaf(pp[i], vv[e], op[i][e]);
      }
    }
    __syncthreads();
  }

  // ---- reduce the per-lane partial outputs: lanes with equal c, then waves
#pragma unroll
  for (int i = 0; i < kQC; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = op[i][e];
      x += __shfl_xor(x, 8, 64);
      x += __shfl_xor(x, 16, 64);
      x += __shfl_xor(x, 32, 64);
      op[i][e] = x;
    }
  float* fin = sc;  // [4 waves][8 chunks][kQC][8]: exactly kKB*kQC floats
  if (lane < 8) {
#pragma unroll
    for (int i = 0; i < kQC; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) fin[((wave * 8 + lane) * kQC + i) * 8 + e] = op[i][e];
  }
  __syncthreads();
  {
    const int i = tid >> 6, d = tid & 63;  // 256 threads = kQC queries x 64 dims
    if (i < nq) {
      const int cc = d >> 3, e = d & 7;
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) acc += fin[((w * 8 + cc) * kQC + i) * 8 + e];
      TO* op_ = (TO*)a.o + fbase + (size_t)(i0 + i) * frs + d;
      *op_ = (TO)(acc / l_i[i]);
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 streaming step on matrix cores (v_mfma_f32_16x16x32_bf16).
//
// One workgroup of kSWaves waves per (stream, head, chunk of up to 16 new
// queries): the 16 query columns of the MFMA hold the chunk (4 in the Voxtral
// schedule; the rest are zero).  The keys' 32-key blocks are cut into one
// contiguous run per wave, so twice as many ring reads are in flight as with
// one wave per ring; the waves' partial (max, sum, O) merge through LDS at the
// end.  Per block and wave:
//   S^T = K' Q'^T  two 16-key MFMA pairs; the A operand (16 keys x 8 dims per
//                  lane).  Ring keys load as whole 128-byte rows (8 lanes per
//                  row, like the values) into this wave's LDS (144-byte rows)
//                  and come back in the operand layout; new keys are rotated
//                  in registers (dims d and d+32 sit in the same lane).
//   softmax        lane (q, g) holds query q's scores for keys 4g..4g+3 and
//                  16+4g..16+4g+3; the row max/sum reduce over the four lanes
//                  of q with v_permlane16_swap / v_permlane32_swap; lazy
//                  running max as in the prefill.
//   O^T += V^T P^T V goes HBM -> VGPR -> this wave's LDS (160-byte rows) and
//                  comes back through ds_read_b64_tr_b16, which hands a lane
//                  four consecutive keys of one dim: exactly the key order
//                  of the score registers.
// The next block's K and V loads (8 KB) are issued before the current block's
// math.  Ring rows are read with non-temporal loads.
constexpr int kSQ = 16;                    // query columns per wave
constexpr int kSWaves = 2;                 // waves per workgroup, each taking half the keys
constexpr int kSRowV = 160;                // LDS bytes per staged V row (conflict-free)
constexpr int kSBufV = 32 * kSRowV;        // one 32-key V block
constexpr int kSRowK = 144;                // LDS bytes per staged K row (conflict-free reads)
constexpr int kSBufK = 32 * kSRowK;        // one 32-key K block
constexpr int kSWaveBuf = kSBufV + kSBufK;  // one wave's staging rows

__device__ __forceinline__ float max16x(float x) {  // max over lanes l, l^16
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max32x(float x) {  // max over lanes l, l^32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum16x(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum32x(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __attribute__((address_space(3))) bf16x4 s_lds_bf16x4;

// Ring rows are streamed once per step: non-temporal loads keep them from
// displacing other lines.
__device__ __forceinline__ u32x4 ring_row_load(const bf16* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

template <typename TO>
__global__ __launch_bounds__(kSWaves * 64, 4) void stream_step_mfma_kernel(StreamArgs a, RopeFreqs fr) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* cs = (float*)smem;                                  // [i1][2][32] cos/sin
  char* work = smem + align16((size_t)a.n * kD * sizeof(float));
  const int H = a.H, W = a.W, n = a.n;
  const int s = blockIdx.x / H, h = blockIdx.x % H;
  const int i0 = blockIdx.y * kSQ;
  const int i1 = min(n, i0 + kSQ);
  const int nq = i1 - i0;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane & 15, g = lane >> 4;
  char* vbuf = work + wave * kSWaveBuf;  // this wave's V block, then its K block
  char* kbuf = vbuf + kSBufV;

  const int64_t P = a.pos[s];
  const size_t frs = (size_t)H * kD;
  const size_t fbase = (size_t)s * n * frs + (size_t)h * kD;
  if (P < 0) {
    // an invalid position: the stream's outputs are NaN, its ring is not
    // written and its position stays as it was (loud, not partial)
    poison_queries<TO>((TO*)a.o + fbase, frs, i0, i1);
    if (a.append && h == 0 && i0 == 0 && tid == 0) a.pos_out[s] = P;
    return;
  }
  const int64_t lo = max((int64_t)0, P + i0 - W + 1);
  const int nring = (int)max((int64_t)0, P - lo);  // ring keys at positions lo .. P-1
  const int nk = nring + i1;                       // then new frames 0 .. i1-1
  const int lo_slot = (int)(lo % W);
  const bf16* __restrict__ qn = (const bf16*)a.q + fbase;
  const bf16* __restrict__ kn = (const bf16*)a.k + fbase;
  const bf16* __restrict__ vn = (const bf16*)a.v + fbase;
  const size_t rbase = ((size_t)s * H + h) * (size_t)W * kD;
  const bf16* rk = (const bf16*)a.ring_k + rbase;  // not restrict: the fused append writes it
  const bf16* rv = (const bf16*)a.ring_v + rbase;
  const bool rope = a.rope;

  // per-block loads: K A-operand rows (2 sub-blocks x 2 dim halves) and V rows
  struct Blk {
    u32x4 k[2][2];  // [sub-block][dim half]
    u32x4 v[4];     // 4 x (8 rows x 16 bytes) of the 32 V rows
  };
  // blocks made only of ring keys (kb + 32 <= nring): unconditional loads.
  // Keys load whole 128-byte rows like the values (k[sb][hf] holds rows
  // 16sb + 8hf + lane/8, 16-byte chunk lane%8) and reach the A-operand layout
  // through the wave's LDS rows: a lane's operand needs one key per lane%16,
  // which would split every row over two load instructions.
  auto load_ring = [&](int kb, Blk& B) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        int slot = lo_slot + kb + 16 * sb + 8 * hf + (lane >> 3);
        if (slot >= W) slot -= W;
        B.k[sb][hf] = ring_row_load(rk + (size_t)slot * kD + 8 * (lane & 7));
      }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int slot = lo_slot + kb + 8 * j + (lane >> 3);
      if (slot >= W) slot -= W;
      B.v[j] = ring_row_load(rv + (size_t)slot * kD + 8 * (lane & 7));
    }
  };

  // the keys' 32-key blocks are split into kSWaves contiguous runs, one per wave
  const int nblk = (nk + 31) / 32;
  const int b0 = wave * nblk / kSWaves, b1 = (wave + 1) * nblk / kSWaves;
  // The first pure-ring block's loads go out before the cos/sin below (float64
  // angles) so that the ring stream starts at once.
  const int bf = min(b1, max(b0, nring >> 5));
  Blk cur, nxt;
  if (b0 < bf) load_ring(32 * b0, cur);

  // cos/sin of the new positions P .. P+i1-1 (float64 angle, as everywhere)
  if (rope) {
    for (int u = tid; u < i1 * kHalf; u += kSWaves * 64) {
      const int j = u / kHalf, f = u % kHalf;
      float cc, ss;
      rope_cs(P + j, fr.f[f], &cc, &ss);
      cs[j * kD + f] = cc;
      cs[j * kD + kHalf + f] = ss;
    }
  }
  __syncthreads();

  // rotated new row j (dims 8g..8g+7 and 32+8g..32+8g+7) as two bf16x8 words
  auto new_row = [&](const bf16* base, int j, u32x4& x, u32x4& y) {
    x = *reinterpret_cast<const u32x4*>(base + (size_t)j * frs + 8 * g);
    y = *reinterpret_cast<const u32x4*>(base + (size_t)j * frs + kHalf + 8 * g);
    if (rope) {
      float xf[8], yf[8];
      unpack8(x, xf);
      unpack8(y, yf);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float xo, yo;
        rope_pair(xf[e], yf[e], cs[j * kD + 8 * g + e], cs[j * kD + kHalf + 8 * g + e], &xo, &yo);
        xf[e] = xo;
        yf[e] = yo;
      }
      x = pack8(xf);
      y = pack8(yf);
    }
  };

  // Q' (B operand): lane (q, g) holds query i0+q, dims 8g.. (m=0) and 32+8g.. (m=1)
  bf16x8 qf[2];
  {
    u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
    if (q < nq) new_row(qn, i0 + q, x, y);
    qf[0] = __builtin_bit_cast(bf16x8, x);
    qf[1] = __builtin_bit_cast(bf16x8, y);
  }

  auto load_blk = [&](int kb, Blk& B) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int kk = kb + 16 * sb + q;  // key of this lane's A row
      if (kk < nring) {
        int slot = lo_slot + kk;
        if (slot >= W) slot -= W;
        const bf16* kr = rk + (size_t)slot * kD + 8 * g;
        B.k[sb][0] = ring_row_load(kr);
        B.k[sb][1] = ring_row_load(kr + kHalf);
      } else if (kk < nk) {
        new_row(kn, kk - nring, B.k[sb][0], B.k[sb][1]);
      } else {
        B.k[sb][0] = u32x4{0, 0, 0, 0};
        B.k[sb][1] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 8 * j + (lane >> 3), c = lane & 7;
      const int kk = kb + row;
      if (kk < nring) {
        int slot = lo_slot + kk;
        if (slot >= W) slot -= W;
        B.v[j] = ring_row_load(rv + (size_t)slot * kD + 8 * c);
      } else if (kk < nk) {
        B.v[j] = *reinterpret_cast<const u32x4*>(vn + (size_t)(kk - nring) * frs + 8 * c);
      } else {
        B.v[j] = u32x4{0, 0, 0, 0};
      }
    }
  };

  // tr16 read address: lane L of group g points at row 4g + L/4, dims 4*(L%4)
  const int v_off = (4 * g + (q >> 2)) * kSRowV + 4 * (q & 3) * 2;
  const float c2 = a.scale_log2;
  const int64_t pq = P + i0 + q;  // this lane's query position
  f32x4 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // One block.  Only the first block (ring keys that leave the window of a
  // later query of the chunk: key index < 15) and the blocks past the ring
  // keys (new frames, padding) can hold masked keys; the others skip the mask.
  // The wave's V and K rows are rewritten every block with no barrier: LDS
  // instructions of one wave execute in order, so a block's writes land after
  // the previous block's reads; the asm statements keep the compiler's order.
  auto step = [&](const Blk& cur, int bi, bool ring_rows) {
    const int kb = 32 * bi;
    char* vb = vbuf;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4*>(vb + (8 * j + (lane >> 3)) * kSRowV + 16 * (lane & 7)) = cur.v[j];
    u32x4 ka[2][2];
    if (ring_rows) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          *reinterpret_cast<u32x4*>(kbuf + (16 * sb + 8 * hf + (lane >> 3)) * kSRowK +
                                    16 * (lane & 7)) = cur.k[sb][hf];
      __asm__ volatile("" ::: "memory");
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          ka[sb][hf] = *reinterpret_cast<const u32x4*>(kbuf + (16 * sb + q) * kSRowK + 64 * hf +
                                                       16 * g);
    } else {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) ka[sb][hf] = cur.k[sb][hf];
    }

    f32x4 sc[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[sb][0]),
                                                    qf[0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[sb][1]),
                                                    qf[1], acc, 0, 0, 0);
      sc[sb] = acc;
    }
    if (kb < kSQ - 1 || kb + 32 > nring) {
      // key kb+16sb+4g+r sits at position lo+kk (ring) or P+(kk-nring) (new)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kk = kb + 16 * sb + 4 * g + r;
          const int64_t pk = kk < nring ? lo + kk : P + (kk - nring);
          const bool ok = (q < nq) && (kk < nk) && (pk <= pq) && (pk > pq - W);
          sc[sb][r] = ok ? sc[sb][r] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[sb][r]);
    mx = max32x(max16x(mx)) * c2;
    const bool need = mx > m_run + 8.0f;
    if (__any(need)) {
      const float m_new = need ? mx : m_run;
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[db][r] *= alpha;
      m_run = m_new;
    }
    const float mu = (m_run == -INFINITY) ? 0.f : m_run;
    float p[8];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 4; ++r) p[4 * sb + r] = __builtin_amdgcn_exp2f(fmaf(sc[sb][r], c2, -mu));
    const u32x4 pw = pack8(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) l_run = dot2_ones(pw[i], l_run);
    const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
    // The V rows written above are read back below by the same wave; LDS
    // instructions of one wave execute in order, so only the compiler must
    // keep the order.
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const char* p0 = vb + v_off + 32 * db;
      const bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((s_lds_bf16x4*)p0);
      const bf16x4 vb2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((s_lds_bf16x4*)(p0 + 16 * kSRowV));
      const bf16x8 vf = __builtin_shufflevector(va, vb2, 0, 1, 2, 3, 4, 5, 6, 7);
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, oacc[db], 0, 0, 0);
    }
    __asm__ volatile("" ::: "memory");
  };
  // this wave's pure-ring blocks [b0, bf) with the next block's loads in
  // flight while one computes (the first block's loads were issued at the
  // start), then the (at most two) blocks that hold new frames or padding
  for (int bi = b0; bi < bf; ++bi) {
    if (bi + 1 < bf) load_ring(32 * (bi + 1), nxt);
    step(cur, bi, true);
    cur = nxt;
  }
  for (int bi = bf; bi < b1; ++bi) {
    load_blk(32 * bi, cur);
    step(cur, bi, false);
  }

  // ---- merge the waves' partial (max, sum, O^T) through LDS
  __syncthreads();  // both waves are done with their V blocks and their ring reads
  float* Mw = reinterpret_cast<float*>(work);  // [kSWaves][16] running max (log2 domain)
  float* Lw = Mw + kSWaves * 16;               // [kSWaves][16] row sums
  float* Ow = Lw + kSWaves * 16;               // [kSWaves][16][64] unnormalised O
  {
    const float l_tot = sum32x(sum16x(l_run));
    if (g == 0) {
      Mw[wave * 16 + q] = m_run;
      Lw[wave * 16 + q] = l_tot;
    }
    // O^T[d = 16db + 4g + r][q]
#pragma unroll
    for (int db = 0; db < 4; ++db)
      *reinterpret_cast<f32x4*>(Ow + (wave * 16 + q) * kD + 16 * db + 4 * g) = oacc[db];
  }
  __syncthreads();

  if (a.append) {
    // fused append (one chunk per (stream, head), so every ring read of this
    // ring is done): rotated new keys and raw values go to slot (P+j) mod W.
    const int j = q;
    if (wave == 0 && j < n) {
      int slot = (int)(((P % W) + W) % W) + j;
      if (slot >= W) slot -= W;
      u32x4 x, y;
      new_row(kn, j, x, y);
      bf16* wk = (bf16*)a.ring_k_w + rbase + (size_t)slot * kD;
      bf16* wv = (bf16*)a.ring_v_w + rbase + (size_t)slot * kD;
      *reinterpret_cast<u32x4*>(wk + 8 * g) = x;
      *reinterpret_cast<u32x4*>(wk + kHalf + 8 * g) = y;
      *reinterpret_cast<u32x4*>(wv + 8 * g) =
          *reinterpret_cast<const u32x4*>(vn + (size_t)j * frs + 8 * g);
      *reinterpret_cast<u32x4*>(wv + kHalf + 8 * g) =
          *reinterpret_cast<const u32x4*>(vn + (size_t)j * frs + kHalf + 8 * g);
    }
    if (h == 0 && tid == 0) a.pos_out[s] = P + n;
  }

  // O rows: query i0+qq, dims d0 .. d0+7 per thread
  for (int t = tid; t < nq * 8; t += kSWaves * 64) {
    const int qq = t >> 3, d0 = 8 * (t & 7);
    float mst = -INFINITY;
#pragma unroll
    for (int w = 0; w < kSWaves; ++w) mst = fmaxf(mst, Mw[w * 16 + qq]);
    float den = 0.f, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int w = 0; w < kSWaves; ++w) {
      const float mw = Mw[w * 16 + qq];
      const float sw = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - mst);
      den = fmaf(sw, Lw[w * 16 + qq], den);
      float ov[8];
      load8(Ow + (w * 16 + qq) * kD + d0, ov);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(sw, ov[e], acc[e]);
    }
    const float inv = 1.f / den;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    store8((TO*)a.o + fbase + (size_t)(i0 + qq) * frs + d0, acc);
  }
}

template <typename TI>
__global__ __launch_bounds__(256) void ring_append_kernel(AppendArgs a, RopeFreqs fr) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* cs = (float*)smem;  // [n][2][32]
  const int s = blockIdx.x;
  const int H = a.H, W = a.W, n = a.n;
  const int tid = threadIdx.x;
  const int64_t P = a.pos[s];
  if (P < 0) {
    // an invalid position: nothing is appended and the position is kept
    if (tid == 0) a.pos_out[s] = P;
    return;
  }
  const int p_slot = (int)(P % W);  // slot of position P
  if (a.rope) {
    for (int u = tid; u < n * kHalf; u += blockDim.x) {
      const int i = u / kHalf, f = u % kHalf;
      float cc, ss;
      rope_cs(P + i, fr.f[f], &cc, &ss);
      cs[i * kD + f] = cc;
      cs[i * kD + kHalf + f] = ss;
    }
  }
  __syncthreads();
  const size_t frs = (size_t)H * kD;
  const int units = n * H * 4;
  for (int u = tid; u < units; u += blockDim.x) {
    const int cp = u & 3;
    const int ih = u >> 2;
    const int h = ih % H, i = ih / H;
    int slot = p_slot + i;  // i < n <= W
    if (slot >= W) slot -= W;
    const size_t src = ((size_t)s * n + i) * frs + (size_t)h * kD + 8 * cp;
    const size_t dst = (((size_t)s * H + h) * W + slot) * kD + 8 * cp;
    const TI* kp = (const TI*)a.k + src;
    const TI* vp = (const TI*)a.v + src;
    float x[8], y[8];
    load8(kp, x);
    load8(kp + kHalf, y);
    if (a.rope) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float xo, yo;
        rope_pair(x[e], y[e], cs[i * kD + 8 * cp + e], cs[i * kD + kHalf + 8 * cp + e], &xo, &yo);
        x[e] = xo;
        y[e] = yo;
      }
    }
    TI* rk = (TI*)a.ring_k + dst;
    store8(rk, x);
    store8(rk + kHalf, y);
    float vx8[8], vy8[8];
    load8(vp, vx8);
    load8(vp + kHalf, vy8);
    TI* rvp = (TI*)a.ring_v + dst;
    store8(rvp, vx8);
    store8(rvp + kHalf, vy8);
  }
  __syncthreads();
  if (tid == 0) a.pos_out[s] = P + n;
}

}  // namespace

hipError_t launch_stream_step(const StreamArgs& a, DT io, DT out, const RopeFreqs& fr,
                              hipStream_t st) {
  dim3 grid((unsigned)(a.S * a.H), (unsigned)((a.n + kQC - 1) / kQC));
  const size_t elem = io == DT::BF16 ? 2 : 4;
  const size_t smem = StepLds(a.n, elem).total;
  if (io == DT::F32) {
    hipLaunchKernelGGL((stream_step_kernel<float, float>), grid, dim3(256), smem, st, a, fr);
    return hipGetLastError();
  }
  // bf16: matrix-core kernel, one wave per (stream, head, 16-query chunk)
  dim3 grid16((unsigned)(a.S * a.H), (unsigned)((a.n + kSQ - 1) / kSQ));
  constexpr size_t kVBufs = (size_t)kSWaves * kSWaveBuf;
  constexpr size_t kMerge = (size_t)kSWaves * (2 * 16 + 16 * kD) * sizeof(float);
  const size_t smem16 = align16((size_t)a.n * kD * sizeof(float)) + (kVBufs > kMerge ? kVBufs : kMerge);
  if (out == DT::BF16)
    hipLaunchKernelGGL((stream_step_mfma_kernel<bf16>), grid16, dim3(kSWaves * 64), smem16, st, a, fr);
  else
    hipLaunchKernelGGL((stream_step_mfma_kernel<float>), grid16, dim3(kSWaves * 64), smem16, st, a, fr);
  return hipGetLastError();
}

hipError_t launch_ring_append(const AppendArgs& a, DT io, const RopeFreqs& fr, hipStream_t st) {
  const size_t smem = (size_t)a.n * kD * sizeof(float);
  if (io == DT::F32)
    hipLaunchKernelGGL(ring_append_kernel<float>, dim3(a.S), dim3(256), smem, st, a, fr);
  else
    hipLaunchKernelGGL(ring_append_kernel<bf16>, dim3(a.S), dim3(256), smem, st, a, fr);
  return hipGetLastError();
}

}  // namespace vx
