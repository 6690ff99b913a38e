// Grouped-query decode step with fused ring append, on bf16 matrix cores
// (gfx950), head_dim 128: one step of the Voxtral Realtime 2602 text decoder
// (transcribe.cpp "Voxtral" family notes, Architecture: 32 query heads over
// 8 key/value heads, head_dim 128, sliding window 8192, RoPE theta 1e6).
//
// One workgroup of NW waves per (stream, key/value head).  The 16 query
// columns of v_mfma_f32_16x16x32_bf16 hold the step's queries of the group:
// column c is new token c / G of query head kvh*G + c % G, so one token of a
// 32/8 decoder fills 4 columns and the key/value rows are read once for all
// four heads.  Every column reads the same keys: the ring slots of positions
// max(0, P-W+1) .. P-1, then the n new tokens.  The keys are cut into NW
// contiguous runs of 32-key blocks, one run per wave, and each wave keeps the
// next block's ring loads in flight while it computes the current one:
//   S^T = K' Q'^T  four MFMAs per 16 keys (128 dims); the A operand: lane
//                  (key, g) holds dims 32m+8g..32m+8g+7 of step m.  Ring
//                  keys load as whole 256-byte rows (16 lanes per row) into
//                  the wave's LDS rows (272 bytes) and come back in that
//                  layout; new keys are rotated in registers (the RoPE
//                  partner dims d+64 sit in the same lane).
//   softmax        lane (c, g) holds column c's scores of keys 4g..4g+3 and
//                  16+4g..16+4g+3; the max and the sum reduce over lanes c,
//                  c^16, c^32, c^48 with permlane swaps; the running max is
//                  lazy (it moves only when a score exceeds it by more than 8
//                  in the log2 domain, so every weight stays <= 256).
//   O^T += V^T P^T V rows pass through the wave's own LDS rows (288 bytes,
//                  so the transpose reads hit distinct banks) and come back
//                  as the A operand through ds_read_b64_tr_b16, four
//                  consecutive keys of one dim per read: the key order of
//                  the score registers.
// The waves' partial (max, sum, O) merge through LDS.  Then the workgroup,
// the only one that touches its ring, writes the rotated new keys and the new
// values into their slots (after all of its reads) and advances pos.
#include "gqa_launch.h"

namespace vx {

namespace {

constexpr int kVRow = 288;          // LDS bytes per staged V row (256 + 32)
constexpr int kVBuf = 32 * kVRow;   // one wave's 32-key V block
constexpr int kKRow = 272;          // LDS bytes per staged K row (256 + 16: conflict-free reads)
constexpr int kKBuf = 32 * kKRow;   // one wave's 32-key K block
constexpr int kWaveBuf = kVBuf + kKBuf;
constexpr float kLazyMax = 8.0f;    // log2-domain slack of the running max

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

__device__ __forceinline__ float lanes16_max(float x) {  // max over lanes l, l^16
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float lanes32_max(float x) {  // max over lanes l, l^32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float lanes16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float lanes32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Ring rows are read once per step and not again until the next step has
// streamed the whole ring set through the caches: non-temporal loads keep
// them from displacing other lines (measured: 10% shorter steps at 8192 slots).
__device__ __forceinline__ u32x4 ring_load(const bf16* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// One 32-key block in registers: K' rows and V rows.  k holds either the
// A-operand layout ([16-key half][32-dim MFMA step]: key 16*half + lane%16)
// or, for pure-ring blocks, whole rows (k[sb][m]: row 16sb + 4m + lane/16,
// 16 bytes at 16*(lane%16)).
struct KvBlock {
  u32x4 k[2][4];
  u32x4 v[8];     // row 4j + lane/16, 16 bytes at 16*(lane%16)
};

template <int NW, typename TO>
__global__ __launch_bounds__(NW * 64) void gqa_decode_kernel(GqaDecodeArgs a, RopeFreqs128 fr) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int Hkv = a.Hkv, W = a.W, n = a.n;
  const int G = a.Hq / Hkv;
  const int ncol = n * G;
  const int s = blockIdx.x / Hkv, kvh = blockIdx.x % Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  float* cs = (float*)smem;  // [n][128]: cos of pair i at j*128+i, sin at j*128+64+i
  char* work = smem + (size_t)n * kGD * sizeof(float);
  char* vb = work + wave * kWaveBuf;
  char* kbuf = vb + kVBuf;

  const int64_t P = a.pos_in[s];
  const int64_t lo = P - W + 1 > 0 ? P - W + 1 : 0;
  const int nring = (int)(P > lo ? P - lo : 0);  // ring keys at positions lo .. P-1
  const int nk = nring + n;                      // then the new tokens
  const int lo_slot = (int)(lo % W);
  const size_t qrs = (size_t)a.Hq * kGD, krs = (size_t)Hkv * kGD;
  const bf16* __restrict__ qn = a.q + (size_t)s * n * qrs + (size_t)kvh * G * kGD;
  const bf16* __restrict__ kn = a.k + (size_t)s * n * krs + (size_t)kvh * kGD;
  const bf16* __restrict__ vn = a.v + (size_t)s * n * krs + (size_t)kvh * kGD;
  const size_t rbase = ((size_t)s * Hkv + kvh) * (size_t)W * kGD;
  const bf16* rk = a.ring_k + rbase;  // not restrict: written at the end
  const bf16* rv = a.ring_v + rbase;
  const bool rope = a.rope;

  // blocks made only of ring keys: no mask except the window edge of later
  // tokens, no new-token rotation
  auto load_ring = [&](int kb, KvBlock& B) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        int slot = lo_slot + kb + 16 * sb + 4 * m + g;
        if (slot >= W) slot -= W;
        B.k[sb][m] = ring_load(rk + (size_t)slot * kGD + 8 * c);
      }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int slot = lo_slot + kb + 4 * j + g;
      if (slot >= W) slot -= W;
      B.v[j] = ring_load(rv + (size_t)slot * kGD + 8 * c);
    }
  };
  // this wave's blocks [b0, b1): first the pure-ring ones [b0, bf), two
  // register sets in turn so that one block's loads fly while the other
  // computes, then the (at most two) blocks that hold new tokens or padding
  const int nblk = (nk + 31) >> 5;
  const int b0 = (int)((int64_t)wave * nblk / NW);
  const int b1 = (int)((int64_t)(wave + 1) * nblk / NW);
  const int nfull = nring >> 5;
  const int bf = min(b1, max(b0, nfull));
  const int edge = n - 1;  // ring keys kk < n-1 can fall out of a later token's window
  // The first pure-ring block's loads go out before the cos/sin below (float64
  // angles) so that the ring stream starts at once.
  KvBlock B0, B1;
  if (b0 < bf) load_ring(32 * b0, B0);

  if (rope) {
    for (int u = tid; u < n * kGHalf; u += NW * 64) {
      const int j = u / kGHalf, i = u % kGHalf;
      float cc, ss;
      rope_cs(P + j, fr.f[i], &cc, &ss);
      cs[j * kGD + i] = cc;
      cs[j * kGD + kGHalf + i] = ss;
    }
  }
  __syncthreads();

  // rotate chunk c8 (dims 8*c8 ..) and its partner chunk c8+8 of new token j
  auto rot = [&](int j, int c8, u32x4& x, u32x4& y) {
    if (!rope) return;
    float xf[8], yf[8], cc[8], ss[8];
    unpack8(x, xf);
    unpack8(y, yf);
    load8(cs + j * kGD + 8 * c8, cc);
    load8(cs + j * kGD + kGHalf + 8 * c8, ss);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float xo, yo;
      rope_pair(xf[e], yf[e], cc[e], ss[e], &xo, &yo);
      xf[e] = xo;
      yf[e] = yo;
    }
    x = pack8(xf);
    y = pack8(yf);
  };

  // Q' (B operand): lane (c, g) holds column c, chunk 4m+g in step m (m = 0, 1)
  // and its partner chunk 4m+g+8 in step m+2
  bf16x8 qf[4];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
    if (c < ncol) {
      const int j = c / G;
      const bf16* qp = qn + (size_t)j * qrs + (size_t)(c - j * G) * kGD + 8 * (4 * m + g);
      x = *reinterpret_cast<const u32x4*>(qp);
      y = *reinterpret_cast<const u32x4*>(qp + kGHalf);
      rot(j, 4 * m + g, x, y);
    }
    qf[m] = __builtin_bit_cast(bf16x8, x);
    qf[m + 2] = __builtin_bit_cast(bf16x8, y);
  }

  // any block: ring keys, new tokens (rotated here) and zero padding past nk
  auto load_any = [&](int kb, KvBlock& B) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int kk = kb + 16 * sb + c;
      if (kk < nring) {
        int slot = lo_slot + kk;
        if (slot >= W) slot -= W;
        const bf16* kr = rk + (size_t)slot * kGD + 8 * g;
#pragma unroll
        for (int m = 0; m < 4; ++m) B.k[sb][m] = ring_load(kr + 32 * m);
      } else if (kk < nk) {
        const int j = kk - nring;
        const bf16* kp = kn + (size_t)j * krs;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          u32x4 x = *reinterpret_cast<const u32x4*>(kp + 8 * (4 * m + g));
          u32x4 y = *reinterpret_cast<const u32x4*>(kp + kGHalf + 8 * (4 * m + g));
          rot(j, 4 * m + g, x, y);
          B.k[sb][m] = x;
          B.k[sb][m + 2] = y;
        }
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) B.k[sb][m] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kk = kb + 4 * j + g;
      if (kk < nring) {
        int slot = lo_slot + kk;
        if (slot >= W) slot -= W;
        B.v[j] = ring_load(rv + (size_t)slot * kGD + 8 * c);
      } else if (kk < nk) {
        B.v[j] = *reinterpret_cast<const u32x4*>(vn + (size_t)(kk - nring) * krs + 8 * c);
      } else {
        B.v[j] = u32x4{0, 0, 0, 0};
      }
    }
  };

  const float c2 = a.scale_log2;
  const int64_t pq = P + (c < ncol ? c / G : 0);  // this lane's query position
  // transpose-read address: lane c of group g points at row 4g + c/4, dims 4*(c%4)
  const int v_off = (4 * g + (c >> 2)) * kVRow + 8 * (c & 3);
  f32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  auto compute = [&](const KvBlock& B, int kb, bool masked, bool ring_rows) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<u32x4*>(vb + (4 * j + g) * kVRow + 16 * c) = B.v[j];
    u32x4 ka[2][4];
    if (ring_rows) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          *reinterpret_cast<u32x4*>(kbuf + (16 * sb + 4 * m + g) * kKRow + 16 * c) = B.k[sb][m];
      __asm__ volatile("" ::: "memory");
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          ka[sb][m] = *reinterpret_cast<const u32x4*>(kbuf + (16 * sb + c) * kKRow + 64 * m + 16 * g);
    } else {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int m = 0; m < 4; ++m) ka[sb][m] = B.k[sb][m];
    }
    f32x4 sc[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[sb][m]),
                                                      qf[m], acc, 0, 0, 0);
      sc[sb] = acc;
    }
    if (masked) {
      // key kb+16sb+4g+r sits at position lo+kk (ring) or P+(kk-nring) (new)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kk = kb + 16 * sb + 4 * g + r;
          const int64_t pk = kk < nring ? lo + kk : P + (kk - nring);
          const bool ok = (kk < nk) && (pk <= pq) && (pk > pq - W);
          sc[sb][r] = ok ? sc[sb][r] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[sb][r]);
    mx = lanes32_max(lanes16_max(mx)) * c2;
    const bool need = mx > m_run + kLazyMax;
    if (__any(need)) {
      const float m_new = need ? mx : m_run;
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db)
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
    // The V rows written above are read back below by the same wave: LDS
    // instructions of one wave execute in order, so only the compiler must
    // keep the order.
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const char* p0 = vb + v_off + 32 * db;
      const bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)p0);
      const bf16x4 vc = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p0 + 16 * kVRow));
      const bf16x8 vf = __builtin_shufflevector(va, vc, 0, 1, 2, 3, 4, 5, 6, 7);
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, oacc[db], 0, 0, 0);
    }
    __asm__ volatile("" ::: "memory");
  };

  if (b0 < bf) {
    for (int bi = b0; bi < bf; bi += 2) {
      if (bi + 1 < bf) load_ring(32 * (bi + 1), B1);
      compute(B0, 32 * bi, 32 * bi < edge, true);
      if (bi + 1 < bf) {
        if (bi + 2 < bf) load_ring(32 * (bi + 2), B0);
        compute(B1, 32 * (bi + 1), 32 * (bi + 1) < edge, true);
      }
    }
  }
  for (int bi = bf; bi < b1; ++bi) {
    KvBlock B;
    load_any(32 * bi, B);
    compute(B, 32 * bi, true, false);
  }

  // ---- merge the waves' partial results through LDS
  __syncthreads();  // every wave is done with its V rows (and its ring reads)
  float* Mw = reinterpret_cast<float*>(work);  // [NW][16] running max (log2 domain)
  float* Lw = Mw + NW * 16;                    // [NW][16] row sums
  float* Ow = Lw + NW * 16;                    // [NW][16][128] unnormalised O
  const float l_tot = lanes32_sum(lanes16_sum(l_run));
  if (g == 0) {
    Mw[wave * 16 + c] = m_run;
    Lw[wave * 16 + c] = l_tot;
  }
#pragma unroll
  for (int db = 0; db < 8; ++db)
    *reinterpret_cast<f32x4*>(Ow + (wave * 16 + c) * kGD + 16 * db + 4 * g) = oacc[db];
  __syncthreads();
  for (int t = tid; t < ncol * 16; t += NW * 64) {
    const int cc = t >> 4, d0 = 8 * (t & 15);
    float mst = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mst = fmaxf(mst, Mw[w * 16 + cc]);
    float den = 0.f, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = Mw[w * 16 + cc];
      const float sc = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - mst);
      den = fmaf(sc, Lw[w * 16 + cc], den);
      float ov[8];
      load8(Ow + (w * 16 + cc) * kGD + d0, ov);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(sc, ov[e], acc[e]);
    }
    const float inv = 1.f / den;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    const int j = cc / G, hq = kvh * G + (cc - j * G);
    TO* op = (TO*)a.o + ((size_t)s * n + j) * qrs + (size_t)hq * kGD + d0;
    store8(op, acc);
  }

  // ---- append: rotated new keys and raw new values to slot (P+j) mod W
  for (int t = tid; t < n * 16; t += NW * 64) {
    const int j = t >> 4, u = t & 15;
    const int64_t pj = P + j;
    const size_t dst = rbase + (size_t)(((pj % W) + W) % W) * kGD;
    if (u < 8) {
      const bf16* kp = kn + (size_t)j * krs + 8 * u;
      u32x4 x = *reinterpret_cast<const u32x4*>(kp);
      u32x4 y = *reinterpret_cast<const u32x4*>(kp + kGHalf);
      rot(j, u, x, y);
      *reinterpret_cast<u32x4*>(a.ring_k + dst + 8 * u) = x;
      *reinterpret_cast<u32x4*>(a.ring_k + dst + kGHalf + 8 * u) = y;
    } else {
      const int cu = u - 8;
      const bf16* vp = vn + (size_t)j * krs + 8 * cu;
      *reinterpret_cast<u32x4*>(a.ring_v + dst + 8 * cu) = *reinterpret_cast<const u32x4*>(vp);
      *reinterpret_cast<u32x4*>(a.ring_v + dst + kGHalf + 8 * cu) =
          *reinterpret_cast<const u32x4*>(vp + kGHalf);
    }
  }
  if (kvh == 0 && tid == 0) a.pos_out[s] = P + n;
}

constexpr int kDecodeWaves = 4;  // 72 KB of LDS; VGPRs allow two waves per SIMD

}  // namespace

hipError_t launch_gqa_decode(const GqaDecodeArgs& a, DT out, const RopeFreqs128& fr,
                             hipStream_t st) {
  constexpr int NW = kDecodeWaves;
  const size_t merge = (size_t)NW * 32 * sizeof(float) + (size_t)NW * 16 * kGD * sizeof(float);
  const size_t work = (size_t)NW * kWaveBuf > merge ? (size_t)NW * kWaveBuf : merge;
  const size_t smem = (size_t)a.n * kGD * sizeof(float) + work;
  const dim3 grid((unsigned)((int64_t)a.S * a.Hkv)), blk(NW * 64);
  if (out == DT::BF16)
    hipLaunchKernelGGL((gqa_decode_kernel<NW, bf16>), grid, blk, smem, st, a, fr);
  else
    hipLaunchKernelGGL((gqa_decode_kernel<NW, float>), grid, blk, smem, st, a, fr);
  return hipGetLastError();
}

}  // namespace vx
