// Grouped-query causal sliding-window prefill with RoPE on bf16 matrix cores
// (gfx950), head_dim 128: the prompt pass of the Voxtral Realtime 2602 text
// decoder (transcribe.cpp "Voxtral" family notes, Architecture: 32 query
// heads over 8 key/value heads, head_dim 128, sliding window 8192, RoPE
// theta 1e6).
//
// Work unit: one workgroup = NW waves for one (batch, key/value head) and a
// tile of BM = 32*NW/G consecutive queries.  Wave w computes query head
// kvh*G + w%G for the 32 queries of block w/G, so the G heads that share a
// key/value head share every staged (and rotated) K/V tile: the tile is read
// from HBM and rotated once per workgroup, not once per query head.  The
// workgroup walks the 64-key tiles that meet the band [q0-W+1, q0+BM-1] and
// each wave skips the 32-key halves outside its own band.
//
// Per 32-key half and wave (v_mfma_f32_32x32x16_bf16, fp32 accumulate):
//   S^T = K' Q'^T  eight MFMAs over the 128 dims: A = K' rows from LDS,
//                  B = Q' in registers (lane l: query l%32; RoPE partner
//                  dims d and d+64 sit in the same lane).
//   P^T = exp2(S^T * scale*log2e - m) with a lazy running max (it moves only
//                  when a score exceeds it by more than 8, so p <= 256).
//   O^T += V^T P^T : B = P^T straight from the score registers; A = V^T from
//                  two LDS transpose reads (ds_read_b64_tr_b16), which give a
//                  lane four consecutive keys of one dim, the key order of
//                  the score registers; four 32-dim blocks.
//   l += P . 1     : row sums of the packed bf16 weights (v_dot2c_f32_bf16).
// LDS rows are padded (K' 272 bytes, V 320 bytes) so the MFMA operand reads
// and the staging writes hit distinct banks; K/V staging is double
// buffered, the next tile's global loads issued before this tile's MFMAs.
#include "gqa_launch.h"

namespace vx {

namespace {

constexpr int kBN = 64;                  // keys per staged tile
constexpr int kRowK = 272;               // LDS bytes per K' row (256 + 16)
constexpr int kRowV = 320;               // LDS bytes per V row (256 + 64)
constexpr int kTileK = kBN * kRowK;
constexpr int kTileV = kBN * kRowV;
constexpr int kStage = kTileK + kTileV;  // 37,888 bytes
constexpr int kRowQT = 4 * kGD + 16;     // LDS bytes per staged cos/sin table row
constexpr float kLazy = 8.0f;
constexpr float kNoMax = -3.0e38f;          // running max before the first score

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_g;

__device__ __forceinline__ float half_swap_max(float x) {  // lanes l, l^32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 tr_pair(const char* p0, const char* p1) {
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_g*)p0);
  const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_g*)p1);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// K unit u in [0, 512) -> (row, chunk pair cp): chunk cp holds dims 8cp.., its
// partner dims 64+8cp..  Four consecutive lanes read 64 contiguous bytes of a
// row; sixteen consecutive lanes write rows {0,4,8,12}+r0 with four chunk
// pairs each, which at the 272-byte stride fall in distinct banks.
__device__ __forceinline__ void k_unit(int u, int& r, int& cp) {
  cp = (u & 3) + 4 * ((u >> 4) & 1);
  r = 4 * ((u >> 2) & 3) + ((u >> 5) & 3) + 16 * (u >> 7);
}
// V unit u in [0, 1024) -> (row, 16-byte chunk): sixteen consecutive lanes
// cover 4 rows x 4 chunks, distinct banks at the 320-byte stride.
__device__ __forceinline__ void v_unit(int u, int& r, int& c) {
  c = (u & 3) + 4 * ((u >> 4) & 3);
  r = ((u >> 2) & 3) + 4 * (u >> 6);
}

template <int NT>
struct GStage {
  static constexpr int UK = 512 / NT;
  static constexpr int UV = 1024 / NT;
  u32x4 kx[UK], ky[UK];
  float kc[UK][8], ks[UK][8];
  u32x4 v[UV];
};

// Global loads of a tile into registers; rows at or past T are clamped to
// T-1 (causality masks them and the values stay finite), so every load is
// unconditional.
template <int NT>
__device__ __forceinline__ void gstage_load(GStage<NT>& st, const bf16* __restrict__ k,
                                            const bf16* __restrict__ v, size_t rs, int T, int kt0,
                                            bool rope, const float* __restrict__ table,
                                            int64_t row0, int tid) {
#pragma unroll
  for (int j = 0; j < GStage<NT>::UK; ++j) {
    int r, cp;
    k_unit(tid + j * NT, r, cp);
    const int key = min(kt0 + r, T - 1);
    const bf16* kp = k + (size_t)key * rs + 8 * cp;
    st.kx[j] = *reinterpret_cast<const u32x4*>(kp);
    st.ky[j] = *reinterpret_cast<const u32x4*>(kp + kGHalf);
    if (rope) {
      const float* cs = table + (row0 + key) * kGD + 8 * cp;
      load8(cs, st.kc[j]);
      load8(cs + kGHalf, st.ks[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < GStage<NT>::UV; ++j) {
    int r, c;
    v_unit(tid + j * NT, r, c);
    const int key = min(kt0 + r, T - 1);
    st.v[j] = *reinterpret_cast<const u32x4*>(v + (size_t)key * rs + 8 * c);
  }
}

// Ring seeding by the staging threads: frames in [s_lo, s_hi) of the tile
// starting at kt0 go to slot (frame mod W) of this (batch, key/value head)'s
// [W, 128] rings.
struct GSeed {
  bf16* ring_k;
  bf16* ring_v;
  int kt0, s_lo, s_hi, W;
  __device__ __forceinline__ bool take(int r, int& slot) const {
    const int t = kt0 + r;
    slot = t % max(W, 1);
    return t >= s_lo && t < s_hi;
  }
};

template <int NT, bool SEED>
__device__ __forceinline__ void gstage_commit(const GStage<NT>& st, char* Kb, char* Vb, bool rope,
                                              int tid, const GSeed& sd) {
#pragma unroll
  for (int j = 0; j < GStage<NT>::UK; ++j) {
    int r, cp;
    k_unit(tid + j * NT, r, cp);
    u32x4 x = st.kx[j], y = st.ky[j];
    if (rope) {
      float xf[8], yf[8];
      unpack8(st.kx[j], xf);
      unpack8(st.ky[j], yf);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float xo, yo;
        rope_pair(xf[e], yf[e], st.kc[j][e], st.ks[j][e], &xo, &yo);
        xf[e] = xo;
        yf[e] = yo;
      }
      x = pack8(xf);
      y = pack8(yf);
    }
    *reinterpret_cast<u32x4*>(Kb + r * kRowK + 16 * cp) = x;
    *reinterpret_cast<u32x4*>(Kb + r * kRowK + 128 + 16 * cp) = y;
    int slot;
    if (SEED && sd.take(r, slot)) {
      bf16* kr = sd.ring_k + (size_t)slot * kGD + 8 * cp;
      *reinterpret_cast<u32x4*>(kr) = x;
      *reinterpret_cast<u32x4*>(kr + kGHalf) = y;
    }
  }
#pragma unroll
  for (int j = 0; j < GStage<NT>::UV; ++j) {
    int r, c;
    v_unit(tid + j * NT, r, c);
    *reinterpret_cast<u32x4*>(Vb + r * kRowV + 16 * c) = st.v[j];
    int slot;
    if (SEED && sd.take(r, slot))
      *reinterpret_cast<u32x4*>(sd.ring_v + (size_t)slot * kGD + 8 * c) = st.v[j];
  }
}

template <int NW, int G, typename TO, bool SEED>
__global__ __launch_bounds__(NW * 64, 8 / NW) void gqa_prefill_kernel(GqaPrefillArgs a,
                                                                      int n_qtiles, int n_short,
                                                                      int hx) {
  static_assert(NW % G == 0, "the waves of a workgroup cover whole groups");
  __shared__ __attribute__((aligned(16))) char lds[2 * kStage];
  constexpr int NT = NW * 64;
  constexpr int BM = 32 * (NW / G);

  // Work order (as in the multi-head prefill): workgroups are dealt to the 8
  // XCDs round-robin; with at least 8 (batch, key/value head) pairs XCD x
  // owns pairs [x*hx, (x+1)*hx) and runs their full-band query tiles first,
  // pair by pair so that neighbouring tiles share K/V in its L2, then the
  // n_short leading tiles whose band is cut at key 0, longest first.
  const int n_pairs = a.B * a.Hkv;
  int pr, qt;
  if (hx > 0) {
    const int i = blockIdx.x >> 3;
    const int n_long = n_qtiles - n_short;
    int pl;
    if (i < hx * n_long) {
      pl = i / n_long;
      qt = n_short + i % n_long;
    } else {
      const int j = i - hx * n_long;
      qt = n_short - 1 - j / hx;
      pl = j % hx;
    }
    pr = (blockIdx.x & 7) * hx + pl;
    if (pr >= n_pairs) return;
  } else {
    const int i = blockIdx.x;
    qt = n_qtiles - 1 - i / n_pairs;
    pr = i % n_pairs;
  }
  const int kvh = pr % a.Hkv, b = pr / a.Hkv;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int gq = wave % G, qb = wave / G;
  const int h = kvh * G + gq;
  const int T = a.T, W = a.W;
  const size_t qrs = (size_t)a.Hq * kGD, krs = (size_t)a.Hkv * kGD;
  const bf16* __restrict__ q = a.q + (size_t)b * T * qrs + (size_t)h * kGD;
  const bf16* __restrict__ k = a.k + (size_t)b * T * krs + (size_t)kvh * kGD;
  const bf16* __restrict__ v = a.v + (size_t)b * T * krs + (size_t)kvh * kGD;
  TO* __restrict__ o = (TO*)a.o + (size_t)b * T * qrs + (size_t)h * kGD;
  const bool rope = a.rope;
  const bool rope_k = a.rope && a.rope_k;

  const int q0 = qt * BM;
  const int qw = q0 + qb * 32;
  const int tq = qw + l32;  // this lane's query

  // ---- Q' fragments (B operand of S^T = K' Q'^T) -------------------------
  // MFMA step m covers dims 16m .. 16m+15; lane half hh holds chunk 2m+hh of
  // 8 dims.  Chunks c and c+8 are RoPE partners (steps m and m+4).  The
  // workgroup's rows of the cos/sin table go through LDS first (coalesced
  // 16-byte pieces); the region is reused by the first K/V tile afterwards.
  static_assert(BM * kRowQT <= 2 * kStage, "Q table rows must fit in LDS");
  if (rope) {
#pragma unroll
    for (int j = 0; j < BM * 32 / NT; ++j) {
      const int i = tid + j * NT;
      const int r = i >> 5, c = i & 31;
      const int row = min(q0 + r, T - 1);
      const u32x4 val =
          *reinterpret_cast<const u32x4*>(a.table + (a.table_row0 + row) * kGD + 4 * c);
      *reinterpret_cast<u32x4*>(lds + r * kRowQT + 16 * c) = val;
    }
    __syncthreads();
  }
  bf16x8 qf[8];
  if (tq < T) {
    const bf16* qp = q + (size_t)tq * qrs;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int c = 2 * m + hh;
      u32x4 x = *reinterpret_cast<const u32x4*>(qp + 8 * c);
      u32x4 y = *reinterpret_cast<const u32x4*>(qp + kGHalf + 8 * c);
      if (rope) {
        const float* cs = reinterpret_cast<const float*>(lds + (tq - q0) * kRowQT) + 8 * c;
        float cc[8], ss[8], xf[8], yf[8];
        load8(cs, cc);
        load8(cs + kGHalf, ss);
        unpack8(x, xf);
        unpack8(y, yf);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float xo, yo;
          rope_pair(xf[e], yf[e], cc[e], ss[e], &xo, &yo);
          xf[e] = xo;
          yf[e] = yo;
        }
        x = pack8(xf);
        y = pack8(yf);
      }
      qf[m] = __builtin_bit_cast(bf16x8, x);
      qf[m + 4] = __builtin_bit_cast(bf16x8, y);
    }
  } else {
#pragma unroll
    for (int m = 0; m < 8; ++m) qf[m] = bf16x8{};
  }

  // per-lane LDS offsets: K' fragment row/col, and the transpose-read address
  // (lane L of each 16-lane group points at row L/4, dims 4*(L%4) of its block)
  const int k_off = l32 * kRowK + 16 * hh;
  const int g = lane >> 4, L = lane & 15;
  const int v_off = (4 * (g >> 1) + (L >> 2)) * kRowV + (16 * (g & 1) + 4 * (L & 3)) * 2;

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  // the running max starts at a finite floor, not -inf: the first finite
  // score always moves it, exp2(floor - m) is 0 (not NaN), and a half whose
  // scores are all masked gives exp2(-inf) = 0 against it, so no selects
  float m_run = kNoMax, l_run = 0.f;
  const float c2 = a.scale_log2;
  const unsigned wm1 = (unsigned)(W - 1);

  const int kbeg = max(0, q0 - W + 1);
  const int klast = min(T, q0 + BM) - 1;
  const int it0 = kbeg / kBN, it1 = klast / kBN;

  GStage<NT> st;
  gstage_load<NT>(st, k, v, krs, T, it0 * kBN, rope_k, a.table, a.table_row0, tid);
  if (rope) __syncthreads();  // every wave has read its Q table rows
  GSeed sd0{};
  if (SEED) {
    const size_t ring = ((size_t)b * a.Hkv + kvh) * (size_t)W * kGD;
    sd0.ring_k = a.ring_k + ring;
    sd0.ring_v = a.ring_v + ring;
    sd0.s_lo = max(q0, T - W);
    sd0.s_hi = min(q0 + BM, T);
    sd0.W = W;
    if (kvh == 0 && qt == 0 && tid == 0) a.pos_out[b] = T;
  }
  auto seed_for = [&](int kt0) {
    GSeed sd = sd0;
    sd.kt0 = kt0;
    return sd;
  };
  gstage_commit<NT, SEED>(st, lds, lds + kTileK, rope_k, tid, seed_for(it0 * kBN));
  __syncthreads();

  for (int it = it0; it <= it1; ++it) {
    const int buf = (it - it0) & 1;
    const bool more = it < it1;
    if (more)
      gstage_load<NT>(st, k, v, krs, T, (it + 1) * kBN, rope_k, a.table, a.table_row0, tid);

    const char* Kb = lds + buf * kStage;
    const char* Vb = Kb + kTileK;
    const int kt0 = it * kBN;

    auto s_half = [&](int sb) {
      f32x16 acc = f32x16{};
      const char* kr = Kb + 32 * sb * kRowK + k_off;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kr + 32 * m);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[m], acc, 0, 0, 0);
      }
      return acc;
    };
    auto pv_half = [&](const f32x16& sc, int sb, float mu) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], c2, -mu));
      const u32x4 w0 = pack8(p), w1 = pack8(p + 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        l_run = dot2_ones(w0[i], l_run);
        l_run = dot2_ones(w1[i], l_run);
      }
      const bf16x8 pf[2] = {__builtin_bit_cast(bf16x8, w0), __builtin_bit_cast(bf16x8, w1)};
      const char* vr = Vb + 32 * sb * kRowV + v_off;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const char* p0 = vr + 16 * ks * kRowV + 64 * db;
          const bf16x8 vf = tr_pair(p0, p0 + 8 * kRowV);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], oacc[db], 0, 0, 0);
        }
      }
    };
    auto update_max = [&](float mx) {
      const float mxs = half_swap_max(mx) * c2;  // log2 domain
      const bool need = mxs > m_run + kLazy;
      if (__any(need)) {
        const float m_new = need ? mxs : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        m_run = m_new;
      }
    };

    bool act[2], msk[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int kb = kt0 + 32 * sb;
      act[sb] = (qw < T) && (kb < T) && (kb + 31 >= qw - W + 1) && (kb <= qw + 31);
      msk[sb] = (kb + 31 > qw) || (kb < qw + 31 - W + 1);
    }
    if (act[0] || act[1]) {
      // the second half's score MFMAs are issued before the first half's
      // softmax, so the matrix core runs while the VALU computes exponentials
      f32x16 s_cur = act[0] ? s_half(0) : s_half(1);
      f32x16 s_nxt = f32x16{};
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        if (!act[sb]) continue;
        if (msk[sb]) {
          // key of register r: kb + 4hh + 8(r/4) + r%4; keep iff 0 <= tq - key <= W-1
          const int d0 = tq - (kt0 + 32 * sb + 4 * hh);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 8 * (r >> 2) + (r & 3);
            s_cur[r] = ((unsigned)(d0 - off) <= wm1) ? s_cur[r] : -INFINITY;
          }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_cur[r]);
        if (sb == 0 && act[1]) s_nxt = s_half(1);
        update_max(mx);
        const float mu = m_run;
        pv_half(s_cur, sb, mu);
        s_cur = s_nxt;
      }
    }

    if (more)
      gstage_commit<NT, SEED>(st, lds + (buf ^ 1) * kStage, lds + (buf ^ 1) * kStage + kTileK,
                              rope_k, tid, seed_for((it + 1) * kBN));
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l; lane holds query tq, dims 32db + 8gg + 4hh + (0..3)
  const float l_tot = half_swap_sum(l_run);
  if (tq < T) {
    const float inv = 1.f / l_tot;
    TO* op = o + (size_t)tq * qrs;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int d0 = 32 * db + 8 * gg + 4 * hh;
        if constexpr (sizeof(TO) == 2) {
          uint2 w;
          w.x = pack_bf16x2(oacc[db][4 * gg] * inv, oacc[db][4 * gg + 1] * inv);
          w.y = pack_bf16x2(oacc[db][4 * gg + 2] * inv, oacc[db][4 * gg + 3] * inv);
          *reinterpret_cast<uint2*>(op + d0) = w;
        } else {
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = oacc[db][4 * gg + e] * inv;
          *reinterpret_cast<f32x4*>(op + d0) = w;
        }
      }
    }
  }
}

template <int NW, int G>
hipError_t launch_g(const GqaPrefillArgs& a, DT out, hipStream_t st) {
  constexpr int BM = 32 * (NW / G);
  const int n_qtiles = (a.T + BM - 1) / BM;
  const int n_short = min(n_qtiles, (a.W - 1 + BM - 1) / BM);  // tiles with q0 < W-1
  const int n_pairs = a.B * a.Hkv;
  const int hx = n_pairs >= 8 ? (n_pairs + 7) / 8 : 0;
  const int64_t grid = hx > 0 ? (int64_t)8 * hx * n_qtiles : (int64_t)n_pairs * n_qtiles;
  const dim3 gr((unsigned)grid), blk(NW * 64);
  if (a.ring_k) {
    if (out == DT::BF16)
      hipLaunchKernelGGL((gqa_prefill_kernel<NW, G, bf16, true>), gr, blk, 0, st, a, n_qtiles, n_short, hx);
    else
      hipLaunchKernelGGL((gqa_prefill_kernel<NW, G, float, true>), gr, blk, 0, st, a, n_qtiles, n_short, hx);
  } else {
    if (out == DT::BF16)
      hipLaunchKernelGGL((gqa_prefill_kernel<NW, G, bf16, false>), gr, blk, 0, st, a, n_qtiles, n_short, hx);
    else
      hipLaunchKernelGGL((gqa_prefill_kernel<NW, G, float, false>), gr, blk, 0, st, a, n_qtiles, n_short, hx);
  }
  return hipGetLastError();
}

// One thread per (frame, head, chunk pair): dims 8cp.. and their partners
// 64+8cp.. rotated with the table row of the frame's position.
__global__ __launch_bounds__(256) void gqa_rope_rows_kernel(const bf16* __restrict__ k,
                                                            bf16* __restrict__ k_rot, int T,
                                                            int Hkv, int64_t units,
                                                            const float* __restrict__ table,
                                                            int64_t row0) {
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= units) return;
  const int cp = (int)(u & 7);
  const int64_t row = u >> 3;                   // (b*T + t)*Hkv + h
  const int t = (int)((row / Hkv) % T);
  const size_t off = (size_t)row * kGD + 8 * cp;
  float x[8], y[8], c[8], sn[8];
  load8(k + off, x);
  load8(k + off + kGHalf, y);
  const float* cs = table + (row0 + t) * kGD + 8 * cp;
  load8(cs, c);
  load8(cs + kGHalf, sn);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float xo, yo;
    rope_pair(x[e], y[e], c[e], sn[e], &xo, &yo);
    x[e] = xo;
    y[e] = yo;
  }
  store8(k_rot + off, x);
  store8(k_rot + off + kGHalf, y);
}

__global__ void gqa_rope_table_kernel(float* __restrict__ table, int64_t p_begin, int count,
                                      RopeFreqs128 fr) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)count * kGHalf) return;
  const int64_t j = idx / kGHalf;
  const int i = (int)(idx % kGHalf);
  float c, s;
  rope_cs(p_begin + j, fr.f[i], &c, &s);
  table[j * kGD + i] = c;
  table[j * kGD + kGHalf + i] = s;
}

}  // namespace

hipError_t launch_gqa_prefill(const GqaPrefillArgs& a, DT out, hipStream_t st) {
  // Groups of 4 (the 32/8 decoder): 8 waves = 4 heads x 64 queries share each
  // staged tile (measured 14% faster than 4 waves x 32 queries at T 16384).
  switch (a.Hq / a.Hkv) {
    case 1: return launch_g<4, 1>(a, out, st);
    case 2: return launch_g<4, 2>(a, out, st);
    case 4: return launch_g<8, 4>(a, out, st);
    case 8: return launch_g<8, 8>(a, out, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gqa_rope_rows(const bf16* k, bf16* k_rot, int B, int T, int Hkv,
                                const float* table, int64_t table_row0, hipStream_t st) {
  const int64_t units = (int64_t)B * T * Hkv * 8;
  const int64_t blocks = (units + 255) / 256;
  hipLaunchKernelGGL(gqa_rope_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, st, k, k_rot, T,
                     Hkv, units, table, table_row0);
  return hipGetLastError();
}

hipError_t launch_gqa_rope_table(float* table, int64_t p_begin, int count,
                                 const RopeFreqs128& fr, hipStream_t st) {
  const int64_t total = (int64_t)count * kGHalf;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(gqa_rope_table_kernel, dim3((unsigned)blocks), dim3(threads), 0, st, table,
                     p_begin, count, fr);
  return hipGetLastError();
}

}  // namespace vx
