// Causal sliding-window prefill with RoPE on bf16 matrix cores (gfx950).
//
// Work unit: one workgroup = NW waves for one (batch, head) and a tile of
// BM = 32*NW consecutive queries; wave w owns queries qw .. qw+31.  The
// workgroup walks the 64-key tiles that intersect the band
// [q0-W+1, q0+BM-1] (banded tile skipping: tiles outside it are never
// loaded), and each wave skips the 32-key halves that lie outside its own
// band and masks only the halves that straddle a band edge.
//
// Per 32-key half and wave (v_mfma_f32_32x32x16_bf16, fp32 accumulate):
//   S^T = K' Q'^T  : A = K' rows from LDS (16 B per lane), B = Q' in registers.
//                    Lane l holds the scores of query l%32 for 16 keys, so
//                    the row max is an in-register max and one swap with
//                    lane l^32.
//   P^T = exp2(S^T * scale*log2e - m)  (lazy max: m moves only when a
//                    score exceeds it by more than 8, so p <= 256)
//   O^T += V^T P^T : B = P^T straight from the score registers (bf16);
//                    A = V^T read from the row-major V tile with two LDS
//                    transpose reads (ds_read_b64_tr_b16), each giving a lane
//                    four consecutive keys of one dimension, exactly the key
//                    order of the score register layout.
//   l += P . 1     : row sums from the packed bf16 P (v_dot2c_f32_bf16), so
//                    the normaliser matches the weights the MFMA multiplies.
// RoPE is fused into the loads: each lane rotates its own Q' row halves
// (pairs (i, i+32) are lane-local) and the staging threads rotate each K
// tile once per workgroup, reading cos/sin from the float32 table; rotated
// values are rounded to bf16 (the storage type of a rotated tensor).
// LDS rows are padded (K' 144 bytes, V 192 bytes) and the staging threads
// are mapped to rows so that the MFMA operand reads and the staging writes
// hit distinct banks.  K/V staging is double buffered: the next tile's buffer
// loads (per-tile descriptors in scalar registers) are issued before the
// current tile's MFMAs.  Masks are applied only to the
// 32-key halves that straddle a band edge, as one unsigned range test per
// score.  Accumulators stay in VGPRs (the build asks for the VGPR form of
// MFMA) so the softmax never moves them between register files.
#include "vx_launch.h"

namespace vx {

namespace {

constexpr int kBN = 64;                    // keys per staged tile
constexpr int kRowK = 144;                 // LDS bytes per K' row: 16-byte reads of 32
                                           // consecutive rows hit distinct banks
constexpr int kRowV = 192;                 // LDS bytes per V row: the 8-byte transpose
                                           // reads of 4 rows x 2 dim blocks hit distinct banks
constexpr int kTileK = 64 * kRowK;         // one K' tile
constexpr int kTileV = 64 * kRowV;         // one V tile
constexpr int kStageBytes = kTileK + kTileV;
constexpr float kLazy = 8.0f;              // log2-domain slack of the running max
constexpr float kNoMax = -3.0e38f;          // running max before the first score

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// max / sum of x over lanes l and l^32 (v_permlane32_swap)
__device__ __forceinline__ float partner_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float partner_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 lds_tr_pair(const char* p0, const char* p1) {
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p0);
  const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p1);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// K unit u -> (row, chunk pair): 16 consecutive lanes write rows {0,4,8,12}+.. so
// that their 16-byte stores at the 144-byte row stride fall in distinct banks.
__device__ __forceinline__ void k_unit(int u, int& r, int& cp) {
  cp = u & 3;
  r = 16 * (u >> 6) + 4 * ((u >> 2) & 3) + ((u >> 4) & 3);
}
// V unit u -> (row, 16-byte chunk): 16 consecutive lanes cover rows 0..3 x 4 chunks,
// conflict-free at the 192-byte row stride; 8 lanes still read each 128-byte row.
__device__ __forceinline__ void v_unit(int u, int& r, int& c) {
  r = 8 * (u >> 6) + 4 * ((u >> 5) & 1) + ((u >> 2) & 3);
  c = 4 * ((u >> 4) & 1) + (u & 3);
}

__device__ __forceinline__ bool work_item(int n_bh, int n_qtiles, int n_short, int hx, int cpx,
                                          int& bh, int& qt) {
  // Work order.  The dispatcher deals workgroups round-robin to the 8 XCDs
  // (workgroup id mod 8), and each XCD has its own L2.  With at least 8
  // (batch, head) pairs, XCD x owns pairs [x*hx, (x+1)*hx).  Its N = hx *
  // n_qtiles tiles, ranked by work (the n_short leading query tiles, whose
  // band is cut at key 0, shortest first, then the full-length ones pair by
  // pair so that neighbouring tiles share K/V in its L2), are dealt to its
  // cpx CUs as follows.
  //  - N <= 2 cpx: the first cpx workgroups land one per CU and the other
  //    R = N - cpx join CUs 0 .. R-1 in the same order; so the largest N - R
  //    tiles go first in ascending order and the R smallest follow in
  //    descending order: the largest of the late ones shares a CU with the
  //    smallest of the early ones, which evens out the work per CU.
  //  - larger grids: full-length tiles first, then the short ones longest
  //    first, which arrive last and pair up with a long workgroup on a CU
  //    that still has room.
  // With fewer pairs every XCD takes query tiles of every pair, longest first.
  if (hx > 0) {
    const int i = blockIdx.x >> 3;
    const int n_long = n_qtiles - n_short;
    const int N = hx * n_qtiles;
    int bl;
    if (N <= 2 * cpx) {
      const int R = max(N - cpx, 0);
      const int k = i < N - R ? R + i : R - 1 - (i - (N - R));
      if (k < hx * n_short) {
        qt = k / hx;
        bl = k % hx;
      } else {
        const int j = k - hx * n_short;
        bl = j / n_long;
        qt = n_short + j % n_long;
      }
    } else if (i < hx * n_long) {
      bl = i / n_long;
      qt = n_short + i % n_long;
    } else {
      const int j = i - hx * n_long;
      qt = n_short - 1 - j / hx;
      bl = j % hx;
    }
    bh = (blockIdx.x & 7) * hx + bl;
  } else {
    const int i = blockIdx.x;
    qt = n_qtiles - 1 - i / n_bh;
    bh = i % n_bh;
  }
  return bh < n_bh;
}

template <int NW>
struct Stage {
  static constexpr int NT = NW * 64;
  static constexpr int UK = 256 / NT;  // K units per thread: (row, chunk pair)
  static constexpr int UV = 512 / NT;  // V units per thread: (row, 16-byte chunk)
  u32x4 kx[UK], ky[UK];
  float kc[UK][8], ks[UK][8];
  u32x4 v[UV];
};

// Global loads of the next tile into registers, as buffer loads: each tile's
// rows get a descriptor (scalar registers) whose size ends at row T, so rows
// at or past T read as zeros (their keys lie after every stored query and
// causality masks them), and every thread keeps fixed byte offsets, so a
// tile costs no vector address arithmetic.  A tile past the end (kt0 >= T)
// gets an empty descriptor: its loads return zeros without touching memory.
// Callers issue the loads unconditionally, past the last tile too: the wait
// counters are counted per wave in issue order, and a load that is issued on
// one path only makes the compiler wait for every load at the join.
template <int NW>
struct StageOffs {
  uint32_t k[Stage<NW>::UK], t[Stage<NW>::UK], v[Stage<NW>::UV];
};

template <int NW>
__device__ __forceinline__ StageOffs<NW> stage_offsets(int tid, size_t rs) {
  constexpr int NT = Stage<NW>::NT;
  const uint32_t rb = (uint32_t)(rs * sizeof(bf16));
  StageOffs<NW> so;
#pragma unroll
  for (int j = 0; j < Stage<NW>::UK; ++j) {
    int r, cp;
    k_unit(tid + j * NT, r, cp);
    so.k[j] = r * rb + 16 * cp;
    so.t[j] = r * (kD * 4) + 32 * cp;
  }
#pragma unroll
  for (int j = 0; j < Stage<NW>::UV; ++j) {
    int r, c;
    v_unit(tid + j * NT, r, c);
    so.v[j] = r * rb + 16 * c;
  }
  return so;
}

// Descriptor of nbytes at p; both are the same in every lane, and reading
// them from lane 0 lets the compiler keep the descriptor in scalar registers
// (a descriptor it cannot prove uniform costs a loop around every load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* p, uint32_t nbytes) {
  const uint64_t u = (uint64_t)p;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(lo | (hi << 32)), (short)0,
                                           __builtin_amdgcn_readfirstlane((int)nbytes),
                                           0x00020000);
}

template <int NW>
__device__ __forceinline__ void stage_load(Stage<NW>& st, const bf16* __restrict__ k,
                                           const bf16* __restrict__ v, size_t rs, int T, int kt0,
                                           bool rope, const float* __restrict__ table,
                                           int64_t row0, const StageOffs<NW>& so) {
  const uint32_t nrows = (uint32_t)max(min(T - kt0, kBN), 0);
  const uint32_t rb = (uint32_t)(rs * sizeof(bf16));
  const auto kr = rows_rsrc(k + (size_t)kt0 * rs, nrows * rb);
  const auto vr = rows_rsrc(v + (size_t)kt0 * rs, nrows * rb);
#pragma unroll
  for (int j = 0; j < Stage<NW>::UK; ++j) {
    st.kx[j] = __builtin_amdgcn_raw_buffer_load_b128(kr, so.k[j], 0, 0);
    st.ky[j] = __builtin_amdgcn_raw_buffer_load_b128(kr, so.k[j] + 2 * kHalf, 0, 0);
    {
      // without RoPE the table loads still go out, against an empty
      // descriptor (zeros, no memory access), so the count of loads per tile
      // does not depend on a runtime flag
      const auto tr = rows_rsrc(table + (row0 + kt0) * kD, rope ? nrows * (kD * 4) : 0u);
      const f32x4 c0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(tr, so.t[j], 0, 0));
      const f32x4 c1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(tr, so.t[j] + 16, 0, 0));
      const f32x4 s0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(tr, so.t[j] + 4 * kHalf, 0, 0));
      const f32x4 s1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(tr, so.t[j] + 4 * kHalf + 16, 0, 0));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        st.kc[j][e] = c0[e];
        st.kc[j][4 + e] = c1[e];
        st.ks[j][e] = s0[e];
        st.ks[j][4 + e] = s1[e];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < Stage<NW>::UV; ++j)
    st.v[j] = __builtin_amdgcn_raw_buffer_load_b128(vr, so.v[j], 0, 0);
}

// Ring seeding by the staging threads: the rotated key rows and value rows of
// frames in [s_lo, s_hi) go to slot (frame mod W) of the stream's rings.
struct Seed {
  bf16* ring_k;  // this (stream, head)'s [W, 64] ring slice
  bf16* ring_v;
  int kt0;       // first frame of the tile being committed
  int s_lo, s_hi, W;
  __device__ __forceinline__ bool take(int r, int& slot) const {
    const int t = kt0 + r;
    slot = t % max(W, 1);
    return t >= s_lo && t < s_hi;
  }
};

template <int NW, bool SEED = false>
__device__ __forceinline__ void stage_commit(const Stage<NW>& st, char* Kb, char* Vb, bool rope,
                                             int tid, const Seed& sd = Seed{}) {
  constexpr int NT = Stage<NW>::NT;
#pragma unroll
  for (int j = 0; j < Stage<NW>::UK; ++j) {
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
    *reinterpret_cast<u32x4*>(Kb + r * kRowK + 64 + 16 * cp) = y;
    int slot;
    if (SEED && sd.take(r, slot)) {
      bf16* kr = sd.ring_k + (size_t)slot * kD + 8 * cp;
      *reinterpret_cast<u32x4*>(kr) = x;
      *reinterpret_cast<u32x4*>(kr + kHalf) = y;
    }
  }
#pragma unroll
  for (int j = 0; j < Stage<NW>::UV; ++j) {
    int r, c;
    v_unit(tid + j * NT, r, c);
    *reinterpret_cast<u32x4*>(Vb + r * kRowV + 16 * c) = st.v[j];
    int slot;
    if (SEED && sd.take(r, slot))
      *reinterpret_cast<u32x4*>(sd.ring_v + (size_t)slot * kD + 8 * c) = st.v[j];
  }
}

template <int NW, typename TO, bool SEED>
__global__ __launch_bounds__(NW * 64, 2) void prefill_mfma_kernel(PrefillArgs a, int n_qtiles,
                                                                  int n_short, int hx, int cpx) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kStageBytes];
  constexpr int BM = NW * 32;

  int bh, qt;
  if (!work_item(a.B * a.H, n_qtiles, n_short, hx, cpx, bh, qt)) return;
  const int h = bh % a.H, b = bh / a.H;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  // fixed batch: stream b at rows b*T ..; varlen: rows cu[b] .. cu[b+1]-1
  int T = a.T;
  size_t row0 = (size_t)b * a.T;
  if (a.cu) {
    const int c0 = min(max(a.cu[b], 0), a.total);
    const int c1 = min(max(a.cu[b + 1], c0), a.total);
    row0 = (size_t)c0;
    T = min(c1 - c0, a.T);
    if (SEED && h == 0 && qt == 0 && threadIdx.x == 0) a.pos_out[b] = T;
    if (qt * NW * 32 >= T) return;
  }
  // T and row0 are the same in every lane; saying so keeps the buffer
  // descriptors built from them in scalar registers
  T = __builtin_amdgcn_readfirstlane(T);
  row0 = ((size_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(row0 >> 32)) << 32) |
         (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)row0);
  const int W = a.W;
  const size_t rs = (size_t)a.H * kD;
  const size_t base = row0 * rs + (size_t)h * kD;
  const bf16* __restrict__ q = (const bf16*)a.q + base;
  const bf16* __restrict__ k = (const bf16*)a.k + base;
  const bf16* __restrict__ v = (const bf16*)a.v + base;
  TO* __restrict__ o = (TO*)a.o + base;
  const bool rope = a.rope;

  const int q0 = qt * BM;
  const int qw = q0 + wave * 32;
  const int tq = qw + l32;  // this lane's query

  const int kbeg = max(0, q0 - W + 1);
  const int klast = min(T, q0 + BM) - 1;
  const int it0 = kbeg / kBN, it1 = klast / kBN;

  // ---- Q' fragments (B operand of S^T = K' Q'^T) -------------------------
  // MFMA step m covers dims 16m .. 16m+15; lane half hh holds dims 16m+8hh+(0..7),
  // i.e. chunk 2m+hh of 8 dims.  Chunks c and c+4 are RoPE partners.
  // The workgroup's rows of the cos/sin table are staged through LDS first:
  // each load instruction then reads 1 KB of consecutive table bytes, where
  // per-lane reads of a lane's own row would touch one 256-byte row per lane.
  // Rows are padded to kRowQT bytes so the per-lane LDS reads below hit
  // distinct banks.  The region is reused by the first K/V tile afterwards.
  // The table rows, the raw query rows and the first K/V tile are all
  // requested before the first wait, so their memory latencies overlap.
  constexpr int kRowQT = 4 * kD + 16;
  constexpr int NT = NW * 64;
  constexpr int NQT = BM * 16 / NT;  // table chunks per thread
  static_assert(BM * kRowQT <= 2 * kStageBytes, "Q table rows must fit in LDS");
  u32x4 tq_rows[NQT];
  if (rope) {
#pragma unroll
    for (int j = 0; j < NQT; ++j) {
      const int i = tid + j * NT;
      const int r = i >> 4, c = i & 15;
      const int row = min(q0 + r, T - 1);
      tq_rows[j] = *reinterpret_cast<const u32x4*>(a.table + (a.table_row0 + row) * kD + 4 * c);
    }
  }
  u32x4 qx[2], qy[2];
  {
    const bf16* qp = q + (size_t)min(tq, T - 1) * rs;
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const int c = 2 * pr + hh;
      qx[pr] = *reinterpret_cast<const u32x4*>(qp + 8 * c);
      qy[pr] = *reinterpret_cast<const u32x4*>(qp + kHalf + 8 * c);
    }
  }
  Stage<NW> st;
  const StageOffs<NW> so = stage_offsets<NW>(tid, rs);
  stage_load<NW>(st, k, v, rs, T, it0 * kBN, rope, a.table, a.table_row0, so);
  if (rope) {
#pragma unroll
    for (int j = 0; j < NQT; ++j) {
      const int i = tid + j * NT;
      *reinterpret_cast<u32x4*>(lds + (i >> 4) * kRowQT + 16 * (i & 15)) = tq_rows[j];
    }
    __syncthreads();
  }
  bf16x8 qf[4];
#pragma unroll
  for (int pr = 0; pr < 2; ++pr) {
    const int c = 2 * pr + hh;
    u32x4 x = qx[pr], y = qy[pr];
    if (rope) {
      const float* cs = reinterpret_cast<const float*>(lds + (min(tq, T - 1) - q0) * kRowQT) + 8 * c;
      float cc[8], ss[8], xf[8], yf[8];
      load8(cs, cc);
      load8(cs + kHalf, ss);
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
    if (tq >= T) x = y = u32x4{0u, 0u, 0u, 0u};
    qf[pr] = __builtin_bit_cast(bf16x8, x);
    qf[pr + 2] = __builtin_bit_cast(bf16x8, y);
  }

  // per-lane LDS offsets: K' fragment row/col, and the transpose-read address
  // (lane L of each 16-lane group points at row L/4, dims 4*(L%4) of its block)
  const int k_off = l32 * kRowK + 16 * hh;
  const int g = lane >> 4, L = lane & 15;
  const int v_off = (4 * (g >> 1) + (L >> 2)) * kRowV + (16 * (g & 1) + 4 * (L & 3)) * 2;

  f32x16 oacc[2];
  oacc[0] = f32x16{};
  oacc[1] = f32x16{};
  // the running max starts at a finite floor, not -inf: the first finite
  // score always moves it, exp2(floor - m) is 0 (not NaN), and a half whose
  // scores are all masked gives exp2(-inf) = 0 against it, so no selects
  float m_run = kNoMax, l_run = 0.f;
  const float c2 = a.scale_log2;
  const unsigned wm1 = (unsigned)(W - 1);

  if (rope) __syncthreads();  // every wave has read its Q table rows
  // ring seeding: this workgroup writes its own query rows, as keys, for
  // frames in the stream's last W
  Seed sd0{};
  if (SEED) {
    const size_t ring = ((size_t)b * a.H + h) * (size_t)W * kD;
    sd0.ring_k = (bf16*)a.ring_k + ring;
    sd0.ring_v = (bf16*)a.ring_v + ring;
    sd0.s_lo = max(q0, T - W);
    sd0.s_hi = min(q0 + BM, T);
    sd0.W = W;
  }
  auto seed_for = [&](int kt0) {
    Seed sd = sd0;
    sd.kt0 = kt0;
    return sd;
  };
  stage_commit<NW, SEED>(st, lds, lds + kTileK, rope, tid, seed_for(it0 * kBN));
  __syncthreads();

  for (int it = it0; it <= it1; ++it) {
    const int buf = (it - it0) & 1;
    // the next tile's loads (past the last tile: an empty descriptor)
    stage_load<NW>(st, k, v, rs, T, (it + 1) * kBN, rope, a.table, a.table_row0, so);

    const char* Kb = lds + buf * kStageBytes;
    const char* Vb = Kb + kTileK;
    const int kt0 = it * kBN;

    // S^T for one 32-key half: 4 MFMAs over the 64 dims
    auto s_half = [&](int sb) {
      f32x16 acc = f32x16{};
      const char* kr = Kb + 32 * sb * kRowK + k_off;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kr + 32 * m);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[m], acc, 0, 0, 0);
      }
      return acc;
    };
    // exp2, bf16 pack, row sum and O^T += V^T P^T for one half
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
        for (int db = 0; db < 2; ++db) {
          const char* p0 = vr + 16 * ks * kRowV + 64 * db;
          const bf16x8 vf = lds_tr_pair(p0, p0 + 8 * kRowV);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], oacc[db], 0, 0, 0);
        }
      }
    };
    // lazy running max: move it only when a score exceeds it by more than kLazy
    auto update_max = [&](float mx) {
      const float mxs = partner_max(mx) * c2;  // log2 domain
      const bool need = mxs > m_run + kLazy;
      if (__any(need)) {
        const float m_new = need ? mxs : m_run;
        // a lane whose keys were all masked so far has nothing to rescale
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          oacc[0][r] *= alpha;
          oacc[1][r] *= alpha;
        }
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
      // Software pipeline over the two 32-key halves: the second half's score
      // MFMAs are issued before the first half's softmax, so the matrix core
      // runs while the VALU computes exponentials.
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

    if (it < it1)
      stage_commit<NW, SEED>(st, lds + (buf ^ 1) * kStageBytes,
                             lds + (buf ^ 1) * kStageBytes + kTileK, rope, tid,
                             seed_for((it + 1) * kBN));
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, lane holds query tq, dims 32db + 8g + 4hh + (0..3)
  const float l_tot = partner_sum(l_run);
  if (tq < T) {
    const float inv = 1.f / l_tot;
    TO* op = o + (size_t)tq * rs;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
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

// Compute units per XCD of the current device (the chip deals workgroups to
// its 8 XCDs round-robin), cached per device.
int cus_per_xcd() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 32;
  int c = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
  if (c == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 8)
      n = 256;
    c = n / 8;
    __atomic_store_n(&cache[dev], c, __ATOMIC_RELAXED);
  }
  return c;
}

template <int NW>
hipError_t launch_nw(const PrefillArgs& a, DT out, hipStream_t st) {
  constexpr int BM = NW * 32;
  const int n_qtiles = (a.T + BM - 1) / BM;
  const int n_short = min(n_qtiles, (a.W - 1 + BM - 1) / BM);  // tiles with q0 < W-1
  const int n_bh = a.B * a.H;
  const int hx = n_bh >= 8 ? (n_bh + 7) / 8 : 0;
  const int cpx = cus_per_xcd();
  const int64_t grid = hx > 0 ? (int64_t)8 * hx * n_qtiles : (int64_t)n_bh * n_qtiles;
  const dim3 g((unsigned)grid), blk(NW * 64);
  if (a.ring_k) {
    if (out == DT::BF16)
      hipLaunchKernelGGL((prefill_mfma_kernel<NW, bf16, true>), g, blk, 0, st, a, n_qtiles, n_short, hx, cpx);
    else
      hipLaunchKernelGGL((prefill_mfma_kernel<NW, float, true>), g, blk, 0, st, a, n_qtiles, n_short, hx, cpx);
  } else {
    if (out == DT::BF16)
      hipLaunchKernelGGL((prefill_mfma_kernel<NW, bf16, false>), g, blk, 0, st, a, n_qtiles, n_short, hx, cpx);
    else
      hipLaunchKernelGGL((prefill_mfma_kernel<NW, float, false>), g, blk, 0, st, a, n_qtiles, n_short, hx, cpx);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillArgs& a, DT out, hipStream_t st) {
  // Four-wave workgroups share each staged (and rotated) K tile among more
  // queries; two-wave ones keep enough workgroups to cover the 256 CUs when
  // the problem is small.
  const int64_t wg4 = (int64_t)((a.T + 127) / 128) * a.H * a.B;
  if (wg4 >= 256) return launch_nw<4>(a, out, st);
  return launch_nw<2>(a, out, st);
}

}  // namespace vx
