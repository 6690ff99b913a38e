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
// tile once per workgroup, reading cos/sin from the float32 table or, with
// no table, computing them from the same float64 angle (the same values);
// rotated values are rounded to bf16 (the storage type of a rotated tensor).
// Frame t of batch entry b sits at position pos0[b] + t; an entry whose
// positions are negative or outside the table, or a varlen stream longer
// than the call allows, gets NaN outputs (loud, never a silent partial).
// LDS rows are padded (K' 144 bytes, V 192 bytes; V in swizzled 128-byte
// rows on rotated keys, see VLayout) and the staging threads are mapped to
// rows so that the MFMA operand reads and the staging writes hit distinct
// banks.  K/V staging is double buffered: the next tile's buffer
// loads (per-tile descriptors in scalar registers) are issued before the
// current tile's MFMAs.  Masks are applied only to the
// 32-key halves that straddle a band edge, as one unsigned range test per
// score.  Accumulators stay in VGPRs (the build asks for the VGPR form of
// MFMA) so the softmax never moves them between register files.
//
// Halves split (HS), the schedule of grids too small to fill the device (at
// most 1.5 four-wave query tiles per CU, e.g. one 1500-frame chunk of 32
// heads): 64-query workgroups of four waves, two per 32-query block, each
// wave taking one 32-key half of every staged tile, so a wave's tile step is
// half as long and the device holds twice the workgroups; the two waves of a
// block merge their partial results through LDS at the end.  Each key tile
// is staged for 64 queries instead of 128, which costs more vector work in
// all, so larger grids keep 128-query workgroups.  The halves split walks
// each band from its newest key tile down to its oldest.
//
// Split walk (on request, with a workspace), for the same small grids: each
// query tile gets two workgroups, the first walking the
// older half of its key tiles and the second the newer half, so each wave's
// chain of dependent tile steps is half as long and the device holds twice
// the waves.  Softmax partials combine exactly: with running maxima m0, m1
// and m = max(m0, m1), the merged sum is l0 2^(m0-m) + l1 2^(m1-m) and
// likewise for O^T.  Per wave, whichever half finishes second does the
// merge: a half that finds its partner's token already in the wave's flag
// word merges at once; otherwise it stores its partial result
// (device-coherent stores, waited for) and swaps its own token into the
// flag, and merges only if the swap returns the partner's token.  The
// merger resets the flag to zero, so every call leaves the flags as it found
// them (also across graph replays), and computes the merge with the halves
// in a fixed order, so the bits do not depend on which finished first.
// Nothing ever waits on another workgroup.
//
// Rotated keys (KROT = false): when the keys were rotated ahead of the
// kernel (large grids, where the staging's rotation of every key tile in
// each of the ~7 workgroups that visit it costs more than one extra pass
// over K) or come pre-rotated, the staging loads neither cos/sin nor
// rotates; queries are still rotated per `rope`.
#include "vx_launch.h"

namespace vx {

namespace {

constexpr int kBN = 64;                    // keys per staged tile
constexpr int kRowK = 144;                 // LDS bytes per K' row: 16-byte reads of 32
                                           // consecutive rows hit distinct banks
constexpr int kTileK = 64 * kRowK;         // one K' tile
// V rows in LDS.  Padded (CV false): 192-byte rows, where the 8-byte transpose
// reads of 4 rows x 2 dim blocks hit distinct banks.  Compact (CV true):
// 128-byte rows with row r's 16-byte chunk c at chunk c ^ 4*((r>>1)&1), which
// keeps the transpose reads and the staging writes on distinct banks (see
// v_unit and the kernel's v_off) in two thirds of the bytes: the kernel on
// rotated keys, at 128 VGPRs, then fits four workgroups per CU (34 KB of LDS
// each instead of 42 KB).
template <bool CV>
struct VLayout {
  static constexpr int kRowV = CV ? 128 : 192;  // LDS bytes per V row
  static constexpr int kTileV = 64 * kRowV;     // one V tile
  static constexpr int kStageBytes = kTileK + kTileV;
  // byte offset of row r's 16-byte chunk c
  static __device__ __forceinline__ int chunk(int r, int c) {
    return r * kRowV + (CV ? ((16 * c) ^ (64 * ((r >> 1) & 1))) : 16 * c);
  }
};
constexpr float kLazy = 8.0f;              // log2-domain slack of the running max
constexpr float kNoMax = -3.0e38f;          // running max before the first score
// split-walk flag tokens: kSplitTok + half (any other flag value counts as
// "partner not done")
constexpr unsigned long long kSplitTok = 0x6a09e667f3bcc908ull;
constexpr int kCoherent = 16;  // buffer cache policy sc1: device-coherent access

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
// V unit u -> (row, 16-byte chunk), 8 lanes reading each 128-byte row.  Padded
// rows: 16 consecutive lanes cover rows 0..3 x 4 chunks, whose stores hit distinct
// banks at the 192-byte stride.  Compact rows: 8 consecutive lanes store one whole
// row, which the chunk swizzle only permutes, so every group of lanes writes whole
// 128-byte rows (with rows 0..3 x 4 chunks the compact layout counted about a
// million bank-conflict cycles per launch at B4 T1500, about 7 per store).
template <bool CV>
__device__ __forceinline__ void v_unit(int u, int& r, int& c) {
  if constexpr (CV) {
    r = u >> 3;
    c = u & 7;
  } else {
    r = 8 * (u >> 6) + 4 * ((u >> 5) & 1) + ((u >> 2) & 3);
    c = 4 * ((u >> 4) & 1) + (u & 3);
  }
}

// Frequency of pair 8c+e, c in 0..3 chosen per lane: selects between
// constant offsets of the kernel argument, so the array is never indexed
// dynamically (that would copy it to scratch memory).
__device__ __forceinline__ double freq8(const RopeFreqs& fr, int c, int e) {
  double f = fr.f[e];
  f = c == 1 ? fr.f[8 + e] : f;
  f = c == 2 ? fr.f[16 + e] : f;
  f = c == 3 ? fr.f[24 + e] : f;
  return f;
}

// Writes NaN over rows [r0, r1) of one head: the loud result for a batch
// entry whose positions are invalid or a stream longer than the call allows.
template <typename TO>
__device__ void poison_rows(TO* o, size_t rs, int r0, int r1) {
  const int n = (r1 - r0) * 16;  // 4-element units
  for (int u = threadIdx.x; u < n; u += blockDim.x) {
    TO* p = o + (size_t)(r0 + u / 16) * rs + 4 * (u % 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = (TO)__builtin_nanf("");
  }
}

template <bool SPLIT>
__device__ __forceinline__ bool work_item(int n_bh, int n_qtiles, int n_short, int hx, int cpx,
                                          int& bh, int& qt, int& half) {
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
  //  - N <= 3 cpx (all resident too, e.g. one 1500-frame chunk of 32 heads
  //    in 64-query workgroups): a snake over the tiles ranked longest first,
  //    CU c taking ranks c, 2 cpx - 1 - c and 2 cpx + c.
  //  - larger grids: full-length tiles first, then the short ones longest
  //    first, which arrive last and pair up with a long workgroup on a CU
  //    that still has room.
  // With fewer pairs every XCD takes query tiles of every pair, longest first.
  // Split walk: the two halves of a query tile are consecutive in their
  // XCD's sequence (ids 16j + x and 16j + 8 + x), and the tiles go in the
  // larger-grid order (every workgroup of such a grid is resident at once).
  int id = blockIdx.x;
  half = 0;
  if (SPLIT) {
    if (hx > 0) {
      half = (id >> 3) & 1;
      id = ((id >> 4) << 3) | (id & 7);
    } else {
      half = id & 1;
      id >>= 1;
    }
  }
  if (hx > 0) {
    const int i = id >> 3;
    const int n_long = n_qtiles - n_short;
    const int N = hx * n_qtiles;
    int bl;
    if (!SPLIT && N <= 3 * cpx) {
      int k;
      if (N <= 2 * cpx) {
        const int R = max(N - cpx, 0);
        k = i < N - R ? R + i : R - 1 - (i - (N - R));
      } else {
        // three rounds: a snake over the tiles ranked longest first (CU c
        // takes ranks c, 2 cpx - 1 - c and 2 cpx + c), so the CUs' sums of
        // tile steps differ by at most about one tile
        const int d = i < cpx ? i : (i < 2 * cpx ? 3 * cpx - 1 - i : i);
        k = N - 1 - d;
      }
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
    bh = (id & 7) * hx + bl;
  } else {
    const int i = id;
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
  int kr[Stage<NW>::UK], kcp[Stage<NW>::UK];  // row and chunk pair of each K unit
};

template <int NW, bool CV>
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
    so.kr[j] = r;
    so.kcp[j] = cp;
  }
#pragma unroll
  for (int j = 0; j < Stage<NW>::UV; ++j) {
    int r, c;
    v_unit<CV>(tid + j * NT, r, c);
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

// With OTF the cos/sin of the staged keys are computed from their positions
// (p0 = position of frame 0) instead of read from the table; without KROT
// the keys arrive rotated and no cos/sin is loaded at all.
template <int NW, bool OTF, bool KROT>
__device__ __forceinline__ void stage_load(Stage<NW>& st, const bf16* __restrict__ k,
                                           const bf16* __restrict__ v, size_t rs, int T, int kt0,
                                           bool rope, const PrefillArgs& a, int64_t trow0,
                                           int64_t p0, const StageOffs<NW>& so) {
  // kt0 <= T on every call (tiles of the band, or T past the last one), so a
  // plain min: a clamp at 0 as well becomes a vector med3 and a vector
  // multiply whose results go back to scalar registers, every tile
  const uint32_t nrows = (uint32_t)min(T - kt0, kBN);
  const uint32_t rb = (uint32_t)(rs * sizeof(bf16));
  const auto kr = rows_rsrc(k + (size_t)kt0 * rs, nrows * rb);
  const auto vr = rows_rsrc(v + (size_t)kt0 * rs, nrows * rb);
#pragma unroll
  for (int j = 0; j < Stage<NW>::UK; ++j) {
    st.kx[j] = __builtin_amdgcn_raw_buffer_load_b128(kr, so.k[j], 0, 0);
    st.ky[j] = __builtin_amdgcn_raw_buffer_load_b128(kr, so.k[j] + 2 * kHalf, 0, 0);
    if constexpr (!KROT) {
      // rotated keys: no cos/sin
    } else if (OTF) {
      if (rope) {
        const int64_t p = p0 + kt0 + so.kr[j];
#pragma unroll
        for (int e = 0; e < 8; ++e) rope_cs(p, freq8(a.fr, so.kcp[j], e), &st.kc[j][e], &st.ks[j][e]);
      }
    } else {
      // without RoPE the table loads still go out, against an empty
      // descriptor (zeros, no memory access), so the count of loads per tile
      // does not depend on a runtime flag
      const auto tr = rows_rsrc(a.table + (trow0 + kt0) * kD, rope ? nrows * (kD * 4) : 0u);
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

template <int NW, bool SEED = false, bool KROT = true, bool CV = false>
__device__ __forceinline__ void stage_commit(const Stage<NW>& st, char* Kb, char* Vb, bool rope,
                                             int tid, const Seed& sd = Seed{}) {
  constexpr int NT = Stage<NW>::NT;
#pragma unroll
  for (int j = 0; j < Stage<NW>::UK; ++j) {
    int r, cp;
    k_unit(tid + j * NT, r, cp);
    u32x4 x = st.kx[j], y = st.ky[j];
    if (KROT && rope) {
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
    v_unit<CV>(tid + j * NT, r, c);
    *reinterpret_cast<u32x4*>(Vb + VLayout<CV>::chunk(r, c)) = st.v[j];
    int slot;
    if (SEED && sd.take(r, slot))
      *reinterpret_cast<u32x4*>(sd.ring_v + (size_t)slot * kD + 8 * c) = st.v[j];
  }
}

// Broadcast of lane 0's 64-bit value (every lane active).
__device__ __forceinline__ unsigned long long lane0_u64(unsigned long long x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((unsigned long long)hi << 32) | lo;
}

template <int NW, typename TO, bool SEED, bool OTF, bool SPLIT, bool KROT, bool HS>
__global__ __launch_bounds__(NW * 64, (NW == 4 && !KROT && !HS) ? 4 : 2) void prefill_mfma_kernel(
    PrefillArgs a, int n_qtiles, int n_short, int hx, int cpx) {
  // compact V rows where they let four workgroups share a CU
  constexpr bool CV = NW == 4 && !KROT && !HS;
  using VL = VLayout<CV>;
  constexpr int kRowV = VL::kRowV, kStageBytes = VL::kStageBytes;
  __shared__ __attribute__((aligned(16))) char lds[2 * kStageBytes];
  // HS (halves split): four waves cover 64 queries, two per 32-query block,
  // each taking one 32-key half of every staged tile; the two merge through
  // LDS at the end
  constexpr int BM = HS ? 64 : NW * 32;
  static_assert(!SPLIT || (!SEED && !OTF), "the split walk serves fixed-length calls with a table");
  static_assert(KROT || (!SEED && !OTF && !SPLIT), "keys arrive rotated only in plain calls");
  static_assert(!HS || (NW == 4 && !SEED && !SPLIT), "halves split: plain four-wave calls");

  int bh, qt, half;
  if (!work_item<SPLIT>(a.B * a.H, n_qtiles, n_short, hx, cpx, bh, qt, half)) return;
  const int h = bh % a.H, b = bh / a.H;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  // fixed batch: stream b at rows b*T ..; varlen: rows cu[b] .. cu[b+1]-1
  int T = a.T;
  size_t row0 = (size_t)b * a.T;
  bool bad = false;
  if (a.cu) {
    const int c0 = min(max(a.cu[b], 0), a.total);
    const int c1 = min(max(a.cu[b + 1], c0), a.total);
    row0 = (size_t)c0;
    T = c1 - c0;
    if (T > a.T) {
      bad = true;  // a stream longer than the call's bound: NaN rows, pos untouched
    } else {
      if (SEED && h == 0 && qt == 0 && threadIdx.x == 0) a.pos_out[b] = T;
      if (qt * BM >= T) return;
    }
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

  // positions: frame t at p0 + t; its cos/sin at table row trow0 + t
  const int64_t p0 = a.pos0 ? a.pos0[b] : 0;
  const int64_t trow0 = a.table_bstride * b + (a.table_pos ? p0 : 0) + a.table_off;
  if (p0 < 0) bad = true;
  if (!OTF && rope && (trow0 < 0 || trow0 + T > a.table_len)) bad = true;
  if (bad) {
    // every row of this entry and head is NaN, written by query tile 0
    if (qt == 0 && half == 0) poison_rows<TO>(o, rs, 0, T);
    return;
  }

  const int q0 = qt * BM;
  const int qblk = HS ? (wave & 1) : wave;  // this wave's 32-query block
  const int hsb = HS ? (wave >> 1) : 0;     // HS: this wave's 32-key half of each tile
  const int qw = q0 + qblk * 32;
  const int tq = qw + l32;  // this lane's query

  const int kbeg = max(0, q0 - W + 1);
  const int klast = min(T, q0 + BM) - 1;
  int it0 = kbeg / kBN, it1 = klast / kBN;
  if (SPLIT) {
    // the older half of the band (the larger, if odd) to half 0, the newer to
    // half 1; a one-tile band leaves half 1 without tiles (it still merges)
    const int mid = it0 + (it1 - it0 + 2) / 2;
    if (half == 0) it1 = mid - 1;
    else it0 = mid;
  }
  // Visiting order of the key tiles it0 .. it1.  P is the number of tiles in
  // the band of a 128-query tile (at least that of any workgroup's band), and
  // the walk starts at the band's tile whose index is a multiple of P,
  // wrapping around to it0: every query tile whose band holds key tile j then
  // visits it at about step j mod P, so workgroups that run side by side read
  // the same K, V and table rows at about the same time and L2 serves all but
  // the first.  (In ascending order a tile's neighbour, BM queries later,
  // reaches the same keys BM/64 steps later, by which time the XCD's resident
  // workgroups have streamed more rows than its L2 keeps on large grids.)
  // A band holds at most one multiple of P; one that holds none (cut at key 0
  // or at T) is walked in ascending order.  So a 32-query block sees its key
  // tiles in an order set by the tile indices alone, the same with two- or
  // four-wave workgroups, and both give the same bits.
  // (The split walk serves grids whose K, V and table rows all stay in L2:
  // its halves go in ascending order.)
  const int P = 2 + (W - 1 + kBN - 1) / kBN;
  int it_start = SPLIT ? it0 : it0 + (P - it0 % P) % P;
  if (it_start > it1) it_start = it0;
  // The halves split (small grids, whose K, V and table rows all stay in L2)
  // walks its band from the newest tile down to the oldest instead: with no
  // reuse to arrange, each wave starts on the tile that holds its own
  // queries' keys (layer workload 21.98 -> 21.72 us, same box, three
  // alternating runs).
  if (HS) it_start = it1;
  // (the same in every lane; the division above is expanded on the vector ALU)
  it_start = __builtin_amdgcn_readfirstlane(it_start);

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
  if (rope && !OTF) {
#pragma unroll
    for (int j = 0; j < NQT; ++j) {
      const int i = tid + j * NT;
      const int r = i >> 4, c = i & 15;
      const int row = min(q0 + r, T - 1);
      tq_rows[j] = *reinterpret_cast<const u32x4*>(a.table + (trow0 + row) * kD + 4 * c);
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
  const StageOffs<NW> so = stage_offsets<NW, CV>(tid, rs);
  stage_load<NW, OTF, KROT>(st, k, v, rs, T, it_start * kBN, rope, a, trow0, p0, so);
  if (rope && !OTF) {
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
      float cc[8], ss[8], xf[8], yf[8];
      if (OTF) {
#pragma unroll
        for (int e = 0; e < 8; ++e) rope_cs(p0 + min(tq, T - 1), freq8(a.fr, c, e), &cc[e], &ss[e]);
      } else {
        const float* cs =
            reinterpret_cast<const float*>(lds + (min(tq, T - 1) - q0) * kRowQT) + 8 * c;
        load8(cs, cc);
        load8(cs + kHalf, ss);
      }
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
  // per 32-dim block db.  In compact V rows the chunk swizzle swaps the row's
  // 64-byte halves for rows with bit 1 set, which for these rows is bit 3 of
  // L; a read of 32 lanes then covers rows 4i..4i+3 at banks 32*(r&1) +
  // [0, 16) and [16, 32).
  const int k_off = l32 * kRowK + 16 * hh;
  const int g = lane >> 4, L = lane & 15;
  const int v_row = (4 * (g >> 1) + (L >> 2)) * kRowV + (16 * (g & 1) + 4 * (L & 3)) * 2;
  const int v_sw = CV ? 64 * (L >> 3) : 0;
  const int v_off[2] = {v_row + v_sw, v_row + (64 ^ v_sw)};

  f32x16 oacc[2];
  oacc[0] = f32x16{};
  oacc[1] = f32x16{};
  // the running max starts at a finite floor, not -inf: the first finite
  // score always moves it, exp2(floor - m) is 0 (not NaN), and a half whose
  // scores are all masked gives exp2(-inf) = 0 against it, so no selects
  float m_run = kNoMax, l_run = 0.f;
  const float c2 = a.scale_log2;
  const unsigned wm1 = (unsigned)(W - 1);

  if (rope && !OTF) __syncthreads();  // every wave has read its Q table rows
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
  stage_commit<NW, SEED, KROT, CV>(st, lds, lds + kTileK, rope, tid, seed_for(it_start * kBN));
  __syncthreads();

  // One step per key tile: the next tile's loads go out first (after the
  // last tile: rows from T on, an empty descriptor), then this tile's scores,
  // softmax and P·V, then the next tile's commit to the other LDS buffer.
  // The walk is two loops with an affine tile index each (it_start .. it1,
  // then it0 .. it_start-1): a wrapped index in one loop makes the compiler
  // keep a staged tile live across the whole step (32 more VGPRs).
  int j = 0;
  auto tile_step = [&](const int it, const int kt_next) {
    const int buf = j & 1;
    stage_load<NW, OTF, KROT>(st, k, v, rs, T, kt_next, rope, a, trow0, p0, so);

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
      const char* vr = Vb + 32 * sb * kRowV;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const char* p0 = vr + 16 * ks * kRowV + v_off[db];
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

    // 32-key half sb: active if it meets this wave's band, masked if it
    // straddles an edge of it
    auto active = [&](int sb) {
      const int kb = kt0 + 32 * sb;
      return (qw < T) && (kb < T) && (kb + 31 >= qw - W + 1) && (kb <= qw + 31);
    };
    auto edge = [&](int sb) {
      const int kb = kt0 + 32 * sb;
      return (kb + 31 > qw) || (kb < qw + 31 - W + 1);
    };
    if constexpr (HS) {
      // only this wave's half: its flags stay scalar
      if (active(hsb)) {
        f32x16 sc = s_half(hsb);
        if (edge(hsb)) {
          const int d0 = tq - (kt0 + 32 * hsb + 4 * hh);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 8 * (r >> 2) + (r & 3);
            sc[r] = ((unsigned)(d0 - off) <= wm1) ? sc[r] : -INFINITY;
          }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
        update_max(mx);
        const float mu = m_run;
        pv_half(sc, hsb, mu);
      }
    } else {
      const bool act[2] = {active(0), active(1)}, msk[2] = {edge(0), edge(1)};
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
    }

    if (kt_next < T)
      stage_commit<NW, SEED, KROT, CV>(st, lds + (buf ^ 1) * kStageBytes,
                             lds + (buf ^ 1) * kStageBytes + kTileK, rope, tid,
                             seed_for(kt_next));
    __syncthreads();
    ++j;
  };
  // split walk: this wave's flag word, read as the last tile starts so that
  // its memory latency hides under that tile (a partner that finishes
  // meanwhile is found by the token swap instead)
  unsigned long long* flag = nullptr;
  unsigned long long seen = 0;
  if (SPLIT) flag = a.split_flags + ((size_t)bh * n_qtiles + qt) * NW + wave;
  if constexpr (HS) {
    for (int it = it1; it >= it0; --it) tile_step(it, it > it0 ? (it - 1) * kBN : T);
  } else {
    const int kt_wrap = it_start > it0 ? it0 * kBN : T;
    for (int it = it_start; it <= it1; ++it) {
      if (SPLIT && it == it1) seen = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      tile_step(it, it < it1 ? (it + 1) * kBN : kt_wrap);
    }
    for (int it = it0; it < it_start; ++it) tile_step(it, it + 1 < it_start ? (it + 1) * kBN : T);
  }

  if constexpr (SPLIT) {
    const size_t slot = ((size_t)bh * n_qtiles + qt) * NW + wave;
    if (qw >= T) {
      // both halves skip a wave past the end alike; its flag is left zero too
      if (half == 0 && lane == 0)
        __hip_atomic_store(flag, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    // The partial results move with device-coherent stores and loads (cache
    // policy sc1, the encoding of device-scope atomic stores and loads): a
    // store is visible to every XCD once the wave's memory counter shows it
    // done, and a load reads the device-coherent value.  So a half waits for
    // its stores before it swaps its token in, and loads its partner's only
    // after seeing the partner's token; no cache is written back or
    // invalidated (device-scope fences would do both to the whole L2).
    const auto pr = rows_rsrc(reinterpret_cast<const char*>(a.split_part) + slot * 2 * kSplitPartBytes,
                              (uint32_t)(2 * kSplitPartBytes));
    const uint32_t v_mine = (uint32_t)(half * kSplitPartBytes) + 16 * lane;
    const uint32_t v_other = (uint32_t)((half ^ 1) * kSplitPartBytes) + 16 * lane;
    const unsigned long long tok_other = kSplitTok + (half ^ 1);
    bool merge = lane0_u64(seen) == tok_other;
    if (!merge) {
#pragma unroll
      for (int r = 0; r < 8; ++r)
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4, f32x4{oacc[r >> 2][4 * (r & 3)], oacc[r >> 2][4 * (r & 3) + 1],
                                            oacc[r >> 2][4 * (r & 3) + 2],
                                            oacc[r >> 2][4 * (r & 3) + 3]}),
            pr, v_mine + r * 1024, 0, kCoherent);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{m_run, l_run, 0.f, 0.f}),
                                             pr, v_mine + 8 * 1024, 0, kCoherent);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      unsigned long long old = 0;
      if (lane == 0)
        old = __hip_atomic_exchange(flag, kSplitTok + half, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
      merge = lane0_u64(old) == tok_other;
      if (!merge) return;  // the partner merges
    }
    asm volatile("" ::: "memory");  // the loads below stay after the token test
    f32x4 po[9];
#pragma unroll
    for (int r = 0; r < 9; ++r)
      po[r] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(pr, v_other + r * 1024,
                                                                              0, kCoherent));
    if (lane == 0) __hip_atomic_store(flag, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // merge with the halves in a fixed order (0 then 1): the same bits
    // whichever half merges
    const float m0 = half ? po[8][0] : m_run, m1 = half ? m_run : po[8][0];
    const float l0 = half ? po[8][1] : l_run, l1 = half ? l_run : po[8][1];
    const float mm = fmaxf(m0, m1);
    const float a0 = __builtin_amdgcn_exp2f(m0 - mm), a1 = __builtin_amdgcn_exp2f(m1 - mm);
    l_run = l0 * a0 + l1 * a1;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = oacc[r >> 2][4 * (r & 3) + e], y = po[r][e];
        const float o0 = half ? y : x, o1 = half ? x : y;
        oacc[r >> 2][4 * (r & 3) + e] = o0 * a0 + o1 * a1;
      }
    }
  }

  if constexpr (HS) {
    // the wave of the second key half hands its partial result (O^T, m, l)
    // to the wave of the first through LDS (the tiles are done with: every
    // wave passed the last step's barrier); the merge takes the halves in a
    // fixed order
    f32x4* part = reinterpret_cast<f32x4*>(lds) + qblk * 9 * 64 + lane;
    if (hsb == 1) {
#pragma unroll
      for (int r = 0; r < 8; ++r)
        part[r * 64] = f32x4{oacc[r >> 2][4 * (r & 3)], oacc[r >> 2][4 * (r & 3) + 1],
                             oacc[r >> 2][4 * (r & 3) + 2], oacc[r >> 2][4 * (r & 3) + 3]};
      part[8 * 64] = f32x4{m_run, l_run, 0.f, 0.f};
    }
    __syncthreads();
    if (hsb == 1) return;
    f32x4 po[9];
#pragma unroll
    for (int r = 0; r < 9; ++r) po[r] = part[r * 64];
    const float m0 = m_run, m1 = po[8][0];
    const float mm = fmaxf(m0, m1);
    const float a0 = __builtin_amdgcn_exp2f(m0 - mm), a1 = __builtin_amdgcn_exp2f(m1 - mm);
    l_run = l_run * a0 + po[8][1] * a1;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        oacc[r >> 2][4 * (r & 3) + e] = oacc[r >> 2][4 * (r & 3) + e] * a0 + po[r][e] * a1;
    }
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

template <int NW, typename TO, bool SEED, bool OTF, bool SPLIT = false, bool KROT = true,
          bool HS = false>
void launch_k(dim3 g, dim3 blk, hipStream_t st, const PrefillArgs& a, int n_qtiles, int n_short,
              int hx, int cpx) {
  hipLaunchKernelGGL((prefill_mfma_kernel<NW, TO, SEED, OTF, SPLIT, KROT, HS>), g, blk, 0, st, a,
                     n_qtiles, n_short, hx, cpx);
}

// Halves split: 64-query workgroups of four waves (see the kernel).
hipError_t launch_hs(const PrefillArgs& a, DT out, hipStream_t st) {
  constexpr int BM = 64;
  const int n_qtiles = (a.T + BM - 1) / BM;
  const int n_short = min(n_qtiles, (a.W - 1 + BM - 1) / BM);
  const int n_bh = a.B * a.H;
  const int hx = n_bh >= 8 ? (n_bh + 7) / 8 : 0;
  const int cpx = cus_per_xcd();
  const int64_t grid = hx > 0 ? (int64_t)8 * hx * n_qtiles : (int64_t)n_bh * n_qtiles;
  const dim3 g((unsigned)grid), blk(256);
  const bool krot = a.rope && !a.k_rotated;
  const bool otf = a.rope && !a.table;  // no table: cos/sin computed in the kernel
  if (out == DT::BF16) {
    if (otf) launch_k<4, bf16, false, true, false, true, true>(g, blk, st, a, n_qtiles, n_short, hx, cpx);
    else if (krot) launch_k<4, bf16, false, false, false, true, true>(g, blk, st, a, n_qtiles, n_short, hx, cpx);
    else launch_k<4, bf16, false, false, false, false, true>(g, blk, st, a, n_qtiles, n_short, hx, cpx);
  } else {
    if (otf) launch_k<4, float, false, true, false, true, true>(g, blk, st, a, n_qtiles, n_short, hx, cpx);
    else if (krot) launch_k<4, float, false, false, false, true, true>(g, blk, st, a, n_qtiles, n_short, hx, cpx);
    else launch_k<4, float, false, false, false, false, true>(g, blk, st, a, n_qtiles, n_short, hx, cpx);
  }
  return hipGetLastError();
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
  const dim3 blk(NW * 64);
  const bool otf = a.rope && !a.table;  // no table: cos/sin computed in the kernel
  if constexpr (NW == 4) {
    if (a.split_flags && !a.cu && !a.ring_k && !otf) {
      const dim3 g2((unsigned)(2 * grid));
      if (out == DT::BF16) launch_k<NW, bf16, false, false, true>(g2, blk, st, a, n_qtiles, n_short, hx, cpx);
      else launch_k<NW, float, false, false, true>(g2, blk, st, a, n_qtiles, n_short, hx, cpx);
      return hipGetLastError();
    }
  }
  const dim3 g((unsigned)grid);
  if constexpr (NW == 4) {
    // keys already rotated (ahead of the kernel, or pre-rotated input): no
    // cos/sin loads or key rotation in the staging
    if (!a.cu && !a.ring_k && !otf && (a.k_rotated || !a.rope)) {
      if (out == DT::BF16) launch_k<NW, bf16, false, false, false, false>(g, blk, st, a, n_qtiles, n_short, hx, cpx);
      else launch_k<NW, float, false, false, false, false>(g, blk, st, a, n_qtiles, n_short, hx, cpx);
      return hipGetLastError();
    }
  }
  if (a.ring_k) {
    // (seeding with in-kernel cos/sin runs four-wave workgroups only: the
    // two-wave variant would need more than 256 VGPRs)
    if constexpr (NW == 4) {
      if (otf) {
        if (out == DT::BF16) launch_k<NW, bf16, true, true>(g, blk, st, a, n_qtiles, n_short, hx, cpx);
        else launch_k<NW, float, true, true>(g, blk, st, a, n_qtiles, n_short, hx, cpx);
        return hipGetLastError();
      }
    }
    if (out == DT::BF16) launch_k<NW, bf16, true, false>(g, blk, st, a, n_qtiles, n_short, hx, cpx);
    else launch_k<NW, float, true, false>(g, blk, st, a, n_qtiles, n_short, hx, cpx);
  } else {
    if (out == DT::BF16) {
      if (otf) launch_k<NW, bf16, false, true>(g, blk, st, a, n_qtiles, n_short, hx, cpx);
      else launch_k<NW, bf16, false, false>(g, blk, st, a, n_qtiles, n_short, hx, cpx);
    } else {
      if (otf) launch_k<NW, float, false, true>(g, blk, st, a, n_qtiles, n_short, hx, cpx);
      else launch_k<NW, float, false, false>(g, blk, st, a, n_qtiles, n_short, hx, cpx);
    }
  }
  return hipGetLastError();
}

}  // namespace

// The split walk pays off against the plain four-wave grid while that grid
// has at most one workgroup per CU and the key bands are long: the merge
// adds about three dependent device-coherent memory round trips to a wave's
// end, which costs more than halving the walk saves once the CUs hold more
// than one query tile each, or when a band is only a few tiles long.
size_t prefill_split_bytes(int B, int T, int H, int W, bool force, size_t* flag_bytes) {
  const int64_t wg4 = (int64_t)((T + 127) / 128) * H * B;
  const int64_t cus = (int64_t)cus_per_xcd() * 8;
  const int64_t band = (int64_t)W + 127 < T ? (int64_t)W + 127 : (int64_t)T;  // longest band
  const int64_t band_tiles = (band + kBN - 1) / kBN;
  // The halves-split workgroups serve the same small grids as well or better
  // (B1 T1500 H16 17.3 against 17.7 us, B1 T500 H32 11.7 against 11.8, B4
  // T150 H32 7.2 against 10.2; the tiniest grids 2 % slower, B1 T1500 H4
  // 16.3 against 16.0) with no workspace, so the split walk runs only on
  // request (VX_FLAG_SPLIT_WALK), on grids whose doubled size is resident.
  (void)band_tiles;
  const bool fits = 2 * wg4 <= 3 * cus;  // the doubled grid is resident at once
  if (wg4 <= 0 || !force || !fits) return 0;
  const size_t slots = (size_t)wg4 * 4;
  const size_t fb = (slots * sizeof(unsigned long long) + 255) & ~(size_t)255;
  if (flag_bytes) *flag_bytes = fb;
  return fb + slots * 2 * kSplitPartBytes;
}

// Rotating the keys ahead of the kernel costs one more read and write of K
// (a launch of its own) and saves the kernel about a quarter of its vector
// work, which sets its pace at full occupancy; the kernel on rotated keys
// also fits four workgroups per CU instead of three (compact V rows).
// Measured against rotating them in the staging: B8 T6000 H32 498 against
// 560 us, B8 T1500 H32 106.7 against 111.6, but B4 T1500 H32 57.6 against
// 56.7 and B2 T3000 H32 65.1 against 64.4 (6 query tiles per CU).  So grids
// of at least 8 query tiles per CU take it.
size_t prefill_krot_bytes(int B, int T, int H) {
  const int64_t wg4 = (int64_t)((T + 127) / 128) * H * B;
  const int64_t cus = (int64_t)cus_per_xcd() * 8;
  if (wg4 < 8 * cus) return 0;
  return (size_t)B * T * H * kD * sizeof(bf16);
}

// Halves split for grids whose 64-query workgroups are all resident at once
// (three per CU): twice the workgroups of the four-wave grid, each wave's
// tile step half as long.
bool prefill_half_split(int B, int T, int H) {
  const int64_t wg4 = (int64_t)((T + 127) / 128) * H * B;
  const int64_t cus = (int64_t)cus_per_xcd() * 8;
  return wg4 > 0 && 2 * wg4 <= 3 * cus;
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, DT out, hipStream_t st) {
  // Four-wave workgroups share each staged (and rotated) K tile among more
  // queries; two-wave ones keep enough workgroups to cover the 256 CUs when
  // the problem is small (unless the split walk is on).
  const int64_t wg4 = (int64_t)((a.T + 127) / 128) * a.H * a.B;
  if (a.half_split && !a.split_flags && !a.cu && !a.ring_k) return launch_hs(a, out, st);
  if (wg4 >= 256 || (a.ring_k && a.rope && !a.table) || a.split_flags) return launch_nw<4>(a, out, st);
  return launch_nw<2>(a, out, st);
}

}  // namespace vx
