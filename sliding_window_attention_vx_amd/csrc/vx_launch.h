// Internal launcher interface between the C ABI (vx_api.hip) and the kernels.
// Arguments reaching these functions have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vx_device.h"

namespace vx {

enum class DT { F32 = 0, BF16 = 1 };

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int B, T, H, W;
  // Frame t of batch entry b sits at position pos0[b] + t (pos0: device int64
  // [B], nullptr = 0).  A negative pos0[b] makes that entry's outputs NaN.
  const int64_t* pos0 = nullptr;
  bool rope;            // rotate q, k on load
  // cos/sin of frame t of batch entry b: table row
  //   b * table_bstride + (table_pos ? pos0[b] : 0) + t + table_off
  // of a [rows][2][32] float32 table with table_len rows; an entry whose rows
  // fall outside [0, table_len) gets NaN outputs.  table == nullptr with rope:
  // cos/sin are computed on the fly from fr (the same float64 angle, so the
  // same values as a table).
  const float* table = nullptr;
  int64_t table_off = 0;
  int64_t table_bstride = 0;
  bool table_pos = true;
  int64_t table_len = 0;
  RopeFreqs fr;
  float scale_log2;     // softmax scale * log2(e)
  // Varlen batch (cu != nullptr): B streams packed along the frame axis,
  // stream b at rows cu[b] .. cu[b+1]-1, each at positions 0 .. length - 1.
  // A stream longer than T gets NaN outputs and its pos_out is left alone.
  // Ring seeding (ring_k != nullptr): the rotated keys and the values of
  // frames t >= length - W go to slot t mod W of the stream's [H, W, 64]
  // rings, and pos_out[b] = length.
  const int32_t* cu = nullptr;
  int total = 0;        // packed rows (offsets are clamped to [0, total])
  void* ring_k = nullptr;
  void* ring_v = nullptr;
  int64_t* pos_out = nullptr;
  // Split walk (split_flags != nullptr; fixed-length batches with a cos/sin
  // table or pre-rotated inputs): two workgroups per 128-query tile, each
  // walking one half of the tile's key band, and per wave the later of the
  // two merges both partial results.  Layout from prefill_split_bytes:
  // one flag word per (b, h, query tile, wave), zero between calls (each
  // call leaves them zero; any value but the kernel's two tokens is taken
  // as zero), then two partial results of kSplitPartBytes per flag.
  unsigned long long* split_flags = nullptr;
  float* split_part = nullptr;
  // k holds keys already rotated (by launch_rope_k_table) while q is rotated
  // per `rope`: the kernel stages the keys as they are
  bool k_rotated = false;
  // 64-query workgroups whose waves take one 32-key half of each tile
  bool half_split = false;
};

// Bytes of one wave's partial result in the split walk: the 64 x 32 float
// O^T accumulators and the running max and sum, as 9 rows of 64 x 16 bytes.
constexpr size_t kSplitPartBytes = (size_t)9 * 64 * 16;

// Workspace bytes of the split walk for a fixed-length prefill of this shape
// and window on the current device (flag words first, *flag_bytes of them,
// 256-byte aligned, then the partial results), or 0 where the walk is not
// taken: always without force (the halves-split workgroups serve small
// grids), and with force on grids whose doubled size is not resident at
// once (more than 1.5 query tiles per CU).
size_t prefill_split_bytes(int B, int T, int H, int W, bool force, size_t* flag_bytes);

// Workspace bytes of the rotated keys for a fixed-length prefill of this
// shape on the current device (B*T*H*64 bf16), or 0 where the grid is too
// small for rotating the keys once, ahead of the kernel, to pay off.
size_t prefill_krot_bytes(int B, int T, int H);

// Whether a fixed-length prefill of this shape takes the halves-split
// workgroups (64 queries, each wave one 32-key half of every tile).
bool prefill_half_split(int B, int T, int H);

struct StreamArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* ring_k;
  const void* ring_v;
  const int64_t* pos;
  void* o;
  int S, n, H, W;
  bool rope;
  float scale_log2;
  // fused append (n <= 16): write rotated new keys/values into the ring after
  // all reads and set pos_out[s] = pos[s] + n (pos_out != pos)
  bool append;
  void* ring_k_w;
  void* ring_v_w;
  int64_t* pos_out;
};

struct AppendArgs {
  void* ring_k;
  void* ring_v;
  const void* k;
  const void* v;
  const int64_t* pos;  // read
  int64_t* pos_out;    // written: pos_out[s] = pos[s] + n (may equal pos)
  int S, n, H, W;
  bool rope;
};

hipError_t launch_rope_table(float* table, int64_t p_begin, int count, const RopeFreqs& fr,
                             hipStream_t st);
// In-place rotation; frame t of batch entry b at position pos0[b] + t
// (pos0: device int64 [B] or nullptr = 0; a negative entry makes its rows NaN).
hipError_t launch_rope_qk(void* q, void* k, int B, int T, int H, const int64_t* pos0, DT io,
                          const RopeFreqs& fr, hipStream_t st);
// Table rows b*T + t = cos/sin of position pos0[b] + t (pos0 nullptr = 0).
hipError_t launch_rope_table_batched(float* table, const int64_t* pos0, int B, int T,
                                     const RopeFreqs& fr, hipStream_t st);
// Rotated keys of a prefill with a cos/sin table (a.table, its row mapping)
// written to k_out ([B, T, H, 64] bf16).
hipError_t launch_rope_k_table(const PrefillArgs& a, void* k_out, hipStream_t st);
hipError_t launch_prefill_valu(const PrefillArgs& a, DT io, DT out, hipStream_t st);
hipError_t launch_prefill_mfma(const PrefillArgs& a, DT out, hipStream_t st);
hipError_t launch_stream_step(const StreamArgs& a, DT io, DT out, const RopeFreqs& fr,
                              hipStream_t st);
hipError_t launch_ring_append(const AppendArgs& a, DT io, const RopeFreqs& fr, hipStream_t st);

constexpr int kStreamMaxNew = 64;  // largest n accepted by the streaming kernels (LDS use)
constexpr int kStreamFusedMaxNew = 16;  // largest n of the fused step + append

}  // namespace vx
