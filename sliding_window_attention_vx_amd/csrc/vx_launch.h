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
  int64_t pos0;
  bool rope;            // rotate q, k on load (table must be valid)
  const float* table;   // [.., 2, 32] cos/sin rows
  int64_t table_row0;   // table row of position pos0 (= pos0 - table_p0)
  float scale_log2;     // softmax scale * log2(e)
  // Varlen batch (cu != nullptr): B streams packed along the frame axis,
  // stream b at rows cu[b] .. cu[b+1]-1 (length at most T), each at positions
  // pos0 .. pos0 + length - 1.  Ring seeding (ring_k != nullptr): the rotated
  // keys and the values of frames t >= length - W go to slot t mod W of the
  // stream's [H, W, 64] rings, and pos_out[b] = length.
  const int32_t* cu = nullptr;
  int total = 0;        // packed rows (offsets are clamped to [0, total])
  void* ring_k = nullptr;
  void* ring_v = nullptr;
  int64_t* pos_out = nullptr;
};

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
hipError_t launch_rope_qk(void* q, void* k, int B, int T, int H, int64_t pos0, DT io,
                          const RopeFreqs& fr, hipStream_t st);
hipError_t launch_prefill_valu(const PrefillArgs& a, DT io, DT out, hipStream_t st);
hipError_t launch_prefill_mfma(const PrefillArgs& a, DT out, hipStream_t st);
hipError_t launch_stream_step(const StreamArgs& a, DT io, DT out, const RopeFreqs& fr,
                              hipStream_t st);
hipError_t launch_ring_append(const AppendArgs& a, DT io, const RopeFreqs& fr, hipStream_t st);

constexpr int kStreamMaxNew = 64;  // largest n accepted by the streaming kernels (LDS use)
constexpr int kStreamFusedMaxNew = 16;  // largest n of the fused step + append

}  // namespace vx
