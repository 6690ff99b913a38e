/*
 * vx.h - C ABI of the MI355X (gfx950) sliding-window RoPE attention library.
 *
 * The operation is the self-attention of the Voxtral Realtime 2602 audio
 * encoder (transcribe.cpp "Voxtral" family notes, section Architecture,
 * Voxtral Realtime 2602): causal attention of each encoder frame over the
 * most recent W = 750 frames including itself, 32 heads of head_dim 64, with
 * rotary position embedding (RoPE, theta = 1e6) on queries and keys.  It comes
 * in two forms:
 *   - prefill: a whole chunk in one call (the Core AI port's batched
 *     first-chunk encoder, "Voxtral Mini 4B Realtime - Core AI", section
 *     "Why two encoders?");
 *   - streaming: 4 new encoder frames per step (same family notes, Streaming
 *     schedule: 8 mel frames = 4 encoder frames = one 80 ms audio token),
 *     attending to a W-slot ring of past rotated keys and values.
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing, frees nothing and keeps no pointer after a call
 *     returns.  Its only state is a per-device cache of the CU count (read
 *     once, to order the prefill's workgroups); it may be called from several
 *     host threads at once.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work on it and never synchronise; a fault in a
 *     kernel surfaces at the caller's next synchronising HIP call.
 *   - Layouts are dense row-major: activations [B,T,H,D] (D fastest), rings
 *     [S,H,W,D].  D (head_dim) must be 64, except for the grouped-query
 *     entry points at the end of this file, which take 128.
 *   - Every argument is checked on the host before anything is launched.  On
 *     any error nothing is launched and no buffer is touched; the status
 *     says why and vx_last_error() gives a message (thread-local).  A failed
 *     kernel launch returns VX_E_HIP.
 *   - Empty work (B == 0, T == 0 or S == 0) returns VX_OK without launching.
 *   - RoPE pairs dimension i with i + D/2 (half-split) and turns the pair by
 *     angle position * theta^(-2i/D); the angle is formed in float64 and its
 *     cosine and sine rounded to float32; the rotation itself is float32 and
 *     the rotated value is rounded to the storage dtype (nearest-even).
 */
#ifndef VX_H
#define VX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VX_OK = 0,
  VX_E_NULL = 1,   /* a required pointer is NULL */
  VX_E_SHAPE = 2,  /* a size is negative, zero where it must not be, or too large */
  VX_E_DTYPE = 3,  /* unsupported dtype or dtype pair */
  VX_E_ALIGN = 4,  /* a tensor pointer is not 16-byte aligned */
  VX_E_RANGE = 5,  /* a value is out of range (window, theta, scale, n > W, positions, table) */
  VX_E_HIP = 6     /* the HIP runtime reported an error when launching */
} vx_status;

typedef enum { VX_F32 = 0, VX_BF16 = 1 } vx_dtype;

/* Flags for vx_attn_cfg.flags. */
#define VX_FLAG_VALU_KERNEL 1u /* prefill: use the float32 vector-ALU kernel instead of the
                                  bf16 matrix-core kernel (a cross-check; bf16 inputs still
                                  get bf16-rounded rotated q and k) */
#define VX_FLAG_SPLIT_WALK 2u  /* prefill: take the split walk (see vx_swa_attn_prefill),
                                  given a workspace, on grids of at most 1.5 query tiles
                                  per compute unit instead of the halves-split workgroups */

typedef struct {
  int32_t head_dim;      /* must be 64                                              */
  int32_t window;        /* W >= 1 (750 for the Voxtral Realtime encoder)           */
  double rope_theta;     /* > 0 (1e6)                                               */
  float softmax_scale;   /* >= 0; 0 means 1/sqrt(head_dim)                          */
  int32_t io_dtype;      /* vx_dtype of q, k, v and of the rings                    */
  int32_t out_dtype;     /* vx_dtype of o; pairs: bf16->bf16, bf16->f32, f32->f32   */
  uint32_t flags;        /* VX_FLAG_* bits, 0 by default                            */
  /* Optional device scratch owned by the caller (NULL/0 = none, 16-byte
   * aligned), used by vx_swa_attn_prefill when it is given no rope_table:
   * the cos/sin rows of the call's positions are built there (see
   * vx_swa_attn_prefill_workspace_size).  No contents are kept between
   * calls; calls that overlap in time must not share a workspace.  Other
   * entry points ignore it. */
  void *workspace;
  size_t workspace_bytes;
} vx_attn_cfg;

/* Fills `cfg` with the Voxtral Realtime encoder defaults: head_dim 64,
 * window 750, theta 1e6, scale 1/8, bf16 in and out, no flags, no workspace. */
void vx_default_cfg(vx_attn_cfg *cfg);

/* RoPE cosine/sine table for `count` consecutive positions starting at
 * `p_begin` (>= 0), for head_dim 64 or 128: the RoPE cache of the rotation
 * defined at the top of this file (transcribe.cpp "Voxtral" family notes,
 * Architecture: RoPE theta 1e6 on the encoder's queries and keys).
 * table: device float32 [count][2][head_dim/2]:
 * table[j][0][i] = cos((p_begin+j) * theta^(-2i/D)), table[j][1][i] = sin(...).
 * Only cfg->head_dim and cfg->rope_theta are read.  The table depends on
 * nothing else, so one table serves every layer and call that uses these
 * positions. */
vx_status vx_rope_table(float *table, int64_t p_begin, int32_t count, const vx_attn_cfg *cfg,
                        void *stream);

/* In-place RoPE of q and k, both [B,T,H,D] of cfg->io_dtype: the rotation
 * the encoder applies to its queries and keys before attention
 * (transcribe.cpp "Voxtral" family notes, Architecture, Voxtral Realtime
 * 2602: RoPE theta 1e6, head_dim 64).  Row t of batch entry b sits at
 * absolute position pos0[b] + t.
 * pos0: device int64 [B] (8-byte aligned), or NULL for position t.  The
 *   values are read on the device, so they are not checked here: an entry
 *   with pos0[b] < 0 has its q and k rows set to NaN (loud, never partial).
 * Either q or k may be NULL (not both).  V is never rotated. */
vx_status vx_rope_qk(void *q, void *k, int32_t B, int32_t T, int32_t H, const int64_t *pos0,
                     const vx_attn_cfg *cfg, void *stream);

/* Causal sliding-window attention over whole chunks (no history), the
 * encoder's self-attention in its whole-chunk form (transcribe.cpp "Voxtral"
 * family notes, Architecture, Voxtral Realtime 2602: causal sliding window
 * of 750 frames, 32 heads x 64, RoPE; run as one call per chunk like the
 * Core AI port's batched first-chunk encoder, "Voxtral Mini 4B Realtime -
 * Core AI", "Why two encoders?"):
 *   o[b,t,h] = sum_j softmax_j(scale * q'[b,t,h] . k'[b,j,h]) v[b,j,h],
 *   j = max(0, t-W+1) .. t,
 * where q', k' are q, k rotated at positions pos0[b] + t.
 * q, k, v: [B,T,H,D] cfg->io_dtype; o: [B,T,H,D] cfg->out_dtype (must not
 * alias the inputs).
 * pos0: device int64 [B] (8-byte aligned), or NULL for positions 0 .. T-1.
 * rope_applied != 0: q and k are already rotated; the table is ignored.
 * rope_applied == 0: the kernel rotates q and k as it loads them, with
 *   cos/sin from
 *   - rope_table (made by vx_rope_table) covering positions table_p0 ..
 *     table_p0 + table_len - 1, which must include every pos0[b] .. pos0[b]
 *     + T - 1: checked here when pos0 is NULL (VX_E_RANGE), on the device
 *     otherwise;
 *   - rope_table == NULL: a table of the call's positions built in the
 *     workspace (one extra launch) when cfg->workspace has room for it,
 *     else cos/sin computed in the kernel from the same float64 angle (the
 *     same values, at a higher cost per tile).
 * A batch entry whose positions are invalid on the device (pos0[b] < 0, or
 * rows outside the given table) gets NaN in all its outputs (loud, never
 * partial); the other entries are unaffected.
 * cfg->workspace (optional): with at least
 * vx_swa_attn_prefill_workspace_size() bytes, a NULL rope_table is served
 * from a table built in it (one extra launch); the results are the same bits
 * as with a caller table or cos/sin computed in the kernel.
 * Schedules (bf16 matrix-core path): grids of at most 1.5 128-query tiles
 * per compute unit (one 1500-frame chunk of 32 heads and smaller) run
 * 64-query workgroups whose two waves per 32-query block each take one
 * 32-key half of every key tile and merge their softmax partials at the
 * end (the exact rescaling of running maxima and sums that flash
 * attention's online softmax uses); larger grids run 128-query workgroups.
 * The two schedules differ in summation order, so a call's bits depend on
 * its grid size (within the same tolerance of the exact result).
 * With VX_FLAG_SPLIT_WALK and a workspace (with a table or rope_applied),
 * such small grids take the split walk instead: two workgroups per 128-query
 * tile, one per half of its key band, the later of the two merging both
 * partials.  Its flag
 * words and partial results follow the table in the workspace (which must
 * then not be shared by calls that overlap in time); each call leaves the
 * flag words zero, and any content other than the kernel's two tokens reads
 * as zero, so the workspace needs no clearing.  Split results are
 * deterministic but not the same bits as the default schedule's (another
 * summation order; within the same tolerance of the exact result).
 * On grids of at least 8 query tiles per compute unit (B8 T1500 H32, say)
 * with a table (the caller's or one built in the workspace), the workspace
 * also takes the keys rotated once ahead of the attention kernel (one more
 * launch, B*T*H*64 bf16 after the table), which then stages them without
 * rotating them again; the rotation reads the same cos/sin rows, so the
 * results keep their bits. */
vx_status vx_swa_attn_prefill(const void *q, const void *k, const void *v, void *o, int32_t B,
                              int32_t T, int32_t H, const int64_t *pos0, int32_t rope_applied,
                              const float *rope_table, int64_t table_p0, int64_t table_len,
                              const vx_attn_cfg *cfg, void *stream);

/* Workspace bytes (cfg->workspace_bytes) with which vx_swa_attn_prefill of
 * this shape and cfg->window, given no rope_table, keeps its cos/sin table in
 * the workspace (B*T rows of 256 bytes, row b*T + t for position pos0[b] + t,
 * rounded up to 256) and, where it takes the split walk on the current
 * device (cfg->flags counts), the walk's flag word per (b, h, 128-query tile,
 * wave of 32 queries), rounded up to 256 bytes, and two 9216-byte partial
 * results per flag word; or, where the keys are rotated ahead of the kernel,
 * B*T*H rows of 128 bytes for them.  Returns 0 for invalid arguments. */
size_t vx_swa_attn_prefill_workspace_size(int32_t B, int32_t T, int32_t H,
                                          const vx_attn_cfg *cfg);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as vx_swa_attn_prefill with rope_table == NULL and a workspace (but
 * never the split walk, nor VX_FLAG_SPLIT_WALK), where
 * the cos/sin rows live in a library-owned static device array of 16 MiB
 * (one per GPU, held until the process ends), so the call allocates nothing.
 * cfg->workspace is ignored.  Requires B*T <= 65536 when rope_applied == 0
 * (VX_E_SHAPE otherwise, nothing launched).  Every call on a GPU shares that
 * GPU's array: calls that overlap in time on one GPU (other streams, other
 * host threads) race and must not be made.  Same results, bit for bit, as
 * vx_swa_attn_prefill given a table of the same positions and no
 * workspace. */
vx_status vx_swa_attn_prefill_noalloc(const void *q, const void *k, const void *v, void *o,
                                      int32_t B, int32_t T, int32_t H, const int64_t *pos0,
                                      int32_t rope_applied, const vx_attn_cfg *cfg,
                                      void *stream);

/* Batched first-chunk prefill over streams of different lengths, which can
 * also seed each stream's KV ring for the streaming step (Voxtral Mini 4B
 * Realtime Core AI page, "Why two encoders?" and the Streaming table: the
 * batched first-chunk encoder, one call for the whole first chunk, then the
 * streaming encoder for later chunks).
 * Stream s has T_s = cu_seqlens[s+1] - cu_seqlens[s] frames at positions
 * 0 .. T_s - 1, packed along the frame axis: q, k, v and o are
 * [total, H, D] with stream s at rows cu_seqlens[s] .. cu_seqlens[s+1]-1;
 * each frame attends as in vx_swa_attn_prefill, within its own stream only.
 * total: the number of packed rows (the host size of q, k, v and o).
 * cu_seqlens: device int32 [S+1], cu_seqlens[0] = 0, non-decreasing, with
 *   cu_seqlens[S] = total.  The kernel clamps every offset to [0, total] and
 *   a negative length counts as 0, so a wrong array cannot reach outside
 *   the buffers.
 * max_T: host bound on every T_s.  A stream with T_s > max_T is an error
 *   found on the device: all its output rows are NaN and its ring and pos
 *   are left untouched (loud, never partial).  max_T <= W is the
 *   full-causal case.
 * bf16 input only (VX_E_DTYPE otherwise); o is bf16 or float32.
 * RoPE as in vx_swa_attn_prefill with pos0 = NULL: a given table must
 *   cover positions 0 .. max_T - 1 (VX_E_RANGE otherwise); a NULL table
 *   means cos/sin computed in the kernel.
 * ring_k, ring_v: [S, H, W, D] bf16 rings, or both NULL for no seeding.
 *   When given, the rotated keys and the values of frames
 *   t >= T_s - W are written to slot t mod W of stream s (other slots keep
 *   their contents) and pos[s] (device int64 [S], required) is set to T_s:
 *   the state after appending the whole first chunk, ready for
 *   vx_swa_attn_stream_step at position T_s.  Seeding needs max_T >= 1. */
vx_status vx_swa_attn_prefill_varlen(const void *q, const void *k, const void *v, void *o,
                                     const int32_t *cu_seqlens, int32_t S, int32_t total,
                                     int32_t max_T, int32_t H, int32_t rope_applied, const float *rope_table,
                                     int64_t table_p0, int64_t table_len, void *ring_k,
                                     void *ring_v, int64_t *pos, const vx_attn_cfg *cfg,
                                     void *stream);

/* One streaming step for S independent streams with n new frames each: the
 * encoder's incremental form (transcribe.cpp "Voxtral" family notes,
 * Streaming schedule: each 80 ms step brings 8 mel frames = 4 encoder frames
 * per stream, attending causally within the 750-frame window over state
 * carried from earlier steps; the Core AI port's streaming encoder, "Why two
 * encoders?").  1 <= n <= min(W, 64): a longer increment is the same
 * computation as consecutive steps of at most 64 frames, each followed by
 * its append (the step attends before it appends, so the ring then holds
 * exactly the keys a longer step would read from the new frames).
 * q_new, k_new, v_new, o: [S,n,H,D]; ring_k (rotated keys) and ring_v:
 * [S,H,W,D] in cfg->io_dtype; slot j of a ring holds the frame at absolute
 * position p with p mod W == j.  pos: device int64 [S], the absolute
 * position of the first new frame of each stream (= frames appended so far;
 * a stream starts at 0 with any ring contents, since slots of positions < 0
 * are never read).  A negative pos[s] is an invalid state found on the
 * device: that stream's outputs are NaN (loud, never partial).  New query i
 * of stream s (position P = pos[s] + i) attends to ring frames at positions
 * max(0, P-W+1) .. pos[s]-1 and to new frames pos[s] .. P.  New q and k are
 * rotated here unless rope_applied != 0.  Reads the ring and pos, never
 * writes them: call vx_kv_ring_append afterwards, on the same stream. */
vx_status vx_swa_attn_stream_step(const void *q_new, const void *k_new, const void *v_new,
                                  const void *ring_k, const void *ring_v, const int64_t *pos,
                                  void *o, int32_t S, int32_t n, int32_t H, int32_t rope_applied,
                                  const vx_attn_cfg *cfg, void *stream);

/* Appends n new frames per stream to the W-slot ring that carries the
 * streaming state (the encoder's cache of past rotated keys and values; the
 * Core AI port keeps an append-only buffer instead, "Voxtral Mini 4B
 * Realtime - Core AI", Usage / Known limitations): rotates k_new (unless
 * rope_applied != 0) at positions pos[s] + i, writes it and v_new to slot
 * (pos[s] + i) mod W of ring_k / ring_v, then sets pos[s] += n on the
 * device.  A stream with pos[s] < 0 is left as it is (nothing written, pos
 * kept).  Shapes and dtypes as in vx_swa_attn_stream_step.  Must follow
 * every read of the ring for this step (same stream): the slots it
 * overwrites still hold keys that the step's queries need. */
vx_status vx_kv_ring_append(void *ring_k, void *ring_v, const void *k_new, const void *v_new,
                            int64_t *pos, int32_t S, int32_t n, int32_t H, int32_t rope_applied,
                            const vx_attn_cfg *cfg, void *stream);

/* One streaming step and its ring append in one call (one launch for bf16):
 * the attention of vx_swa_attn_stream_step, then the rotated new keys and the
 * new values are written to slots (pos_in[s] + i) mod W of the rings, and
 * pos_out[s] = pos_in[s] + n (the per-step schedule of transcribe.cpp
 * "Voxtral" family notes, Streaming schedule).  Same shapes and dtypes as
 * the two separate calls, and the same results bit for bit.  Requires
 * 1 <= n <= min(W, 16) (one workgroup per ring, which writes it only after
 * all its reads).  A stream with pos_in[s] < 0 gets NaN outputs, no ring
 * write and pos_out[s] = pos_in[s].  pos_in and pos_out must be distinct
 * arrays: some workgroups still read pos_in while another writes pos_out;
 * swap the two for the next step. */
vx_status vx_swa_attn_stream_step_append(const void *q_new, const void *k_new, const void *v_new,
                                         void *ring_k, void *ring_v, const int64_t *pos_in,
                                         int64_t *pos_out, void *o, int32_t S, int32_t n,
                                         int32_t H, int32_t rope_applied, const vx_attn_cfg *cfg,
                                         void *stream);

/* ---- Grouped-query attention, head_dim 128 ---------------------------------
 * The text decoder of Voxtral Realtime 2602 (transcribe.cpp "Voxtral" family
 * notes, Architecture: 32 query heads over 8 key/value heads, head_dim 128,
 * sliding window 8192, RoPE theta 1e6): the same causal sliding-window
 * attention with RoPE, where query head h reads key/value head h / G,
 * G = Hq / Hkv (each key/value head serves G consecutive query heads).
 * These entry points take cfg->head_dim == 128, bf16 input (VX_E_DTYPE
 * otherwise), a bf16 or float32 output and no flags; RoPE pairs dimension i
 * with i + 64.  q and o have Hq heads, k, v and the rings Hkv heads. */

/* Fills `cfg` with the Voxtral Realtime text-decoder defaults: head_dim 128,
 * window 8192, theta 1e6, scale 1/sqrt(128) (softmax_scale 0), bf16 in and
 * out, no flags. */
void vx_default_gqa_cfg(vx_attn_cfg *cfg);

/* Prompt prefill:
 *   o[b,t,h] = sum_j softmax_j(scale * q'[b,t,h] . k'[b,j,h/G]) v[b,j,h/G],
 *   j = max(0, t-W+1) .. t,
 * q', k' rotated at positions pos0 + t.  q, o: [B,T,Hq,128]; k, v:
 * [B,T,Hkv,128].  Hq must be a multiple of Hkv with G in {1, 2, 4, 8}
 * (VX_E_SHAPE otherwise).  RoPE arguments as in vx_swa_attn_prefill, with a
 * table made by vx_rope_table at head_dim 128.
 * ring_k, ring_v: [B,Hkv,W,128] bf16 rings, or both NULL.  When given
 * (needs pos0 == 0), the rotated keys and the values of frames t >= T - W
 * go to slot t mod W of batch entry b's rings (other slots keep their
 * contents) and pos[b] (device int64 [B], required) is set to T: the state
 * from which vx_gqa_attn_decode continues at position T.
 * k_rot: NULL, or a caller-owned [B,T,Hkv,128] bf16 buffer (rope_applied
 *   must be 0, VX_E_RANGE otherwise; it must not overlap any other tensor).
 *   When given, the call first writes the rotated keys k' there (bf16, the
 *   exact values the attention uses) and then attends over them, so the keys
 *   are rotated once instead of once per query tile: two launches, same
 *   results bit for bit, and faster on long prompts. */
vx_status vx_gqa_attn_prefill(const void *q, const void *k, const void *v, void *o, int32_t B,
                              int32_t T, int32_t Hq, int32_t Hkv, int64_t pos0,
                              int32_t rope_applied, const float *rope_table, int64_t table_p0,
                              int64_t table_len, void *ring_k, void *ring_v, int64_t *pos,
                              void *k_rot, const vx_attn_cfg *cfg, void *stream);

/* One decode step of S independent streams with n new tokens each, and its
 * ring append, in one launch.  q_new, o: [S,n,Hq,128]; k_new, v_new:
 * [S,n,Hkv,128]; ring_k (rotated keys) and ring_v: [S,Hkv,W,128], slot j
 * holding the token at position p with p mod W == j.  pos_in[s] (device
 * int64) is the position of the first new token (= tokens appended so far;
 * a stream starts at 0 with any ring contents).  New token i of stream s
 * (position P = pos_in[s] + i) of query head h attends, on key/value head
 * h/G, to ring tokens at positions max(0, P-W+1) .. pos_in[s]-1 and to new
 * tokens pos_in[s] .. P.  q_new and k_new are rotated here unless
 * rope_applied != 0.  After every read of its ring the call writes the
 * rotated new keys and the new values to slots (pos_in[s] + i) mod W and
 * sets pos_out[s] = pos_in[s] + n; pos_in and pos_out must be distinct
 * arrays (swap them for the next step).  Requires 1 <= n <= W and
 * n * Hq/Hkv <= 16 (one token of a 32/8 decoder uses 4 of the 16 query
 * columns of a workgroup). */
vx_status vx_gqa_attn_decode(const void *q_new, const void *k_new, const void *v_new,
                             void *ring_k, void *ring_v, const int64_t *pos_in, int64_t *pos_out,
                             void *o, int32_t S, int32_t n, int32_t Hq, int32_t Hkv,
                             int32_t rope_applied, const vx_attn_cfg *cfg, void *stream);

/* ---- Projections around the encoder's attention -----------------------------
 * Each Voxtral Realtime 2602 encoder layer projects its normalised hidden
 * state (width d_model = 1280) to q, k, v of 32 heads x 64, k_proj without a
 * bias, applies RoPE to q and k, attends, and projects back to d_model with
 * the output projection (transcribe.cpp "Voxtral" family notes, Architecture,
 * Voxtral Realtime 2602).  The Core AI port fuses the q/k/v projections into
 * one matrix product ([Core AI] "Voxtral Mini 4B Realtime - Core AI",
 * artifact manifest: fused QKV).  Weights are bf16 [out, in] row-major (the
 * layout of a linear layer's weight), activations bf16 row-major, fp32
 * accumulation on matrix cores. */

/* y = x w^T (+ bias): x [M, K], w [N, K], bias [N] or NULL, all bf16;
 * y [M, N] in out_dtype (VX_BF16 or VX_F32).  K must be a multiple of 128 and
 * N of 32 (VX_E_SHAPE otherwise); M == 0 is a no-op. */
vx_status vx_linear(const void *x, const void *w, const void *bias, void *y, int32_t M,
                    int32_t N, int32_t K, int32_t out_dtype, void *stream);

/* Fused q/k/v projection with RoPE for S streams of n new frames:
 * x [S, n, d_model]; w_qkv [3*H*64, d_model] holds the q rows, then k, then
 * v; b_q, b_v [H*64] or NULL (k has no bias).  Writes q' = rope(x Wq^T + b_q),
 * k' = rope(x Wk^T) and v = x Wv^T + b_v as [S, n, H, 64] bf16 (rounded once
 * after the rotation), frame i of stream s rotated at position pos[s] + i
 * (pos: device int64 [S]).  Only cfg->rope_theta and cfg->io_dtype (bf16)
 * are used.  d_model and H*64 must be multiples of 128. */
vx_status vx_enc_qkv_rope(const void *x, const void *w_qkv, const void *b_q, const void *b_v,
                          const int64_t *pos, int32_t S, int32_t n, int32_t H, int32_t d_model,
                          void *q, void *k, void *v, const vx_attn_cfg *cfg, void *stream);

/* One streaming step of the encoder's attention block, three launches on
 * `stream`: vx_enc_qkv_rope at positions pos_in, the fused streaming step and
 * ring append of vx_swa_attn_stream_step_append over the rotated q', k' (with
 * pos_out[s] = pos_in[s] + n), and y = o W_o^T + b_o (w_o [d_model, H*64],
 * b_o [d_model] or NULL).  q, k, v, o: caller-owned [S, n, H, 64] bf16 work
 * buffers; y [S, n, d_model] in cfg->out_dtype.  Requires 1 <= n <=
 * min(W, 16), bf16, H*64 and d_model multiples of 128; no buffer the call
 * writes may overlap another argument. */
vx_status vx_enc_attn_step(const void *x, const void *w_qkv, const void *b_q, const void *b_v,
                           const void *w_o, const void *b_o, void *ring_k, void *ring_v,
                           const int64_t *pos_in, int64_t *pos_out, void *q, void *k, void *v,
                           void *o, void *y, int32_t S, int32_t n, int32_t H, int32_t d_model,
                           const vx_attn_cfg *cfg, void *stream);

/* ---- The streaming encoder step ---------------------------------------------
 * One step of the Voxtral Realtime 2602 audio encoder turns 2n new log-mel
 * frames (n_mels = 128 bins) of each of S streams into n encoder frames of
 * width d_model (transcribe.cpp "Voxtral" family notes, Architecture and
 * Streaming schedule: 8 mel frames -> 4 encoder frames per 80 ms token):
 *   - a stem of two causal convolutions with kernel 3, each followed by GELU
 *     (exact erf form): n_mels -> d_model at stride 1, then d_model ->
 *     d_model at stride 2.  Causal means left padding of k-1 = 2 frames,
 *     which in a stream are the previous step's last two input frames of
 *     each convolution (zeros at the start of a stream);
 *   - L pre-norm layers, each  x += attn(rmsnorm(x) * g_attn)  and then
 *     x += W_down (silu(h W_gate^T) * (h W_up^T)) + b_down  with
 *     h = rmsnorm(x) * g_ffn; the attention is vx_enc_attn_step's block
 *     (q/k/v + RoPE, the windowed attention over each layer's ring with the
 *     append, the output projection).
 * RMSNorm: x / sqrt(mean(x^2) + eps), eps = 1e-5 in this model.  The
 * residual stream x is float32 ([S, n, d_model]); every other tensor stored
 * between launches (normalised states, q', k', v, attention output, SwiGLU
 * hidden state, conv1 output) is bf16, accumulation fp32 on matrix cores.
 * Weights are bf16; convolution weights are [out, tap, in] (tap 2 multiplies
 * the newest frame).  ffn (5120 in this model), d_model (1280), n_mels and
 * H*64 must be multiples of 128. */

typedef struct {
  const void *w1; /* [d_model, 3, n_mels] */
  const void *b1; /* [d_model] or NULL */
  const void *w2; /* [d_model, 3, d_model] */
  const void *b2; /* [d_model] or NULL */
} vx_enc_stem_weights;

typedef struct {
  const void *g_attn; /* [d_model] RMSNorm gain in front of the attention */
  const void *w_qkv;  /* [3*H*64, d_model]: the q rows, then k, then v */
  const void *b_q;    /* [H*64] or NULL (k has no bias) */
  const void *b_v;    /* [H*64] or NULL */
  const void *w_o;    /* [d_model, H*64] */
  const void *b_o;    /* [d_model] or NULL */
  const void *g_ffn;  /* [d_model] RMSNorm gain in front of the feed-forward */
  const void *w_gate; /* [ffn, d_model] */
  const void *w_up;   /* [ffn, d_model] */
  const void *w_down; /* [d_model, ffn] */
  const void *b_down; /* [d_model] or NULL */
} vx_enc_layer_weights;

/* Caller-owned work buffers of a layer step (reused by every layer). */
typedef struct {
  void *h;   /* [S*n, d_model] bf16 normalised state */
  void *q;   /* [S*n, H*64] bf16 rotated queries */
  void *k;   /* [S*n, H*64] bf16 rotated keys */
  void *v;   /* [S*n, H*64] bf16 values */
  void *o;   /* [S*n, H*64] bf16 attention output */
  void *u;   /* [S*n, ffn] bf16 SwiGLU hidden state */
  void *acc; /* [2, S*n, d_model] float32 partial sums of the projections
                added into the residual (K split in two parts) */
} vx_enc_work;

/* y = x / sqrt(mean(x^2) + eps) * g per row: x float32 [M, dim], g bf16
 * [dim], y bf16 [M, dim] (fp32 arithmetic, y rounded once).  dim must be a
 * multiple of 8, eps finite and >= 0; y must not overlap x or g. */
vx_status vx_rmsnorm(const float *x, const void *g, void *y, int32_t M, int32_t dim, float eps,
                     void *stream);

/* The stem for one step, three launches on `stream`.
 * mel_buf [S, 2n+2, n_mels] bf16: slots 0-1 hold the stream's two previous
 * mel frames (zeros at its start), slots 2 .. 2n+1 this step's 2n frames,
 * written by the caller.  c1_buf [S, 2n+2, d_model] bf16: slots 0-1 hold
 * the first convolution's two previous output frames (zeros at the start);
 * the call writes this step's outputs to slots 2 .. 2n+1.  x_out [S, n,
 * d_model] float32 receives the n new frames.  On return slots 0-1 of both
 * buffers hold slots 2n and 2n+1 (the state for the next step).  Buffers
 * the call writes must not overlap any other argument; each buffer and w2
 * must be smaller than 2^30 bytes. */
vx_status vx_enc_stem_step(void *mel_buf, void *c1_buf, const vx_enc_stem_weights *w,
                           float *x_out, int32_t S, int32_t n, int32_t n_mels, int32_t d_model,
                           void *stream);

/* One pre-norm layer for one step, eight launches on `stream`, updating the
 * residual x [S, n, d_model] float32 in place.  The output and down
 * projections each run as two K halves whose fp32 sums a row-wise reduction
 * adds, in order, with the bias into x; the reduction after the output
 * projection also writes the FFN's normalised state.  ring_k, ring_v [S, H, W, 64]
 * bf16 rotated keys and values of this layer; frame i of stream s is at
 * position pos_in[s] + i; the call appends the new keys and values and sets
 * pos_out[s] = pos_in[s] + n (distinct arrays).  Requires 1 <= n <=
 * min(W, 16), cfg->io_dtype bf16, cfg->head_dim 64, no flags; cfg->window,
 * rope_theta and softmax_scale apply.  No written buffer (x, rings, work,
 * pos_out) may overlap another argument. */
vx_status vx_enc_layer_step(float *x, const vx_enc_layer_weights *w, void *ring_k, void *ring_v,
                            const int64_t *pos_in, int64_t *pos_out, const vx_enc_work *work,
                            int32_t S, int32_t n, int32_t H, int32_t d_model, int32_t ffn,
                            float eps, const vx_attn_cfg *cfg, void *stream);

/* A whole encoder step: vx_enc_stem_step into x, then layers[0 .. L-1] in
 * order as vx_enc_layer_step, layer l on rings ring_k + l*S*H*W*64 (ring_k,
 * ring_v [L, S, H, W, 64] bf16); all layers read positions pos_in and write
 * pos_out.  The last reduction of layer l also writes layer l+1's normalised
 * input, so the result equals the calls made one by one, bit for bit, in
 * 3 + 1 + 7L launches on `stream`; 1 <= L <= 4096, d_model <= 4096.  Same
 * buffer rules as the two calls above. */
vx_status vx_enc_step(void *mel_buf, void *c1_buf, const vx_enc_stem_weights *stem,
                      const vx_enc_layer_weights *layers, int32_t L, void *ring_k, void *ring_v,
                      const int64_t *pos_in, int64_t *pos_out, float *x, const vx_enc_work *work,
                      int32_t S, int32_t n, int32_t n_mels, int32_t H, int32_t d_model,
                      int32_t ffn, float eps, const vx_attn_cfg *cfg, void *stream);

/* Static description of a status code. */
const char *vx_status_string(vx_status s);

/* Message for the last non-OK status returned on the calling thread
 * ("" if none).  Valid until the next vx_* call on this thread. */
const char *vx_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t vx_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VX_H */
