// C ABI of the vx library: argument validation on the host, then kernel
// selection and launch on the caller's stream.  Nothing here allocates,
// synchronises or keeps state between calls (apart from the thread-local
// text of the last error).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <string>
#include <vector>

#include "enc_launch.h"
#include "gqa_launch.h"
#include "linear_launch.h"
#include "vx.h"
#include "vx_launch.h"

namespace {

thread_local std::string g_err;

vx_status fail(vx_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

vx_status ok() {
  g_err.clear();
  return VX_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Largest sizes accepted: every offset fits comfortably in 64-bit, and every
// launch stays below 2^32 work-items (at most 4 work-items per frame row of
// one head in the prefill and rotation kernels).
constexpr int64_t kMaxElems = (int64_t)1 << 40;
constexpr int32_t kMaxDim = 1 << 24;
constexpr int64_t kMaxRows = (int64_t)1 << 30;  // B*T*H for prefill and rotation

vx::DT to_dt(int32_t d) { return d == VX_BF16 ? vx::DT::BF16 : vx::DT::F32; }
size_t elem_size(int32_t d) { return d == VX_BF16 ? 2 : 4; }

vx_status check_cfg(const vx_attn_cfg* cfg) {
  if (!cfg) return fail(VX_E_NULL, "cfg is NULL");
  if (cfg->head_dim != vx::kD) return fail(VX_E_SHAPE, "head_dim must be 64 (got %d)", cfg->head_dim);
  if (cfg->window < 1) return fail(VX_E_RANGE, "window must be >= 1 (got %d)", cfg->window);
  if (!(cfg->rope_theta > 0.0) || !isfinite(cfg->rope_theta))
    return fail(VX_E_RANGE, "rope_theta must be finite and > 0");
  if (!(cfg->softmax_scale >= 0.0f) || !isfinite(cfg->softmax_scale))
    return fail(VX_E_RANGE, "softmax_scale must be finite and >= 0");
  const int32_t io = cfg->io_dtype, out = cfg->out_dtype;
  if ((io != VX_F32 && io != VX_BF16) || (out != VX_F32 && out != VX_BF16))
    return fail(VX_E_DTYPE, "unknown dtype (io %d, out %d)", io, out);
  if (io == VX_F32 && out == VX_BF16)
    return fail(VX_E_DTYPE, "float32 inputs with bfloat16 output is not supported");
  if (cfg->flags & ~(VX_FLAG_VALU_KERNEL | VX_FLAG_SPLIT_WALK))
    return fail(VX_E_RANGE, "unknown flag bits 0x%x", cfg->flags);
  if (cfg->workspace_bytes > 0 && !cfg->workspace)
    return fail(VX_E_NULL, "workspace is NULL but workspace_bytes is %zu", cfg->workspace_bytes);
  if (cfg->workspace && !aligned16(cfg->workspace))
    return fail(VX_E_ALIGN, "workspace is not 16-byte aligned");
  return VX_OK;
}

vx::RopeFreqs rope_freqs(double theta) {
  vx::RopeFreqs f;
  for (int i = 0; i < vx::kHalf; ++i) f.f[i] = pow(theta, -2.0 * i / (double)vx::kD);
  return f;
}

float scale_log2(const vx_attn_cfg* cfg) {
  const double s = cfg->softmax_scale > 0.0f ? (double)cfg->softmax_scale
                                             : 1.0 / sqrt((double)cfg->head_dim);
  return (float)(s * 1.4426950408889634073599);  // log2(e)
}

// Grouped-query entry points: head_dim 128, bf16 input, no flags.
vx_status check_gqa_cfg(const char* what, const vx_attn_cfg* cfg) {
  if (!cfg) return fail(VX_E_NULL, "%s: cfg is NULL", what);
  if (cfg->head_dim != vx::kGD)
    return fail(VX_E_SHAPE, "%s: head_dim must be 128 (got %d)", what, cfg->head_dim);
  if (cfg->window < 1) return fail(VX_E_RANGE, "%s: window must be >= 1 (got %d)", what, cfg->window);
  if (!(cfg->rope_theta > 0.0) || !isfinite(cfg->rope_theta))
    return fail(VX_E_RANGE, "%s: rope_theta must be finite and > 0", what);
  if (!(cfg->softmax_scale >= 0.0f) || !isfinite(cfg->softmax_scale))
    return fail(VX_E_RANGE, "%s: softmax_scale must be finite and >= 0", what);
  if (cfg->io_dtype != VX_BF16) return fail(VX_E_DTYPE, "%s: only bf16 input is supported", what);
  if (cfg->out_dtype != VX_BF16 && cfg->out_dtype != VX_F32)
    return fail(VX_E_DTYPE, "%s: unknown output dtype %d", what, cfg->out_dtype);
  if (cfg->flags != 0) return fail(VX_E_RANGE, "%s: no flags are defined (got 0x%x)", what, cfg->flags);
  return VX_OK;
}

vx::RopeFreqs128 rope_freqs128(double theta) {
  vx::RopeFreqs128 f;
  for (int i = 0; i < vx::kGHalf; ++i) f.f[i] = pow(theta, -2.0 * i / (double)vx::kGD);
  return f;
}

vx_status check_heads(const char* what, int32_t Hq, int32_t Hkv) {
  if (Hq < 1 || Hkv < 1) return fail(VX_E_SHAPE, "%s: Hq and Hkv must be >= 1", what);
  if (Hq > 65535) return fail(VX_E_SHAPE, "%s: Hq must be <= 65535", what);
  if (Hq % Hkv != 0)
    return fail(VX_E_SHAPE, "%s: Hq (%d) must be a multiple of Hkv (%d)", what, Hq, Hkv);
  return VX_OK;
}

vx_status check_dims(const char* what, int64_t a, int64_t b, int64_t c) {
  if (a < 0 || b < 0 || c < 0) return fail(VX_E_SHAPE, "%s: negative size", what);
  if (a > kMaxDim || b > kMaxDim || c > kMaxDim) return fail(VX_E_SHAPE, "%s: size too large", what);
  if (a * b * c * vx::kD > kMaxElems) return fail(VX_E_SHAPE, "%s: tensor too large", what);
  return VX_OK;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

vx_status launched(hipError_t e) {
  if (e != hipSuccess) return fail(VX_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

// ---- Library-owned scratch for vx_swa_attn_prefill_noalloc -----------------
// A file-scope device array: every GPU the library runs on holds its own copy
// until the process ends.  Host code never uses the array's name as an
// address (in host code it is a stand-in, not device memory); it uses the
// address hipGetSymbolAddress returns, looked up once per device with that
// device current and kept per device.
constexpr size_t kNoAllocBytes = (size_t)16 << 20;  // 65536 cos/sin rows of 256 bytes
static __device__ __align__(256) char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of this device's `scratch`, or NULL with *err set.
void* scratch_address(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

void vx_default_cfg(vx_attn_cfg* cfg) {
  if (!cfg) return;
  cfg->head_dim = 64;
  cfg->window = 750;
  cfg->rope_theta = 1e6;
  cfg->softmax_scale = 0.125f;
  cfg->io_dtype = VX_BF16;
  cfg->out_dtype = VX_BF16;
  cfg->flags = 0;
  cfg->workspace = nullptr;
  cfg->workspace_bytes = 0;
}

void vx_default_gqa_cfg(vx_attn_cfg* cfg) {
  if (!cfg) return;
  cfg->head_dim = 128;
  cfg->window = 8192;
  cfg->rope_theta = 1e6;
  cfg->softmax_scale = 0.0f;  // 1/sqrt(128)
  cfg->io_dtype = VX_BF16;
  cfg->out_dtype = VX_BF16;
  cfg->flags = 0;
  cfg->workspace = nullptr;
  cfg->workspace_bytes = 0;
}

vx_status vx_rope_table(float* table, int64_t p_begin, int32_t count, const vx_attn_cfg* cfg,
                        void* stream) {
  if (!cfg) return fail(VX_E_NULL, "cfg is NULL");
  if (cfg->head_dim != vx::kD && cfg->head_dim != vx::kGD)
    return fail(VX_E_SHAPE, "head_dim must be 64 or 128 (got %d)", cfg->head_dim);
  if (!(cfg->rope_theta > 0.0) || !isfinite(cfg->rope_theta))
    return fail(VX_E_RANGE, "rope_theta must be finite and > 0");
  if (count < 0 || count > kMaxDim) return fail(VX_E_SHAPE, "count out of range (%d)", count);
  if (p_begin < 0 || p_begin > ((int64_t)1 << 52)) return fail(VX_E_RANGE, "p_begin out of range");
  if (count == 0) return ok();
  if (!table) return fail(VX_E_NULL, "table is NULL");
  if (!aligned16(table)) return fail(VX_E_ALIGN, "table is not 16-byte aligned");
  (void)hipGetLastError();
  if (cfg->head_dim == vx::kGD)
    return launched(vx::launch_gqa_rope_table(table, p_begin, count,
                                              rope_freqs128(cfg->rope_theta), (hipStream_t)stream));
  return launched(vx::launch_rope_table(table, p_begin, count, rope_freqs(cfg->rope_theta),
                                        (hipStream_t)stream));
}

vx_status vx_rope_qk(void* q, void* k, int32_t B, int32_t T, int32_t H, const int64_t* pos0,
                     const vx_attn_cfg* cfg, void* stream) {
  vx_status st = check_cfg(cfg);
  if (st) return st;
  if ((st = check_dims("rope_qk", B, T, H))) return st;
  if (pos0 && ((uintptr_t)pos0 & 7u) != 0) return fail(VX_E_ALIGN, "pos0 is not 8-byte aligned");
  if ((int64_t)B * T == 0) return ok();
  if (H < 1) return fail(VX_E_SHAPE, "H must be >= 1");
  if ((int64_t)B * T * H > kMaxRows) return fail(VX_E_SHAPE, "B*T*H too large");
  if (!q && !k) return fail(VX_E_NULL, "q and k are both NULL");
  if ((q && !aligned16(q)) || (k && !aligned16(k))) return fail(VX_E_ALIGN, "q/k not 16-byte aligned");
  const size_t bytes = (size_t)B * T * H * vx::kD * elem_size(cfg->io_dtype);
  if (q && k && overlap(q, bytes, k, bytes)) return fail(VX_E_RANGE, "q and k overlap");
  (void)hipGetLastError();
  return launched(vx::launch_rope_qk(q, k, B, T, H, pos0, to_dt(cfg->io_dtype),
                                     rope_freqs(cfg->rope_theta), (hipStream_t)stream));
}

// Bytes of the cos/sin table the prefill builds in the workspace: B*T rows.
size_t prefill_table_bytes(int32_t B, int32_t T) {
  return (size_t)B * T * vx::kD * sizeof(float);
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

}  // extern "C"

namespace {

// vx_swa_attn_prefill; allow_split = false keeps the unsplit walk whatever
// the workspace holds (the allocation-free entry point's bits).
vx_status prefill_impl(const void* q, const void* k, const void* v, void* o, int32_t B,
                       int32_t T, int32_t H, const int64_t* pos0, int32_t rope_applied,
                       const float* rope_table, int64_t table_p0, int64_t table_len,
                       const vx_attn_cfg* cfg, void* stream, bool allow_split) {
  vx_status st = check_cfg(cfg);
  if (st) return st;
  if ((st = check_dims("prefill", B, T, H))) return st;
  if (pos0 && ((uintptr_t)pos0 & 7u) != 0) return fail(VX_E_ALIGN, "pos0 is not 8-byte aligned");
  if ((int64_t)B * T == 0) return ok();
  if (H < 1) return fail(VX_E_SHAPE, "H must be >= 1");
  if (B > 65535 || H > 65535) return fail(VX_E_SHAPE, "B and H must be <= 65535");
  if ((int64_t)B * T * H > kMaxRows) return fail(VX_E_SHAPE, "B*T*H too large");
  if (!q || !k || !v || !o) return fail(VX_E_NULL, "q, k, v and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(VX_E_ALIGN, "q, k, v and o must be 16-byte aligned");
  const size_t n = (size_t)B * T * H * vx::kD;
  const size_t ib = n * elem_size(cfg->io_dtype), ob = n * elem_size(cfg->out_dtype);
  if (overlap(o, ob, q, ib) || overlap(o, ob, k, ib) || overlap(o, ob, v, ib))
    return fail(VX_E_RANGE, "o overlaps an input");
  if (cfg->workspace &&
      (overlap(cfg->workspace, cfg->workspace_bytes, o, ob) ||
       overlap(cfg->workspace, cfg->workspace_bytes, q, ib) ||
       overlap(cfg->workspace, cfg->workspace_bytes, k, ib) ||
       overlap(cfg->workspace, cfg->workspace_bytes, v, ib)))
    return fail(VX_E_RANGE, "the workspace overlaps a tensor");
  vx::PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.B = B;
  a.T = T;
  a.H = H;
  a.W = cfg->window;
  a.pos0 = pos0;
  a.rope = rope_applied == 0;
  a.scale_log2 = scale_log2(cfg);
  a.fr = rope_freqs(cfg->rope_theta);
  const bool valu = (cfg->flags & VX_FLAG_VALU_KERNEL) || cfg->io_dtype == VX_F32;
  bool build_table = false;
  if (a.rope) {
    if (rope_table) {
      if (!aligned16(rope_table)) return fail(VX_E_ALIGN, "rope_table is not 16-byte aligned");
      if (table_p0 < 0 || table_len < 0) return fail(VX_E_RANGE, "table_p0 and table_len must be >= 0");
      if (!pos0 && (table_p0 > 0 || table_len < T))
        return fail(VX_E_RANGE,
                    "rope_table covers positions [%lld, %lld) but the chunk needs [0, %d)",
                    (long long)table_p0, (long long)(table_p0 + table_len), T);
      a.table = rope_table;
      a.table_off = -table_p0;
      a.table_len = table_len;
    } else if (cfg->workspace && cfg->workspace_bytes >= prefill_table_bytes(B, T)) {
      // a table of exactly the call's positions, row b*T + t, in the workspace
      build_table = true;
      a.table = (const float*)cfg->workspace;
      a.table_bstride = T;
      a.table_pos = false;
      a.table_len = (int64_t)B * T;
    }  // else: cos/sin computed in the kernel
  }
  // After the table if one is built there: the split walk's flags and
  // partial results (small grids, with a table or pre-rotated inputs), or
  // the keys rotated ahead of the kernel (large grids with a table); the two
  // never apply to the same grid.
  const size_t ws_off = build_table ? align256(prefill_table_bytes(B, T)) : 0;
  void* k_rot = nullptr;
  if (!valu && cfg->workspace && a.rope && a.table) {
    const size_t kb = vx::prefill_krot_bytes(B, T, H);
    if (kb && cfg->workspace_bytes >= ws_off + kb) k_rot = (char*)cfg->workspace + ws_off;
  }
  if (allow_split && !valu && cfg->workspace && (!a.rope || a.table)) {
    const size_t off = ws_off;
    size_t fb = 0;
    const size_t sb = vx::prefill_split_bytes(B, T, H, cfg->window,
                                              (cfg->flags & VX_FLAG_SPLIT_WALK) != 0, &fb);
    if (sb && cfg->workspace_bytes >= off + sb) {
      a.split_flags = (unsigned long long*)((char*)cfg->workspace + off);
      a.split_part = (float*)((char*)cfg->workspace + off + fb);
    }
  }
  (void)hipGetLastError();
  if (build_table) {
    vx_status s1 = launched(vx::launch_rope_table_batched((float*)a.table, pos0, B, T, a.fr,
                                                          (hipStream_t)stream));
    if (s1) return s1;
  }
  if (valu)
    return launched(vx::launch_prefill_valu(a, to_dt(cfg->io_dtype), to_dt(cfg->out_dtype),
                                            (hipStream_t)stream));
  a.half_split = vx::prefill_half_split(B, T, H);
  if (k_rot) {
    vx_status s2 = launched(vx::launch_rope_k_table(a, k_rot, (hipStream_t)stream));
    if (s2) return s2;
    a.k = k_rot;
    a.k_rotated = true;
  }
  return launched(vx::launch_prefill_mfma(a, to_dt(cfg->out_dtype), (hipStream_t)stream));
}

}  // namespace

extern "C" {

vx_status vx_swa_attn_prefill(const void* q, const void* k, const void* v, void* o, int32_t B,
                              int32_t T, int32_t H, const int64_t* pos0, int32_t rope_applied,
                              const float* rope_table, int64_t table_p0, int64_t table_len,
                              const vx_attn_cfg* cfg, void* stream) {
  return prefill_impl(q, k, v, o, B, T, H, pos0, rope_applied, rope_table, table_p0, table_len,
                      cfg, stream, true);
}

size_t vx_swa_attn_prefill_workspace_size(int32_t B, int32_t T, int32_t H,
                                          const vx_attn_cfg* cfg) {
  if (check_cfg(cfg) != VX_OK || check_dims("prefill", B, T, H) != VX_OK) return 0;
  return align256(prefill_table_bytes(B, T)) +
         vx::prefill_split_bytes(B, T, H, cfg->window, (cfg->flags & VX_FLAG_SPLIT_WALK) != 0,
                                 nullptr) +
         vx::prefill_krot_bytes(B, T, H);
}

vx_status vx_swa_attn_prefill_noalloc(const void* q, const void* k, const void* v, void* o,
                                      int32_t B, int32_t T, int32_t H, const int64_t* pos0,
                                      int32_t rope_applied, const vx_attn_cfg* cfg,
                                      void* stream) {
  vx_status st = check_cfg(cfg);
  if (st) return st;
  if ((st = check_dims("prefill_noalloc", B, T, H))) return st;
  if (rope_applied == 0 && prefill_table_bytes(B, T) > kNoAllocBytes)
    return fail(VX_E_SHAPE,
                "prefill_noalloc: B*T = %lld rows exceed the library scratch (%zu rows); "
                "use vx_swa_attn_prefill with a workspace or a table",
                (long long)B * T, kNoAllocBytes / (vx::kD * sizeof(float)));
  if ((int64_t)B * T == 0) return ok();
  vx_attn_cfg c = *cfg;
  c.workspace = nullptr;
  c.workspace_bytes = 0;
  if (rope_applied == 0) {
    hipError_t e = hipSuccess;
    void* p = scratch_address(&e);
    if (!p) return fail(VX_E_HIP, "prefill_noalloc: no scratch address: %s", hipGetErrorString(e));
    c.workspace = p;
    c.workspace_bytes = kNoAllocBytes;
  }
  return prefill_impl(q, k, v, o, B, T, H, pos0, rope_applied, nullptr, 0, 0, &c, stream, false);
}

vx_status vx_swa_attn_prefill_varlen(const void* q, const void* k, const void* v, void* o,
                                     const int32_t* cu_seqlens, int32_t S, int32_t total,
                                     int32_t max_T, int32_t H, int32_t rope_applied,
                                     const float* rope_table,
                                     int64_t table_p0, int64_t table_len, void* ring_k,
                                     void* ring_v, int64_t* pos, const vx_attn_cfg* cfg,
                                     void* stream) {
  vx_status st = check_cfg(cfg);
  if (st) return st;
  if ((st = check_dims("prefill_varlen", S, max_T, H))) return st;
  if (total < 0 || (int64_t)total > (int64_t)S * max_T)
    return fail(VX_E_SHAPE, "prefill_varlen: total must be in [0, S*max_T]");
  if (cfg->io_dtype != VX_BF16)
    return fail(VX_E_DTYPE, "prefill_varlen: only bf16 input is supported");
  const bool seed = ring_k || ring_v;
  if (S == 0 || ((max_T == 0 || total == 0) && !seed)) return ok();
  if (seed && max_T == 0) return fail(VX_E_SHAPE, "prefill_varlen: seeding needs max_T >= 1");
  if (H < 1) return fail(VX_E_SHAPE, "H must be >= 1");
  if (S > 65535 || H > 65535) return fail(VX_E_SHAPE, "S and H must be <= 65535");
  if ((int64_t)S * max_T * H > kMaxRows) return fail(VX_E_SHAPE, "S*max_T*H too large");
  if (!q || !k || !v || !o || !cu_seqlens)
    return fail(VX_E_NULL, "q, k, v, o and cu_seqlens must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(VX_E_ALIGN, "q, k, v and o must be 16-byte aligned");
  if (((uintptr_t)cu_seqlens & 3u) != 0) return fail(VX_E_ALIGN, "cu_seqlens is not 4-byte aligned");
  const size_t n = (size_t)total * H * vx::kD;
  const size_t ib = n * elem_size(cfg->io_dtype), ob = n * elem_size(cfg->out_dtype);
  if (overlap(o, ob, q, ib) || overlap(o, ob, k, ib) || overlap(o, ob, v, ib))
    return fail(VX_E_RANGE, "o overlaps an input");
  if (seed) {
    if (!ring_k || !ring_v || !pos)
      return fail(VX_E_NULL, "ring seeding needs ring_k, ring_v and pos");
    if (!aligned16(ring_k) || !aligned16(ring_v))
      return fail(VX_E_ALIGN, "ring_k and ring_v must be 16-byte aligned");
    if (((uintptr_t)pos & 7u) != 0) return fail(VX_E_ALIGN, "pos is not 8-byte aligned");
    if ((int64_t)S * H * cfg->window * vx::kD > kMaxElems)
      return fail(VX_E_SHAPE, "prefill_varlen: ring too large");
    const size_t rb = (size_t)S * H * cfg->window * vx::kD * elem_size(cfg->io_dtype);
    if (overlap(ring_k, rb, ring_v, rb)) return fail(VX_E_RANGE, "ring_k and ring_v overlap");
    if (overlap(o, ob, ring_k, rb) || overlap(o, ob, ring_v, rb))
      return fail(VX_E_RANGE, "o overlaps a ring");
  }
  vx::PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.B = S;
  a.T = max_T;
  a.H = H;
  a.W = cfg->window;
  a.rope = rope_applied == 0;
  a.scale_log2 = scale_log2(cfg);
  a.fr = rope_freqs(cfg->rope_theta);
  a.cu = cu_seqlens;
  a.total = total;
  if (seed) {
    a.ring_k = ring_k;
    a.ring_v = ring_v;
    a.pos_out = pos;
  }
  if (a.rope && rope_table) {  // without a table: cos/sin computed in the kernel
    if (!aligned16(rope_table)) return fail(VX_E_ALIGN, "rope_table is not 16-byte aligned");
    if (table_p0 < 0 || table_len < 0 || table_p0 > 0 || max_T > table_p0 + table_len)
      return fail(VX_E_RANGE,
                  "rope_table covers positions [%lld, %lld) but the chunks need [0, %d)",
                  (long long)table_p0, (long long)(table_p0 + table_len), max_T);
    a.table = rope_table;
    a.table_off = -table_p0;
    a.table_len = table_len;
  }
  (void)hipGetLastError();
  return launched(vx::launch_prefill_mfma(a, to_dt(cfg->out_dtype), (hipStream_t)stream));
}

static vx_status check_stream_common(const char* what, int32_t S, int32_t n, int32_t H,
                                     const vx_attn_cfg* cfg) {
  vx_status st = check_cfg(cfg);
  if (st) return st;
  if ((st = check_dims(what, S, n, H))) return st;
  if (n < 1 || n > cfg->window)
    return fail(VX_E_RANGE, "%s: need 1 <= n <= window (n %d, window %d)", what, n, cfg->window);
  if (n > vx::kStreamMaxNew)
    return fail(VX_E_RANGE, "%s: at most %d new frames per step (got %d)", what,
                vx::kStreamMaxNew, n);
  if (H < 1) return fail(VX_E_SHAPE, "%s: H must be >= 1", what);
  if ((int64_t)S * H * ((n + 3) / 4) * 256 >= ((int64_t)1 << 32))
    return fail(VX_E_SHAPE, "%s: S*H*n too large", what);
  if ((int64_t)S * H * cfg->window * vx::kD > kMaxElems) return fail(VX_E_SHAPE, "%s: ring too large", what);
  return VX_OK;
}

vx_status vx_swa_attn_stream_step(const void* q_new, const void* k_new, const void* v_new,
                                  const void* ring_k, const void* ring_v, const int64_t* pos,
                                  void* o, int32_t S, int32_t n, int32_t H, int32_t rope_applied,
                                  const vx_attn_cfg* cfg, void* stream) {
  vx_status st = check_stream_common("stream_step", S, n, H, cfg);
  if (st) return st;
  if (S == 0) return ok();
  if (!q_new || !k_new || !v_new || !ring_k || !ring_v || !pos || !o)
    return fail(VX_E_NULL, "stream_step: a tensor pointer is NULL");
  if (!aligned16(q_new) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(ring_k) ||
      !aligned16(ring_v) || !aligned16(o))
    return fail(VX_E_ALIGN, "stream_step: tensors must be 16-byte aligned");
  if (((uintptr_t)pos & 7u) != 0) return fail(VX_E_ALIGN, "stream_step: pos must be 8-byte aligned");
  const size_t nf = (size_t)S * n * H * vx::kD;
  const size_t ob = nf * elem_size(cfg->out_dtype), ib = nf * elem_size(cfg->io_dtype);
  const size_t rb = (size_t)S * H * cfg->window * vx::kD * elem_size(cfg->io_dtype);
  if (overlap(o, ob, q_new, ib) || overlap(o, ob, k_new, ib) || overlap(o, ob, v_new, ib) ||
      overlap(o, ob, ring_k, rb) || overlap(o, ob, ring_v, rb))
    return fail(VX_E_RANGE, "stream_step: o overlaps an input");
  vx::StreamArgs a{};
  a.q = q_new;
  a.k = k_new;
  a.v = v_new;
  a.ring_k = ring_k;
  a.ring_v = ring_v;
  a.pos = pos;
  a.o = o;
  a.S = S;
  a.n = n;
  a.H = H;
  a.W = cfg->window;
  a.rope = rope_applied == 0;
  a.scale_log2 = scale_log2(cfg);
  (void)hipGetLastError();
  return launched(vx::launch_stream_step(a, to_dt(cfg->io_dtype), to_dt(cfg->out_dtype),
                                         rope_freqs(cfg->rope_theta), (hipStream_t)stream));
}

vx_status vx_kv_ring_append(void* ring_k, void* ring_v, const void* k_new, const void* v_new,
                            int64_t* pos, int32_t S, int32_t n, int32_t H, int32_t rope_applied,
                            const vx_attn_cfg* cfg, void* stream) {
  vx_status st = check_stream_common("ring_append", S, n, H, cfg);
  if (st) return st;
  if (S == 0) return ok();
  if (!ring_k || !ring_v || !k_new || !v_new || !pos)
    return fail(VX_E_NULL, "ring_append: a tensor pointer is NULL");
  if (!aligned16(ring_k) || !aligned16(ring_v) || !aligned16(k_new) || !aligned16(v_new))
    return fail(VX_E_ALIGN, "ring_append: tensors must be 16-byte aligned");
  if (((uintptr_t)pos & 7u) != 0) return fail(VX_E_ALIGN, "ring_append: pos must be 8-byte aligned");
  const size_t rb = (size_t)S * H * cfg->window * vx::kD * elem_size(cfg->io_dtype);
  if (overlap(ring_k, rb, ring_v, rb)) return fail(VX_E_RANGE, "ring_append: ring_k and ring_v overlap");
  vx::AppendArgs a{};
  a.ring_k = ring_k;
  a.ring_v = ring_v;
  a.k = k_new;
  a.v = v_new;
  a.pos = pos;
  a.pos_out = pos;
  a.S = S;
  a.n = n;
  a.H = H;
  a.W = cfg->window;
  a.rope = rope_applied == 0;
  (void)hipGetLastError();
  return launched(vx::launch_ring_append(a, to_dt(cfg->io_dtype), rope_freqs(cfg->rope_theta),
                                         (hipStream_t)stream));
}

vx_status vx_swa_attn_stream_step_append(const void* q_new, const void* k_new, const void* v_new,
                                         void* ring_k, void* ring_v, const int64_t* pos_in,
                                         int64_t* pos_out, void* o, int32_t S, int32_t n,
                                         int32_t H, int32_t rope_applied, const vx_attn_cfg* cfg,
                                         void* stream) {
  vx_status st = check_stream_common("stream_step_append", S, n, H, cfg);
  if (st) return st;
  if (n > vx::kStreamFusedMaxNew)
    return fail(VX_E_RANGE, "stream_step_append: at most %d new frames per step (got %d)",
                vx::kStreamFusedMaxNew, n);
  if (S == 0) return ok();
  if (!q_new || !k_new || !v_new || !ring_k || !ring_v || !pos_in || !pos_out || !o)
    return fail(VX_E_NULL, "stream_step_append: a tensor pointer is NULL");
  if (!aligned16(q_new) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(ring_k) ||
      !aligned16(ring_v) || !aligned16(o))
    return fail(VX_E_ALIGN, "stream_step_append: tensors must be 16-byte aligned");
  if (((uintptr_t)pos_in & 7u) != 0 || ((uintptr_t)pos_out & 7u) != 0)
    return fail(VX_E_ALIGN, "stream_step_append: pos_in/pos_out must be 8-byte aligned");
  const size_t nf = (size_t)S * n * H * vx::kD;
  const size_t ob = nf * elem_size(cfg->out_dtype), ib = nf * elem_size(cfg->io_dtype);
  const size_t rb = (size_t)S * H * cfg->window * vx::kD * elem_size(cfg->io_dtype);
  const size_t pb = (size_t)S * sizeof(int64_t);
  if (overlap(pos_in, pb, pos_out, pb))
    return fail(VX_E_RANGE, "stream_step_append: pos_in and pos_out must not overlap");
  if (overlap(ring_k, rb, ring_v, rb))
    return fail(VX_E_RANGE, "stream_step_append: ring_k and ring_v overlap");
  if (overlap(o, ob, q_new, ib) || overlap(o, ob, k_new, ib) || overlap(o, ob, v_new, ib) ||
      overlap(o, ob, ring_k, rb) || overlap(o, ob, ring_v, rb))
    return fail(VX_E_RANGE, "stream_step_append: o overlaps an input");
  vx::StreamArgs a{};
  a.q = q_new;
  a.k = k_new;
  a.v = v_new;
  a.ring_k = ring_k;
  a.ring_v = ring_v;
  a.pos = pos_in;
  a.o = o;
  a.S = S;
  a.n = n;
  a.H = H;
  a.W = cfg->window;
  a.rope = rope_applied == 0;
  a.scale_log2 = scale_log2(cfg);
  const vx::RopeFreqs fr = rope_freqs(cfg->rope_theta);
  (void)hipGetLastError();
  if (cfg->io_dtype == VX_BF16) {
    a.append = true;
    a.ring_k_w = ring_k;
    a.ring_v_w = ring_v;
    a.pos_out = pos_out;
    return launched(vx::launch_stream_step(a, vx::DT::BF16, to_dt(cfg->out_dtype), fr,
                                           (hipStream_t)stream));
  }
  // float32: the two kernels back to back on the same stream
  vx_status s1 = launched(vx::launch_stream_step(a, vx::DT::F32, vx::DT::F32, fr, (hipStream_t)stream));
  if (s1) return s1;
  vx::AppendArgs b{};
  b.ring_k = ring_k;
  b.ring_v = ring_v;
  b.k = k_new;
  b.v = v_new;
  b.pos = pos_in;
  b.pos_out = pos_out;
  b.S = S;
  b.n = n;
  b.H = H;
  b.W = cfg->window;
  b.rope = a.rope;
  return launched(vx::launch_ring_append(b, vx::DT::F32, fr, (hipStream_t)stream));
}

vx_status vx_gqa_attn_prefill(const void* q, const void* k, const void* v, void* o, int32_t B,
                              int32_t T, int32_t Hq, int32_t Hkv, int64_t pos0,
                              int32_t rope_applied, const float* rope_table, int64_t table_p0,
                              int64_t table_len, void* ring_k, void* ring_v, int64_t* pos,
                              void* k_rot, const vx_attn_cfg* cfg, void* stream) {
  const char* what = "gqa_prefill";
  vx_status st = check_gqa_cfg(what, cfg);
  if (st) return st;
  if (B < 0 || T < 0) return fail(VX_E_SHAPE, "%s: negative size", what);
  if ((st = check_heads(what, Hq, Hkv))) return st;
  const int32_t G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(VX_E_SHAPE, "%s: Hq/Hkv must be 1, 2, 4 or 8 (got %d)", what, G);
  if (pos0 < 0 || pos0 > ((int64_t)1 << 52)) return fail(VX_E_RANGE, "%s: pos0 out of range", what);
  const bool seed = ring_k || ring_v;
  if (seed && pos0 != 0) return fail(VX_E_RANGE, "%s: ring seeding needs pos0 == 0", what);
  if ((int64_t)B * T == 0) return ok();
  if (B > 65535 || T > kMaxDim) return fail(VX_E_SHAPE, "%s: B or T too large", what);
  if ((int64_t)B * T * Hq * vx::kGD > kMaxElems) return fail(VX_E_SHAPE, "%s: tensor too large", what);
  if (!q || !k || !v || !o) return fail(VX_E_NULL, "%s: q, k, v and o must be non-NULL", what);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(VX_E_ALIGN, "%s: q, k, v and o must be 16-byte aligned", what);
  const size_t qb = (size_t)B * T * Hq * vx::kGD * 2, kb = (size_t)B * T * Hkv * vx::kGD * 2;
  const size_t ob = (size_t)B * T * Hq * vx::kGD * elem_size(cfg->out_dtype);
  if (overlap(o, ob, q, qb) || overlap(o, ob, k, kb) || overlap(o, ob, v, kb))
    return fail(VX_E_RANGE, "%s: o overlaps an input", what);
  vx::GqaPrefillArgs a{};
  a.q = (const vx::bf16*)q;
  a.k = (const vx::bf16*)k;
  a.v = (const vx::bf16*)v;
  a.o = o;
  a.B = B;
  a.T = T;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.W = cfg->window;
  a.rope = rope_applied == 0;
  a.scale_log2 = scale_log2(cfg);
  if (seed) {
    if (!ring_k || !ring_v || !pos) return fail(VX_E_NULL, "%s: seeding needs ring_k, ring_v and pos", what);
    if (!aligned16(ring_k) || !aligned16(ring_v))
      return fail(VX_E_ALIGN, "%s: ring_k and ring_v must be 16-byte aligned", what);
    if (((uintptr_t)pos & 7u) != 0) return fail(VX_E_ALIGN, "%s: pos is not 8-byte aligned", what);
    if ((int64_t)B * Hkv * cfg->window * vx::kGD > kMaxElems)
      return fail(VX_E_SHAPE, "%s: ring too large", what);
    const size_t rb = (size_t)B * Hkv * cfg->window * vx::kGD * 2;
    if (overlap(ring_k, rb, ring_v, rb)) return fail(VX_E_RANGE, "%s: ring_k and ring_v overlap", what);
    if (overlap(o, ob, ring_k, rb) || overlap(o, ob, ring_v, rb))
      return fail(VX_E_RANGE, "%s: o overlaps a ring", what);
    a.ring_k = (vx::bf16*)ring_k;
    a.ring_v = (vx::bf16*)ring_v;
    a.pos_out = pos;
  }
  if (k_rot) {
    if (!a.rope) return fail(VX_E_RANGE, "%s: k_rot needs rope_applied == 0", what);
    if (!aligned16(k_rot)) return fail(VX_E_ALIGN, "%s: k_rot is not 16-byte aligned", what);
    if (overlap(k_rot, kb, q, qb) || overlap(k_rot, kb, k, kb) || overlap(k_rot, kb, v, kb) ||
        overlap(k_rot, kb, o, ob))
      return fail(VX_E_RANGE, "%s: k_rot overlaps q, k, v or o", what);
    if (seed) {
      const size_t rb = (size_t)B * Hkv * cfg->window * vx::kGD * 2;
      if (overlap(k_rot, kb, ring_k, rb) || overlap(k_rot, kb, ring_v, rb))
        return fail(VX_E_RANGE, "%s: k_rot overlaps a ring", what);
    }
  }
  if (a.rope) {
    if (!rope_table) return fail(VX_E_NULL, "%s: rope_table is NULL and rope_applied == 0", what);
    if (!aligned16(rope_table)) return fail(VX_E_ALIGN, "%s: rope_table is not 16-byte aligned", what);
    if (table_p0 < 0 || table_len < 0 || pos0 < table_p0 || pos0 + T > table_p0 + table_len)
      return fail(VX_E_RANGE,
                  "%s: rope_table covers positions [%lld, %lld) but the prompt needs [%lld, %lld)",
                  what, (long long)table_p0, (long long)(table_p0 + table_len), (long long)pos0,
                  (long long)(pos0 + T));
    a.table = rope_table;
    a.table_row0 = pos0 - table_p0;
  }
  (void)hipGetLastError();
  if (k_rot) {
    // rotate the keys once into k_rot, then attend over them with only q rotated in the kernel
    vx_status s1 = launched(vx::launch_gqa_rope_rows(a.k, (vx::bf16*)k_rot, B, T, Hkv, a.table,
                                                     a.table_row0, (hipStream_t)stream));
    if (s1) return s1;
    a.k = (const vx::bf16*)k_rot;
    a.rope_k = false;
  }
  return launched(vx::launch_gqa_prefill(a, to_dt(cfg->out_dtype), (hipStream_t)stream));
}

vx_status vx_gqa_attn_decode(const void* q_new, const void* k_new, const void* v_new,
                             void* ring_k, void* ring_v, const int64_t* pos_in, int64_t* pos_out,
                             void* o, int32_t S, int32_t n, int32_t Hq, int32_t Hkv,
                             int32_t rope_applied, const vx_attn_cfg* cfg, void* stream) {
  const char* what = "gqa_decode";
  vx_status st = check_gqa_cfg(what, cfg);
  if (st) return st;
  if (S < 0 || S > kMaxDim) return fail(VX_E_SHAPE, "%s: S out of range", what);
  if ((st = check_heads(what, Hq, Hkv))) return st;
  const int32_t G = Hq / Hkv;
  if (n < 1 || n > cfg->window)
    return fail(VX_E_RANGE, "%s: need 1 <= n <= window (n %d, window %d)", what, n, cfg->window);
  if ((int64_t)n * G > vx::kGqaMaxCols)
    return fail(VX_E_RANGE, "%s: n * Hq/Hkv must be <= %d (got %lld)", what, vx::kGqaMaxCols,
                (long long)n * G);
  if ((int64_t)S * Hkv >= ((int64_t)1 << 31)) return fail(VX_E_SHAPE, "%s: S*Hkv too large", what);
  if ((int64_t)S * Hkv * cfg->window * vx::kGD > kMaxElems)
    return fail(VX_E_SHAPE, "%s: ring too large", what);
  if (S == 0) return ok();
  if (!q_new || !k_new || !v_new || !ring_k || !ring_v || !pos_in || !pos_out || !o)
    return fail(VX_E_NULL, "%s: a tensor pointer is NULL", what);
  if (!aligned16(q_new) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(ring_k) ||
      !aligned16(ring_v) || !aligned16(o))
    return fail(VX_E_ALIGN, "%s: tensors must be 16-byte aligned", what);
  if (((uintptr_t)pos_in & 7u) != 0 || ((uintptr_t)pos_out & 7u) != 0)
    return fail(VX_E_ALIGN, "%s: pos_in/pos_out must be 8-byte aligned", what);
  const size_t qb = (size_t)S * n * Hq * vx::kGD * 2, kb = (size_t)S * n * Hkv * vx::kGD * 2;
  const size_t ob = (size_t)S * n * Hq * vx::kGD * elem_size(cfg->out_dtype);
  const size_t rb = (size_t)S * Hkv * cfg->window * vx::kGD * 2;
  const size_t pb = (size_t)S * sizeof(int64_t);
  if (overlap(pos_in, pb, pos_out, pb))
    return fail(VX_E_RANGE, "%s: pos_in and pos_out must not overlap", what);
  if (overlap(ring_k, rb, ring_v, rb)) return fail(VX_E_RANGE, "%s: ring_k and ring_v overlap", what);
  if (overlap(o, ob, q_new, qb) || overlap(o, ob, k_new, kb) || overlap(o, ob, v_new, kb) ||
      overlap(o, ob, ring_k, rb) || overlap(o, ob, ring_v, rb))
    return fail(VX_E_RANGE, "%s: o overlaps an input", what);
  if (overlap(ring_k, rb, k_new, kb) || overlap(ring_k, rb, v_new, kb) ||
      overlap(ring_v, rb, k_new, kb) || overlap(ring_v, rb, v_new, kb))
    return fail(VX_E_RANGE, "%s: a ring overlaps the new keys or values", what);
  vx::GqaDecodeArgs a{};
  a.q = (const vx::bf16*)q_new;
  a.k = (const vx::bf16*)k_new;
  a.v = (const vx::bf16*)v_new;
  a.ring_k = (vx::bf16*)ring_k;
  a.ring_v = (vx::bf16*)ring_v;
  a.pos_in = pos_in;
  a.pos_out = pos_out;
  a.o = o;
  a.S = S;
  a.n = n;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.W = cfg->window;
  a.rope = rope_applied == 0;
  a.scale_log2 = scale_log2(cfg);
  (void)hipGetLastError();
  return launched(vx::launch_gqa_decode(a, to_dt(cfg->out_dtype), rope_freqs128(cfg->rope_theta),
                                        (hipStream_t)stream));
}

// ---- projections around the encoder's attention ---------------------------

static vx_status check_linear_shape(const char* what, int32_t M, int32_t N, int32_t K) {
  if (M < 0 || N < 1 || K < 1) return fail(VX_E_SHAPE, "%s: need M >= 0, N >= 1, K >= 1", what);
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return fail(VX_E_SHAPE, "%s: size too large", what);
  if (K % vx::kLinKStep != 0)
    return fail(VX_E_SHAPE, "%s: K (%d) must be a multiple of %d", what, K, vx::kLinKStep);
  if (N % 32 != 0) return fail(VX_E_SHAPE, "%s: N (%d) must be a multiple of 32", what, N);
  if ((int64_t)M * K > kMaxElems || (int64_t)N * K > kMaxElems || (int64_t)M * N > kMaxElems)
    return fail(VX_E_SHAPE, "%s: tensor too large", what);
  if ((int64_t)((M + 63) / 64) > 65535) return fail(VX_E_SHAPE, "%s: M too large", what);
  // the kernel addresses x and w with 32-bit byte offsets
  if ((int64_t)M * K * 2 >= ((int64_t)1 << 30) || (int64_t)N * K * 2 >= ((int64_t)1 << 30))
    return fail(VX_E_SHAPE, "%s: x and w must each be smaller than 2^30 bytes", what);
  return VX_OK;
}

vx_status vx_linear(const void* x, const void* w, const void* bias, void* y, int32_t M, int32_t N,
                    int32_t K, int32_t out_dtype, void* stream) {
  const char* what = "linear";
  vx_status st = check_linear_shape(what, M, N, K);
  if (st) return st;
  if (out_dtype != VX_BF16 && out_dtype != VX_F32)
    return fail(VX_E_DTYPE, "%s: unknown output dtype %d", what, out_dtype);
  if (M == 0) return ok();
  if (!x || !w || !y) return fail(VX_E_NULL, "%s: x, w and y must be non-NULL", what);
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (bias && !aligned16(bias)))
    return fail(VX_E_ALIGN, "%s: x, w, bias and y must be 16-byte aligned", what);
  const size_t yb = (size_t)M * N * elem_size(out_dtype);
  if (overlap(y, yb, x, (size_t)M * K * 2) || overlap(y, yb, w, (size_t)N * K * 2) ||
      (bias && overlap(y, yb, bias, (size_t)N * 2)))
    return fail(VX_E_RANGE, "%s: y overlaps an input", what);
  vx::LinearArgs a{};
  a.x = (const vx::bf16*)x;
  a.w = (const vx::bf16*)w;
  a.M = M;
  a.N = N;
  a.K = K;
  a.bias = (const vx::bf16*)bias;
  a.y = y;
  vx::dense_rows(a);
  (void)hipGetLastError();
  return launched(vx::launch_linear(a, to_dt(out_dtype), (hipStream_t)stream));
}

static vx_status check_block(const char* what, int32_t S, int32_t n, int32_t H, int32_t d_model,
                             const vx_attn_cfg* cfg) {
  vx_status st = check_cfg(cfg);
  if (st) return st;
  if (cfg->io_dtype != VX_BF16) return fail(VX_E_DTYPE, "%s: only bf16 is supported", what);
  if (cfg->flags != 0) return fail(VX_E_RANGE, "%s: no flags apply (got 0x%x)", what, cfg->flags);
  if (S < 0 || n < 1 || H < 1) return fail(VX_E_SHAPE, "%s: need S >= 0, n >= 1, H >= 1", what);
  if ((int64_t)S * n > kMaxDim) return fail(VX_E_SHAPE, "%s: S*n too large", what);
  if ((st = check_linear_shape(what, S * n, 3 * H * vx::kD, d_model))) return st;
  if ((st = check_linear_shape(what, S * n, d_model, H * vx::kD))) return st;
  return VX_OK;
}

vx_status vx_enc_qkv_rope(const void* x, const void* w_qkv, const void* b_q, const void* b_v,
                          const int64_t* pos, int32_t S, int32_t n, int32_t H, int32_t d_model,
                          void* q, void* k, void* v, const vx_attn_cfg* cfg, void* stream) {
  const char* what = "enc_qkv_rope";
  vx_status st = check_cfg(cfg);
  if (st) return st;
  if (cfg->io_dtype != VX_BF16) return fail(VX_E_DTYPE, "%s: only bf16 is supported", what);
  if (S < 0 || n < 1 || H < 1) return fail(VX_E_SHAPE, "%s: need S >= 0, n >= 1, H >= 1", what);
  if ((int64_t)S * n > kMaxDim) return fail(VX_E_SHAPE, "%s: S*n too large", what);
  if ((st = check_linear_shape(what, S * n, 3 * H * vx::kD, d_model))) return st;
  if ((H * vx::kD) % 128 != 0) return fail(VX_E_SHAPE, "%s: H*64 must be a multiple of 128", what);
  if (S == 0) return ok();
  if (!x || !w_qkv || !pos || !q || !k || !v)
    return fail(VX_E_NULL, "%s: x, w_qkv, pos, q, k and v must be non-NULL", what);
  if (!aligned16(x) || !aligned16(w_qkv) || !aligned16(q) || !aligned16(k) || !aligned16(v) ||
      (b_q && !aligned16(b_q)) || (b_v && !aligned16(b_v)))
    return fail(VX_E_ALIGN, "%s: tensors must be 16-byte aligned", what);
  if (((uintptr_t)pos & 7u) != 0) return fail(VX_E_ALIGN, "%s: pos must be 8-byte aligned", what);
  const size_t ob = (size_t)S * n * H * vx::kD * 2;
  const size_t xb = (size_t)S * n * d_model * 2, wb = (size_t)3 * H * vx::kD * d_model * 2;
  const void* outs[3] = {q, k, v};
  for (int i = 0; i < 3; ++i) {
    if (overlap(outs[i], ob, x, xb) || overlap(outs[i], ob, w_qkv, wb))
      return fail(VX_E_RANGE, "%s: an output overlaps an input", what);
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], ob, outs[j], ob)) return fail(VX_E_RANGE, "%s: q, k, v overlap", what);
  }
  vx::LinearArgs a{};
  a.x = (const vx::bf16*)x;
  a.w = (const vx::bf16*)w_qkv;
  a.M = S * n;
  a.N = 3 * H * vx::kD;
  a.K = d_model;
  a.HD = H * vx::kD;
  a.n = n;
  a.pos = pos;
  a.b_q = (const vx::bf16*)b_q;
  a.b_v = (const vx::bf16*)b_v;
  a.q = (vx::bf16*)q;
  a.k = (vx::bf16*)k;
  a.v = (vx::bf16*)v;
  vx::dense_rows(a);
  (void)hipGetLastError();
  return launched(vx::launch_qkv_rope(a, rope_freqs(cfg->rope_theta), (hipStream_t)stream));
}

vx_status vx_enc_attn_step(const void* x, const void* w_qkv, const void* b_q, const void* b_v,
                           const void* w_o, const void* b_o, void* ring_k, void* ring_v,
                           const int64_t* pos_in, int64_t* pos_out, void* q, void* k, void* v,
                           void* o, void* y, int32_t S, int32_t n, int32_t H, int32_t d_model,
                           const vx_attn_cfg* cfg, void* stream) {
  const char* what = "enc_attn_step";
  vx_status st = check_block(what, S, n, H, d_model, cfg);
  if (st) return st;
  if ((st = check_stream_common(what, S, n, H, cfg))) return st;
  if (n > vx::kStreamFusedMaxNew)
    return fail(VX_E_RANGE, "%s: at most %d new frames per step (got %d)", what,
                vx::kStreamFusedMaxNew, n);
  if (S == 0) return ok();
  if (!x || !w_qkv || !w_o || !ring_k || !ring_v || !pos_in || !pos_out || !q || !k || !v || !o ||
      !y)
    return fail(VX_E_NULL, "%s: a required pointer is NULL", what);
  const void* al[] = {x, w_qkv, w_o, ring_k, ring_v, q, k, v, o, y};
  for (const void* p : al)
    if (!aligned16(p)) return fail(VX_E_ALIGN, "%s: tensors must be 16-byte aligned", what);
  if ((b_q && !aligned16(b_q)) || (b_v && !aligned16(b_v)) || (b_o && !aligned16(b_o)))
    return fail(VX_E_ALIGN, "%s: biases must be 16-byte aligned", what);
  if (((uintptr_t)pos_in & 7u) != 0 || ((uintptr_t)pos_out & 7u) != 0)
    return fail(VX_E_ALIGN, "%s: pos_in/pos_out must be 8-byte aligned", what);
  const size_t M = (size_t)S * n;
  const size_t act = M * H * vx::kD * 2, xb = M * d_model * 2;
  const size_t yb = M * d_model * elem_size(cfg->out_dtype);
  const size_t rb = (size_t)S * H * cfg->window * vx::kD * 2, pb = (size_t)S * sizeof(int64_t);
  // the buffers the block writes must not overlap anything else it touches
  const void* wr[] = {q, k, v, o, y, ring_k, ring_v};
  const size_t wrb[] = {act, act, act, act, yb, rb, rb};
  const void* all[] = {x, w_qkv, w_o, q, k, v, o, y, ring_k, ring_v};
  const size_t allb[] = {xb, (size_t)3 * H * vx::kD * d_model * 2, (size_t)d_model * H * vx::kD * 2,
                         act, act, act, act, yb, rb, rb};
  for (int i = 0; i < 7; ++i)
    for (int j = 0; j < 10; ++j)
      if (wr[i] != all[j] && overlap(wr[i], wrb[i], all[j], allb[j]))
        return fail(VX_E_RANGE, "%s: buffers overlap", what);
  if (overlap(pos_in, pb, pos_out, pb))
    return fail(VX_E_RANGE, "%s: pos_in and pos_out must not overlap", what);
  (void)hipGetLastError();
  const hipStream_t hs = (hipStream_t)stream;
  const vx::RopeFreqs fr = rope_freqs(cfg->rope_theta);
  // 1. q', k' (rotated at pos_in[s] + i) and v from the hidden state
  vx::LinearArgs a{};
  a.x = (const vx::bf16*)x;
  a.w = (const vx::bf16*)w_qkv;
  a.M = (int)M;
  a.N = 3 * H * vx::kD;
  a.K = d_model;
  a.HD = H * vx::kD;
  a.n = n;
  a.pos = pos_in;
  a.b_q = (const vx::bf16*)b_q;
  a.b_v = (const vx::bf16*)b_v;
  a.q = (vx::bf16*)q;
  a.k = (vx::bf16*)k;
  a.v = (vx::bf16*)v;
  vx::dense_rows(a);
  if ((st = launched(vx::launch_qkv_rope(a, fr, hs)))) return st;
  // 2. attention over the ring and the new frames, then the append (q, k already rotated)
  vx::StreamArgs sa{};
  sa.q = q;
  sa.k = k;
  sa.v = v;
  sa.ring_k = ring_k;
  sa.ring_v = ring_v;
  sa.pos = pos_in;
  sa.o = o;
  sa.S = S;
  sa.n = n;
  sa.H = H;
  sa.W = cfg->window;
  sa.rope = false;
  sa.scale_log2 = scale_log2(cfg);
  sa.append = true;
  sa.ring_k_w = ring_k;
  sa.ring_v_w = ring_v;
  sa.pos_out = pos_out;
  if ((st = launched(vx::launch_stream_step(sa, vx::DT::BF16, vx::DT::BF16, fr, hs)))) return st;
  // 3. output projection
  vx::LinearArgs b{};
  b.x = (const vx::bf16*)o;
  b.w = (const vx::bf16*)w_o;
  b.M = (int)M;
  b.N = d_model;
  b.K = H * vx::kD;
  b.bias = (const vx::bf16*)b_o;
  b.y = y;
  vx::dense_rows(b);
  return launched(vx::launch_linear(b, to_dt(cfg->out_dtype), hs));
}

// ---- the streaming encoder step ---------------------------------------------

namespace {

struct Region {
  const void* p;
  size_t bytes;
  bool written;
};

// Every region the call writes must be disjoint from every other region it
// touches (NULL regions, the optional biases left out, are skipped).
bool regions_disjoint(const std::vector<Region>& r) {
  for (size_t i = 0; i < r.size(); ++i) {
    if (!r[i].written || !r[i].p) continue;
    for (size_t j = 0; j < r.size(); ++j)
      if (j != i && r[j].p && overlap(r[i].p, r[i].bytes, r[j].p, r[j].bytes)) return false;
  }
  return true;
}

vx_status check_eps(const char* what, float eps) {
  if (!(eps >= 0.0f) || !isfinite(eps)) return fail(VX_E_RANGE, "%s: eps must be finite and >= 0", what);
  return VX_OK;
}

// Row maps of the two stem convolutions as products over frame windows.
// conv1: output frame t of stream s (row s*2n + t) reads mel slots t .. t+2,
// i.e. 3*n_mels contiguous elements from slot t; writes c1 slot t + 2.
// conv2: output frame t (row s*n + t) reads c1 slots 2t .. 2t+2; writes x.
void stem_args(vx::LinearArgs& c1, vx::LinearArgs& c2, void* mel_buf, void* c1_buf,
               const vx_enc_stem_weights* w, float* x_out, int S, int n, int n_mels, int d_model) {
  const int F = 2 * n + 2;
  c1 = vx::LinearArgs{};
  c1.x = (const vx::bf16*)mel_buf;
  c1.w = (const vx::bf16*)w->w1;
  c1.M = S * 2 * n;
  c1.N = d_model;
  c1.K = 3 * n_mels;
  c1.rpg = 2 * n;
  c1.xgs = (int64_t)F * n_mels;
  c1.xrs = n_mels;
  c1.ygs = (int64_t)F * d_model;
  c1.yrs = d_model;
  c1.x_bytes = (int64_t)S * F * n_mels * 2;
  c1.bias = (const vx::bf16*)w->b1;
  c1.y = (vx::bf16*)c1_buf + 2 * (int64_t)d_model;
  c2 = vx::LinearArgs{};
  c2.x = (const vx::bf16*)c1_buf;
  c2.w = (const vx::bf16*)w->w2;
  c2.M = S * n;
  c2.N = d_model;
  c2.K = 3 * d_model;
  c2.rpg = n;
  c2.xgs = (int64_t)F * d_model;
  c2.xrs = 2 * (int64_t)d_model;
  c2.ygs = (int64_t)n * d_model;
  c2.yrs = d_model;
  c2.x_bytes = (int64_t)S * F * d_model * 2;
  c2.bias = (const vx::bf16*)w->b2;
  c2.y = x_out;
}

vx_status check_stem(const char* what, const void* mel_buf, const void* c1_buf,
                     const vx_enc_stem_weights* w, const float* x_out, int32_t S, int32_t n,
                     int32_t n_mels, int32_t d_model) {
  if (S < 0 || n < 1 || n_mels < 1 || d_model < 1)
    return fail(VX_E_SHAPE, "%s: need S >= 0, n >= 1, n_mels >= 1, d_model >= 1", what);
  if (n > kMaxDim / 2 || (int64_t)S * (2 * n + 2) > kMaxDim)
    return fail(VX_E_SHAPE, "%s: S*(2n+2) too large", what);
  if (n_mels % 128 != 0 || d_model % 128 != 0)
    return fail(VX_E_SHAPE, "%s: n_mels (%d) and d_model (%d) must be multiples of 128", what,
                n_mels, d_model);
  const int64_t F = 2 * (int64_t)n + 2;
  if ((int64_t)S * F * d_model * 2 >= ((int64_t)1 << 30) ||
      (int64_t)d_model * 3 * d_model * 2 >= ((int64_t)1 << 30))
    return fail(VX_E_SHAPE, "%s: buffers and weights must each be smaller than 2^30 bytes", what);
  vx_status st;
  if ((st = check_linear_shape(what, S * 2 * n, d_model, 3 * n_mels))) return st;
  if ((st = check_linear_shape(what, S * n, d_model, 3 * d_model))) return st;
  if (S == 0) return VX_OK;
  if (!w) return fail(VX_E_NULL, "%s: stem weights are NULL", what);
  if (!mel_buf || !c1_buf || !x_out || !w->w1 || !w->w2)
    return fail(VX_E_NULL, "%s: mel_buf, c1_buf, x_out, w1 and w2 must be non-NULL", what);
  const void* al[] = {mel_buf, c1_buf, x_out, w->w1, w->w2, w->b1, w->b2};
  for (const void* p : al)
    if (p && !aligned16(p)) return fail(VX_E_ALIGN, "%s: tensors must be 16-byte aligned", what);
  return VX_OK;
}

vx_status launch_stem(void* mel_buf, void* c1_buf, const vx_enc_stem_weights* w, float* x_out,
                      int S, int n, int n_mels, int d_model, hipStream_t hs) {
  vx::LinearArgs c1, c2;
  stem_args(c1, c2, mel_buf, c1_buf, w, x_out, S, n, n_mels, d_model);
  vx_status st;
  if ((st = launched(vx::launch_linear(c1, vx::DT::BF16, hs, vx::LinEpi::Gelu)))) return st;
  if ((st = launched(vx::launch_linear(c2, vx::DT::F32, hs, vx::LinEpi::Gelu)))) return st;
  return launched(vx::launch_stem_shift((vx::bf16*)mel_buf, 2 * n + 2, n_mels, (vx::bf16*)c1_buf,
                                        2 * n + 2, d_model, S, hs));
}

vx_status check_layer_shape(const char* what, int32_t S, int32_t n, int32_t H, int32_t d_model,
                            int32_t ffn, float eps, const vx_attn_cfg* cfg) {
  vx_status st = check_block(what, S, n, H, d_model, cfg);
  if (st) return st;
  if ((st = check_stream_common(what, S, n, H, cfg))) return st;
  if ((st = check_eps(what, eps))) return st;
  if (n > vx::kStreamFusedMaxNew)
    return fail(VX_E_RANGE, "%s: at most %d new frames per step (got %d)", what,
                vx::kStreamFusedMaxNew, n);
  if ((H * vx::kD) % 128 != 0 || d_model % 128 != 0)
    return fail(VX_E_SHAPE, "%s: H*64 and d_model must be multiples of 128", what);
  if (ffn < 1 || ffn % 128 != 0)
    return fail(VX_E_SHAPE, "%s: ffn (%d) must be a positive multiple of 128", what, ffn);
  if ((st = check_linear_shape(what, S * n, 2 * ffn, d_model))) return st;
  if ((st = check_linear_shape(what, S * n, d_model, ffn))) return st;
  if (d_model > vx::kReduceMaxDim)
    return fail(VX_E_SHAPE, "%s: d_model (%d) must be at most %d", what, d_model, vx::kReduceMaxDim);
  return VX_OK;
}

vx_status check_layer_weights(const char* what, const vx_enc_layer_weights* w) {
  if (!w) return fail(VX_E_NULL, "%s: layer weights are NULL", what);
  if (!w->g_attn || !w->w_qkv || !w->w_o || !w->g_ffn || !w->w_gate || !w->w_up || !w->w_down)
    return fail(VX_E_NULL, "%s: a required layer weight is NULL", what);
  const void* al[] = {w->g_attn, w->w_qkv, w->b_q, w->b_v, w->w_o, w->b_o,
                      w->g_ffn,  w->w_gate, w->w_up, w->w_down, w->b_down};
  for (const void* p : al)
    if (p && !aligned16(p)) return fail(VX_E_ALIGN, "%s: weights must be 16-byte aligned", what);
  return VX_OK;
}

vx_status check_work(const char* what, const vx_enc_work* wk) {
  if (!wk) return fail(VX_E_NULL, "%s: work is NULL", what);
  const void* al[] = {wk->h, wk->q, wk->k, wk->v, wk->o, wk->u, wk->acc};
  for (const void* p : al) {
    if (!p) return fail(VX_E_NULL, "%s: a work buffer is NULL", what);
    if (!aligned16(p)) return fail(VX_E_ALIGN, "%s: work buffers must be 16-byte aligned", what);
  }
  return VX_OK;
}

// Appends the regions of one layer's weights (read) to r.
void weight_regions(std::vector<Region>& r, const vx_enc_layer_weights* w, int H, int dm, int ffn) {
  const size_t hd = (size_t)H * vx::kD;
  const Region add[] = {
      {w->g_attn, (size_t)dm * 2, false},       {w->w_qkv, 3 * hd * dm * 2, false},
      {w->b_q, hd * 2, false},                  {w->b_v, hd * 2, false},
      {w->w_o, (size_t)dm * hd * 2, false},     {w->b_o, (size_t)dm * 2, false},
      {w->g_ffn, (size_t)dm * 2, false},        {w->w_gate, (size_t)ffn * dm * 2, false},
      {w->w_up, (size_t)ffn * dm * 2, false},   {w->w_down, (size_t)dm * ffn * 2, false},
      {w->b_down, (size_t)dm * 2, false}};
  for (const Region& a : add) r.push_back(a);
}

// K parts of the output and down projections: two when the K stages split
// evenly (every tile shape's stage divides 128), else one.
int residual_splits(int K) { return K % (2 * vx::kLinKStep) == 0 ? 2 : 1; }

// The product x w^T of a projection added into the residual stream: the K
// parts' fp32 sums into acc, then x += sum + bias, and h = rmsnorm(x) * g_next
// when g_next is given (the next product's input).
vx_status residual_product(float* x, const vx::bf16* in, const vx::bf16* w, const vx::bf16* bias,
                           int M, int N, int K, const vx_enc_work* wk, const vx::bf16* g_next,
                           float eps, hipStream_t hs) {
  vx::LinearArgs a{};
  a.x = in;
  a.w = w;
  a.M = M;
  a.N = N;
  a.K = K;
  a.y = wk->acc;
  a.splits = residual_splits(K);
  vx::dense_rows(a);
  vx_status st;
  if ((st = launched(vx::launch_linear(a, vx::DT::F32, hs, vx::LinEpi::Partial)))) return st;
  return launched(vx::launch_residual_reduce(x, (const float*)wk->acc, a.splits, bias, g_next,
                                             (vx::bf16*)wk->h, M, N, eps, hs));
}

// One pre-norm layer (arguments validated): [RMSNorm,] q/k/v + RoPE, the
// attention step with the append, the output projection into the residual
// with the FFN's RMSNorm, gate/up + SwiGLU, the down projection into the
// residual, with h = rmsnorm(x) * g_next when g_next is given.  norm_in:
// compute h = rmsnorm(x) * g_attn first; without it h must already hold that
// (the previous layer's g_next).
vx_status launch_layer(float* x, const vx_enc_layer_weights* w, void* ring_k, void* ring_v,
                       const int64_t* pos_in, int64_t* pos_out, const vx_enc_work* wk, int S,
                       int n, int H, int dm, int ffn, float eps, const vx_attn_cfg* cfg,
                       const vx::RopeFreqs& fr, bool norm_in, const void* g_next, hipStream_t hs) {
  const int M = S * n, HD = H * vx::kD;
  vx_status st;
  // 1. h = rmsnorm(x) * g_attn
  if (norm_in &&
      (st = launched(vx::launch_rmsnorm(x, (const vx::bf16*)w->g_attn, (vx::bf16*)wk->h, M, dm, eps,
                                        hs))))
    return st;
  // 2. q', k' (rotated at pos_in[s] + i), v
  vx::LinearArgs a{};
  a.x = (const vx::bf16*)wk->h;
  a.w = (const vx::bf16*)w->w_qkv;
  a.M = M;
  a.N = 3 * HD;
  a.K = dm;
  a.HD = HD;
  a.n = n;
  a.pos = pos_in;
  a.b_q = (const vx::bf16*)w->b_q;
  a.b_v = (const vx::bf16*)w->b_v;
  a.q = (vx::bf16*)wk->q;
  a.k = (vx::bf16*)wk->k;
  a.v = (vx::bf16*)wk->v;
  vx::dense_rows(a);
  if ((st = launched(vx::launch_qkv_rope(a, fr, hs)))) return st;
  // 3. attention over the ring and the new frames, then the append
  vx::StreamArgs sa{};
  sa.q = wk->q;
  sa.k = wk->k;
  sa.v = wk->v;
  sa.ring_k = ring_k;
  sa.ring_v = ring_v;
  sa.pos = pos_in;
  sa.o = wk->o;
  sa.S = S;
  sa.n = n;
  sa.H = H;
  sa.W = cfg->window;
  sa.rope = false;
  sa.scale_log2 = scale_log2(cfg);
  sa.append = true;
  sa.ring_k_w = ring_k;
  sa.ring_v_w = ring_v;
  sa.pos_out = pos_out;
  if ((st = launched(vx::launch_stream_step(sa, vx::DT::BF16, vx::DT::BF16, fr, hs)))) return st;
  // 4-5. x += o W_o^T + b_o; h = rmsnorm(x) * g_ffn
  if ((st = residual_product(x, (const vx::bf16*)wk->o, (const vx::bf16*)w->w_o,
                             (const vx::bf16*)w->b_o, M, dm, HD, wk, (const vx::bf16*)w->g_ffn,
                             eps, hs)))
    return st;
  // 6. u = silu(h W_gate^T) * (h W_up^T)
  vx::LinearArgs g{};
  g.x = (const vx::bf16*)wk->h;
  g.w = (const vx::bf16*)w->w_gate;
  g.w2 = (const vx::bf16*)w->w_up;
  g.M = M;
  g.N = 2 * ffn;
  g.K = dm;
  g.y = wk->u;
  vx::dense_rows(g);
  if ((st = launched(vx::launch_linear(g, vx::DT::BF16, hs, vx::LinEpi::SwiGLU)))) return st;
  // 7. x += u W_down^T + b_down [; h = rmsnorm(x) * g_next]
  return residual_product(x, (const vx::bf16*)wk->u, (const vx::bf16*)w->w_down,
                          (const vx::bf16*)w->b_down, M, dm, ffn, wk,
                          (const vx::bf16*)g_next, eps, hs);
}

}  // namespace

vx_status vx_rmsnorm(const float* x, const void* g, void* y, int32_t M, int32_t dim, float eps,
                     void* stream) {
  const char* what = "rmsnorm";
  if (M < 0 || dim < 1) return fail(VX_E_SHAPE, "%s: need M >= 0 and dim >= 1", what);
  if (dim % 8 != 0) return fail(VX_E_SHAPE, "%s: dim (%d) must be a multiple of 8", what, dim);
  if (M > kMaxDim * 4 || dim > kMaxDim || (int64_t)M * dim > kMaxElems)
    return fail(VX_E_SHAPE, "%s: size too large", what);
  vx_status st = check_eps(what, eps);
  if (st) return st;
  if (M == 0) return ok();
  if (!x || !g || !y) return fail(VX_E_NULL, "%s: x, g and y must be non-NULL", what);
  if (!aligned16(x) || !aligned16(g) || !aligned16(y))
    return fail(VX_E_ALIGN, "%s: x, g and y must be 16-byte aligned", what);
  const size_t yb = (size_t)M * dim * 2;
  if (overlap(y, yb, x, (size_t)M * dim * 4) || overlap(y, yb, g, (size_t)dim * 2))
    return fail(VX_E_RANGE, "%s: y overlaps an input", what);
  (void)hipGetLastError();
  return launched(vx::launch_rmsnorm(x, (const vx::bf16*)g, (vx::bf16*)y, M, dim, eps,
                                     (hipStream_t)stream));
}

vx_status vx_enc_stem_step(void* mel_buf, void* c1_buf, const vx_enc_stem_weights* w,
                           float* x_out, int32_t S, int32_t n, int32_t n_mels, int32_t d_model,
                           void* stream) {
  const char* what = "enc_stem_step";
  vx_status st = check_stem(what, mel_buf, c1_buf, w, x_out, S, n, n_mels, d_model);
  if (st) return st;
  if (S == 0) return ok();
  const size_t F = 2 * (size_t)n + 2;
  const std::vector<Region> r = {{mel_buf, S * F * n_mels * 2, true},
                      {c1_buf, S * F * d_model * 2, true},
                      {x_out, (size_t)S * n * d_model * 4, true},
                      {w->w1, (size_t)d_model * 3 * n_mels * 2, false},
                      {w->b1, (size_t)d_model * 2, false},
                      {w->w2, (size_t)d_model * 3 * d_model * 2, false},
                      {w->b2, (size_t)d_model * 2, false}};
  if (!regions_disjoint(r)) return fail(VX_E_RANGE, "%s: buffers overlap", what);
  (void)hipGetLastError();
  return launch_stem(mel_buf, c1_buf, w, x_out, S, n, n_mels, d_model, (hipStream_t)stream);
}

vx_status vx_enc_layer_step(float* x, const vx_enc_layer_weights* w, void* ring_k, void* ring_v,
                            const int64_t* pos_in, int64_t* pos_out, const vx_enc_work* work,
                            int32_t S, int32_t n, int32_t H, int32_t d_model, int32_t ffn,
                            float eps, const vx_attn_cfg* cfg, void* stream) {
  return vx_enc_step(nullptr, nullptr, nullptr, w, 1, ring_k, ring_v, pos_in, pos_out, x, work, S,
                     n, 0, H, d_model, ffn, eps, cfg, stream);
}

vx_status vx_enc_step(void* mel_buf, void* c1_buf, const vx_enc_stem_weights* stem,
                      const vx_enc_layer_weights* layers, int32_t L, void* ring_k, void* ring_v,
                      const int64_t* pos_in, int64_t* pos_out, float* x, const vx_enc_work* work,
                      int32_t S, int32_t n, int32_t n_mels, int32_t H, int32_t d_model,
                      int32_t ffn, float eps, const vx_attn_cfg* cfg, void* stream) {
  const bool with_stem = stem != nullptr;
  const char* what = with_stem ? "enc_step" : "enc_layer_step";
  vx_status st = check_layer_shape(what, S, n, H, d_model, ffn, eps, cfg);
  if (st) return st;
  if (L < 1 || L > 4096) return fail(VX_E_SHAPE, "%s: L (%d) must be in [1, 4096]", what, L);
  if (with_stem && (st = check_stem(what, mel_buf, c1_buf, stem, x, S, n, n_mels, d_model)))
    return st;
  if (S == 0) return ok();
  if (!layers) return fail(VX_E_NULL, "%s: layers is NULL", what);
  for (int l = 0; l < L; ++l)
    if ((st = check_layer_weights(what, &layers[l]))) return st;
  if (!x || !pos_in || !pos_out || !ring_k || !ring_v)
    return fail(VX_E_NULL, "%s: x, rings, pos_in and pos_out must be non-NULL", what);
  if (!aligned16(x) || !aligned16(ring_k) || !aligned16(ring_v))
    return fail(VX_E_ALIGN, "%s: x and the rings must be 16-byte aligned", what);
  if (((uintptr_t)pos_in & 7u) != 0 || ((uintptr_t)pos_out & 7u) != 0)
    return fail(VX_E_ALIGN, "%s: pos_in/pos_out must be 8-byte aligned", what);
  if ((st = check_work(what, work))) return st;
  const size_t M = (size_t)S * n, act = M * H * vx::kD * 2;
  const size_t ring1 = (size_t)S * H * cfg->window * vx::kD * 2, pb = (size_t)S * 8;
  // every written region against everything else
  std::vector<Region> r;
  r.reserve(19 + 11 * (size_t)L);
  const size_t F = 2 * (size_t)n + 2;
  r.push_back({x, M * d_model * 4, true});
  r.push_back({pos_in, pb, false});
  r.push_back({pos_out, pb, true});
  r.push_back({ring_k, ring1 * L, true});
  r.push_back({ring_v, ring1 * L, true});
  r.push_back({work->h, M * d_model * 2, true});
  r.push_back({work->q, act, true});
  r.push_back({work->k, act, true});
  r.push_back({work->v, act, true});
  r.push_back({work->o, act, true});
  r.push_back({work->u, M * ffn * 2, true});
  r.push_back({work->acc, 2 * M * d_model * 4, true});
  if (with_stem) {
    r.push_back({mel_buf, S * F * n_mels * 2, true});
    r.push_back({c1_buf, S * F * d_model * 2, true});
    r.push_back({stem->w1, (size_t)d_model * 3 * n_mels * 2, false});
    r.push_back({stem->b1, (size_t)d_model * 2, false});
    r.push_back({stem->w2, (size_t)d_model * 3 * d_model * 2, false});
    r.push_back({stem->b2, (size_t)d_model * 2, false});
  }
  for (int l = 0; l < L; ++l) weight_regions(r, &layers[l], H, d_model, ffn);
  if (!regions_disjoint(r)) return fail(VX_E_RANGE, "%s: buffers overlap", what);
  (void)hipGetLastError();
  const hipStream_t hs = (hipStream_t)stream;
  if (with_stem && (st = launch_stem(mel_buf, c1_buf, stem, x, S, n, n_mels, d_model, hs)))
    return st;
  const vx::RopeFreqs fr = rope_freqs(cfg->rope_theta);
  // layer l > 0 takes its normalised input from layer l-1's last reduction
  for (int l = 0; l < L; ++l) {
    char* rk = (char*)ring_k + ring1 * l;
    char* rv = (char*)ring_v + ring1 * l;
    const void* g_next = l + 1 < L ? layers[l + 1].g_attn : nullptr;
    if ((st = launch_layer(x, &layers[l], rk, rv, pos_in, pos_out, work, S, n, H, d_model, ffn,
                           eps, cfg, fr, l == 0, g_next, hs)))
      return st;
  }
  return ok();
}

const char* vx_status_string(vx_status s) {
  switch (s) {
    case VX_OK: return "ok";
    case VX_E_NULL: return "null pointer";
    case VX_E_SHAPE: return "bad shape";
    case VX_E_DTYPE: return "unsupported dtype";
    case VX_E_ALIGN: return "misaligned pointer";
    case VX_E_RANGE: return "value out of range";
    case VX_E_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* vx_last_error(void) { return g_err.c_str(); }

int32_t vx_version(void) { return 100; }

}  // extern "C"
