"""Sliding-window RoPE attention for MI355X (gfx950): Python binding of libvx.

Causal attention of each frame over the last `window` frames (itself
included) with half-split RoPE on queries and keys -- the self-attention of
the Voxtral Realtime 2602 audio encoder (W = 750, 32 heads x 64, theta 1e6;
transcribe.cpp "Voxtral" family notes, section Architecture).  Every call
marshals torch tensors into the C ABI of include/vx.h; all arithmetic runs in
the HIP kernels of libvx.so.  PyTorch only provides device memory and
streams.  There is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "VxError", "Config", "lib", "rope_table", "rope_qk", "prefill", "prefill_workspace_size",
    "prefill_workspace", "prefill_noalloc", "prefill_varlen", "stream_step", "ring_append",
    "stream_step_append", "gqa_prefill", "gqa_decode", "linear", "enc_qkv_rope",
    "enc_attn_step", "rmsnorm", "enc_work", "enc_stem_step", "enc_layer_step", "enc_step",
    "LAYER_KEYS", "STEM_KEYS",
    "WINDOW", "THETA", "HEAD_DIM", "DEC_WINDOW", "DEC_HEAD_DIM",
]

WINDOW = 750
THETA = 1e6
HEAD_DIM = 64
# text decoder (grouped-query attention): 32 query / 8 key-value heads
DEC_WINDOW = 8192
DEC_HEAD_DIM = 128

VX_F32, VX_BF16 = 0, 1
VX_FLAG_VALU_KERNEL = 1
VX_FLAG_SPLIT_WALK = 2
_STATUS = {0: "ok", 1: "null pointer", 2: "bad shape", 3: "unsupported dtype",
           4: "misaligned pointer", 5: "value out of range", 6: "HIP runtime error"}

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvx.so")


class VxError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        self.status = status
        super().__init__(f"{func}: {_STATUS.get(status, status)}: {msg}")


class _Cfg(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("window", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("softmax_scale", ctypes.c_float),
                ("io_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]



_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64

# encoder-step weight and work structs (field order of include/vx.h)
STEM_KEYS = ("w1", "b1", "w2", "b2")
LAYER_KEYS = ("g_attn", "w_qkv", "b_q", "b_v", "w_o", "b_o", "g_ffn", "w_gate", "w_up", "w_down",
              "b_down")
WORK_KEYS = ("h", "q", "k", "v", "o", "u", "acc")


class _StemW(ctypes.Structure):
    _fields_ = [(k, _vp) for k in STEM_KEYS]


class _LayerW(ctypes.Structure):
    _fields_ = [(k, _vp) for k in LAYER_KEYS]


class _Work(ctypes.Structure):
    _fields_ = [(k, _vp) for k in WORK_KEYS]

_SIGS = {
    "vx_default_cfg": (None, [ctypes.POINTER(_Cfg)]),
    "vx_rope_table": (ctypes.c_int, [_vp, _i64, _i32, ctypes.POINTER(_Cfg), _vp]),
    "vx_rope_qk": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _vp, ctypes.POINTER(_Cfg), _vp]),
    "vx_swa_attn_prefill": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp,
                                           _i64, _i64, ctypes.POINTER(_Cfg), _vp]),
    "vx_swa_attn_prefill_workspace_size": (ctypes.c_size_t, [_i32, _i32, _i32,
                                                             ctypes.POINTER(_Cfg)]),
    "vx_swa_attn_prefill_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp,
                                                   _i32, ctypes.POINTER(_Cfg), _vp]),
    "vx_swa_attn_stream_step": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                               _i32, _i32, ctypes.POINTER(_Cfg), _vp]),
    "vx_kv_ring_append": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                         ctypes.POINTER(_Cfg), _vp]),
    "vx_swa_attn_stream_step_append": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                      _i32, _i32, _i32, _i32,
                                                      ctypes.POINTER(_Cfg), _vp]),
    "vx_swa_attn_prefill_varlen": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                                  _vp, ctypes.c_int64, ctypes.c_int64, _vp, _vp,
                                                  _vp, ctypes.POINTER(_Cfg), _vp]),
    "vx_default_gqa_cfg": (None, [ctypes.POINTER(_Cfg)]),
    "vx_gqa_attn_prefill": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, _i32,
                                           _vp, _i64, _i64, _vp, _vp, _vp, _vp,
                                           ctypes.POINTER(_Cfg), _vp]),
    "vx_gqa_attn_decode": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                          _i32, _i32, ctypes.POINTER(_Cfg), _vp]),
    "vx_linear": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]),
    "vx_enc_qkv_rope": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp,
                                       _vp, ctypes.POINTER(_Cfg), _vp]),
    "vx_enc_attn_step": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                        ctypes.POINTER(_Cfg), _vp]),
    "vx_rmsnorm": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, ctypes.c_float, _vp]),
    "vx_enc_stem_step": (ctypes.c_int, [_vp, _vp, ctypes.POINTER(_StemW), _vp, _i32, _i32, _i32,
                                        _i32, _vp]),
    "vx_enc_layer_step": (ctypes.c_int, [_vp, ctypes.POINTER(_LayerW), _vp, _vp, _vp, _vp,
                                         ctypes.POINTER(_Work), _i32, _i32, _i32, _i32, _i32,
                                         ctypes.c_float, ctypes.POINTER(_Cfg), _vp]),
    "vx_enc_step": (ctypes.c_int, [_vp, _vp, ctypes.POINTER(_StemW), ctypes.POINTER(_LayerW), _i32,
                                   _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(_Work), _i32, _i32, _i32,
                                   _i32, _i32, _i32, ctypes.c_float, ctypes.POINTER(_Cfg), _vp]),
    "vx_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "vx_last_error": (ctypes.c_char_p, []),
    "vx_version": (_i32, []),
}
_lib = None


def lib():
    """The loaded libvx.so (ctypes).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sliding_window_attention_vx_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


class Config:
    """Attention parameters (mirrors vx_attn_cfg)."""

    def __init__(self, window=WINDOW, theta=THETA, scale=0.0, io_dtype="bf16", out_dtype=None,
                 valu=False, head_dim=HEAD_DIM, workspace=None, force_split=False):
        self.head_dim = int(head_dim)
        self.window = int(window)
        self.theta = float(theta)
        self.scale = float(scale)
        self.io_dtype = io_dtype
        self.out_dtype = out_dtype or io_dtype
        self.valu = bool(valu)
        self.workspace = workspace  # device tensor or None
        self.force_split = bool(force_split)

    def c(self):
        d = {"bf16": VX_BF16, "f32": VX_F32}
        ws = self.workspace
        return _Cfg(self.head_dim, self.window, self.theta, self.scale, d[self.io_dtype],
                    d[self.out_dtype],
                    (VX_FLAG_VALU_KERNEL if self.valu else 0)
                    | (VX_FLAG_SPLIT_WALK if self.force_split else 0),
                    None if ws is None else ws.data_ptr(),
                    0 if ws is None else ws.numel() * ws.element_size())


def _check(status, func):
    if status != 0:
        raise VxError(status, func, lib().vx_last_error().decode())


def _dt(t):
    import torch
    if t.dtype == torch.bfloat16:
        return "bf16"
    if t.dtype == torch.float32:
        return "f32"
    raise ValueError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev_tensor(t, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def rope_table(p_begin, count, theta=THETA, device="cuda", out=None, head_dim=HEAD_DIM):
    """cos/sin table [count, 2, head_dim/2] float32 for positions p_begin .. p_begin+count-1."""
    import torch
    if out is None:
        out = torch.empty((count, 2, head_dim // 2), dtype=torch.float32, device=device)
    _dev_tensor(out, "out")
    cfg = Config(theta=theta, head_dim=head_dim).c()
    _check(lib().vx_rope_table(_ptr(out), int(p_begin), int(count), ctypes.byref(cfg),
                               _stream(out)), "vx_rope_table")
    return out


def _pos0(pos0, B, device):
    """pos0 as a device int64 [B] tensor (None: positions start at 0)."""
    import torch
    if pos0 is None:
        return None
    if isinstance(pos0, torch.Tensor):
        _dev_tensor(pos0, "pos0")
        if pos0.dtype != torch.int64 or pos0.shape != (B,):
            raise ValueError(f"pos0 must be an int64 tensor of shape ({B},)")
        return pos0
    return torch.full((B,), int(pos0), dtype=torch.int64, device=device)


def _table(table, head_dim):
    """A caller's cos/sin table: float32 [rows, 2, head_dim/2] on the GPU."""
    import torch
    _dev_tensor(table, "table")
    if table.dtype != torch.float32 or table.dim() != 3 or table.shape[1:] != (2, head_dim // 2):
        raise ValueError(f"table must be float32 [rows, 2, {head_dim // 2}] (from rope_table "
                         f"with head_dim {head_dim})")
    return table


def rope_qk(q, k, pos0=None, theta=THETA):
    """Rotate q and k [B,T,H,64] in place (either may be None).

    pos0: None (row t at position t), an int (the same first position for
    every batch entry) or a device int64 tensor [B] (entry b starts at pos0[b]).
    """
    t = q if q is not None else k
    for name, x in (("q", q), ("k", k)):
        if x is not None:
            _dev_tensor(x, name)
            if x.shape != t.shape or x.dtype != t.dtype:
                raise ValueError("q and k must have the same shape and dtype")
    if t.dim() != 4 or t.shape[-1] != HEAD_DIM:
        raise ValueError("expected [B, T, H, 64]")
    B, T, H, _ = t.shape
    p0 = _pos0(pos0, B, t.device)
    cfg = Config(theta=theta, io_dtype=_dt(t)).c()
    _check(lib().vx_rope_qk(_ptr(q), _ptr(k), B, T, H, _ptr(p0), ctypes.byref(cfg), _stream(t)),
           "vx_rope_qk")


def prefill_workspace_size(B, T, H, window=WINDOW, theta=THETA, force_split=False):
    """Bytes of workspace with which prefill() of this shape keeps its cos/sin table
    there and takes the split walk (small grids) or rotates its keys ahead (large ones)."""
    cfg = Config(window, theta, force_split=force_split).c()
    return int(lib().vx_swa_attn_prefill_workspace_size(int(B), int(T), int(H), ctypes.byref(cfg)))


def prefill_workspace(B, T, H, window=WINDOW, device="cuda", force_split=False):
    """A workspace of prefill_workspace_size() bytes (reusable across calls on one stream)."""
    import torch
    n = prefill_workspace_size(B, T, H, window, force_split=force_split)
    return torch.empty((n + 15) // 16 * 16, dtype=torch.uint8, device=device)


def prefill(q, k, v, window=WINDOW, pos0=None, theta=THETA, scale=0.0, rope_applied=False,
            table=None, table_p0=0, out=None, out_dtype=None, valu=False, workspace=None,
            auto_table=True, force_split=False):
    """Causal sliding-window attention over whole chunks; q,k,v [B,T,H,64] -> o [B,T,H,64].

    pos0: None (positions 0..T-1), an int, or a device int64 tensor [B] (entry b
    at positions pos0[b] .. pos0[b]+T-1).  With rope_applied=False the kernel
    rotates q and k with cos/sin from `table` (rope_table rows starting at
    position table_p0).  Without a table: for pos0 None or an int a table of
    the chunk's positions is made here (auto_table=True); otherwise the
    library builds one in the workspace if it has room, else computes cos/sin
    in the kernel.  workspace: a uint8 device tensor (prefill_workspace), reused
    across calls; None runs without one.  With a workspace and force_split,
    grids of at most 1.5 128-query tiles per compute unit take the split
    walk (two workgroups per query tile).  Grids of at least 8 tiles per
    unit with a table rotate their keys once, into the workspace, ahead of
    the attention kernel (the same bits).
    """
    import torch
    for name, x in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(x, name)
    if not (q.shape == k.shape == v.shape) or q.dim() != 4 or q.shape[-1] != HEAD_DIM:
        raise ValueError("q, k, v must all be [B, T, H, 64]")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    B, T, H, _ = q.shape
    io = _dt(q)
    od = out_dtype or (_dt(out) if out is not None else io)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16 if od == "bf16" else torch.float32,
                          device=q.device)
    _dev_tensor(out, "out")
    if out.shape != q.shape or _dt(out) != od:
        raise ValueError("out has the wrong shape or dtype")
    p0 = _pos0(pos0, B, q.device)
    tlen = 0
    if not rope_applied and table is None and not isinstance(pos0, torch.Tensor) and auto_table:
        # one position range for every entry: a table of exactly those rows
        first = 0 if pos0 is None else int(pos0)
        table = rope_table(first, max(T, 1), theta, device=q.device)
        table_p0 = first
    if not rope_applied and table is not None:
        _table(table, HEAD_DIM)
        tlen = table.shape[0]
    if workspace is not None:
        _dev_tensor(workspace, "workspace")
        if workspace.dtype != torch.uint8:
            raise ValueError("workspace must be a uint8 tensor (see prefill_workspace)")
    cfg = Config(window, theta, scale, io, od, valu, workspace=workspace,
                 force_split=force_split).c()
    _check(lib().vx_swa_attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, T, H, _ptr(p0),
                                     int(bool(rope_applied)),
                                     _ptr(table) if not rope_applied else None, int(table_p0),
                                     int(tlen), ctypes.byref(cfg), _stream(q)),
           "vx_swa_attn_prefill")
    return out


def prefill_noalloc(q, k, v, window=WINDOW, pos0=None, theta=THETA, scale=0.0,
                    rope_applied=False, out=None, out_dtype=None):
    """prefill() whose cos/sin rows live in the library's static device scratch
    (no workspace, nothing allocated by the library); B*T <= 65536 rows."""
    import torch
    for name, x in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(x, name)
    if not (q.shape == k.shape == v.shape) or q.dim() != 4 or q.shape[-1] != HEAD_DIM:
        raise ValueError("q, k, v must all be [B, T, H, 64]")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    B, T, H, _ = q.shape
    io = _dt(q)
    od = out_dtype or (_dt(out) if out is not None else io)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16 if od == "bf16" else torch.float32,
                          device=q.device)
    _dev_tensor(out, "out")
    if out.shape != q.shape or _dt(out) != od:
        raise ValueError("out has the wrong shape or dtype")
    p0 = _pos0(pos0, B, q.device)
    cfg = Config(window, theta, scale, io, od).c()
    _check(lib().vx_swa_attn_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, T, H,
                                             _ptr(p0), int(bool(rope_applied)),
                                             ctypes.byref(cfg), _stream(q)),
           "vx_swa_attn_prefill_noalloc")
    return out


def prefill_varlen(q, k, v, cu_seqlens, max_T, window=WINDOW, theta=THETA, scale=0.0,
                   rope_applied=False, table=None, ring_k=None, ring_v=None, pos=None, out=None,
                   out_dtype=None):
    """Batched first-chunk prefill: streams packed along the frame axis.

    q, k, v: bf16 [total, H, 64]; stream s is rows cu_seqlens[s] .. cu_seqlens[s+1]-1
    (cu_seqlens: int32 device tensor [S+1]), at positions 0 .. T_s-1, T_s <= max_T.
    With ring_k, ring_v ([S, H, W, 64] bf16) and pos (int64 [S]) the rings are
    seeded with the chunk's last W rotated keys and values and pos[s] = T_s.
    """
    import torch
    for name, x in (("q", q), ("k", k), ("v", v), ("cu_seqlens", cu_seqlens)):
        _dev_tensor(x, name)
    if not (q.shape == k.shape == v.shape) or q.dim() != 3 or q.shape[-1] != HEAD_DIM:
        raise ValueError("q, k, v must all be [total, H, 64]")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be int32 [S+1]")
    S = cu_seqlens.numel() - 1
    H = q.shape[1]
    io = _dt(q)
    od = out_dtype or (_dt(out) if out is not None else io)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16 if od == "bf16" else torch.float32,
                          device=q.device)
    _dev_tensor(out, "out")
    if out.shape != q.shape or _dt(out) != od:
        raise ValueError("out has the wrong shape or dtype")
    tlen = 0
    if not rope_applied and table is not None:
        _table(table, HEAD_DIM)
        tlen = table.shape[0]
    if ring_k is not None:
        for name, x in (("ring_k", ring_k), ("ring_v", ring_v), ("pos", pos)):
            if x is None:
                raise ValueError("ring seeding needs ring_k, ring_v and pos")
            _dev_tensor(x, name)
        if ring_k.shape != (S, H, window, HEAD_DIM) or ring_v.shape != ring_k.shape:
            raise ValueError(f"rings must be [S, H, W, 64] = {(S, H, window, HEAD_DIM)}")
        if pos.dtype != torch.int64 or pos.shape != (S,):
            raise ValueError("pos must be int64 [S]")
    cfg = Config(window, theta, scale, io, od).c()
    _check(lib().vx_swa_attn_prefill_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(cu_seqlens), S, q.shape[0], int(max_T), H,
        int(bool(rope_applied)), _ptr(table) if not rope_applied else None, 0, int(tlen),
        _ptr(ring_k), _ptr(ring_v), _ptr(pos),
        ctypes.byref(cfg), _stream(q)), "vx_swa_attn_prefill_varlen")
    return out


def _stream_shapes(q_new, ring_k, ring_v, pos, window):
    if q_new.dim() != 4 or q_new.shape[-1] != HEAD_DIM:
        raise ValueError("new frames must be [S, n, H, 64]")
    S, n, H, _ = q_new.shape
    if ring_k.shape != (S, H, window, HEAD_DIM) or ring_v.shape != ring_k.shape:
        raise ValueError(f"rings must be [S, H, W, 64] = {(S, H, window, HEAD_DIM)}")
    import torch
    if pos.dtype != torch.int64 or pos.shape != (S,):
        raise ValueError("pos must be int64 [S]")
    return S, n, H


def stream_step(q_new, k_new, v_new, ring_k, ring_v, pos, window=WINDOW, theta=THETA, scale=0.0,
                rope_applied=False, out=None, out_dtype=None):
    """One streaming step (reads the rings and pos, writes o [S,n,H,64])."""
    import torch
    for name, x in (("q_new", q_new), ("k_new", k_new), ("v_new", v_new), ("ring_k", ring_k),
                    ("ring_v", ring_v), ("pos", pos)):
        _dev_tensor(x, name)
    S, n, H = _stream_shapes(q_new, ring_k, ring_v, pos, window)
    if k_new.shape != q_new.shape or v_new.shape != q_new.shape:
        raise ValueError("q_new, k_new, v_new must have the same shape")
    io = _dt(q_new)
    if any(_dt(x) != io for x in (k_new, v_new, ring_k, ring_v)):
        raise ValueError("new frames and rings must share a dtype")
    od = out_dtype or (_dt(out) if out is not None else io)
    if out is None:
        out = torch.empty(q_new.shape, dtype=torch.bfloat16 if od == "bf16" else torch.float32,
                          device=q_new.device)
    _dev_tensor(out, "out")
    if out.shape != q_new.shape or _dt(out) != od:
        raise ValueError("out has the wrong shape or dtype")
    cfg = Config(window, theta, scale, io, od).c()
    _check(lib().vx_swa_attn_stream_step(_ptr(q_new), _ptr(k_new), _ptr(v_new), _ptr(ring_k),
                                         _ptr(ring_v), _ptr(pos), _ptr(out), S, n, H,
                                         int(bool(rope_applied)), ctypes.byref(cfg),
                                         _stream(q_new)), "vx_swa_attn_stream_step")
    return out


def ring_append(ring_k, ring_v, k_new, v_new, pos, window=WINDOW, theta=THETA, rope_applied=False):
    """Append the new frames to the rings in place and advance pos by n."""
    for name, x in (("k_new", k_new), ("v_new", v_new), ("ring_k", ring_k), ("ring_v", ring_v),
                    ("pos", pos)):
        _dev_tensor(x, name)
    S, n, H = _stream_shapes(k_new, ring_k, ring_v, pos, window)
    if v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must have the same shape")
    io = _dt(k_new)
    cfg = Config(window, theta, 0.0, io, io).c()
    _check(lib().vx_kv_ring_append(_ptr(ring_k), _ptr(ring_v), _ptr(k_new), _ptr(v_new), _ptr(pos),
                                   S, n, H, int(bool(rope_applied)), ctypes.byref(cfg),
                                   _stream(k_new)), "vx_kv_ring_append")


def stream_step_append(q_new, k_new, v_new, ring_k, ring_v, pos_in, pos_out, window=WINDOW,
                       theta=THETA, scale=0.0, rope_applied=False, out=None, out_dtype=None):
    """Streaming step plus ring append in one call; pos_out[s] = pos_in[s] + n (distinct arrays)."""
    import torch
    for name, x in (("q_new", q_new), ("k_new", k_new), ("v_new", v_new), ("ring_k", ring_k),
                    ("ring_v", ring_v), ("pos_in", pos_in), ("pos_out", pos_out)):
        _dev_tensor(x, name)
    S, n, H = _stream_shapes(q_new, ring_k, ring_v, pos_in, window)
    if pos_out.shape != pos_in.shape or pos_out.dtype != pos_in.dtype:
        raise ValueError("pos_out must be int64 [S]")
    if k_new.shape != q_new.shape or v_new.shape != q_new.shape:
        raise ValueError("q_new, k_new, v_new must have the same shape")
    io = _dt(q_new)
    if any(_dt(x) != io for x in (k_new, v_new, ring_k, ring_v)):
        raise ValueError("new frames and rings must share a dtype")
    od = out_dtype or (_dt(out) if out is not None else io)
    if out is None:
        out = torch.empty(q_new.shape, dtype=torch.bfloat16 if od == "bf16" else torch.float32,
                          device=q_new.device)
    _dev_tensor(out, "out")
    if out.shape != q_new.shape or _dt(out) != od:
        raise ValueError("out has the wrong shape or dtype")
    cfg = Config(window, theta, scale, io, od).c()
    _check(lib().vx_swa_attn_stream_step_append(
        _ptr(q_new), _ptr(k_new), _ptr(v_new), _ptr(ring_k), _ptr(ring_v), _ptr(pos_in),
        _ptr(pos_out), _ptr(out), S, n, H, int(bool(rope_applied)), ctypes.byref(cfg),
        _stream(q_new)), "vx_swa_attn_stream_step_append")
    return out


# ---------------------------------------------------------------------------
# grouped-query attention, head_dim 128 (the text decoder)
# ---------------------------------------------------------------------------

def gqa_prefill(q, k, v, window=DEC_WINDOW, pos0=0, theta=THETA, scale=0.0, rope_applied=False,
                table=None, table_p0=0, ring_k=None, ring_v=None, pos=None, out=None,
                out_dtype=None, k_rot=None):
    """Grouped-query prompt prefill: q [B,T,Hq,128], k, v [B,T,Hkv,128] bf16 -> o [B,T,Hq,128].

    Query head h reads key/value head h // (Hq // Hkv).  With ring_k, ring_v
    ([B, Hkv, W, 128] bf16) and pos (int64 [B]) the rings are seeded with the
    prompt's last W rotated keys and values and pos[b] = T (needs pos0 = 0).
    With k_rot (bf16, k's shape) the keys are rotated once into k_rot first
    and the attention reads them from there (same results, faster).
    """
    import torch
    for name, x in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(x, name)
    if q.dim() != 4 or q.shape[-1] != DEC_HEAD_DIM or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, T, Hq, 128] and k, v [B, T, Hkv, 128]")
    B, T, Hq, _ = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, T, Hkv, DEC_HEAD_DIM):
        raise ValueError("k and v must be [B, T, Hkv, 128] with q's B and T")
    if any(_dt(x) != "bf16" for x in (q, k, v)):
        raise ValueError("q, k, v must be bfloat16")
    od = out_dtype or (_dt(out) if out is not None else "bf16")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16 if od == "bf16" else torch.float32,
                          device=q.device)
    _dev_tensor(out, "out")
    if out.shape != q.shape or _dt(out) != od:
        raise ValueError("out has the wrong shape or dtype")
    tlen = 0
    if not rope_applied:
        if table is None:
            table = rope_table(pos0, max(T, 1), theta, device=q.device, head_dim=DEC_HEAD_DIM)
            table_p0 = pos0
        _table(table, DEC_HEAD_DIM)
        tlen = table.shape[0]
    if ring_k is not None or ring_v is not None:
        for name, x in (("ring_k", ring_k), ("ring_v", ring_v), ("pos", pos)):
            if x is None:
                raise ValueError("ring seeding needs ring_k, ring_v and pos")
            _dev_tensor(x, name)
        want = (B, Hkv, window, DEC_HEAD_DIM)
        if ring_k.shape != want or ring_v.shape != want:
            raise ValueError(f"rings must be [B, Hkv, W, 128] = {want}")
        if pos.dtype != torch.int64 or pos.shape != (B,):
            raise ValueError("pos must be int64 [B]")
    if k_rot is not None:
        _dev_tensor(k_rot, "k_rot")
        if k_rot.shape != k.shape or _dt(k_rot) != "bf16":
            raise ValueError("k_rot must be bfloat16 with k's shape")
    cfg = Config(window, theta, scale, "bf16", od, head_dim=DEC_HEAD_DIM).c()
    _check(lib().vx_gqa_attn_prefill(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, T, Hq, Hkv, int(pos0), int(bool(rope_applied)),
        _ptr(table), int(table_p0), int(tlen), _ptr(ring_k), _ptr(ring_v), _ptr(pos),
        _ptr(k_rot), ctypes.byref(cfg), _stream(q)), "vx_gqa_attn_prefill")
    return out


def gqa_decode(q_new, k_new, v_new, ring_k, ring_v, pos_in, pos_out, window=DEC_WINDOW,
               theta=THETA, scale=0.0, rope_applied=False, out=None, out_dtype=None):
    """One grouped-query decode step with its ring append.

    q_new [S,n,Hq,128], k_new/v_new [S,n,Hkv,128] bf16; rings [S,Hkv,W,128]
    bf16; pos_in/pos_out int64 [S], distinct (pos_out = pos_in + n).
    """
    import torch
    for name, x in (("q_new", q_new), ("k_new", k_new), ("v_new", v_new), ("ring_k", ring_k),
                    ("ring_v", ring_v), ("pos_in", pos_in), ("pos_out", pos_out)):
        _dev_tensor(x, name)
    if q_new.dim() != 4 or q_new.shape[-1] != DEC_HEAD_DIM:
        raise ValueError("q_new must be [S, n, Hq, 128]")
    S, n, Hq, _ = q_new.shape
    Hkv = k_new.shape[2] if k_new.dim() == 4 else -1
    if k_new.shape != (S, n, Hkv, DEC_HEAD_DIM) or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must be [S, n, Hkv, 128]")
    want = (S, Hkv, window, DEC_HEAD_DIM)
    if ring_k.shape != want or ring_v.shape != want:
        raise ValueError(f"rings must be [S, Hkv, W, 128] = {want}")
    for x in (pos_in, pos_out):
        if x.dtype != torch.int64 or x.shape != (S,):
            raise ValueError("pos_in and pos_out must be int64 [S]")
    if any(_dt(x) != "bf16" for x in (q_new, k_new, v_new, ring_k, ring_v)):
        raise ValueError("new tokens and rings must be bfloat16")
    od = out_dtype or (_dt(out) if out is not None else "bf16")
    if out is None:
        out = torch.empty(q_new.shape, dtype=torch.bfloat16 if od == "bf16" else torch.float32,
                          device=q_new.device)
    _dev_tensor(out, "out")
    if out.shape != q_new.shape or _dt(out) != od:
        raise ValueError("out has the wrong shape or dtype")
    cfg = Config(window, theta, scale, "bf16", od, head_dim=DEC_HEAD_DIM).c()
    _check(lib().vx_gqa_attn_decode(
        _ptr(q_new), _ptr(k_new), _ptr(v_new), _ptr(ring_k), _ptr(ring_v), _ptr(pos_in),
        _ptr(pos_out), _ptr(out), S, n, Hq, Hkv, int(bool(rope_applied)), ctypes.byref(cfg),
        _stream(q_new)), "vx_gqa_attn_decode")
    return out


# ---------------------------------------------------------------------------
# projections around the encoder's attention (bf16 matrix cores)
# ---------------------------------------------------------------------------

def _bf16_dev(t, name):
    _dev_tensor(t, name)
    if _dt(t) != "bf16":
        raise ValueError(f"{name} must be bfloat16")
    return t


def linear(x, w, bias=None, out=None, out_dtype="bf16"):
    """y = x w^T (+ bias): x [M, K], w [N, K], bias [N] bf16 -> y [M, N] (bf16 or f32).

    K must be a multiple of 128 and N of 32.
    """
    import torch
    _bf16_dev(x, "x")
    _bf16_dev(w, "w")
    if bias is not None:
        _bf16_dev(bias, "bias")
    if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("x must be [M, K] and w [N, K]")
    M, K = x.shape
    N = w.shape[0]
    if bias is not None and bias.shape != (N,):
        raise ValueError("bias must be [N]")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32,
                          device=x.device)
    _dev_tensor(out, "out")
    if out.shape != (M, N):
        raise ValueError("out must be [M, N]")
    od = VX_BF16 if _dt(out) == "bf16" else VX_F32
    _check(lib().vx_linear(_ptr(x), _ptr(w), _ptr(bias), _ptr(out), M, N, K, od, _stream(x)),
           "vx_linear")
    return out


def enc_qkv_rope(x, w_qkv, b_q, b_v, pos, H=32, theta=THETA, q=None, k=None, v=None):
    """Fused q/k/v projection with RoPE: x [S, n, d_model] -> q', k', v [S, n, H, 64] bf16.

    w_qkv [3*H*64, d_model] holds the q rows, then k, then v; k has no bias;
    frame i of stream s sits at position pos[s] + i.
    """
    import torch
    for name, t in (("x", x), ("w_qkv", w_qkv)):
        _bf16_dev(t, name)
    for name, t in (("b_q", b_q), ("b_v", b_v)):
        if t is not None:
            _bf16_dev(t, name)
    _dev_tensor(pos, "pos")
    if x.dim() != 3:
        raise ValueError("x must be [S, n, d_model]")
    S, n, dm = x.shape
    if w_qkv.shape != (3 * H * HEAD_DIM, dm):
        raise ValueError(f"w_qkv must be [3*H*64, d_model] = {(3 * H * HEAD_DIM, dm)}")
    if pos.dtype != torch.int64 or pos.shape != (S,):
        raise ValueError("pos must be int64 [S]")
    outs = []
    for t in (q, k, v):
        if t is None:
            t = torch.empty((S, n, H, HEAD_DIM), dtype=torch.bfloat16, device=x.device)
        _bf16_dev(t, "q/k/v")
        if t.shape != (S, n, H, HEAD_DIM):
            raise ValueError("q, k, v must be [S, n, H, 64]")
        outs.append(t)
    cfg = Config(theta=theta).c()
    _check(lib().vx_enc_qkv_rope(_ptr(x), _ptr(w_qkv), _ptr(b_q), _ptr(b_v), _ptr(pos), S, n, H,
                                 dm, _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]),
                                 ctypes.byref(cfg), _stream(x)), "vx_enc_qkv_rope")
    return tuple(outs)


def enc_attn_step(x, w_qkv, b_q, b_v, w_o, b_o, ring_k, ring_v, pos_in, pos_out, window=WINDOW,
                  theta=THETA, scale=0.0, H=32, work=None, out=None, out_dtype="bf16"):
    """One streaming step of the encoder's attention block (three launches):
    q', k', v = x W_qkv^T (+ b_q, b_v) rotated at pos_in[s] + i; attention over
    the rings and the new frames, with the ring append; y = o W_o^T + b_o.

    x [S, n, d_model] bf16; rings [S, H, W, 64] bf16; pos_in/pos_out int64 [S]
    (distinct); work: optional dict of bf16 [S, n, H, 64] buffers q, k, v, o.
    Returns y [S, n, d_model].
    """
    import torch
    for name, t in (("x", x), ("w_qkv", w_qkv), ("w_o", w_o), ("ring_k", ring_k),
                    ("ring_v", ring_v)):
        _bf16_dev(t, name)
    for name, t in (("b_q", b_q), ("b_v", b_v), ("b_o", b_o)):
        if t is not None:
            _bf16_dev(t, name)
    for name, t in (("pos_in", pos_in), ("pos_out", pos_out)):
        _dev_tensor(t, name)
    if x.dim() != 3:
        raise ValueError("x must be [S, n, d_model]")
    S, n, dm = x.shape
    if w_qkv.shape != (3 * H * HEAD_DIM, dm) or w_o.shape != (dm, H * HEAD_DIM):
        raise ValueError("w_qkv must be [3*H*64, d_model] and w_o [d_model, H*64]")
    if ring_k.shape != (S, H, window, HEAD_DIM) or ring_v.shape != ring_k.shape:
        raise ValueError(f"rings must be [S, H, W, 64] = {(S, H, window, HEAD_DIM)}")
    for t in (pos_in, pos_out):
        if t.dtype != torch.int64 or t.shape != (S,):
            raise ValueError("pos_in and pos_out must be int64 [S]")
    work = dict(work or {})
    for key in ("q", "k", "v", "o"):
        if key not in work:
            work[key] = torch.empty((S, n, H, HEAD_DIM), dtype=torch.bfloat16, device=x.device)
        _bf16_dev(work[key], key)
        if work[key].shape != (S, n, H, HEAD_DIM):
            raise ValueError("work buffers must be [S, n, H, 64]")
    if out is None:
        out = torch.empty((S, n, dm), dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32,
                          device=x.device)
    _dev_tensor(out, "out")
    if out.shape != (S, n, dm):
        raise ValueError("out must be [S, n, d_model]")
    cfg = Config(window, theta, scale, "bf16", _dt(out)).c()
    _check(lib().vx_enc_attn_step(
        _ptr(x), _ptr(w_qkv), _ptr(b_q), _ptr(b_v), _ptr(w_o), _ptr(b_o), _ptr(ring_k),
        _ptr(ring_v), _ptr(pos_in), _ptr(pos_out), _ptr(work["q"]), _ptr(work["k"]),
        _ptr(work["v"]), _ptr(work["o"]), _ptr(out), S, n, H, dm, ctypes.byref(cfg),
        _stream(x)), "vx_enc_attn_step")
    return out


# ---------------------------------------------------------------------------
# the streaming encoder step: stem, pre-norm layers (residual stream float32)
# ---------------------------------------------------------------------------

def rmsnorm(x, g, eps=1e-5, out=None):
    """y = x / sqrt(mean(x^2) + eps) * g per row: x float32 [..., dim], g bf16 [dim] -> bf16."""
    import torch
    _dev_tensor(x, "x")
    if x.dtype != torch.float32:
        raise ValueError("x must be float32")
    _bf16_dev(g, "g")
    dim = x.shape[-1]
    if g.shape != (dim,):
        raise ValueError("g must be [dim]")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    _bf16_dev(out, "out")
    if out.shape != x.shape:
        raise ValueError("out must have x's shape")
    M = x.numel() // dim if dim else 0
    _check(lib().vx_rmsnorm(_ptr(x), _ptr(g), _ptr(out), M, dim, float(eps), _stream(x)),
           "vx_rmsnorm")
    return out


def enc_work(S, n, H, d_model, ffn, device="cuda"):
    """Work buffers of a layer step: bf16 h, q, k, v, o, u and the float32
    partial sums acc [2, S*n, d_model]."""
    import torch
    M = S * n
    shapes = dict(h=(M, d_model), q=(M, H * HEAD_DIM), k=(M, H * HEAD_DIM), v=(M, H * HEAD_DIM),
                  o=(M, H * HEAD_DIM), u=(M, ffn))
    work = {k: torch.empty(v, dtype=torch.bfloat16, device=device) for k, v in shapes.items()}
    work["acc"] = torch.empty((2, M, d_model), dtype=torch.float32, device=device)
    return work


def _stem_struct(stem):
    for k in ("w1", "w2"):
        _bf16_dev(stem[k], k)
    for k in ("b1", "b2"):
        if stem.get(k) is not None:
            _bf16_dev(stem[k], k)
    return _StemW(*[_ptr(stem.get(k)) for k in STEM_KEYS])


def _layer_struct(w, H, dm, ffn):
    shapes = dict(g_attn=(dm,), w_qkv=(3 * H * HEAD_DIM, dm), b_q=(H * HEAD_DIM,),
                  b_v=(H * HEAD_DIM,), w_o=(dm, H * HEAD_DIM), b_o=(dm,), g_ffn=(dm,),
                  w_gate=(ffn, dm), w_up=(ffn, dm), w_down=(dm, ffn), b_down=(dm,))
    for k in LAYER_KEYS:
        t = w.get(k)
        if t is None:
            if not k.startswith("b_"):
                raise ValueError(f"layer weight {k} is required")
            continue
        _bf16_dev(t, k)
        if tuple(t.shape) != shapes[k]:
            raise ValueError(f"layer weight {k} must be {shapes[k]}, got {tuple(t.shape)}")
    return _LayerW(*[_ptr(w.get(k)) for k in LAYER_KEYS])


def _work_struct(work, S, n, H, dm, ffn, device):
    import torch
    work = dict(work) if work is not None else enc_work(S, n, H, dm, ffn, device)
    for k in WORK_KEYS[:-1]:
        _bf16_dev(work[k], k)
    _dev_tensor(work["acc"], "acc")
    if work["acc"].dtype != torch.float32 or work["acc"].numel() < 2 * S * n * dm:
        raise ValueError("work['acc'] must be float32 with 2 * S * n * d_model elements")
    return work, _Work(*[_ptr(work[k]) for k in WORK_KEYS])


def _stem_shapes(mel_buf, c1_buf):
    _bf16_dev(mel_buf, "mel_buf")
    _bf16_dev(c1_buf, "c1_buf")
    if mel_buf.dim() != 3 or c1_buf.dim() != 3 or mel_buf.shape[:2] != c1_buf.shape[:2]:
        raise ValueError("mel_buf must be [S, 2n+2, n_mels] and c1_buf [S, 2n+2, d_model]")
    S, F, n_mels = mel_buf.shape
    if F < 4 or F % 2:
        raise ValueError("the buffers hold 2n+2 frame slots (n >= 1)")
    return S, (F - 2) // 2, n_mels, c1_buf.shape[2]


def enc_stem_step(mel_buf, c1_buf, stem, x_out=None):
    """The stem for one step: both causal convolutions (+ GELU) over the frame
    buffers, then the move of each buffer's last two slots to slots 0-1.

    mel_buf [S, 2n+2, n_mels] bf16 (slots 2.. hold the step's 2n mel frames),
    c1_buf [S, 2n+2, d_model] bf16, stem: dict w1 [d_model, 3, n_mels], b1,
    w2 [d_model, 3, d_model], b2.  Returns x_out [S, n, d_model] float32.
    """
    import torch
    S, n, n_mels, dm = _stem_shapes(mel_buf, c1_buf)
    if x_out is None:
        x_out = torch.empty((S, n, dm), dtype=torch.float32, device=mel_buf.device)
    _dev_tensor(x_out, "x_out")
    if x_out.dtype != torch.float32 or x_out.shape != (S, n, dm):
        raise ValueError("x_out must be float32 [S, n, d_model]")
    sw = _stem_struct(stem)
    _check(lib().vx_enc_stem_step(_ptr(mel_buf), _ptr(c1_buf), ctypes.byref(sw), _ptr(x_out), S, n,
                                  n_mels, dm, _stream(mel_buf)), "vx_enc_stem_step")
    return x_out


def _layer_common(x, ring_k, ring_v, pos_in, pos_out, window, H, L=None):
    import torch
    _dev_tensor(x, "x")
    if x.dtype != torch.float32 or x.dim() != 3:
        raise ValueError("x must be float32 [S, n, d_model]")
    S, n, dm = x.shape
    want = (S, H, window, HEAD_DIM) if L is None else (L, S, H, window, HEAD_DIM)
    for name, t in (("ring_k", ring_k), ("ring_v", ring_v)):
        _bf16_dev(t, name)
        if t.shape != want:
            raise ValueError(f"{name} must be {want}")
    for name, t in (("pos_in", pos_in), ("pos_out", pos_out)):
        _dev_tensor(t, name)
        if t.dtype != torch.int64 or t.shape != (S,):
            raise ValueError("pos_in and pos_out must be int64 [S]")
    return S, n, dm


def enc_layer_step(x, wts, ring_k, ring_v, pos_in, pos_out, window=WINDOW, theta=THETA, scale=0.0,
                   H=32, eps=1e-5, work=None):
    """One pre-norm layer (seven launches), updating the float32 residual x
    [S, n, d_model] in place: x += attn(rmsnorm(x) g_attn), then
    x += W_down(silu(h W_gate^T) (h W_up^T)) + b_down, h = rmsnorm(x) g_ffn.
    wts: dict of bf16 tensors (LAYER_KEYS; biases optional); rings
    [S, H, W, 64] bf16; pos_in/pos_out int64 [S] (distinct)."""
    S, n, dm = _layer_common(x, ring_k, ring_v, pos_in, pos_out, window, H)
    ffn = wts["w_gate"].shape[0]
    lw = _layer_struct(wts, H, dm, ffn)
    work, ws = _work_struct(work, S, n, H, dm, ffn, x.device)
    cfg = Config(window, theta, scale, "bf16", "bf16").c()
    _check(lib().vx_enc_layer_step(_ptr(x), ctypes.byref(lw), _ptr(ring_k), _ptr(ring_v),
                                   _ptr(pos_in), _ptr(pos_out), ctypes.byref(ws), S, n, H, dm, ffn,
                                   float(eps), ctypes.byref(cfg), _stream(x)), "vx_enc_layer_step")
    return x


def enc_step(mel_buf, c1_buf, stem, layers, ring_k, ring_v, pos_in, pos_out, x=None,
             window=WINDOW, theta=THETA, scale=0.0, H=32, eps=1e-5, work=None):
    """A whole encoder step: the stem into x [S, n, d_model] float32, then
    the L = len(layers) layers in order (ring_k, ring_v [L, S, H, W, 64] bf16;
    every layer reads pos_in and writes pos_out).  Returns x."""
    import torch
    S, n, n_mels, dm = _stem_shapes(mel_buf, c1_buf)
    if x is None:
        x = torch.empty((S, n, dm), dtype=torch.float32, device=mel_buf.device)
    L = len(layers)
    if L < 1:
        raise ValueError("need at least one layer")
    _layer_common(x, ring_k, ring_v, pos_in, pos_out, window, H, L)
    ffn = layers[0]["w_gate"].shape[0]
    arr = (_LayerW * L)(*[_layer_struct(w, H, dm, ffn) for w in layers])
    sw = _stem_struct(stem)
    work, ws = _work_struct(work, S, n, H, dm, ffn, x.device)
    cfg = Config(window, theta, scale, "bf16", "bf16").c()
    _check(lib().vx_enc_step(_ptr(mel_buf), _ptr(c1_buf), ctypes.byref(sw), arr, L, _ptr(ring_k),
                             _ptr(ring_v), _ptr(pos_in), _ptr(pos_out), _ptr(x), ctypes.byref(ws),
                             S, n, n_mels, H, dm, ffn, float(eps), ctypes.byref(cfg),
                             _stream(mel_buf)), "vx_enc_step")
    return x
