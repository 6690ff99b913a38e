"""Python access to the float64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the benchmark's CPU-baseline leg, never by the product package.  It shares
no code with the HIP library; inputs reach it as float64 copies of the
stored values.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def build():
    """Compile oracle.c into liboracle.so (gcc, OpenMP)."""
    subprocess.run(["sh", os.path.join(_HERE, "build.sh")], check=True)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    _lib = _configure(ctypes.CDLL(_LIB_PATH))
    return _lib


@contextlib.contextmanager
def using_library(path):
    """Temporarily route every oracle call to another build of oracle.c (tests only)."""
    global _lib
    saved = _load()
    _lib = _configure(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = saved


def _configure(lib):
    lib.oracle_bf16_round.restype = ctypes.c_double
    lib.oracle_bf16_round.argtypes = [ctypes.c_double]
    lib.oracle_bf16_round_array.restype = None
    lib.oracle_bf16_round_array.argtypes = [_dp, _i64]
    lib.oracle_rope.restype = None
    lib.oracle_rope.argtypes = [_dp, _i64, _i64, _i64, _i64, _i64p, ctypes.c_double, ctypes.c_int]
    lib.oracle_prefill.restype = ctypes.c_int
    lib.oracle_prefill.argtypes = [_dp, _dp, _dp, _dp, _i64, _i64, _i64, _i64, _i64, _i64p,
                                   ctypes.c_double, ctypes.c_double, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int]
    lib.oracle_stream_step.restype = ctypes.c_int
    lib.oracle_stream_step.argtypes = [_dp, _dp, _dp, _dp, _dp, _i64p, _dp, _i64, _i64, _i64,
                                       _i64, _i64, ctypes.c_double, ctypes.c_double, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int]
    lib.oracle_ring_append.restype = ctypes.c_int
    lib.oracle_ring_append.argtypes = [_dp, _dp, _dp, _dp, _i64p, _i64, _i64, _i64, _i64, _i64,
                                       ctypes.c_double, ctypes.c_int, ctypes.c_int]
    lib.oracle_gqa_prefill.restype = ctypes.c_int
    lib.oracle_gqa_prefill.argtypes = [_dp, _dp, _dp, _dp, _i64, _i64, _i64, _i64, _i64, _i64,
                                       _i64p, ctypes.c_double, ctypes.c_double, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int]
    lib.oracle_gqa_stream_step.restype = ctypes.c_int
    lib.oracle_gqa_stream_step.argtypes = [_dp, _dp, _dp, _dp, _dp, _i64p, _dp, _i64, _i64, _i64,
                                           _i64, _i64, _i64, ctypes.c_double, ctypes.c_double,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    return lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, t=_dp):
    return a.ctypes.data_as(t)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def bf16_round(x):
    """Round float64 values to the nearest bfloat16 value (ties to even)."""
    a = _f64(x).copy()
    _load().oracle_bf16_round_array(_ptr(a), a.size)
    return a


def rope(x, pos=None, theta=1e6, bf16=False):
    """Rotate x [B,T,H,D] (copy) with half-split RoPE; pos [B,T] absolute positions or None (= t)."""
    a = _f64(x).copy()
    B, T, H, D = a.shape
    p = None
    if pos is not None:
        p = np.ascontiguousarray(np.broadcast_to(np.asarray(pos, dtype=np.int64), (B, T)))
    _load().oracle_rope(_ptr(a), B, T, H, D, None if p is None else _ptr(p, _i64p),
                        float(theta), int(bool(bf16)))
    return a


def prefill(q, k, v, W, pos=None, theta=1e6, scale=None, bf16=False, rope_applied=False,
            nthreads=0):
    """Causal sliding-window attention over whole chunks; q,k,v [B,T,H,D] -> o [B,T,H,D] float64.

    pos: None (positions 0..T-1), an int offset (positions pos+t), or an array [B,T].
    bf16=True applies the bfloat16 contract (rotated q,k rounded to bf16).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, D = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    p = None
    if pos is not None:
        if np.isscalar(pos):
            p = (np.int64(pos) + np.arange(T, dtype=np.int64))[None, :].repeat(B, 0)
        else:
            p = np.broadcast_to(np.asarray(pos, dtype=np.int64), (B, T))
        p = np.ascontiguousarray(p, dtype=np.int64)
    o = np.zeros_like(q)
    rc = _load().oracle_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, T, H, D, int(W),
                                None if p is None else _ptr(p, _i64p), float(theta), float(scale),
                                int(bool(bf16)), int(bool(rope_applied)), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_prefill rejected its arguments")
    return o


def prefill_varlen(q, k, v, cu, W, ring_k=None, ring_v=None, pos=None, theta=1e6, bf16=False,
                   rope_applied=False):
    """Batched first-chunk prefill (Voxtral Mini 4B Realtime Core AI page: the
    batched first-chunk encoder runs a stream's whole first chunk in one call,
    the streaming encoder then continues from it).

    q, k, v: [total, H, D]; stream s is rows cu[s] .. cu[s+1]-1, an independent
    chunk at positions 0 .. T_s-1, attended exactly as prefill() does.  With
    rings ([S,H,W,D] float64, modified in place) and pos (int64 [S]), the chunk
    is then appended to stream s's ring from position 0 exactly as
    ring_append() does, so pos[s] = T_s and the last W frames sit in their
    slots.  A composition of prefill() and ring_append(); no new arithmetic.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = [int(c) for c in cu]
    o = np.zeros_like(q)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if b > a:
            o[a:b] = prefill(q[None, a:b], k[None, a:b], v[None, a:b], W, theta=theta, bf16=bf16,
                             rope_applied=rope_applied)[0]
        if ring_k is not None:
            pos[s] = 0
            for c in range(a, b, int(W)):  # ring_append takes at most W frames per call
                e = min(b, c + int(W))
                ring_append(ring_k[s:s + 1], ring_v[s:s + 1], k[None, c:e], v[None, c:e],
                            pos[s:s + 1], W, theta=theta, bf16=bf16, rope_applied=rope_applied)
    return o


def stream_step(q_new, k_new, v_new, ring_k, ring_v, pos, W, theta=1e6, scale=None, bf16=False,
                rope_applied=False, nthreads=0):
    """One streaming step; q/k/v_new [S,n,H,D], rings [S,H,W,D], pos [S] -> o [S,n,H,D]."""
    q_new, k_new, v_new = _f64(q_new), _f64(k_new), _f64(v_new)
    ring_k, ring_v = _f64(ring_k), _f64(ring_v)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    S, n, H, D = q_new.shape
    assert ring_k.shape == (S, H, W, D) and ring_v.shape == (S, H, W, D)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.zeros_like(q_new)
    rc = _load().oracle_stream_step(_ptr(q_new), _ptr(k_new), _ptr(v_new), _ptr(ring_k),
                                    _ptr(ring_v), _ptr(pos, _i64p), _ptr(o), S, n, H, D, int(W),
                                    float(theta), float(scale), int(bool(bf16)),
                                    int(bool(rope_applied)), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_stream_step rejected its arguments")
    return o


def ring_append(ring_k, ring_v, k_new, v_new, pos, W, theta=1e6, bf16=False, rope_applied=False):
    """Append in place: ring_k/ring_v float64 [S,H,W,D] and pos int64 [S] are modified."""
    for a in (ring_k, ring_v):
        assert a.dtype == np.float64 and a.flags.c_contiguous
    assert pos.dtype == np.int64 and pos.flags.c_contiguous
    k_new, v_new = _f64(k_new), _f64(v_new)
    S, n, H, D = k_new.shape
    rc = _load().oracle_ring_append(_ptr(ring_k), _ptr(ring_v), _ptr(k_new), _ptr(v_new),
                                    _ptr(pos, _i64p), S, n, H, D, int(W), float(theta),
                                    int(bool(bf16)), int(bool(rope_applied)))
    if rc != 0:
        raise ValueError("oracle_ring_append rejected its arguments")


def gqa_prefill(q, k, v, W, pos=None, theta=1e6, scale=None, bf16=False, rope_applied=False,
                nthreads=0):
    """Grouped-query causal sliding-window attention over whole chunks.

    Voxtral Realtime 2602 text decoder (transcribe.cpp "Voxtral" family notes,
    Architecture: 32 query heads over 8 key/value heads, head_dim 128, window
    8192).  q [B,T,Hq,D], k,v [B,T,Hkv,D] -> o [B,T,Hq,D] float64; query head
    h reads key/value head h // (Hq // Hkv).  pos as in prefill().
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    assert k.shape == (B, T, Hkv, D) and v.shape == k.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    p = None
    if pos is not None:
        if np.isscalar(pos):
            p = (np.int64(pos) + np.arange(T, dtype=np.int64))[None, :].repeat(B, 0)
        else:
            p = np.broadcast_to(np.asarray(pos, dtype=np.int64), (B, T))
        p = np.ascontiguousarray(p, dtype=np.int64)
    o = np.zeros_like(q)
    rc = _load().oracle_gqa_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, T, Hq, Hkv, D, int(W),
                                    None if p is None else _ptr(p, _i64p), float(theta),
                                    float(scale), int(bool(bf16)), int(bool(rope_applied)),
                                    int(nthreads))
    if rc != 0:
        raise ValueError("oracle_gqa_prefill rejected its arguments")
    return o


def gqa_stream_step(q_new, k_new, v_new, ring_k, ring_v, pos, W, theta=1e6, scale=None,
                    bf16=False, rope_applied=False, nthreads=0):
    """One grouped-query streaming (decode) step.

    q_new [S,n,Hq,D], k_new/v_new [S,n,Hkv,D], rings [S,Hkv,W,D], pos [S]
    -> o [S,n,Hq,D].  Reads the rings only; ring_append() with the key/value
    heads appends the step's frames.
    """
    q_new, k_new, v_new = _f64(q_new), _f64(k_new), _f64(v_new)
    ring_k, ring_v = _f64(ring_k), _f64(ring_v)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    S, n, Hq, D = q_new.shape
    Hkv = k_new.shape[2]
    assert k_new.shape == (S, n, Hkv, D) and v_new.shape == k_new.shape
    assert ring_k.shape == (S, Hkv, W, D) and ring_v.shape == (S, Hkv, W, D)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.zeros_like(q_new)
    rc = _load().oracle_gqa_stream_step(_ptr(q_new), _ptr(k_new), _ptr(v_new), _ptr(ring_k),
                                        _ptr(ring_v), _ptr(pos, _i64p), _ptr(o), S, n, Hq, Hkv,
                                        D, int(W), float(theta), float(scale), int(bool(bf16)),
                                        int(bool(rope_applied)), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_gqa_stream_step rejected its arguments")
    return o


# ---------------------------------------------------------------------------
# Encoder attention block around the streaming step (projections)
# ---------------------------------------------------------------------------
# Voxtral Realtime 2602 audio encoder (transcribe.cpp "Voxtral" family notes,
# Architecture): each layer projects its normalised hidden state (width 1280)
# to q, k, v (32 heads x 64), k_proj without a bias, applies RoPE to q and k,
# attends, and projects back to 1280 with the output projection.  The
# projections are plain matrix products (numpy matmul in float64 is the step);
# everything else is the pinned functions above.

def linear(x, w, b=None):
    """y = x w^T (+ b) in float64; x [M,K], w [N,K], b [N] -> [M,N]."""
    y = _f64(x) @ _f64(w).T
    if b is not None:
        y = y + _f64(b)[None, :]
    return y


def enc_qkv_rope(x, w_qkv, b_q, b_v, pos_rows, H, theta=1e6, bf16=False):
    """Fused q/k/v projection and RoPE.

    x [M, d_model]; w_qkv [3*H*64, d_model] with the q rows first, then k,
    then v; b_q, b_v [H*64] (k has no bias); pos_rows [M] absolute positions.
    Returns q', k' (rotated) and v as [M, H, 64] float64.  bf16=True rounds
    the three stored tensors to bfloat16 (the rotated q and k after rotation).
    """
    HD = H * 64
    w = _f64(w_qkv)
    q = linear(x, w[:HD], b_q)
    k = linear(x, w[HD:2 * HD])
    v = linear(x, w[2 * HD:], b_v)
    M = q.shape[0]
    p = np.asarray(pos_rows, dtype=np.int64).reshape(1, M)
    q = rope(q.reshape(1, M, H, 64), pos=p, theta=theta)[0]
    k = rope(k.reshape(1, M, H, 64), pos=p, theta=theta)[0]
    v = v.reshape(M, H, 64)
    if bf16:
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    return q, k, v


def enc_attn_step(x, w_qkv, b_q, b_v, w_o, b_o, ring_k, ring_v, pos, W, H, theta=1e6,
                  bf16=False):
    """One streaming step of the encoder's attention block for S streams.

    x [S, n, d_model] (frames pos[s] .. pos[s]+n-1 of stream s); rings
    [S, H, W, 64] float64 and pos int64 [S] are advanced in place exactly as
    ring_append does.  Returns y [S, n, d_model] = attention(q', k', v) w_o^T
    + b_o.  bf16=True rounds every tensor the block stores between its steps
    (q', k', v and the attention output o) to bfloat16.
    """
    x = _f64(x)
    S, n, dm = x.shape
    pos_rows = (np.asarray(pos, dtype=np.int64)[:, None] + np.arange(n)[None, :]).reshape(-1)
    q, k, v = enc_qkv_rope(x.reshape(S * n, dm), w_qkv, b_q, b_v, pos_rows, H, theta, bf16)
    shp = (S, n, H, 64)
    o = stream_step(q.reshape(shp), k.reshape(shp), v.reshape(shp), ring_k, ring_v, pos, W,
                    theta=theta, rope_applied=True)
    ring_append(ring_k, ring_v, k.reshape(shp), v.reshape(shp), pos, W, theta=theta,
                rope_applied=True)
    if bf16:
        o = bf16_round(o)
    return linear(o.reshape(S * n, H * 64), w_o, b_o).reshape(S, n, dm)


# ---------------------------------------------------------------------------
# Whole streaming encoder step: conv stem and transformer layers
# ---------------------------------------------------------------------------
# Voxtral Realtime 2602 audio encoder (transcribe.cpp "Voxtral" family notes,
# Architecture): a causal (left-pad-only) conv stem, conv1 128 -> 1280 kernel
# 3 stride 1 and conv2 1280 -> 1280 kernel 3 stride 2, each followed by GELU;
# then 32 pre-norm layers: RMSNorm, the attention block, residual add,
# RMSNorm, a SwiGLU MLP (bias only on the down projection), residual add.
# Streaming feeds 8 mel frames per step (4 encoder frames, one audio token).

def rmsnorm(x, g, eps=1e-5):
    """x / sqrt(mean(x^2) + eps) * g over the last axis, float64."""
    x = _f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * _f64(g)


def gelu(x):
    """GELU with the exact error function: x * (1 + erf(x / sqrt(2))) / 2."""
    from scipy.special import erf
    x = _f64(x)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def silu(x):
    x = _f64(x)
    return x / (1.0 + np.exp(-x))


def causal_conv1d(xpad, w, b, stride):
    """Causal 1-D convolution over frames.

    xpad [S, P + T, C_in]: each stream's input frames preceded by its P = k-1
    cached frames; w [C_out, k, C_in]; b [C_out].  Output frame t (0 <= t <
    (T - 1) // stride + 1 ... for T a multiple of stride, T // stride) reads
    padded frames stride*t .. stride*t + k - 1, i.e. input frames up to
    stride*t (left padding only).  Returns [S, T // stride, C_out].
    """
    xpad, w = _f64(xpad), _f64(w)
    S, TP, Ci = xpad.shape
    Co, k, _ = w.shape
    T = TP - (k - 1)
    n_out = T // stride
    out = np.empty((S, n_out, Co))
    for t in range(n_out):
        win = xpad[:, stride * t:stride * t + k, :].reshape(S, k * Ci)
        out[:, t] = win @ w.reshape(Co, k * Ci).T
    return out + _f64(b)[None, None, :]


def enc_stem_step(mel_new, mel_cache, c1_cache, w1, b1, w2, b2, bf16=False):
    """One streaming step of the conv stem for S streams.

    mel_new [S, 8, 128]; mel_cache [S, 2, 128] and c1_cache [S, 2, 1280] are
    each conv's last two input frames (updated in place).  Returns the 4 new
    encoder frames [S, 4, 1280].  bf16=True rounds the stored first-conv
    output; the second conv's output starts the residual stream, which is
    held in float32 and so compared unrounded.
    """
    xp = np.concatenate([_f64(mel_cache), _f64(mel_new)], axis=1)
    c1 = gelu(causal_conv1d(xp, w1, b1, 1))
    if bf16:
        c1 = bf16_round(c1)
    c1p = np.concatenate([_f64(c1_cache), c1], axis=1)
    out = gelu(causal_conv1d(c1p, w2, b2, 2))
    mel_cache[:] = xp[:, -2:]
    c1_cache[:] = c1p[:, -2:]
    return out


def enc_layer_step(x, wts, ring_k, ring_v, pos, W, H, theta=1e6, eps=1e-5, bf16=False):
    """One pre-norm encoder layer on the streaming residual x [S, n, d_model]
    (float64, returned updated).  wts: g_attn, w_qkv, b_q, b_v, w_o, b_o,
    g_ffn, w_gate, w_up, w_down, b_down.  Rings and pos advance in place.
    bf16=True rounds every tensor stored between launches (the normalised
    states, q', k', v, o and the SwiGLU hidden state)."""
    x = _f64(x)
    S, n, dm = x.shape
    h = rmsnorm(x, wts["g_attn"], eps)
    if bf16:
        h = bf16_round(h)
    x = x + enc_attn_step(h, wts["w_qkv"], wts["b_q"], wts["b_v"], wts["w_o"], wts["b_o"], ring_k,
                          ring_v, pos, W, H, theta=theta, bf16=bf16)
    h = rmsnorm(x, wts["g_ffn"], eps)
    if bf16:
        h = bf16_round(h)
    h2 = h.reshape(S * n, dm)
    u = silu(linear(h2, wts["w_gate"])) * linear(h2, wts["w_up"])
    if bf16:
        u = bf16_round(u)
    return x + linear(u, wts["w_down"], wts["b_down"]).reshape(S, n, dm)
