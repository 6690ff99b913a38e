"""Seeded synthetic inputs for the sliding-window RoPE attention path.

This module only *draws* inputs: it holds none of the attention arithmetic
(no rotation, no scores, no softmax).  Both the GPU path and the CPU oracle
consume what it returns, so the same seed gives the same bytes on both sides.

Workloads (shapes follow the Voxtral Realtime 2602 audio encoder: 32 heads of
head_dim 64, window 750, RoPE theta 1e6, 4 encoder frames per streaming step;
see the transcribe.cpp "Voxtral" family notes, section Architecture, Voxtral
Realtime 2602):

  tiny      B1  T64   H4  W16   fp32, N(0,1)
  layer     B1  T1500 H32 W750  bf16, 0.5*N(0,1)
  stack     32 layers x (B4 T1500 H32) W750 bf16, 0.5*N(0,1), one seed per layer
  stream    64 streams x 4 new frames, H32, W750, bf16 ring pre-filled N(0,1),
            first new position per stream ~ U{750..20000}
  long      B8  T6000 H32 W750  bf16, N(0,1), 1% of key rows scaled x8

Draw order for a prefill set: Q, K, V (each standard_normal float32 of shape
[B,T,H,64]), then (long only) the stressed key-row choice.  Scaling happens in
float32 (a power of two, so exact), then round-to-nearest-even to bfloat16
for bf16 workloads.
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

HEAD_DIM = 64


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    T: int
    H: int
    W: int
    dtype: str  # "f32" or "bf16"
    scale: float  # multiplier applied to N(0,1) draws
    seed: int
    stress_frac: float = 0.0  # fraction of key rows multiplied by stress_mult
    stress_mult: float = 1.0
    layers: int = 1
    theta: float = 1e6
    D: int = HEAD_DIM


@dataclasses.dataclass(frozen=True)
class StreamConfig:
    name: str
    S: int
    n: int
    H: int
    W: int
    dtype: str
    seed: int
    pos_lo: int
    pos_hi: int
    theta: float = 1e6
    D: int = HEAD_DIM


CONFIGS = {
    "tiny": PrefillConfig("tiny", B=1, T=64, H=4, W=16, dtype="f32", scale=1.0, seed=1),
    "layer": PrefillConfig("layer", B=1, T=1500, H=32, W=750, dtype="bf16", scale=0.5, seed=2),
    "stack": PrefillConfig("stack", B=4, T=1500, H=32, W=750, dtype="bf16", scale=0.5, seed=3,
                           layers=32),
    "stream": StreamConfig("stream", S=64, n=4, H=32, W=750, dtype="bf16", seed=4,
                           pos_lo=750, pos_hi=20000),
    "long": PrefillConfig("long", B=8, T=6000, H=32, W=750, dtype="bf16", scale=1.0, seed=5,
                          stress_frac=0.01, stress_mult=8.0),
}


# ---------------------------------------------------------------------------
# bfloat16 storage conversion (input preparation only)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array holding exactly the bfloat16-representable nearest values."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


# ---------------------------------------------------------------------------
# prefill sets
# ---------------------------------------------------------------------------

def make_prefill(B: int, T: int, H: int, *, seed, dtype: str = "bf16", scale: float = 1.0,
                 stress_frac: float = 0.0, stress_mult: float = 1.0, D: int = HEAD_DIM):
    """Draw Q, K, V of shape [B,T,H,D] as float32 arrays holding storage-dtype values.

    `seed` is an int or a sequence of ints (numpy SeedSequence entropy).
    Returns dict(q, k, v, stressed_rows) where stressed_rows is the sorted flat
    index (over B*T*H rows of K) of the rows that were multiplied.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    shape = (B, T, H, D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        s = np.float32(scale)
        q *= s
        k *= s
        v *= s
    stressed = np.zeros(0, dtype=np.int64)
    if stress_frac > 0.0:
        nrows = B * T * H
        count = int(round(stress_frac * nrows))
        stressed = np.sort(rng.choice(nrows, size=count, replace=False)).astype(np.int64)
        kr = k.reshape(nrows, D)
        kr[stressed] *= np.float32(stress_mult)
    return dict(q=_store(q, dtype), k=_store(k, dtype), v=_store(v, dtype), stressed_rows=stressed)


def make_config(name: str, layer: int = 0):
    """Prefill set for a named workload (for 'stack', one layer's set)."""
    c = CONFIGS[name]
    assert isinstance(c, PrefillConfig)
    seed = [c.seed, layer] if c.layers > 1 else c.seed
    return make_prefill(c.B, c.T, c.H, seed=seed, dtype=c.dtype, scale=c.scale,
                        stress_frac=c.stress_frac, stress_mult=c.stress_mult, D=c.D)


# ---------------------------------------------------------------------------
# streaming sets
# ---------------------------------------------------------------------------

def make_stream_state(S: int, H: int, W: int, *, seed, pos_lo: int, pos_hi: int,
                      dtype: str = "bf16", D: int = HEAD_DIM, full: bool = True):
    """Pre-filled ring state for S streams.

    Returns dict(ring_k, ring_v [S,H,W,D] float32 holding storage values, pos [S] int64).
    pos[s] is the absolute position of the next frame to arrive, drawn
    uniformly from {pos_lo..pos_hi}.  Ring slot j holds the frame whose
    position p satisfies p mod W == j; with full=True all W slots hold the
    frames pos-W..pos-1 (pos_lo must then be >= W).  The ring contents are
    N(0,1) draws and are taken to be keys that are already rotated.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    ring_k = rng.standard_normal((S, H, W, D), dtype=np.float32)
    ring_v = rng.standard_normal((S, H, W, D), dtype=np.float32)
    pos = rng.integers(pos_lo, pos_hi, size=S, endpoint=True, dtype=np.int64)
    if full and pos_lo < W:
        raise ValueError("a full ring needs pos_lo >= W")
    return dict(ring_k=_store(ring_k, dtype), ring_v=_store(ring_v, dtype), pos=pos)


def make_stream_frames(S: int, n: int, H: int, *, seed, step: int, dtype: str = "bf16",
                       D: int = HEAD_DIM, scale: float = 1.0):
    """Fresh new-frame q, k, v [S,n,H,D] for streaming step `step`."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1000003, step])))
    shape = (S, n, H, D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        s = np.float32(scale)
        q *= s
        k *= s
        v *= s
    return dict(q=_store(q, dtype), k=_store(k, dtype), v=_store(v, dtype))


def make_stream_config(name: str = "stream"):
    c = CONFIGS[name]
    assert isinstance(c, StreamConfig)
    return make_stream_state(c.S, c.H, c.W, seed=c.seed, pos_lo=c.pos_lo, pos_hi=c.pos_hi,
                             dtype=c.dtype, D=c.D)


# Batched first chunks: 64 streams whose first chunks hold 120..156 encoder
# frames (156 = the 312-mel first chunk after the stride-2 stem), 32 heads.
FIRST_CHUNK = dict(S=64, t_lo=120, t_hi=156, H=32, W=750, dtype="bf16", scale=0.5, seed=6)


def make_first_chunks(S: int, H: int, lengths, *, seed, dtype: str = "bf16", scale: float = 0.5,
                      D: int = HEAD_DIM):
    """Packed first chunks: q, k, v [total, H, D] with stream s at rows cu[s] .. cu[s+1]-1.

    Draws Q, K, V for all frames at once (order Q, K, V, as make_prefill).
    Returns dict(q, k, v, cu) with cu an int32 array of S+1 offsets.
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    assert lengths.shape == (S,) and np.all(lengths >= 0)
    cu = np.zeros(S + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    x = make_prefill(1, int(cu[-1]), H, seed=seed, dtype=dtype, scale=scale, D=D)
    return dict(q=x["q"][0], k=x["k"][0], v=x["v"][0], cu=cu)


def first_chunk_lengths(S: int, t_lo: int, t_hi: int, *, seed) -> np.ndarray:
    """Chunk lengths drawn uniformly from t_lo..t_hi (inclusive)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    return rng.integers(t_lo, t_hi + 1, size=S).astype(np.int64)


def band_pairs(T: int, W: int) -> int:
    """Number of (query, key) pairs with 0 <= t-j < W, 0 <= j <= t < T (counting only)."""
    if T <= W:
        return T * (T + 1) // 2
    return W * (W + 1) // 2 + (T - W) * W


# ---------------------------------------------------------------------------
# text-decoder sets (grouped-query attention)
# ---------------------------------------------------------------------------
# The Voxtral Realtime 2602 text decoder (transcribe.cpp "Voxtral" family
# notes, Architecture): 32 query heads over 8 key/value heads, head_dim 128,
# sliding window 8192, RoPE theta 1e6.
#
#   dec_tiny     prefill B2 T200 Hq8 Hkv2 W64 bf16, N(0,1)
#   dec_prefill  prefill B1 T16384 Hq32 Hkv8 W8192 bf16, N(0,1): a prompt two
#                windows long
#   dec_decode   64 streams x 1 new token, Hq32 Hkv8 W8192 bf16, rings
#                pre-filled N(0,1), next position per stream ~ U{8192..65536}

@dataclasses.dataclass(frozen=True)
class GqaConfig:
    name: str
    kind: str  # "prefill" or "decode"
    B: int     # batch (prefill) or streams (decode)
    T: int     # prompt length (prefill) or new tokens per step (decode)
    Hq: int
    Hkv: int
    W: int
    dtype: str
    seed: int
    scale: float = 1.0
    pos_lo: int = 0
    pos_hi: int = 0
    theta: float = 1e6
    D: int = 128


GQA_CONFIGS = {
    "dec_tiny": GqaConfig("dec_tiny", "prefill", B=2, T=200, Hq=8, Hkv=2, W=64, dtype="bf16",
                          seed=21),
    "dec_prefill": GqaConfig("dec_prefill", "prefill", B=1, T=16384, Hq=32, Hkv=8, W=8192,
                             dtype="bf16", seed=22),
    "dec_decode": GqaConfig("dec_decode", "decode", B=64, T=1, Hq=32, Hkv=8, W=8192,
                            dtype="bf16", seed=23, pos_lo=8192, pos_hi=65536),
}


def make_gqa_prefill(B: int, T: int, Hq: int, Hkv: int, *, seed, dtype: str = "bf16",
                     scale: float = 1.0, D: int = 128):
    """Q [B,T,Hq,D], then K and V [B,T,Hkv,D], as float32 arrays of storage values."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    out = {}
    for name, H in (("q", Hq), ("k", Hkv), ("v", Hkv)):
        x = rng.standard_normal((B, T, H, D), dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[name] = _store(x, dtype)
    return out


def make_gqa_frames(S: int, n: int, Hq: int, Hkv: int, *, seed, step: int,
                    dtype: str = "bf16", D: int = 128):
    """New-token q [S,n,Hq,D], k and v [S,n,Hkv,D] for decode step `step`."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1000003, step])))
    return {name: _store(rng.standard_normal((S, n, H, D), dtype=np.float32), dtype)
            for name, H in (("q", Hq), ("k", Hkv), ("v", Hkv))}


def make_gqa_config(name: str):
    c = GQA_CONFIGS[name]
    assert c.kind == "prefill"
    return make_gqa_prefill(c.B, c.T, c.Hq, c.Hkv, seed=c.seed, dtype=c.dtype, scale=c.scale,
                            D=c.D)


def make_gqa_decode_state(name: str = "dec_decode"):
    """Full rings [S,Hkv,W,D] and next positions for a decode workload."""
    c = GQA_CONFIGS[name]
    assert c.kind == "decode"
    return make_stream_state(c.B, c.Hkv, c.W, seed=c.seed, pos_lo=c.pos_lo, pos_hi=c.pos_hi,
                             dtype=c.dtype, D=c.D)


# ---------------------------------------------------------------------------
# encoder attention block (projections around the streaming step)
# ---------------------------------------------------------------------------
# One encoder layer's q/k/v and output projections (d_model 1280, 32 heads x
# 64, k_proj without a bias) around the streaming step of the stream
# workload: 64 streams x 4 new frames.

ENC_BLOCK = dict(S=64, n=4, H=32, d_model=1280, W=750, seed=8, pos_lo=750, pos_hi=20000)


def make_enc_block_weights(d_model: int, H: int, *, seed):
    """Synthetic projection weights at a trained layer's scale, bf16 values in float32 arrays.

    w_qkv [3*H*64, d_model] (q rows, then k, then v) and w_o [d_model, H*64]
    are N(0, 1/fan_in); b_q, b_v [H*64] and b_o [d_model] are 0.02*N(0,1).
    Draw order: w_qkv, b_q, b_v, w_o, b_o.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 2024])))
    HD = H * 64
    w_qkv = rng.standard_normal((3 * HD, d_model), dtype=np.float32) * np.float32(d_model ** -0.5)
    b_q = rng.standard_normal(HD, dtype=np.float32) * np.float32(0.02)
    b_v = rng.standard_normal(HD, dtype=np.float32) * np.float32(0.02)
    w_o = rng.standard_normal((d_model, HD), dtype=np.float32) * np.float32(HD ** -0.5)
    b_o = rng.standard_normal(d_model, dtype=np.float32) * np.float32(0.02)
    return {name: _store(a, "bf16") for name, a in
            (("w_qkv", w_qkv), ("b_q", b_q), ("b_v", b_v), ("w_o", w_o), ("b_o", b_o))}


def make_enc_block_input(S: int, n: int, d_model: int, *, seed, step: int):
    """Normalised hidden states x [S, n, d_model] (N(0,1), bf16) for streaming step `step`."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 77, step])))
    return _store(rng.standard_normal((S, n, d_model), dtype=np.float32), "bf16")


# Whole streaming encoder step: stem + L pre-norm layers, 64 streams x 4 new
# frames (8 mel frames of 128 bins), d_model 1280, 32 heads x 64, FFN 5120.
ENC_STEP = dict(S=64, n=4, H=32, d_model=1280, ffn=5120, n_mels=128, L=32, W=750, seed=9,
                pos_lo=750, pos_hi=20000)


def make_enc_stem_weights(d_model: int, n_mels: int, *, seed):
    """Synthetic stem weights (bf16 values in float32 arrays).

    w1 [d_model, 3, n_mels] and w2 [d_model, 3, d_model] (output, tap, input)
    are N(0, 1/fan_in) with fan_in = 3 * input channels; b1, b2 [d_model] are
    0.02*N(0,1).  Draw order: w1, b1, w2, b2.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 2025])))
    w1 = rng.standard_normal((d_model, 3, n_mels), dtype=np.float32) * np.float32((3 * n_mels) ** -0.5)
    b1 = rng.standard_normal(d_model, dtype=np.float32) * np.float32(0.02)
    w2 = rng.standard_normal((d_model, 3, d_model), dtype=np.float32) * np.float32((3 * d_model) ** -0.5)
    b2 = rng.standard_normal(d_model, dtype=np.float32) * np.float32(0.02)
    return {name: _store(a, "bf16") for name, a in (("w1", w1), ("b1", b1), ("w2", w2), ("b2", b2))}


def make_enc_layer_weights(d_model: int, H: int, ffn: int, *, seed, layer: int):
    """Synthetic weights of one pre-norm layer (bf16 values in float32 arrays).

    The attention projections are make_enc_block_weights' recipe (seeded by
    [seed, layer]); the RMSNorm gains g_attn, g_ffn [d_model] are 1 + 0.1*N(0,1);
    w_gate, w_up [ffn, d_model] are N(0, 1/d_model), w_down [d_model, ffn]
    N(0, 1/ffn), b_down 0.02*N(0,1).  Draw order: g_attn, g_ffn, w_gate,
    w_up, w_down, b_down.
    """
    wts = make_enc_block_weights(d_model, H, seed=[seed, layer])
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 2026, layer])))
    g_attn = 1 + rng.standard_normal(d_model, dtype=np.float32) * np.float32(0.1)
    g_ffn = 1 + rng.standard_normal(d_model, dtype=np.float32) * np.float32(0.1)
    w_gate = rng.standard_normal((ffn, d_model), dtype=np.float32) * np.float32(d_model ** -0.5)
    w_up = rng.standard_normal((ffn, d_model), dtype=np.float32) * np.float32(d_model ** -0.5)
    w_down = rng.standard_normal((d_model, ffn), dtype=np.float32) * np.float32(ffn ** -0.5)
    b_down = rng.standard_normal(d_model, dtype=np.float32) * np.float32(0.02)
    for name, a in (("g_attn", g_attn), ("g_ffn", g_ffn), ("w_gate", w_gate), ("w_up", w_up),
                    ("w_down", w_down), ("b_down", b_down)):
        wts[name] = _store(a, "bf16")
    return wts


def make_mel(S: int, frames: int, n_mels: int, *, seed, step: int):
    """Log-mel frames [S, frames, n_mels] for streaming step `step`: 0.5*N(0,1)
    (the spread of normalised log-mel features), bf16."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 79, step])))
    return _store(rng.standard_normal((S, frames, n_mels), dtype=np.float32) * np.float32(0.5), "bf16")
