"""Independent formulations used to pin the oracle (CPU, numpy / torch fp64).

These are written differently from oracle.c on purpose:
  * RoPE as complex multiplication of z_i = x_i + 1j*x_{i+D/2} by exp(1j*angle),
    with the frequency taken as exp(-(2i/D) ln theta);
  * attention as a dense T x T score matrix with -inf outside the band, one
    numpy softmax per row; or torch's scaled_dot_product_attention.
"""
import numpy as np


def complex_rope(x, pos, theta=1e6):
    """x [..., T, H, D] float64, pos [T] ints -> rotated copy."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    i = np.arange(half, dtype=np.float64)
    freq = np.exp(-(2.0 * i / D) * np.log(theta))
    ang = np.asarray(pos, dtype=np.float64)[:, None, None] * freq[None, None, :]
    z = (x[..., :half] + 1j * x[..., half:]) * np.exp(1j * ang)
    return np.concatenate([z.real, z.imag], axis=-1)


def band_mask(T, W):
    t = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    return (j <= t) & (j > t - W)


def dense_band_attention(qr, kr, v, W, scale=None):
    """qr, kr, v [T,H,D] (already rotated) -> o [T,H,D]."""
    T, H, D = qr.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    s = np.einsum("thd,jhd->htj", qr, kr) * scale
    s = np.where(band_mask(T, W)[None], s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return np.einsum("htj,jhd->thd", p, v)


def sdpa_band(qr, kr, v, W, causal_flag=False):
    """torch SDPA in float64 on CPU; qr,kr,v [B,T,H,D] -> [B,T,H,D]."""
    import torch
    import torch.nn.functional as F
    q = torch.from_numpy(np.ascontiguousarray(qr.transpose(0, 2, 1, 3)))
    k = torch.from_numpy(np.ascontiguousarray(kr.transpose(0, 2, 1, 3)))
    vv = torch.from_numpy(np.ascontiguousarray(v.transpose(0, 2, 1, 3)))
    if causal_flag:
        o = F.scaled_dot_product_attention(q, k, vv, is_causal=True)
    else:
        T = qr.shape[1]
        m = torch.from_numpy(band_mask(T, W))
        o = F.scaled_dot_product_attention(q, k, vv, attn_mask=m)
    return o.numpy().transpose(0, 2, 1, 3)
