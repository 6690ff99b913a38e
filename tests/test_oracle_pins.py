"""Pins for the float64 CPU oracle, against facts fixed outside the oracle.

Each test names what pins it: a brute-force dense formulation, torch's
scaled_dot_product_attention, a closed form, an invariant the pages state
(offline == streaming; full causal attention when T <= W), or a constant the
pages print (tests/golden/voxtral_realtime_constants.json).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from sliding_window_attention_vx_amd import synth
from tests.refimpl import complex_rope, dense_band_attention, sdpa_band

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# --------------------------------------------------------------------------
# bfloat16 rounding
# --------------------------------------------------------------------------

def test_bf16_round_matches_bit_rounding_of_float32():
    # Independent implementation: integer round-to-nearest-even on float32 bits.
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-39, -2.5e-40], dtype=np.float32)])
    x = x.astype(np.float32)
    want = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x)).astype(np.float64)
    got = oracle.bf16_round(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_bf16_round_ties_and_closed_forms():
    u = 2.0 ** -7  # spacing of bf16 in [1, 2)
    cases = {
        1.0 + u / 2: 1.0,                  # tie -> even significand (1.0)
        1.0 + 3 * u / 2: 1.0 + 2 * u,      # tie -> even (1 + 2u)
        1.0 + u / 2 + 2.0 ** -40: 1.0 + u,  # just above the tie
        -(1.0 + u / 2): -1.0,
        1.0 / 3.0: 0.333984375,            # 171/512
        math.pi: 3.140625,
    }
    for x, want in cases.items():
        assert oracle.bf16_round(np.array([x]))[0] == want, x


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------

def test_rope_position_zero_is_identity():
    x = rnd((1, 3, 2, 64), 1)
    np.testing.assert_array_equal(oracle.rope(x, pos=np.zeros((1, 3), np.int64)), x)


def test_rope_matches_complex_multiplication():
    x = rnd((2, 5, 3, 64), 2)
    pos = np.array([[0, 1, 749, 750, 19999], [3, 17, 1500, 6000, 123456]], dtype=np.int64)
    got = oracle.rope(x, pos=pos, theta=1e6)
    for b in range(2):
        want = complex_rope(x[b], pos[b], theta=1e6)
        np.testing.assert_allclose(got[b], want, rtol=0, atol=1e-9)


def test_rope_d2_is_rotation_by_position_radians():
    # D = 2: one pair with frequency theta^0 = 1, so the angle is the position itself.
    x = rnd((1, 4, 1, 2), 3)
    pos = np.array([[0, 1, 2, 1000]], dtype=np.int64)
    got = oracle.rope(x, pos=pos, theta=12345.0)
    z = (x[0, :, 0, 0] + 1j * x[0, :, 0, 1]) * np.exp(1j * pos[0].astype(float))
    np.testing.assert_allclose(got[0, :, 0, 0], z.real, atol=1e-12)
    np.testing.assert_allclose(got[0, :, 0, 1], z.imag, atol=1e-12)


def test_rope_frequencies_closed_form_theta_1e6():
    # theta = 1e6, D = 64: f_i = 1e6^(-2i/64) = 10^(-3i/16).  Rotating the basis
    # vector e_i at position 1 turns it by exactly f_i radians into (cos, sin)
    # on dims (i, i+32).
    D = 64
    closed = {0: 1.0, 8: 10 ** -1.5, 16: 1e-3, 24: 10 ** -4.5, 31: 10 ** (-93 / 16)}
    for i, f in closed.items():
        x = np.zeros((1, 1, 1, D))
        x[0, 0, 0, i] = 1.0
        r = oracle.rope(x, pos=np.array([[1]]), theta=1e6)[0, 0, 0]
        assert abs(math.atan2(r[i + 32], r[i]) - f) < 1e-15 * max(1.0, f) + 1e-18, i
        assert abs(r[i] ** 2 + r[i + 32] ** 2 - 1.0) < 1e-15
        others = np.delete(r, [i, i + 32])
        assert np.all(others == 0.0)


def test_rope_preserves_pair_norms():
    x = rnd((1, 6, 4, 64), 4)
    pos = np.arange(6, dtype=np.int64)[None] * 3331
    r = oracle.rope(x, pos=pos)
    n0 = x[..., :32] ** 2 + x[..., 32:] ** 2
    n1 = r[..., :32] ** 2 + r[..., 32:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-13)


@pytest.mark.parametrize("shift", [1, 7, 750, 19999])
def test_rope_relative_position_property(shift):
    # <R(m)q, R(n)k> depends only on n - m.
    q = rnd((1, 4, 2, 64), 5)
    k = rnd((1, 4, 2, 64), 6)
    m = np.array([[0, 5, 100, 749]])
    n = np.array([[3, 5, 40, 0]])
    s0 = np.sum(oracle.rope(q, pos=m) * oracle.rope(k, pos=n), axis=-1)
    s1 = np.sum(oracle.rope(q, pos=m + shift) * oracle.rope(k, pos=n + shift), axis=-1)
    np.testing.assert_allclose(s1, s0, rtol=1e-9, atol=1e-9)


# --------------------------------------------------------------------------
# prefill attention
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,W,H,D", [(1, 1, 1, 2), (2, 3, 1, 8), (5, 3, 2, 8), (16, 16, 1, 64),
                                     (16, 1, 2, 8), (64, 16, 4, 64), (64, 69, 1, 64),
                                     (40, 7, 3, 16)])
def test_prefill_matches_dense_brute_force(T, W, H, D):
    q, k, v = (rnd((1, T, H, D), s) for s in (10, 11, 12))
    pos = np.arange(T)
    got = oracle.prefill(q, k, v, W)[0]
    want = dense_band_attention(complex_rope(q[0], pos), complex_rope(k[0], pos), v[0], W)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_prefill_full_causal_when_T_le_W():
    # With T <= W the window never bites: plain causal attention (torch SDPA, is_causal).
    B, T, H, D, W = 2, 48, 3, 64, 750
    q, k, v = (rnd((B, T, H, D), s) for s in (20, 21, 22))
    pos = np.arange(T)
    qr = np.stack([complex_rope(q[b], pos) for b in range(B)])
    kr = np.stack([complex_rope(k[b], pos) for b in range(B)])
    want = sdpa_band(qr, kr, v, W, causal_flag=True)
    np.testing.assert_allclose(oracle.prefill(q, k, v, W), want, rtol=0, atol=1e-12)


def test_prefill_band_matches_sdpa_with_mask():
    B, T, H, D, W = 1, 100, 2, 64, 37
    q, k, v = (rnd((B, T, H, D), s) for s in (23, 24, 25))
    pos = np.arange(T)
    qr = complex_rope(q[0], pos)[None]
    kr = complex_rope(k[0], pos)[None]
    want = sdpa_band(qr, kr, v, W)
    np.testing.assert_allclose(oracle.prefill(q, k, v, W), want, rtol=0, atol=1e-12)


def test_window_one_returns_values_exactly():
    q, k, v = (rnd((2, 9, 3, 64), s) for s in (30, 31, 32))
    np.testing.assert_array_equal(oracle.prefill(q, k, v, 1), v)


def test_constant_values_give_constant_output():
    q, k = rnd((1, 30, 2, 64), 33), rnd((1, 30, 2, 64), 34)
    v = np.full((1, 30, 2, 64), -2.75)
    np.testing.assert_allclose(oracle.prefill(q, k, v, 11), v, rtol=0, atol=1e-14)


def test_prefill_invariant_under_position_offset():
    q, k, v = (rnd((1, 50, 2, 64), s) for s in (35, 36, 37))
    o0 = oracle.prefill(q, k, v, 20, pos=0)
    for off in (1, 750, 19999):
        np.testing.assert_allclose(oracle.prefill(q, k, v, 20, pos=off), o0, rtol=0, atol=1e-9)


def test_window_locality():
    # Query t sees frames t-W+1..t: changing frame t-W leaves it unchanged,
    # changing frame t-W+1 does not.
    T, W, t = 40, 10, 30
    q, k, v = (rnd((1, T, 1, 64), s) for s in (40, 41, 42))
    o0 = oracle.prefill(q, k, v, W)
    k1, v1 = k.copy(), v.copy()
    k1[0, t - W] += 5.0
    v1[0, t - W] += 5.0
    o1 = oracle.prefill(q, k1, v1, W)
    np.testing.assert_array_equal(o1[0, t], o0[0, t])
    assert np.any(o1[0, t - W] != o0[0, t - W])
    k2, v2 = k.copy(), v.copy()
    k2[0, t - W + 1] += 5.0
    v2[0, t - W + 1] += 5.0
    o2 = oracle.prefill(q, k2, v2, W)
    assert np.max(np.abs(o2[0, t] - o0[0, t])) > 1e-3


def test_batch_and_heads_are_independent():
    q, k, v = (rnd((3, 20, 4, 64), s) for s in (43, 44, 45))
    full = oracle.prefill(q, k, v, 6)
    for b in range(3):
        for h in range(4):
            one = oracle.prefill(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1],
                                 v[b:b + 1, :, h:h + 1], 6)
            np.testing.assert_array_equal(one[0, :, 0], full[b, :, h])


def test_bf16_contract_rounds_rotated_qk():
    # bf16 mode = brute force on bf16-rounded complex-rotated q, k (v untouched).
    T, H, D, W = 33, 2, 64, 9
    q, k, v = (rnd((1, T, H, D), s) for s in (46, 47, 48))
    pos = np.arange(T)
    qr = oracle.bf16_round(complex_rope(q[0], pos))
    kr = oracle.bf16_round(complex_rope(k[0], pos))
    want = dense_band_attention(qr, kr, v[0], W)
    got = oracle.prefill(q, k, v, W, bf16=True)[0]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # and it differs from the exact mode by about bf16 resolution, not more
    exact = oracle.prefill(q, k, v, W)[0]
    d = np.max(np.abs(got - exact))
    assert 1e-6 < d < 0.05


def test_rope_applied_skips_rotation():
    q, k, v = (rnd((1, 12, 2, 64), s) for s in (49, 50, 51))
    pos = np.arange(12)
    qr, kr = complex_rope(q[0], pos)[None], complex_rope(k[0], pos)[None]
    np.testing.assert_allclose(oracle.prefill(qr, kr, v, 5, rope_applied=True),
                               oracle.prefill(q, k, v, 5), rtol=0, atol=1e-12)


def test_thread_count_does_not_change_results():
    q, k, v = (rnd((2, 70, 3, 64), s) for s in (52, 53, 54))
    a = oracle.prefill(q, k, v, 25, nthreads=1)
    b = oracle.prefill(q, k, v, 25, nthreads=4)
    np.testing.assert_array_equal(a, b)


# --------------------------------------------------------------------------
# streaming: ring of W slots, attend then append
# --------------------------------------------------------------------------

def run_stream(q, k, v, W, chunks, bf16=False, start_pos=0):
    """Feed [1,T,H,D] frames through stream_step + ring_append in chunks."""
    B, T, H, D = q.shape
    S = 1
    ring_k = np.zeros((S, H, W, D))
    ring_v = np.zeros((S, H, W, D))
    # fill the ring with garbage: slots for positions < 0 must never be read
    ring_k[:] = 1e3
    ring_v[:] = -1e3
    pos = np.array([start_pos], dtype=np.int64)
    out = np.zeros_like(q)
    t = 0
    ci = 0
    while t < T:
        n = min(chunks[ci % len(chunks)], T - t)
        ci += 1
        sl = slice(t, t + n)
        o = oracle.stream_step(q[:, sl], k[:, sl], v[:, sl], ring_k, ring_v, pos, W, bf16=bf16)
        oracle.ring_append(ring_k, ring_v, k[:, sl], v[:, sl], pos, W, bf16=bf16)
        out[:, sl] = o
        t += n
    assert pos[0] == start_pos + T
    return out, ring_k, ring_v


@pytest.mark.parametrize("chunks", [[1], [3], [4], [7], [50], [4, 1, 7, 3]])
def test_streaming_equals_prefill(chunks):
    # Offline and streaming encoders compute the same thing: chunked streaming
    # over a W-slot ring equals whole-sequence prefill, across ring wraps.
    W, T, H, D = 50, 160, 2, 64
    q, k, v = (rnd((1, T, H, D), s) for s in (60, 61, 62))
    got, _, _ = run_stream(q, k, v, W, chunks)
    np.testing.assert_allclose(got, oracle.prefill(q, k, v, W), rtol=0, atol=1e-12)


def test_streaming_equals_prefill_chunk_equal_to_window():
    W, T = 16, 70
    q, k, v = (rnd((1, T, 2, 64), s) for s in (63, 64, 65))
    got, _, _ = run_stream(q, k, v, W, [W])
    np.testing.assert_allclose(got, oracle.prefill(q, k, v, W), rtol=0, atol=1e-12)


def test_streaming_equals_prefill_bf16_contract():
    W, T = 24, 90
    q, k, v = (rnd((1, T, 2, 64), s) for s in (66, 67, 68))
    got, _, _ = run_stream(q, k, v, W, [4], bf16=True)
    np.testing.assert_allclose(got, oracle.prefill(q, k, v, W, bf16=True), rtol=0, atol=1e-12)


def test_streaming_at_real_window_three_wraps():
    W, T = 750, 3 * 750 + 13
    q, k, v = (rnd((1, T, 1, 64), s, 0.5) for s in (69, 70, 71))
    got, _, _ = run_stream(q, k, v, W, [4])
    np.testing.assert_allclose(got, oracle.prefill(q, k, v, W), rtol=0, atol=1e-12)


def test_ring_holds_rotated_keys_at_position_mod_w():
    W, T, H = 8, 21, 2
    q, k, v = (rnd((1, T, H, 64), s) for s in (72, 73, 74))
    _, rk, rv = run_stream(q, k, v, W, [3], start_pos=5)
    kr = complex_rope(k[0], np.arange(5, 5 + T))
    for t in range(T - W, T):
        p = 5 + t
        np.testing.assert_allclose(rk[0, :, p % W], kr[t], atol=1e-12)
        np.testing.assert_array_equal(rv[0, :, p % W], v[0, t])


def test_stream_step_from_absolute_positions_matches_prefill_slice():
    # A ring pre-filled with rotated keys of positions P-W..P-1 behaves like the
    # tail of a prefill over positions P-W..P+n-1.
    W, n, H, P = 30, 4, 2, 12345
    T = W + n
    q, k, v = (rnd((1, T, H, 64), s) for s in (75, 76, 77))
    posv = np.arange(P - W, P + n)
    kr = complex_rope(k[0], posv)
    ring_k = np.zeros((1, H, W, 64))
    ring_v = np.zeros((1, H, W, 64))
    for t in range(W):
        ring_k[0, :, posv[t] % W] = kr[t]
        ring_v[0, :, posv[t] % W] = v[0, t]
    o = oracle.stream_step(q[:, W:], k[:, W:], v[:, W:], ring_k, ring_v,
                           np.array([P], np.int64), W)
    want = oracle.prefill(q, k, v, W, pos=P - W)[:, W:]
    np.testing.assert_allclose(o, want, rtol=0, atol=1e-9)


def test_stream_snapshot_resume_is_identical():
    W, T = 20, 60
    q, k, v = (rnd((1, T, 2, 64), s) for s in (78, 79, 80))
    a, rk, rv = run_stream(q[:, :30], k[:, :30], v[:, :30], W, [4])
    # resume twice from the same snapshot
    outs = []
    for _ in range(2):
        rk2, rv2, pos = rk.copy(), rv.copy(), np.array([30], np.int64)
        o = oracle.stream_step(q[:, 30:34], k[:, 30:34], v[:, 30:34], rk2, rv2, pos, W)
        outs.append(o)
    np.testing.assert_array_equal(outs[0], outs[1])


def test_stream_rejects_chunk_larger_than_window():
    ring = np.zeros((1, 1, 4, 64))
    x = np.zeros((1, 5, 1, 64))
    with pytest.raises(ValueError):
        oracle.stream_step(x, x, x, ring, ring, np.array([0], np.int64), 4)


# --------------------------------------------------------------------------
# constants the pages print
# --------------------------------------------------------------------------

def test_workload_constants_match_pages():
    c = json.load(open(os.path.join(GOLDEN, "voxtral_realtime_constants.json")))
    W = c["encoder_window_frames"]["value"]
    for name in ("layer", "stack", "long", "stream"):
        cfg = synth.CONFIGS[name]
        assert cfg.W == W
        assert cfg.theta == c["encoder_rope_theta"]["value"]
        assert cfg.D == c["encoder_head_dim"]["value"]
        assert cfg.H == c["encoder_heads"]["value"]
    assert synth.CONFIGS["stream"].n == c["encoder_frames_per_step"]["value"]
    # 30 s of audio at 16 kHz / hop 160 / stride 2 = 1500 encoder frames
    frames = 30 * c["sample_rate_hz"]["value"] // c["mel_hop"]["value"] // c["conv2_stride"]["value"]
    assert frames == synth.CONFIGS["layer"].T == 1500
    assert c["mel_frames_per_audio_token"]["value"] // c["conv2_stride"]["value"] == 4


def test_oracle_regression_record_tiny():
    # Written by tests/golden/make_oracle_golden.py (oracle only); guards
    # against unintended changes of the oracle's arithmetic.
    rec = json.load(open(os.path.join(GOLDEN, "oracle_tiny.json")))
    c = synth.CONFIGS["tiny"]
    x = synth.make_config("tiny")
    assert {k: synth.sha256(x[k]) for k in ("q", "k", "v")} == rec["input_sha256"]
    o = oracle.prefill(x["q"], x["k"], x["v"], c.W, theta=c.theta)
    assert abs(o.sum() - rec["sum"]) < 1e-9
    assert abs((o * o).sum() - rec["sum_sq"]) < 1e-9
    for key, val in rec["samples"].items():
        t, h, d = map(int, key.split(","))
        assert abs(o[0, t, h, d] - val) < 1e-12


def test_prefill_varlen_is_per_stream_prefill_plus_ring_seed():
    """The batched first-chunk composition: each packed stream equals its own
    prefill, and its ring holds the last W frames (value rows exactly, key rows
    rotated at their own positions) in slot t mod W; an empty stream leaves
    its ring untouched."""
    from sliding_window_attention_vx_amd import synth
    lengths = [5, 0, 9]
    x = synth.make_first_chunks(3, 2, lengths, seed=11, dtype="f32", scale=1.0)
    W = 4
    rk = np.full((3, 2, W, 64), 5.0)
    rv = rk.copy()
    pos = np.full(3, -1, dtype=np.int64)
    o = oracle.prefill_varlen(x["q"], x["k"], x["v"], x["cu"], W, ring_k=rk, ring_v=rv, pos=pos)
    assert list(pos) == lengths
    cu = x["cu"]
    for s, T in enumerate(lengths):
        a, b = int(cu[s]), int(cu[s + 1])
        if T == 0:
            assert np.all(rk[s] == 5.0) and np.all(rv[s] == 5.0)
            continue
        want = oracle.prefill(x["q"][None, a:b], x["k"][None, a:b], x["v"][None, a:b], W)[0]
        np.testing.assert_array_equal(o[a:b], want)
        krot = oracle.rope(x["k"][None, a:b])[0]  # positions 0 .. T-1
        for t in range(max(0, T - W), T):
            np.testing.assert_array_equal(rv[s][:, t % W], x["v"][a + t])
            np.testing.assert_array_equal(rk[s][:, t % W], krot[t])
        if T < W:  # slots past the chunk keep their contents
            assert np.all(rk[s][:, T:] == 5.0)


# --------------------------------------------------------------------------
# grouped-query attention (text decoder: 32 query heads over 8 key/value
# heads, head_dim 128, window 8192, RoPE theta 1e6)
# --------------------------------------------------------------------------

def _expand_kv(x, G):
    """Copy each key/value head to G consecutive query heads (the
    repeat_interleave form of GQA the Core AI page compares against a
    broadcast form); axis 2 is the head axis of [B,T,H,D]."""
    return np.repeat(x, G, axis=2)


@pytest.mark.parametrize("T,W,Hq,Hkv,D", [(40, 7, 4, 2, 16), (48, 16, 8, 2, 128),
                                           (33, 40, 4, 1, 8), (20, 5, 3, 3, 8)])
def test_gqa_prefill_matches_dense_brute_force(T, W, Hq, Hkv, D):
    q = rnd((1, T, Hq, D), 80)
    k, v = rnd((1, T, Hkv, D), 81), rnd((1, T, Hkv, D), 82)
    pos = np.arange(T)
    G = Hq // Hkv
    kr = _expand_kv(complex_rope(k[0], pos)[None], G)[0]
    want = dense_band_attention(complex_rope(q[0], pos), kr, _expand_kv(v, G)[0], W)
    np.testing.assert_allclose(oracle.gqa_prefill(q, k, v, W)[0], want, rtol=0, atol=1e-12)


def test_gqa_prefill_matches_sdpa_grouped_mode():
    # torch SDPA's own grouped mode (enable_gqa: query head h reads key/value
    # head h // (Hq/Hkv)) with a band mask, at the decoder's head_dim 128.
    import torch
    import torch.nn.functional as F
    from tests.refimpl import band_mask
    B, T, Hq, Hkv, D, W = 2, 80, 8, 2, 128, 30
    q, k, v = rnd((B, T, Hq, D), 83), rnd((B, T, Hkv, D), 84), rnd((B, T, Hkv, D), 85)
    pos = np.arange(T)
    qr = np.stack([complex_rope(q[b], pos) for b in range(B)])
    kr = np.stack([complex_rope(k[b], pos) for b in range(B)])
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(0, 2, 1, 3)))
    want = F.scaled_dot_product_attention(t(qr), t(kr), t(v),
                                          attn_mask=torch.from_numpy(band_mask(T, W)),
                                          enable_gqa=True).numpy().transpose(0, 2, 1, 3)
    np.testing.assert_allclose(oracle.gqa_prefill(q, k, v, W), want, rtol=0, atol=1e-12)


def test_gqa_with_one_group_is_multi_head():
    q, k, v = (rnd((2, 30, 4, 16), s) for s in (86, 87, 88))
    np.testing.assert_array_equal(oracle.gqa_prefill(q, k, v, 9), oracle.prefill(q, k, v, 9))


def test_gqa_key_value_head_touches_only_its_group():
    # Changing key/value head j changes the outputs of query heads jG .. jG+G-1 only.
    T, Hq, Hkv, D, W = 24, 8, 4, 16, 10
    G = Hq // Hkv
    q, k, v = rnd((1, T, Hq, D), 89), rnd((1, T, Hkv, D), 90), rnd((1, T, Hkv, D), 91)
    base = oracle.gqa_prefill(q, k, v, W)
    for j in range(Hkv):
        k2, v2 = k.copy(), v.copy()
        k2[:, :, j] += 1.0
        v2[:, :, j] *= -2.0
        o = oracle.gqa_prefill(q, k2, v2, W)
        changed = np.any(o != base, axis=(0, 1, 3))
        assert list(np.nonzero(changed)[0]) == list(range(j * G, (j + 1) * G)), j


def test_gqa_rope_frequencies_closed_form_head_dim_128():
    # theta = 1e6, D = 128: f_i = 1e6^(-2i/128) = 10^(-3i/32); the basis vector
    # e_i at position 1 turns by f_i radians into dims (i, i+64).
    D = 128
    for i in (0, 1, 32, 63):
        f = 10.0 ** (-3.0 * i / 32.0)
        x = np.zeros((1, 1, 1, D))
        x[0, 0, 0, i] = 1.0
        r = oracle.rope(x, pos=np.array([[1]]), theta=1e6)[0, 0, 0]
        assert abs(math.atan2(r[i + 64], r[i]) - f) < 1e-15 * max(1.0, f) + 1e-18, i
        assert np.all(np.delete(r, [i, i + 64]) == 0.0)


def run_gqa_decode(q, k, v, W, n=1, bf16=False, prefix=0):
    """Feed q [1,T,Hq,D], k/v [1,T,Hkv,D] through gqa_stream_step + ring_append,
    n tokens per step, over garbage-filled W-slot rings.  The first `prefix`
    tokens are only appended (no attention), so decoding starts at that
    position with a full history; returns the outputs of the decoded tokens."""
    _, T, Hq, D = q.shape
    Hkv = k.shape[2]
    ring_k = np.full((1, Hkv, W, D), 1e3)
    ring_v = np.full((1, Hkv, W, D), -1e3)
    pos = np.array([0], dtype=np.int64)
    for t in range(0, prefix, W):
        sl = slice(t, min(prefix, t + W))
        oracle.ring_append(ring_k, ring_v, k[:, sl], v[:, sl], pos, W, bf16=bf16)
    out = np.zeros_like(q[:, prefix:])
    for t in range(prefix, T, n):
        sl = slice(t, min(T, t + n))
        out[:, t - prefix:sl.stop - prefix] = oracle.gqa_stream_step(
            q[:, sl], k[:, sl], v[:, sl], ring_k, ring_v, pos, W, bf16=bf16)
        oracle.ring_append(ring_k, ring_v, k[:, sl], v[:, sl], pos, W, bf16=bf16)
    return out


@pytest.mark.parametrize("n", [1, 3])
def test_gqa_decode_equals_prefill_across_ring_wraps(n):
    # Token-by-token decode over a W-slot ring equals whole-prompt prefill.
    W, T, Hq, Hkv, D = 16, 53, 8, 2, 128
    q, k, v = rnd((1, T, Hq, D), 92), rnd((1, T, Hkv, D), 93), rnd((1, T, Hkv, D), 94)
    got = run_gqa_decode(q, k, v, W, n=n)
    np.testing.assert_allclose(got, oracle.gqa_prefill(q, k, v, W), rtol=0, atol=1e-12)


def test_gqa_decode_equals_prefill_bf16_contract_past_the_window():
    # Decode from position 8190 (rings wrapped many times) in the bf16
    # contract: the decoded tail equals the tail of one prefill over all tokens.
    W, p0, T, Hq, Hkv, D = 12, 8190, 8230, 4, 1, 32
    q, k, v = rnd((1, T, Hq, D), 95), rnd((1, T, Hkv, D), 96), rnd((1, T, Hkv, D), 97)
    got = run_gqa_decode(q, k, v, W, bf16=True, prefix=p0)
    want = oracle.gqa_prefill(q, k, v, W, bf16=True)[:, p0:]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_gqa_rejects_indivisible_heads():
    x6, x4 = np.zeros((1, 3, 6, 8)), np.zeros((1, 3, 4, 8))
    with pytest.raises(ValueError):
        oracle.gqa_prefill(x6, x4, x4, 2)
    with pytest.raises(ValueError):
        oracle.gqa_stream_step(x6, x4, x4, np.zeros((1, 4, 2, 8)), np.zeros((1, 4, 2, 8)),
                               np.array([0], np.int64), 2)


def test_decoder_constants_match_pages():
    c = json.load(open(os.path.join(GOLDEN, "voxtral_realtime_constants.json")))
    for name in ("dec_prefill", "dec_decode"):
        cfg = synth.GQA_CONFIGS[name]
        assert cfg.Hq == c["text_decoder_heads_q"]["value"]
        assert cfg.Hkv == c["text_decoder_heads_kv"]["value"]
        assert cfg.D == c["text_decoder_head_dim"]["value"]
        assert cfg.W == c["text_decoder_window"]["value"]
        assert cfg.theta == c["text_decoder_rope_theta"]["value"]


# --------------------------------------------------------------------------
# encoder attention block: projections around the streaming step
# --------------------------------------------------------------------------

def test_linear_matches_loops():
    x, w, b = rnd((3, 5), 100), rnd((4, 5), 101), rnd(4, 102)
    got = oracle.linear(x, w, b)
    for m in range(3):
        for n in range(4):
            want = b[n] + sum(x[m, kk] * w[n, kk] for kk in range(5))
            assert abs(got[m, n] - want) < 1e-12
    np.testing.assert_allclose(oracle.linear(x, w), got - b[None, :], rtol=0, atol=1e-12)


def test_qkv_rope_split_order_bias_and_positions():
    # d_model 64, one head: q rows = I (plus b_q), k rows = 2I (no bias), v rows = a
    # permutation (plus b_v); so q' and k' are rotations of known vectors at the
    # row positions, and v is the permuted input plus its bias.
    M, H = 5, 1
    x = rnd((M, 64), 103)
    perm = np.random.default_rng(104).permutation(64)
    w = np.concatenate([np.eye(64), 2 * np.eye(64), np.eye(64)[perm]])
    bq, bv = rnd(64, 105), rnd(64, 106)
    pos = np.array([0, 1, 749, 750, 123456])
    q, k, v = oracle.enc_qkv_rope(x, w, bq, bv, pos, H)
    np.testing.assert_allclose(q[:, 0], complex_rope((x + bq)[:, None], pos)[:, 0], atol=1e-12)
    np.testing.assert_allclose(k[:, 0], complex_rope((2 * x)[:, None], pos)[:, 0], atol=1e-12)
    np.testing.assert_array_equal(v[:, 0], x[:, perm] + bv)


def test_enc_attn_step_zero_output_weights_give_bias():
    S, n, H, W, dm = 2, 3, 2, 8, 16
    x = rnd((S, n, dm), 107)
    w_qkv, bq, bv = rnd((3 * H * 64, dm), 108), rnd(H * 64, 109), rnd(H * 64, 110)
    b_o = rnd(dm, 111)
    rk, rv = np.zeros((S, H, W, 64)), np.zeros((S, H, W, 64))
    pos = np.array([0, 5], dtype=np.int64)
    y = oracle.enc_attn_step(x, w_qkv, bq, bv, np.zeros((dm, H * 64)), b_o, rk, rv, pos, W, H)
    np.testing.assert_array_equal(y, np.broadcast_to(b_o, y.shape))
    assert list(pos) == [3, 8]


@pytest.mark.parametrize("bf16", [False, True])
def test_enc_attn_step_streamed_equals_prefill_of_projected_sequence(bf16):
    # Streaming the block n frames at a time over a W-slot ring gives the same
    # y as projecting the whole sequence, one prefill over it, and the output
    # projection (the bf16 contract rounds q', k', v and o on both sides).
    T, H, W, dm, n = 40, 2, 12, 32, 4
    x = rnd((1, T, dm), 112) * 0.5
    w_qkv = rnd((3 * H * 64, dm), 113) / np.sqrt(dm)
    bq, bv = rnd(H * 64, 114) * 0.1, rnd(H * 64, 115) * 0.1
    w_o, b_o = rnd((dm, H * 64), 116) / np.sqrt(H * 64), rnd(dm, 117) * 0.1
    rk, rv = np.full((1, H, W, 64), 1e3), np.full((1, H, W, 64), -1e3)
    pos = np.zeros(1, dtype=np.int64)
    got = np.concatenate([oracle.enc_attn_step(x[:, t:t + n], w_qkv, bq, bv, w_o, b_o, rk, rv, pos,
                                               W, H, bf16=bf16) for t in range(0, T, n)], axis=1)
    q, k, v = oracle.enc_qkv_rope(x[0], w_qkv, bq, bv, np.arange(T), H, bf16=bf16)
    o = oracle.prefill(q[None], k[None], v[None], W, rope_applied=True)[0]
    if bf16:
        o = oracle.bf16_round(o)
    want = oracle.linear(o.reshape(T, H * 64), w_o, b_o)
    np.testing.assert_allclose(got[0], want, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# whole encoder step: norms, activations, conv stem, layer
# --------------------------------------------------------------------------

def test_rmsnorm_closed_forms():
    g = rnd(6, 120)
    c = 2.5
    y = oracle.rmsnorm(np.full((1, 6), c), g, eps=0.0)
    np.testing.assert_allclose(y[0], g * np.sign(c), atol=1e-15)
    y = oracle.rmsnorm(np.full((1, 6), 0.1), np.ones(6), eps=0.01)
    np.testing.assert_allclose(y, 0.1 / math.sqrt(0.01 + 0.01), atol=1e-15)
    x = rnd((3, 1280), 121)
    r = oracle.rmsnorm(x, np.ones(1280), eps=0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(r * r, axis=-1)), 1.0, atol=1e-12)


def test_gelu_and_silu_against_standard_library():
    xs = np.linspace(-6, 6, 97)
    want = [0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in xs]
    np.testing.assert_allclose(oracle.gelu(xs), want, rtol=0, atol=1e-15)
    assert oracle.gelu(np.array([1.0]))[0] == pytest.approx(0.8413447460685429, abs=1e-15)
    # silu(ln 3) = ln 3 * sigmoid(ln 3) = 0.75 ln 3
    assert oracle.silu(np.array([math.log(3)]))[0] == pytest.approx(0.75 * math.log(3), abs=1e-15)
    np.testing.assert_allclose(oracle.silu(xs), [v / (1 + math.exp(-v)) for v in xs], atol=1e-15)


@pytest.mark.parametrize("stride", [1, 2])
def test_causal_conv1d_brute_force_and_causality(stride):
    S, T, Ci, Co, k = 2, 8, 3, 4, 3
    xp = rnd((S, T + k - 1, Ci), 122)
    w, b = rnd((Co, k, Ci), 123), rnd(Co, 124)
    y = oracle.causal_conv1d(xp, w, b, stride)
    assert y.shape == (S, T // stride, Co)
    for s in range(S):
        for t in range(T // stride):
            for o in range(Co):
                want = b[o] + sum(w[o, j, c] * xp[s, stride * t + j, c]
                                  for j in range(k) for c in range(Ci))
                assert abs(y[s, t, o] - want) < 1e-12
    # output t reads padded frames up to stride*t + k - 1 only
    xq = xp.copy()
    xq[:, stride * 2 + k:] += 100.0
    np.testing.assert_array_equal(oracle.causal_conv1d(xq, w, b, stride)[:, :3], y[:, :3])


@pytest.mark.parametrize("bf16", [False, True])
def test_stem_streamed_equals_offline_with_zero_history(bf16):
    # 5 steps of 8 mel frames through the cached stem equal one causal pass over
    # all 40 frames with two zero frames of left padding for each conv
    S, n_mel, C = 2, 6, 10
    w1, b1 = rnd((C, 3, n_mel), 125) * 0.3, rnd(C, 126) * 0.1
    w2, b2 = rnd((C, 3, C), 127) * 0.3, rnd(C, 128) * 0.1
    mel = rnd((S, 40, n_mel), 129)
    mc, cc = np.zeros((S, 2, n_mel)), np.zeros((S, 2, C))
    got = np.concatenate([oracle.enc_stem_step(mel[:, 8 * i:8 * i + 8], mc, cc, w1, b1, w2, b2,
                                               bf16=bf16) for i in range(5)], axis=1)
    c1 = oracle.gelu(oracle.causal_conv1d(np.concatenate([np.zeros((S, 2, n_mel)), mel], 1), w1, b1, 1))
    if bf16:
        c1 = oracle.bf16_round(c1)
    want = oracle.gelu(oracle.causal_conv1d(np.concatenate([np.zeros((S, 2, C)), c1], 1), w2, b2, 2))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(mc, mel[:, -2:])


def _layer_weights(dm, H, ffn, seed):
    r = lambda shape, s, sc: rnd(shape, seed + s) * sc
    return dict(g_attn=1 + r(dm, 0, 0.1), w_qkv=r((3 * H * 64, dm), 1, dm ** -0.5),
                b_q=r(H * 64, 2, 0.1), b_v=r(H * 64, 3, 0.1), w_o=r((dm, H * 64), 4, (H * 64) ** -0.5),
                b_o=r(dm, 5, 0.1), g_ffn=1 + r(dm, 6, 0.1), w_gate=r((ffn, dm), 7, dm ** -0.5),
                w_up=r((ffn, dm), 8, dm ** -0.5), w_down=r((dm, ffn), 9, ffn ** -0.5),
                b_down=r(dm, 10, 0.1))


@pytest.mark.parametrize("bf16", [False, True])
def test_layer_streamed_equals_offline_layer(bf16):
    # the layer streamed 4 frames at a time over W-slot rings equals the same
    # layer over the whole sequence with one prefill for its attention
    T, H, W, dm, ffn, n = 24, 2, 10, 32, 48, 4
    wts = _layer_weights(dm, H, ffn, 130)
    x = rnd((1, T, dm), 131)
    rk, rv = np.full((1, H, W, 64), 1e3), np.full((1, H, W, 64), -1e3)
    pos = np.zeros(1, dtype=np.int64)
    got = np.concatenate([oracle.enc_layer_step(x[:, t:t + n], wts, rk, rv, pos, W, H, bf16=bf16)
                          for t in range(0, T, n)], axis=1)
    rd = oracle.bf16_round if bf16 else (lambda a: a)
    h = rd(oracle.rmsnorm(x[0], wts["g_attn"]))
    q, k, v = oracle.enc_qkv_rope(h, wts["w_qkv"], wts["b_q"], wts["b_v"], np.arange(T), H, bf16=bf16)
    o = rd(oracle.prefill(q[None], k[None], v[None], W, rope_applied=True)[0])
    x1 = x[0] + oracle.linear(o.reshape(T, H * 64), wts["w_o"], wts["b_o"])
    h = rd(oracle.rmsnorm(x1, wts["g_ffn"]))
    u = rd(oracle.silu(oracle.linear(h, wts["w_gate"])) * oracle.linear(h, wts["w_up"]))
    want = x1 + oracle.linear(u, wts["w_down"], wts["b_down"])
    np.testing.assert_allclose(got[0], want, rtol=0, atol=1e-11)
