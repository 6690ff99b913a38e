"""GPU parity of the projections around the encoder's attention
(vx_linear, vx_enc_qkv_rope, vx_enc_attn_step) against the float64 oracle.

Tolerances: the projections accumulate bf16 products in float32, so a
plain product in float32 output is within 1e-4 relative to its scale of the
float64 product of the same bf16 inputs; a value stored as bf16 (q', k', v)
is within one bf16 rounding (2^-7 relative) plus 1e-4 of the float64 value.
The block's output y is checked like the attention (max |err| <= 2e-2,
relative RMS <= 1e-2) against the bf16-contract oracle, which rounds every
tensor the block stores between its launches (q', k', v, o) to bf16.
"""
import numpy as np
import pytest

import oracle
import sliding_window_attention_vx_amd as vx
from sliding_window_attention_vx_amd import synth
from tests.test_gpu_parity import check_bf16, dev, host, say

pytestmark = pytest.mark.gpu


def _rnd(shape, seed, scale=1.0):
    return synth.round_to_bf16(
        np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * np.float32(scale))


@pytest.mark.parametrize("M,N,K,bias", [(1, 32, 128, False), (5, 96, 256, True),
                                        (64, 64, 128, True), (100, 1280, 2048, True),
                                        (256, 6144, 1280, False), (256, 1280, 2048, True),
                                        (37, 192, 384, True)])
def test_linear_matches_float64_product(M, N, K, bias):
    say(f"linear M{M} N{N} K{K} bias {bias}")
    x, w = _rnd((M, K), 1), _rnd((N, K), 2, K ** -0.5)
    b = _rnd(N, 3, 0.1) if bias else None
    want = oracle.linear(x, w, b)
    y32 = host(vx.linear(dev(x, "bf16"), dev(w, "bf16"), None if b is None else dev(b, "bf16"),
                         out_dtype="f32"))
    scale = np.sqrt(np.mean(want ** 2))
    err = np.max(np.abs(y32 - want))
    say(f"  f32 out: max|err| {err:.3e} (scale {scale:.3e})")
    assert err <= 1e-4 * scale
    y16 = host(vx.linear(dev(x, "bf16"), dev(w, "bf16"), None if b is None else dev(b, "bf16")))
    assert np.all(np.abs(y16 - want) <= np.abs(want) * 2.0 ** -7 + 1e-4 * scale)


def _close_bf16(got, want, what):
    scale = np.sqrt(np.mean(want ** 2))
    bad = np.abs(got - want) > np.abs(want) * 2.0 ** -7 + 1e-4 * scale
    say(f"{what}: {int(bad.sum())} of {bad.size} beyond one bf16 rounding")
    assert not bad.any()


@pytest.mark.parametrize("S,n,H,dm,bias", [(3, 4, 2, 128, True), (64, 4, 32, 1280, True),
                                           (1, 1, 4, 256, False), (5, 3, 2, 384, True)])
def test_enc_qkv_rope_matches_oracle(S, n, H, dm, bias):
    import torch
    say(f"qkv+rope S{S} n{n} H{H} d_model {dm}")
    wts = synth.make_enc_block_weights(dm, H, seed=[5, dm])
    x = synth.make_enc_block_input(S, n, dm, seed=5, step=0)
    pos = np.random.default_rng(6).integers(0, 30000, size=S).astype(np.int64)
    bq, bv = (wts["b_q"], wts["b_v"]) if bias else (None, None)
    q, k, v = vx.enc_qkv_rope(dev(x, "bf16"), dev(wts["w_qkv"], "bf16"),
                              None if bq is None else dev(bq, "bf16"),
                              None if bv is None else dev(bv, "bf16"),
                              torch.from_numpy(pos).cuda(), H=H)
    pos_rows = (pos[:, None] + np.arange(n)[None, :]).reshape(-1)
    wq, wk, wv = oracle.enc_qkv_rope(x.reshape(S * n, dm), wts["w_qkv"], bq, bv, pos_rows, H)
    for name, got, want in (("q'", q, wq), ("k'", k, wk), ("v", v, wv)):
        _close_bf16(host(got).reshape(S * n, H, 64), want, name)


def _block_inputs(S, n, H, dm, W, seed):
    import torch
    wts = synth.make_enc_block_weights(dm, H, seed=seed)
    st = synth.make_stream_state(S, H, W, seed=[seed, 1], pos_lo=W, pos_hi=20000)
    d = {k_: dev(v_, "bf16") for k_, v_ in wts.items()}
    rk, rv = dev(st["ring_k"], "bf16"), dev(st["ring_v"], "bf16")
    pin = torch.from_numpy(st["pos"].copy()).cuda()
    return wts, st, d, rk, rv, pin, torch.empty_like(pin)


def test_enc_attn_step_full_workload_sampled_streams():
    c = synth.ENC_BLOCK
    S, n, H, dm, W = c["S"], c["n"], c["H"], c["d_model"], c["W"]
    say(f"encoder attention block step S{S} n{n} H{H} d_model {dm} W{W}; oracle on sampled streams")
    wts, st, d, rk, rv, pin, pout = _block_inputs(S, n, H, dm, W, c["seed"])
    x = synth.make_enc_block_input(S, n, dm, seed=c["seed"], step=0)
    y = host(vx.enc_attn_step(dev(x, "bf16"), d["w_qkv"], d["b_q"], d["b_v"], d["w_o"], d["b_o"],
                              rk, rv, pin, pout, window=W, H=H, out_dtype="f32"))
    np.testing.assert_array_equal(host(pout.double()), st["pos"] + n)
    for s in (0, 21, 63):
        sl = slice(s, s + 1)
        rk_o = st["ring_k"][sl].astype(np.float64)
        rv_o = st["ring_v"][sl].astype(np.float64)
        p_o = st["pos"][sl].copy()
        want = oracle.enc_attn_step(x[sl], wts["w_qkv"], wts["b_q"], wts["b_v"], wts["w_o"],
                                    wts["b_o"], rk_o, rv_o, p_o, W, H, bf16=True)
        check_bf16(y[sl], want, f"block y stream {s}")
        # appended rows: the projected v and rotated k, each one bf16 rounding of an fp32
        # accumulation, so within one rounding of the oracle's float64 values
        _close_bf16(host(rv[sl]), rv_o, f"ring v stream {s}")
        _close_bf16(host(rk[sl]), rk_o, f"ring k stream {s}")


def test_enc_attn_step_consecutive_steps_match_oracle():
    # several steps in a row, rings wrapping, against the oracle stepped alongside
    import torch
    S, n, H, dm, W = 3, 4, 2, 256, 16
    say(f"block steps S{S} n{n} H{H} d_model {dm} W{W}")
    wts, st, d, rk, rv, pin, pout = _block_inputs(S, n, H, dm, W, 9)
    rk_o, rv_o = st["ring_k"].astype(np.float64), st["ring_v"].astype(np.float64)
    p_o = st["pos"].copy()
    for step in range(9):
        x = synth.make_enc_block_input(S, n, dm, seed=9, step=step)
        y = host(vx.enc_attn_step(dev(x, "bf16"), d["w_qkv"], d["b_q"], d["b_v"], d["w_o"],
                                  d["b_o"], rk, rv, pin, pout, window=W, H=H, out_dtype="f32"))
        want = oracle.enc_attn_step(x, wts["w_qkv"], wts["b_q"], wts["b_v"], wts["w_o"],
                                    wts["b_o"], rk_o, rv_o, p_o, W, H, bf16=True)
        check_bf16(y, want, f"step {step}")
        pin, pout = pout, pin
    np.testing.assert_array_equal(host(pin.double()), p_o)
    torch.cuda.synchronize()
