"""GPU parity of the grouped-query (text decoder) entry points against the
float64 oracle: vx_gqa_attn_prefill and vx_gqa_attn_decode, head_dim 128.

Tolerances as in test_gpu_parity: bf16 max |err| <= 2e-2 and relative RMS
<= 1e-2 against the bf16-contract oracle (rotated q, k rounded to bf16, the
rest exact).  Ring contents: values bit-exact, rotated keys within one bf16
rounding of the oracle's (a float32 rotation can round the other way at a
tie).  At the full prompt size (T 16384, W 8192) the oracle computes sampled
query rows: the rows t0 .. t0+n-1 of a prefill equal a decode step of those
rows over a ring holding the W-1 frames before t0 (a composition of
oracle.ring_append and oracle.gqa_stream_step, pinned against oracle
prefill on the CPU).
"""
import numpy as np
import pytest

import oracle
import sliding_window_attention_vx_amd as vx
from sliding_window_attention_vx_amd import synth
from tests.test_gpu_parity import check_bf16, dev, host, say

pytestmark = pytest.mark.gpu

D = 128


def _prefill(x, W, out_dtype="f32", rings=False, fill=0.0, rope_applied=False, k_rot=False):
    import torch
    q, k, v = (dev(x[n], "bf16") for n in ("q", "k", "v"))
    B, T, Hkv = k.shape[0], k.shape[1], k.shape[2]
    rk = rv = pos = None
    if rings:
        rk = torch.full((B, Hkv, W, D), fill, device="cuda").to(torch.bfloat16)
        rv = rk.clone()
        pos = torch.full((B,), -7, dtype=torch.int64, device="cuda")
    o = vx.gqa_prefill(q, k, v, window=W, ring_k=rk, ring_v=rv, pos=pos, out_dtype=out_dtype,
                       rope_applied=rope_applied, k_rot=torch.empty_like(k) if k_rot else None)
    return o, rk, rv, pos


def _oracle_rows(x, b, t0, n, W):
    """Exact bf16-contract prefill outputs of rows t0 .. t0+n-1 of batch entry b."""
    Hkv = x["k"].shape[2]
    s0 = max(0, t0 - W + 1)
    rk = np.zeros((1, Hkv, W, D))
    rv = np.zeros((1, Hkv, W, D))
    pos = np.array([s0], dtype=np.int64)
    if t0 > s0:
        oracle.ring_append(rk, rv, x["k"][b:b + 1, s0:t0], x["v"][b:b + 1, s0:t0], pos, W,
                           bf16=True)
    sl = (slice(b, b + 1), slice(t0, t0 + n))
    return oracle.gqa_stream_step(x["q"][sl], x["k"][sl], x["v"][sl], rk, rv, pos, W,
                                  bf16=True)[0]


def test_gqa_rope_table_values_head_dim_128():
    say("rope_table head_dim 128, p 0..20000")
    t = host(vx.rope_table(0, 20001, head_dim=D))
    p = np.arange(20001, dtype=np.float64)[:, None]
    f = 1e6 ** (-2.0 * np.arange(64) / 128.0)
    assert np.max(np.abs(t[:, 0] - np.cos(p * f))) <= 6.0e-8
    assert np.max(np.abs(t[:, 1] - np.sin(p * f))) <= 6.0e-8


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_gqa_prefill_tiny(out_dtype):
    c = synth.GQA_CONFIGS["dec_tiny"]
    say(f"gqa prefill B{c.B} T{c.T} Hq{c.Hq} Hkv{c.Hkv} W{c.W} -> {out_dtype}")
    x = synth.make_gqa_config("dec_tiny")
    o, *_ = _prefill(x, c.W, out_dtype)
    want = oracle.gqa_prefill(x["q"], x["k"], x["v"], c.W, bf16=True)
    check_bf16(host(o), want, f"gqa tiny {out_dtype}")


@pytest.mark.parametrize("B,T,Hq,Hkv,W", [(1, 130, 8, 8, 50), (2, 97, 8, 4, 40), (1, 200, 8, 1, 70),
                                          (1, 1, 4, 1, 16), (2, 33, 4, 1, 1), (1, 64, 4, 1, 64),
                                          (1, 65, 4, 1, 64), (1, 300, 16, 4, 300),
                                          (3, 150, 32, 8, 100)])
def test_gqa_prefill_group_sizes_and_edges(B, T, Hq, Hkv, W):
    say(f"gqa prefill B{B} T{T} Hq{Hq} Hkv{Hkv} W{W}")
    x = synth.make_gqa_prefill(B, T, Hq, Hkv, seed=[31, T, Hq, Hkv, W])
    o, *_ = _prefill(x, W)
    want = oracle.gqa_prefill(x["q"], x["k"], x["v"], W, bf16=True)
    check_bf16(host(o), want, f"gqa B{B} T{T} G{Hq // Hkv} W{W}")


def test_gqa_prefill_pre_rotated_input_equals_fused_rope():
    import torch
    x = synth.make_gqa_prefill(1, 180, 8, 2, seed=32)
    o_fused, *_ = _prefill(x, 60, out_dtype="bf16")
    # rotate on the host in the bf16 contract, then call with rope_applied
    qr = oracle.bf16_round(oracle.rope(x["q"]))
    kr = oracle.bf16_round(oracle.rope(x["k"]))
    y = dict(q=qr, k=kr, v=x["v"])
    o_pre, *_ = _prefill(y, 60, out_dtype="bf16", rope_applied=True)
    torch.cuda.synchronize()
    want = oracle.gqa_prefill(x["q"], x["k"], x["v"], 60, bf16=True)
    check_bf16(host(o_pre), want, "pre-rotated")
    check_bf16(host(o_fused), host(o_pre), "fused vs pre-rotated")


@pytest.mark.parametrize("k_rot", [True, False])
def test_gqa_prefill_full_size_sampled_rows(k_rot):
    c = synth.GQA_CONFIGS["dec_prefill"]
    say(f"gqa prefill full size B{c.B} T{c.T} Hq{c.Hq} Hkv{c.Hkv} W{c.W} k_rot {k_rot}; "
        "oracle on sampled rows")
    x = synth.make_gqa_config("dec_prefill")
    o, *_ = _prefill(x, c.W, out_dtype="bf16", k_rot=k_rot)
    got = host(o)
    assert np.all(np.isfinite(got))
    for t0 in (0, 1000, c.W - 3, c.W + 517, c.T - 4):
        n = 4
        want = _oracle_rows(x, 0, t0, n, c.W)
        check_bf16(got[0, t0:t0 + n], want, f"rows {t0}..{t0 + n - 1}")


def test_gqa_prefill_seeds_rings():
    B, T, Hq, Hkv, W = 2, 150, 8, 2, 64
    say(f"gqa prefill seeding B{B} T{T} W{W}")
    x = synth.make_gqa_prefill(B, T, Hq, Hkv, seed=33)
    o, rk, rv, pos = _prefill(x, W, rings=True, fill=5.0)
    check_bf16(host(o), oracle.gqa_prefill(x["q"], x["k"], x["v"], W, bf16=True), "seeded prefill")
    rk_o = np.full((B, Hkv, W, D), 5.0)
    rv_o = rk_o.copy()
    pos_o = np.zeros(B, dtype=np.int64)
    for s in range(0, T, W):
        e = min(T, s + W)
        oracle.ring_append(rk_o, rv_o, x["k"][:, s:e], x["v"][:, s:e], pos_o, W, bf16=True)
    np.testing.assert_array_equal(host(pos.double()), pos_o)
    np.testing.assert_array_equal(host(rv), rv_o)
    gk = host(rk)
    assert np.all(np.abs(gk - rk_o) <= np.abs(rk_o) * 2.0 ** -7 + 1e-30)
    assert (gk != rk_o).mean() < 1e-3


def test_gqa_prefill_deterministic():
    import torch
    x = synth.make_gqa_prefill(1, 700, 32, 8, seed=34)
    a, *_ = _prefill(x, 256, out_dtype="bf16")
    b, *_ = _prefill(x, 256, out_dtype="bf16")
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------

def _decode_state(st):
    import torch
    rk, rv = dev(st["ring_k"], "bf16"), dev(st["ring_v"], "bf16")
    pos = torch.from_numpy(st["pos"].copy()).cuda()
    return rk, rv, pos, torch.empty_like(pos)


def test_gqa_decode_full_workload():
    import torch
    c = synth.GQA_CONFIGS["dec_decode"]
    say(f"gqa decode S{c.B} n{c.T} Hq{c.Hq} Hkv{c.Hkv} W{c.W}; oracle on sampled streams")
    st = synth.make_gqa_decode_state("dec_decode")
    fr = synth.make_gqa_frames(c.B, c.T, c.Hq, c.Hkv, seed=c.seed, step=0)
    rk, rv, pin, pout = _decode_state(st)
    rk0, rv0 = rk.clone(), rv.clone()
    qn, kn, vn = (dev(fr[n], "bf16") for n in ("q", "k", "v"))
    o = host(vx.gqa_decode(qn, kn, vn, rk, rv, pin, pout, window=c.W, out_dtype="f32"))
    assert np.all(np.isfinite(o))
    np.testing.assert_array_equal(host(pout.double()), st["pos"] + c.T)
    np.testing.assert_array_equal(host(pin.double()), st["pos"])
    for s in (0, 17, 40, 63):
        sl = slice(s, s + 1)
        want = oracle.gqa_stream_step(fr["q"][sl], fr["k"][sl], fr["v"][sl], st["ring_k"][sl],
                                      st["ring_v"][sl], st["pos"][sl], c.W, bf16=True)
        check_bf16(o[sl], want, f"decode stream {s}")
    # the append wrote slot pos mod W of every ring and nothing else
    slots = torch.from_numpy(st["pos"] % c.W).cuda()
    sidx = torch.arange(c.B, device="cuda")
    for new, old, src in ((rk, rk0, None), (rv, rv0, vn)):
        keep = torch.ones(c.B, c.W, dtype=torch.bool, device="cuda")
        keep[sidx, slots] = False
        assert torch.equal(new.permute(0, 2, 1, 3)[keep], old.permute(0, 2, 1, 3)[keep])
        if src is not None:
            assert torch.equal(new[sidx, :, slots], src[:, 0])
    krot = oracle.bf16_round(oracle.rope(fr["k"], pos=st["pos"][:, None]))
    gk = host(rk[sidx, :, slots])
    assert np.all(np.abs(gk - krot[:, 0]) <= np.abs(krot[:, 0]) * 2.0 ** -7 + 1e-30)


@pytest.mark.parametrize("Hq,Hkv,n,W", [(32, 8, 1, 64), (32, 8, 4, 40), (8, 1, 2, 100),
                                        (4, 4, 16, 64), (8, 4, 3, 8192)])
def test_gqa_decode_matches_oracle_at_varied_positions(Hq, Hkv, n, W):
    # positions: empty history, partial ring, exactly full, wrapped many times
    S = 6
    pos = np.array([0, 1, W - 1, W, W + 5, 7 * W + 3], dtype=np.int64)
    say(f"gqa decode Hq{Hq} Hkv{Hkv} n{n} W{W} pos {list(pos)}")
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([35, Hq, n, W])))
    st = dict(ring_k=synth.round_to_bf16(rng.standard_normal((S, Hkv, W, D), dtype=np.float32)),
              ring_v=synth.round_to_bf16(rng.standard_normal((S, Hkv, W, D), dtype=np.float32)),
              pos=pos)
    fr = synth.make_gqa_frames(S, n, Hq, Hkv, seed=[36, Hq, n, W], step=0)
    rk, rv, pin, pout = _decode_state(st)
    qn, kn, vn = (dev(fr[k], "bf16") for k in ("q", "k", "v"))
    o = host(vx.gqa_decode(qn, kn, vn, rk, rv, pin, pout, window=W, out_dtype="f32"))
    want = oracle.gqa_stream_step(fr["q"], fr["k"], fr["v"], st["ring_k"], st["ring_v"], pos, W,
                                  bf16=True)
    check_bf16(o, want, f"decode Hq{Hq} Hkv{Hkv} n{n} W{W}")
    rk_o, rv_o = st["ring_k"].astype(np.float64), st["ring_v"].astype(np.float64)
    p_o = pos.copy()
    oracle.ring_append(rk_o, rv_o, fr["k"], fr["v"], p_o, W, bf16=True)
    np.testing.assert_array_equal(host(pout.double()), p_o)
    np.testing.assert_array_equal(host(rv), rv_o)
    gk = host(rk)
    assert np.all(np.abs(gk - rk_o) <= np.abs(rk_o) * 2.0 ** -7 + 1e-30)


def _decode_run(x, W, n, rk, rv, p0):
    """Decode tokens p0.. of x (q [1,T,Hq,D], k/v [1,T,Hkv,D]) n at a time on the GPU."""
    import torch
    T = x["q"].shape[1]
    qd, kd, vd = (dev(x[k], "bf16") for k in ("q", "k", "v"))
    pin = torch.full((1,), p0, dtype=torch.int64, device="cuda")
    pout = torch.empty_like(pin)
    outs = []
    for t in range(p0, T, n):
        sl = slice(t, min(T, t + n))
        qn, kn, vn = (a[:, sl].contiguous() for a in (qd, kd, vd))
        outs.append(vx.gqa_decode(qn, kn, vn, rk, rv, pin, pout, window=W, out_dtype="f32"))
        pin, pout = pout, pin
    return host(torch.cat(outs, dim=1)), int(host(pin.double())[0])


@pytest.mark.parametrize("n,W,T", [(1, 64, 200), (4, 40, 130), (1, 8192, 300)])
def test_gqa_decode_token_by_token_equals_prefill(n, W, T):
    import torch
    Hq, Hkv = 32, 8
    say(f"gqa decode==prefill n{n} W{W} T{T}")
    x = synth.make_gqa_prefill(1, T, Hq, Hkv, seed=[37, n, W, T])
    rk = torch.full((1, Hkv, W, D), float("nan"), device="cuda").to(torch.bfloat16)
    rv = rk.clone()
    got, p = _decode_run(x, W, n, rk, rv, 0)
    assert p == T
    check_bf16(got, oracle.gqa_prefill(x["q"], x["k"], x["v"], W, bf16=True), "decoded vs oracle")
    pre, *_ = _prefill(x, W)
    check_bf16(got, host(pre), "decoded vs GPU prefill")


def test_gqa_prefill_seed_then_decode():
    # the prompt's prefill seeds the rings, decode continues from position T
    import torch
    Hq, Hkv, W, T0, T = 32, 8, 128, 300, 340
    say(f"gqa seed then decode W{W} T0 {T0} T {T}")
    x = synth.make_gqa_prefill(1, T, Hq, Hkv, seed=38)
    head = {k: v[:, :T0] for k, v in x.items()}
    _, rk, rv, pos = _prefill(head, W, rings=True, fill=float("nan"))
    torch.cuda.synchronize()
    assert int(host(pos.double())[0]) == T0
    got, p = _decode_run(x, W, 1, rk, rv, T0)
    assert p == T
    want = oracle.gqa_prefill(x["q"], x["k"], x["v"], W, bf16=True)[:, T0:]
    check_bf16(got, want, "decode after seeded prefill")


def test_gqa_decode_batch_invariance():
    import torch
    W, Hq, Hkv, S = 256, 32, 8, 12
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(39)))
    st = dict(ring_k=synth.round_to_bf16(rng.standard_normal((S, Hkv, W, D), dtype=np.float32)),
              ring_v=synth.round_to_bf16(rng.standard_normal((S, Hkv, W, D), dtype=np.float32)),
              pos=rng.integers(0, 3 * W, size=S).astype(np.int64))
    fr = synth.make_gqa_frames(S, 1, Hq, Hkv, seed=40, step=0)
    rk, rv, pin, pout = _decode_state(st)
    qn, kn, vn = (dev(fr[k], "bf16") for k in ("q", "k", "v"))
    full = vx.gqa_decode(qn, kn, vn, rk.clone(), rv.clone(), pin, pout, window=W)
    for s in (0, 5, 11):
        one = vx.gqa_decode(qn[s:s + 1].contiguous(), kn[s:s + 1].contiguous(),
                            vn[s:s + 1].contiguous(), rk[s:s + 1].clone(), rv[s:s + 1].clone(),
                            pin[s:s + 1].clone(), pout[s:s + 1].clone(), window=W)
        torch.cuda.synchronize()
        assert torch.equal(one[0], full[s])


@pytest.mark.parametrize("B,T,Hq,Hkv,W", [(2, 150, 8, 2, 64), (1, 700, 32, 8, 256)])
def test_gqa_prefill_k_rot_path_equals_fused(B, T, Hq, Hkv, W):
    # keys rotated once into k_rot, then attended: the same outputs and seeded
    # rings bit for bit as the single fused kernel, and k_rot holds the
    # bf16-rounded rotated keys
    import torch
    say(f"gqa prefill k_rot path B{B} T{T} Hq{Hq} Hkv{Hkv} W{W}")
    x = synth.make_gqa_prefill(B, T, Hq, Hkv, seed=[41, T])
    q, k, v = (dev(x[n], "bf16") for n in ("q", "k", "v"))
    outs = []
    for use_krot in (False, True):
        rk = torch.full((B, Hkv, W, D), 3.0, device="cuda").to(torch.bfloat16)
        rv = rk.clone()
        pos = torch.zeros(B, dtype=torch.int64, device="cuda")
        kr = torch.empty_like(k) if use_krot else None
        o = vx.gqa_prefill(q, k, v, window=W, ring_k=rk, ring_v=rv, pos=pos, k_rot=kr)
        outs.append((o, rk, rv, pos, kr))
    torch.cuda.synchronize()
    (o0, rk0, rv0, p0, _), (o1, rk1, rv1, p1, kr) = outs
    assert torch.equal(o0, o1) and torch.equal(rk0, rk1) and torch.equal(rv0, rv1)
    assert torch.equal(p0, p1)
    want = oracle.bf16_round(oracle.rope(x["k"]))
    got = host(kr)
    assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -7 + 1e-30)
    assert (got != want).mean() < 1e-3
    check_bf16(host(o1), oracle.gqa_prefill(x["q"], x["k"], x["v"], W, bf16=True), "k_rot path")
