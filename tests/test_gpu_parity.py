"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Tolerances (stated for this operation): float32 mode max |err| <= 1e-5
against the exact oracle; bf16 mode max |err| <= 2e-2 and relative RMS
<= 1e-2 against the bf16-contract oracle (rotated q, k rounded to bf16, the
rest exact).  Inputs are the seeded synthetic workloads of synth.py.
"""
import numpy as np
import pytest

import oracle
import sliding_window_attention_vx_amd as vx
from sliding_window_attention_vx_amd import synth

pytestmark = pytest.mark.gpu

F32_TOL = 1e-5
BF16_MAX = 2e-2
BF16_RRMS = 1e-2


def say(*a):
    print(*a, flush=True)


def dev(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.float().cpu().numpy().astype(np.float64)


def check_bf16(got, want, what=""):
    err = np.abs(got - want)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx = float(err.max())
    rrms = float(np.sqrt(np.mean(err ** 2)) / np.sqrt(np.mean(want ** 2)))
    say(f"{what}: max|err| {mx:.3e}  rel-rms {rrms:.3e}")
    assert mx <= BF16_MAX, f"{what}: max|err| {mx}"
    assert rrms <= BF16_RRMS, f"{what}: rel rms {rrms}"


def check_f32(got, want, what="", tol=F32_TOL):
    mx = float(np.max(np.abs(got - want)))
    say(f"{what}: max|err| {mx:.3e}")
    assert np.all(np.isfinite(got))
    assert mx <= tol, f"{what}: max|err| {mx}"


def run_prefill(x, W, dtype, out_dtype=None, valu=False, pos0=0, table=None, table_p0=0):
    q, k, v = (dev(x[n], dtype) for n in ("q", "k", "v"))
    o = vx.prefill(q, k, v, window=W, pos0=pos0, out_dtype=out_dtype, valu=valu, table=table,
                   table_p0=table_p0)
    return host(o)


# --------------------------------------------------------------------------
# RoPE pieces
# --------------------------------------------------------------------------

def test_rope_table_values():
    import torch
    say("rope_table p 0..20000")
    t = host(vx.rope_table(0, 20001))
    p = np.arange(20001, dtype=np.float64)[:, None]
    f = 1e6 ** (-2.0 * np.arange(32) / 64.0)
    want_c, want_s = np.cos(p * f), np.sin(p * f)
    # float32 rounding of the exact values: <= half an ulp (6e-8 near 1)
    assert np.max(np.abs(t[:, 0] - want_c)) <= 6.0e-8
    assert np.max(np.abs(t[:, 1] - want_s)) <= 6.0e-8
    assert torch.cuda.is_available()


@pytest.mark.parametrize("p0", [2_147_000_000, (1 << 52) - 4096])
def test_rope_table_values_large_positions(p0):
    """Large angles (positions near 2^31 and near the 2^52 the ABI allows): the
    float64 reduction by pi/2 must still give each cos/sin of the float64 angle
    within half a float32 ulp of its exact value.  At such positions the angle
    p*f moves by about f for one ulp of f, so the frequencies here are the
    correctly rounded ones (libm pow, as the library and the C oracle use;
    numpy's vectorised power is one ulp low for i = 11 and 25)."""
    import math
    say(f"rope_table p {p0} .. {p0 + 4095}")
    t = host(vx.rope_table(p0, 4096))
    p = (p0 + np.arange(4096, dtype=np.int64)).astype(np.float64)[:, None]
    f = np.array([math.pow(1e6, -2.0 * i / 64.0) for i in range(32)])
    want_c, want_s = np.cos(p * f), np.sin(p * f)
    assert np.max(np.abs(t[:, 0] - want_c)) <= 6.0e-8
    assert np.max(np.abs(t[:, 1] - want_s)) <= 6.0e-8


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rope_qk_matches_oracle(dtype):
    say(f"rope_qk {dtype}")
    x = synth.make_prefill(2, 300, 3, seed=11, dtype=dtype)
    q, k = dev(x["q"], dtype), dev(x["k"], dtype)
    vx.rope_qk(q, k, pos0=777)
    pos = 777 + np.arange(300)
    for got, src in ((host(q), x["q"]), (host(k), x["k"])):
        want = oracle.rope(src, pos=pos, bf16=(dtype == "bf16"))
        if dtype == "f32":
            check_f32(got, want, "rope f32", tol=2e-6)
        else:
            # float32 rotation rounded to bf16 vs float64 rotation rounded to bf16:
            # one bf16 ulp of the result, or the float32 rounding of the rotation
            # itself where x*c - y*s nearly cancels; and rarely different at all.
            diff = got != want
            bound = np.abs(want) * 2.0 ** -7 + 4 * 2.0 ** -24 * 8.0
            assert np.all(np.abs(got - want) <= bound)
            assert diff.mean() < 1e-3, diff.mean()


# --------------------------------------------------------------------------
# prefill
# --------------------------------------------------------------------------

def test_tiny_fp32_prefill():
    c = synth.CONFIGS["tiny"]
    x = synth.make_config("tiny")
    say("tiny fp32 prefill B1 T64 H4 W16")
    got = run_prefill(x, c.W, "f32")
    want = oracle.prefill(x["q"], x["k"], x["v"], c.W)
    check_f32(got, want, "tiny fp32")


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_layer_bf16_prefill(out_dtype):
    c = synth.CONFIGS["layer"]
    x = synth.make_config("layer")
    say(f"layer bf16 prefill B1 T1500 H32 W750 out {out_dtype}")
    got = run_prefill(x, c.W, "bf16", out_dtype=out_dtype)
    want = oracle.prefill(x["q"], x["k"], x["v"], c.W, bf16=True)
    check_bf16(got, want, f"layer out={out_dtype}")
    exact = oracle.prefill(x["q"], x["k"], x["v"], c.W)
    say(f"  vs exact oracle: max|err| {np.max(np.abs(got - exact)):.3e}")


def test_layer_valu_kernel_cross_check():
    c = synth.CONFIGS["layer"]
    x = synth.make_prefill(1, 1500, 4, seed=2, dtype="bf16", scale=0.5)
    say("layer-shaped VALU kernel (H4) vs contract oracle")
    got = run_prefill(x, c.W, "bf16", out_dtype="f32", valu=True)
    want = oracle.prefill(x["q"], x["k"], x["v"], c.W, bf16=True)
    check_f32(got, want, "valu bf16-in f32-out", tol=2e-5)


def test_fused_rope_equals_pre_rotated_input():
    # RoPE fused into the tile loads == vx_rope_qk then prefill(rope_applied): bit for bit.
    x = synth.make_prefill(2, 700, 4, seed=12, dtype="bf16", scale=0.5)
    say("fused vs pre-rotated B2 T700 H4")
    q, k, v = (dev(x[n], "bf16") for n in ("q", "k", "v"))
    fused = vx.prefill(q, k, v, window=750)
    q2, k2 = q.clone(), k.clone()
    vx.rope_qk(q2, k2)
    pre = vx.prefill(q2, k2, v, window=750, rope_applied=True)
    import torch
    torch.cuda.synchronize()
    assert torch.equal(fused.view(torch.int16), pre.view(torch.int16))


@pytest.mark.parametrize("T,W", [(1, 750), (2, 1), (31, 16), (33, 16), (64, 64), (65, 64),
                                 (127, 33), (129, 100), (200, 1), (300, 750), (749, 750),
                                 (750, 750), (751, 750), (1000, 97)])
def test_prefill_edge_shapes(T, W):
    say(f"edge T{T} W{W}")
    x = synth.make_prefill(2, T, 3, seed=100 + T + W, dtype="bf16", scale=0.5)
    got = run_prefill(x, W, "bf16")
    want = oracle.prefill(x["q"], x["k"], x["v"], W, bf16=True)
    check_bf16(got, want, f"mfma T{T} W{W}")
    x32 = synth.make_prefill(1, T, 2, seed=200 + T + W, dtype="f32")
    got32 = run_prefill(x32, W, "f32")
    check_f32(got32, oracle.prefill(x32["q"], x32["k"], x32["v"], W), f"fp32 T{T} W{W}")


@pytest.mark.parametrize("B,T,H,W", [(4, 64, 64, 64), (1, 129, 128, 16), (2, 300, 48, 97),
                                     (1, 1000, 40, 750), (1, 2000, 20, 1), (2, 1501, 16, 751)])
def test_prefill_many_heads_edge_shapes(B, T, H, W):
    """Grids of at least 256 query tiles (sixteen-query waves): ragged T, T below one
    tile, W = 1, W not a multiple of 32, W above T; sampled (b, h) against the oracle."""
    say(f"many heads B{B} T{T} H{H} W{W}")
    x = synth.make_prefill(B, T, H, seed=300 + T + W, dtype="bf16", scale=0.5)
    got = run_prefill(x, W, "bf16")
    rng = np.random.default_rng(T + W)
    picks = [(0, 0), (B - 1, H - 1)] + [tuple(int(v) for v in rng.integers([0, 0], [B, H]))
                                        for _ in range(2)]
    for b, h in picks:
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        want = oracle.prefill(x["q"][sl], x["k"][sl], x["v"][sl], W, bf16=True)
        check_bf16(got[sl], want, f"B{B} T{T} H{H} W{W} b{b} h{h}")


def test_prefill_at_the_head_and_batch_limits():
    """H = 65535 and B = 65535, the largest the boundary accepts, with short
    chunks: sampled (b, h) against the oracle."""
    for B, T, H, W, picks in ((1, 3, 65535, 2, [(0, 0), (0, 1), (0, 32767), (0, 65534)]),
                              (65535, 2, 1, 750, [(0, 0), (12345, 0), (65534, 0)])):
        say(f"limits: B{B} T{T} H{H} W{W}")
        x = synth.make_prefill(B, T, H, seed=400 + T, dtype="bf16", scale=0.5)
        got = run_prefill(x, W, "bf16")
        for b, h in picks:
            sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
            want = oracle.prefill(x["q"][sl], x["k"][sl], x["v"][sl], W, bf16=True)
            check_bf16(got[sl], want, f"B{B} T{T} H{H} b{b} h{h}")


def test_prefill_position_offset_and_table_window():
    say("prefill pos0 12345, table 12000..14000")
    x = synth.make_prefill(1, 400, 4, seed=13, dtype="bf16", scale=0.5)
    table = vx.rope_table(12000, 2000)
    got = run_prefill(x, 750, "bf16", pos0=12345, table=table, table_p0=12000)
    want = oracle.prefill(x["q"], x["k"], x["v"], 750, pos=12345, bf16=True)
    check_bf16(got, want, "pos0 12345")
    # positions 13700 .. 14099 run past the table: found on the device, loud
    assert np.all(np.isnan(run_prefill(x, 750, "bf16", pos0=13700, table=table, table_p0=12000)))


def _check_picks(x, got, picks, W, what):
    """The oracle on the chosen (b, h) pairs at once: each pair's head slice
    becomes one batch entry of a single oracle call (threads over entries)."""
    sel = lambda a: np.stack([a[b, :, h] for b, h in picks])[:, :, None]  # noqa: E731
    want = oracle.prefill(sel(x["q"]), sel(x["k"]), sel(x["v"]), W, bf16=True)
    for i, (b, h) in enumerate(picks):
        check_bf16(got[b, :, h], want[i, :, 0], f"{what} b{b} h{h}")


def test_stack_layers_sampled():
    """Stack workload (B4 T1500 H32 per layer): 16 (b, h) pairs of layer 0 and
    8 of layer 31 against the oracle, corners included."""
    c = synth.CONFIGS["stack"]
    rng = np.random.default_rng(3)
    for layer, n in ((0, 16), (c.layers - 1, 8)):
        say(f"stack layer {layer}: B4 T1500 H32, oracle on {n} sampled (b,h)")
        x = synth.make_config("stack", layer=layer)
        got = run_prefill(x, c.W, "bf16")
        picks = [(0, 0), (c.B - 1, c.H - 1)]
        while len(picks) < n:
            p_ = tuple(int(v) for v in rng.integers([0, 0], [c.B, c.H]))
            if p_ not in picks:
                picks.append(p_)
        _check_picks(x, got, picks, c.W, f"stack layer {layer}")


def test_long_sampled():
    """Long-form workload (B8 T6000 H32, 1 % of key rows x8): every (b, h)
    that holds one of the 16 largest stressed key rows, plus sampled pairs
    (32 in all), against the oracle."""
    c = synth.CONFIGS["long"]
    say("long: B8 T6000 H32 with stressed key rows, oracle on 32 (b,h)")
    x = synth.make_config("long")
    got = run_prefill(x, c.W, "bf16")
    assert np.all(np.isfinite(got))
    stressed = x["stressed_rows"]  # flat indices of (b, t, h) rows
    k_rows = x["k"].reshape(-1, x["k"].shape[-1])
    norms = np.linalg.norm(k_rows[stressed].astype(np.float64), axis=1)
    top = stressed[np.argsort(-norms)[:16]]
    picks = []
    for r in top:
        p_ = (int(r // (c.T * c.H)), int(r % c.H))
        if p_ not in picks:
            picks.append(p_)
    rng = np.random.default_rng(5)
    for p_ in [(0, 0), (c.B - 1, c.H - 1)]:
        if p_ not in picks:
            picks.append(p_)
    while len(picks) < 32:
        p_ = tuple(int(v) for v in rng.integers([0, 0], [c.B, c.H]))
        if p_ not in picks:
            picks.append(p_)
    _check_picks(x, got, picks, c.W, "long")


def test_prefill_deterministic():
    import torch
    x = synth.make_prefill(1, 1500, 8, seed=14, dtype="bf16", scale=0.5)
    q, k, v = (dev(x[n], "bf16") for n in ("q", "k", "v"))
    a = vx.prefill(q, k, v)
    b = vx.prefill(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# --------------------------------------------------------------------------
# streaming
# --------------------------------------------------------------------------

def _stream_state_dev(st, dtype):
    import torch
    return (dev(st["ring_k"], dtype), dev(st["ring_v"], dtype),
            torch.from_numpy(st["pos"].copy()).cuda())


@pytest.mark.parametrize("io,out", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32")])
def test_stream_step_full_workload(io, out):
    c = synth.CONFIGS["stream"]
    say(f"stream S64 n4 H32 W750 io {io} out {out}")
    st = synth.make_stream_state(c.S, c.H, c.W, seed=c.seed, pos_lo=c.pos_lo, pos_hi=c.pos_hi,
                                 dtype=io)
    fr = synth.make_stream_frames(c.S, c.n, c.H, seed=c.seed, step=0, dtype=io)
    rk, rv, pos = _stream_state_dev(st, io)
    qn, kn, vn = (dev(fr[n], io) for n in ("q", "k", "v"))
    o = host(vx.stream_step(qn, kn, vn, rk, rv, pos, window=c.W, out_dtype=out))
    want = oracle.stream_step(fr["q"], fr["k"], fr["v"], st["ring_k"], st["ring_v"], st["pos"],
                              c.W, bf16=(io == "bf16"))
    if io == "f32":
        check_f32(o, want, "stream f32")
    else:
        check_bf16(o, want, f"stream {io}->{out}")
    # append: rotated keys and values land in slot (pos+i) mod W, pos advances by n
    vx.ring_append(rk, rv, kn, vn, pos, window=c.W)
    rk_o = st["ring_k"].astype(np.float64)
    rv_o = st["ring_v"].astype(np.float64)
    pos_o = st["pos"].copy()
    oracle.ring_append(rk_o, rv_o, fr["k"], fr["v"], pos_o, c.W, bf16=(io == "bf16"))
    np.testing.assert_array_equal(host(pos.double()), pos_o)
    np.testing.assert_array_equal(host(rv), rv_o)
    gk = host(rk)
    if io == "f32":
        check_f32(gk, rk_o, "append f32", tol=2e-6)
    else:
        assert np.all(np.abs(gk - rk_o) <= np.abs(rk_o) * 2.0 ** -7 + 1e-30)
        assert (gk != rk_o).mean() < 1e-3


def test_stream_step_at_the_stream_limit():
    """S = 65535 streams, the largest the boundary accepts: sampled streams of
    the step and of the append against the oracle."""
    S, n, H, W = 65535, 1, 1, 4
    say(f"stream limits: S{S} n{n} H{H} W{W}")
    st = synth.make_stream_state(S, H, W, seed=71, pos_lo=W, pos_hi=20000)
    fr = synth.make_stream_frames(S, n, H, seed=71, step=0)
    rk, rv, pos = _stream_state_dev(st, "bf16")
    qn, kn, vn = (dev(fr[c], "bf16") for c in ("q", "k", "v"))
    o = host(vx.stream_step(qn, kn, vn, rk, rv, pos, window=W, out_dtype="f32"))
    vx.ring_append(rk, rv, kn, vn, pos, window=W)
    grk, grv, gpos = host(rk), host(rv), host(pos.double())
    for s in (0, 1, 40000, S - 1):
        sl = slice(s, s + 1)
        want = oracle.stream_step(fr["q"][sl], fr["k"][sl], fr["v"][sl], st["ring_k"][sl],
                                  st["ring_v"][sl], st["pos"][sl], W, bf16=True)
        check_bf16(o[sl], want, f"stream {s}")
        rk_o = st["ring_k"][sl].astype(np.float64)
        rv_o = st["ring_v"][sl].astype(np.float64)
        pos_o = st["pos"][sl].copy()
        oracle.ring_append(rk_o, rv_o, fr["k"][sl], fr["v"][sl], pos_o, W, bf16=True)
        np.testing.assert_array_equal(gpos[sl], pos_o)
        np.testing.assert_array_equal(grv[sl], rv_o)
        assert np.all(np.abs(grk[sl] - rk_o) <= np.abs(rk_o) * 2.0 ** -7 + 4 * 2.0 ** -24 * 8.0)


def feed_stream(q, k, v, W, chunks, S=1, ring_fill=np.nan, io="bf16"):
    """Run frames [S,T,H,D] through stream_step + ring_append from position 0."""
    import torch
    S_, T, H, D = q.shape
    rk = torch.full((S_, H, W, D), ring_fill, device="cuda").to(
        torch.bfloat16 if io == "bf16" else torch.float32)
    rv = rk.clone()
    pos = torch.zeros(S_, dtype=torch.int64, device="cuda")
    outs = []
    t, ci = 0, 0
    qd, kd, vd = (dev(a, io) for a in (q, k, v))
    while t < T:
        n = min(chunks[ci % len(chunks)], T - t)
        ci += 1
        sl = slice(t, t + n)
        qn, kn, vn = (a[:, sl].contiguous() for a in (qd, kd, vd))
        outs.append(vx.stream_step(qn, kn, vn, rk, rv, pos, window=W, out_dtype="f32"))
        vx.ring_append(rk, rv, kn, vn, pos, window=W)
        t += n
    return host(torch.cat(outs, dim=1)), host(pos.double())


@pytest.mark.parametrize("chunks,W,T", [([4], 750, 800), ([1], 40, 130), ([7, 3, 4], 64, 300),
                                        ([64], 64, 200)])
def test_streaming_equals_prefill_on_gpu(chunks, W, T):
    say(f"stream==prefill chunks {chunks} W{W} T{T}")
    x = synth.make_prefill(2, T, 2, seed=300 + T, dtype="bf16", scale=0.5)
    got, pos = feed_stream(x["q"], x["k"], x["v"], W, chunks)
    assert np.all(pos == T)
    want = oracle.prefill(x["q"], x["k"], x["v"], W, bf16=True)
    check_bf16(got, want, "streamed vs oracle prefill")
    pre = run_prefill(x, W, "bf16", out_dtype="f32")
    check_bf16(got, pre, "streamed vs GPU prefill")


def test_stream_f32_equals_oracle_prefill():
    x = synth.make_prefill(1, 150, 2, seed=301, dtype="f32")
    got, _ = feed_stream(x["q"], x["k"], x["v"], 50, [4], io="f32")
    check_f32(got, oracle.prefill(x["q"], x["k"], x["v"], 50), "stream f32 vs oracle prefill")


def test_stream_batch_invariance_and_determinism():
    import torch
    c = synth.CONFIGS["stream"]
    S, H = 16, 4
    st = synth.make_stream_state(S, H, c.W, seed=9, pos_lo=0 + c.W, pos_hi=20000)
    fr = synth.make_stream_frames(S, 4, H, seed=9, step=0)
    rk, rv, pos = _stream_state_dev(st, "bf16")
    qn, kn, vn = (dev(fr[n], "bf16") for n in ("q", "k", "v"))
    full = vx.stream_step(qn, kn, vn, rk, rv, pos)
    again = vx.stream_step(qn, kn, vn, rk, rv, pos)
    torch.cuda.synchronize()
    assert torch.equal(full, again)
    for s in (0, 5, 15):
        one = vx.stream_step(qn[s:s + 1].contiguous(), kn[s:s + 1].contiguous(),
                             vn[s:s + 1].contiguous(), rk[s:s + 1].contiguous(),
                             rv[s:s + 1].contiguous(), pos[s:s + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(one[0], full[s])


def test_stream_snapshot_resume_bitwise():
    import torch
    x = synth.make_prefill(1, 120, 2, seed=302, dtype="bf16", scale=0.5)
    W = 50
    # run 100 frames, snapshot, then continue twice from the snapshot
    qd, kd, vd = (dev(x[n], "bf16") for n in ("q", "k", "v"))
    rk = torch.zeros((1, 2, W, 64), dtype=torch.bfloat16, device="cuda")
    rv = rk.clone()
    pos = torch.zeros(1, dtype=torch.int64, device="cuda")
    for t in range(0, 100, 4):
        sl = slice(t, t + 4)
        vx.stream_step(qd[:, sl].contiguous(), kd[:, sl].contiguous(), vd[:, sl].contiguous(),
                       rk, rv, pos, window=W)
        vx.ring_append(rk, rv, kd[:, sl].contiguous(), vd[:, sl].contiguous(), pos, window=W)
    snap = (rk.clone(), rv.clone(), pos.clone())
    outs = []
    for _ in range(2):
        a, b, p = (t.clone() for t in snap)
        sl = slice(100, 104)
        outs.append(vx.stream_step(qd[:, sl].contiguous(), kd[:, sl].contiguous(),
                                   vd[:, sl].contiguous(), a, b, p, window=W))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("T,W", [(1, 750), (5, 750), (97, 33), (300, 64), (1500, 750)])
def test_prefill_uniform_scores_closed_form(T, W):
    # q = k = 0 makes every score 0, so o[t] is the plain mean of v[t-W+1..t]:
    # exact for small-integer values (bf16 weights 1, integer sums in fp32).
    import torch
    say(f"uniform scores T{T} W{W}")
    H = 2
    v = (np.arange(T)[None, :, None, None] % 7 * 3 + np.arange(64)[None, None, None, :] % 5
         + np.arange(H)[None, None, :, None]).astype(np.float32) * np.ones((1, T, H, 64), np.float32)
    z = torch.zeros((1, T, H, 64), dtype=torch.bfloat16, device="cuda")
    o = host(vx.prefill(z, z, dev(v, "bf16"), window=W, out_dtype="f32"))
    c = np.cumsum(np.concatenate([np.zeros((1, 1, H, 64)), v], axis=1), axis=1)
    t = np.arange(T)
    lo = np.maximum(0, t - W + 1)
    want = (c[:, t + 1] - c[:, lo]) / (t - lo + 1)[None, :, None, None]
    np.testing.assert_allclose(o, want, rtol=0, atol=1e-5)


@pytest.mark.parametrize("io,n", [("bf16", 1), ("bf16", 4), ("bf16", 16), ("f32", 4)])
def test_fused_step_append_equals_two_calls(io, n):
    # vx_swa_attn_stream_step_append == vx_swa_attn_stream_step + vx_kv_ring_append, bit for bit
    import torch
    S, H, W = 6, 4, 750
    say(f"fused step+append io {io} n {n}")
    st = synth.make_stream_state(S, H, W, seed=21, pos_lo=0 + W, pos_hi=20000, dtype=io)
    fr = synth.make_stream_frames(S, n, H, seed=21, step=0, dtype=io)
    rk, rv, pos = _stream_state_dev(st, io)
    qn, kn, vn = (dev(fr[x], io) for x in ("q", "k", "v"))
    rk2, rv2, pos_in = rk.clone(), rv.clone(), pos.clone()
    o1 = vx.stream_step(qn, kn, vn, rk, rv, pos, window=W)
    vx.ring_append(rk, rv, kn, vn, pos, window=W)
    pos_out = torch.full_like(pos_in, -1)
    o2 = vx.stream_step_append(qn, kn, vn, rk2, rv2, pos_in, pos_out, window=W)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(rk, rk2) and torch.equal(rv, rv2)
    assert torch.equal(pos, pos_out)
    assert torch.equal(pos_in, torch.from_numpy(st["pos"]).cuda())  # pos_in untouched


def test_fused_stream_equals_prefill():
    import torch
    W, T = 64, 200
    x = synth.make_prefill(3, T, 2, seed=303, dtype="bf16", scale=0.5)
    qd, kd, vd = (dev(x[n], "bf16") for n in ("q", "k", "v"))
    rk = torch.full((3, 2, W, 64), float("nan"), device="cuda").bfloat16()
    rv = rk.clone()
    pa = torch.zeros(3, dtype=torch.int64, device="cuda")
    pb = torch.empty_like(pa)
    outs = []
    for t in range(0, T, 4):
        sl = slice(t, t + 4)
        outs.append(vx.stream_step_append(qd[:, sl].contiguous(), kd[:, sl].contiguous(),
                                          vd[:, sl].contiguous(), rk, rv, pa, pb, window=W,
                                          out_dtype="f32"))
        pa, pb = pb, pa
    got = host(torch.cat(outs, dim=1))
    assert np.all(host(pa.double()) == T)
    check_bf16(got, oracle.prefill(x["q"], x["k"], x["v"], W, bf16=True), "fused stream vs oracle")
