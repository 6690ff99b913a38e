"""GPU parity of the streaming encoder step (vx_rmsnorm, vx_enc_stem_step,
vx_enc_layer_step, vx_enc_step) against the float64 oracle in bf16-contract
mode, which rounds to bf16 every tensor the GPU stores in bf16 between its
launches (conv1 output, normalised states, q', k', v, o, SwiGLU hidden
state) and keeps the float32 residual stream unrounded.

Tolerances (float32 outputs; err = got - want, rms = RMS of want):
  - RMSNorm output (bf16): within one bf16 rounding of the float64 value.
  - stem output, one layer: max|err| <= 2e-2 * rms and rel RMS <= 1e-2, the
    attention's bar scaled to the residual's size.  Both sides round at the
    same points; they differ where the GPU's float32 sum lands on the other
    side of a bf16 rounding boundary, a one-ulp (2^-8 relative) change of a
    few elements that the next product spreads at far below 1e-2.
    (The attention kernel also feeds its probabilities to the matrix cores
    in bf16, one more rounding of o's order; that dominates a layer's
    deviation, about 1e-3 relative.)
  - several layers: with random weights a deviation in one layer's output is
    amplified by every later layer (the oracle's own bf16 contract drifts
    from exact float64 by 2.3e-2 relative RMS over 32 layers, from 1e-3 for
    one), so a fixed end-to-end bar would test the weights, not the code.
    The step is instead checked three ways:
      1. vx_enc_step equals the stem and layer calls made one by one, bit
         for bit (the same deterministic kernels in the same order);
      2. teacher forcing: each GPU layer against the oracle layer given the
         same input (the GPU's residual before it) and its own oracle rings,
         to the one-layer bar above;
      3. free running, as a coarse net for a skipped, repeated or reordered
         layer: the GPU's distance from the contract oracle stays within
         twice the contract's distance from exact float64 (max and RMS).
    The measured figures are printed.
"""
import numpy as np
import pytest

import oracle
import sliding_window_attention_vx_amd as vx
from sliding_window_attention_vx_amd import synth
from tests.test_gpu_parity import dev, host, say

pytestmark = pytest.mark.gpu


def _close_bf16(got, want, what):
    scale = np.sqrt(np.mean(want ** 2))
    bad = np.abs(got - want) > np.abs(want) * 2.0 ** -7 + 1e-4 * scale
    say(f"{what}: {int(bad.sum())} of {bad.size} beyond one bf16 rounding")
    assert not bad.any()


def _check_resid(got, want, what, exact=None):
    """One piece: the fixed bar.  Free-running layers (exact given): twice the
    contract's own distance from exact arithmetic."""
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = got - want
    rms = float(np.sqrt(np.mean(want ** 2)))
    mx = float(np.max(np.abs(err)))
    rrms = float(np.sqrt(np.mean(err ** 2))) / rms
    say(f"{what}: max|err| {mx:.3e} ({mx / rms:.2e} rms)  rel-rms {rrms:.3e}  (rms {rms:.3f})")
    if exact is None:
        max_tol, rrms_tol = 2e-2 * rms, 1e-2
    else:
        d = want - exact
        max_tol = 2 * float(np.max(np.abs(d)))
        rrms_tol = 2 * float(np.sqrt(np.mean(d ** 2))) / rms
        say(f"    contract vs exact: max {max_tol / 2:.3e}  rel-rms {rrms_tol / 2:.3e}")
    assert mx <= max_tol, f"{what}: max|err| {mx} > {max_tol}"
    assert rrms <= rrms_tol, f"{what}: rel rms {rrms} > {rrms_tol}"


# ---------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,dim", [(1, 8), (5, 1280), (300, 1280), (7, 5120), (3, 72), (2, 640),
                                   (9, 2048), (4, 4096)])
def test_rmsnorm_matches_oracle(M, dim):
    import torch
    say(f"rmsnorm M{M} dim {dim}")
    rng = np.random.default_rng(M * 7 + dim)
    x = (rng.standard_normal((M, dim)) * rng.uniform(0.1, 30.0, size=(M, 1))).astype(np.float32)
    g = synth.round_to_bf16((1 + 0.1 * rng.standard_normal(dim)).astype(np.float32))
    y = vx.rmsnorm(torch.from_numpy(x).cuda(), dev(g, "bf16"), eps=1e-5)
    _close_bf16(host(y), oracle.rmsnorm(x, g, 1e-5), "rmsnorm")


def test_rmsnorm_zero_row_gives_zero():
    import torch
    x = torch.zeros((2, 1280), dtype=torch.float32, device="cuda")
    g = torch.ones(1280, dtype=torch.bfloat16, device="cuda")
    assert host(vx.rmsnorm(x, g, eps=1e-5)).max() == 0.0


# ---------------------------------------------------------------------------
# stem
# ---------------------------------------------------------------------------

def _stem_run(S, n, n_mels, dm, steps, seed):
    import torch
    sw = synth.make_enc_stem_weights(dm, n_mels, seed=seed)
    dsw = {k: dev(v, "bf16") for k, v in sw.items()}
    F = 2 * n + 2
    mel_buf = torch.zeros((S, F, n_mels), dtype=torch.bfloat16, device="cuda")
    c1_buf = torch.zeros((S, F, dm), dtype=torch.bfloat16, device="cuda")
    mc, cc = np.zeros((S, 2, n_mels)), np.zeros((S, 2, dm))
    for step in range(steps):
        mel = synth.make_mel(S, 2 * n, n_mels, seed=seed, step=step)
        mel_buf[:, 2:] = dev(mel, "bf16")
        say(f"stem S{S} n{n} n_mels {n_mels} d_model {dm} step {step}")
        x = host(vx.enc_stem_step(mel_buf, c1_buf, dsw))
        want = oracle.enc_stem_step(mel, mc, cc, sw["w1"], sw["b1"], sw["w2"], sw["b2"], bf16=True)
        _check_resid(x, want, f"  stem out step {step}")
        # the carried state: mel slots 0-1 are the step's last two frames exactly,
        # c1 slots 0-1 the first convolution's last two outputs
        np.testing.assert_array_equal(host(mel_buf[:, :2]), mel[:, -2:])
        _close_bf16(host(c1_buf[:, :2]), cc, "  conv1 cache")


@pytest.mark.parametrize("S,n,n_mels,dm,steps", [(3, 4, 128, 256, 3), (2, 1, 256, 128, 4),
                                                 (5, 3, 128, 384, 2)])
def test_stem_consecutive_steps_match_oracle(S, n, n_mels, dm, steps):
    _stem_run(S, n, n_mels, dm, steps, seed=[31, S, n])


def test_stem_full_workload():
    c = synth.ENC_STEP
    _stem_run(c["S"], c["n"], c["n_mels"], c["d_model"], 2, seed=c["seed"])


# ---------------------------------------------------------------------------
# layers
# ---------------------------------------------------------------------------

def _dev_layer(w):
    return {k: dev(v, "bf16") for k, v in w.items()}


@pytest.mark.parametrize("S,n,H,dm,ffn,W,steps,pos_lo", [
    (3, 4, 2, 256, 512, 16, 6, 16),     # full rings, several wraps
    (2, 4, 2, 128, 256, 16, 5, 0),      # stream start: empty history
    (4, 3, 4, 256, 384, 10, 4, 10),     # ragged n, W not a multiple of n
])
def test_layer_consecutive_steps_match_oracle(S, n, H, dm, ffn, W, steps, pos_lo):
    import torch
    seed = [41, S, dm]
    w = synth.make_enc_layer_weights(dm, H, ffn, seed=seed, layer=0)
    dw = _dev_layer(w)
    st = synth.make_stream_state(S, H, W, seed=[seed, 1], pos_lo=pos_lo, pos_hi=pos_lo + 3 * W,
                                 full=pos_lo >= W)
    rk_h, rv_h = st["ring_k"].astype(np.float64), st["ring_v"].astype(np.float64)
    pos = st["pos"].copy()
    rk, rv = dev(st["ring_k"], "bf16"), dev(st["ring_v"], "bf16")
    pin = torch.from_numpy(pos.copy()).cuda()
    pout = torch.empty_like(pin)
    work = vx.enc_work(S, n, H, dm, ffn)
    for step in range(steps):
        x = synth.make_enc_block_input(S, n, dm, seed=seed, step=step).astype(np.float32) * 2
        xg = torch.from_numpy(x).cuda()
        say(f"layer S{S} n{n} H{H} d_model {dm} ffn {ffn} W{W} step {step} pos {pos.tolist()}")
        vx.enc_layer_step(xg, dw, rk, rv, pin, pout, window=W, H=H, work=work)
        want = oracle.enc_layer_step(x, w, rk_h, rv_h, pos, W, H, bf16=True)
        _check_resid(host(xg), want, f"  layer out step {step}")
        assert host(pout).tolist() == pos.tolist()
        pin, pout = pout, pin
    _close_bf16(host(rk), rk_h, "  ring_k after the steps")
    _close_bf16(host(rv), rv_h, "  ring_v after the steps")


def test_layer_full_workload_sampled_streams():
    import torch
    c = synth.ENC_STEP
    S, n, H, dm, ffn, W = c["S"], c["n"], c["H"], c["d_model"], c["ffn"], c["W"]
    w = synth.make_enc_layer_weights(dm, H, ffn, seed=c["seed"], layer=0)
    st = synth.make_stream_state(S, H, W, seed=[c["seed"], 1], pos_lo=c["pos_lo"],
                                 pos_hi=c["pos_hi"])
    x = synth.make_enc_block_input(S, n, dm, seed=c["seed"], step=0).astype(np.float32) * 2
    pin = torch.from_numpy(st["pos"].copy()).cuda()
    pout = torch.empty_like(pin)
    rk, rv = dev(st["ring_k"], "bf16"), dev(st["ring_v"], "bf16")
    xg = torch.from_numpy(x).cuda()
    say(f"layer full workload S{S} n{n} H{H} d_model {dm} ffn {ffn} W{W}")
    vx.enc_layer_step(xg, _dev_layer(w), rk, rv, pin, pout, window=W, H=H)
    got = host(xg)
    sel = [0, 1, 17, 38, 63]
    rk_h, rv_h = st["ring_k"][sel].astype(np.float64), st["ring_v"][sel].astype(np.float64)
    pos = st["pos"][sel].copy()
    want = oracle.enc_layer_step(x[sel], w, rk_h, rv_h, pos, W, H, bf16=True)
    _check_resid(got[sel], want, "  layer out (5 streams)")
    _close_bf16(host(rk[sel]), rk_h, "  ring_k (5 streams)")
    assert host(pout).tolist() == (st["pos"] + n).tolist()


# ---------------------------------------------------------------------------
# whole step: stem + L layers
# ---------------------------------------------------------------------------

class _Model:
    """Weights of a synthetic encoder (host float32 arrays and device copies)."""

    def __init__(self, L, H, dm, ffn, n_mels, seed):
        self.stem = synth.make_enc_stem_weights(dm, n_mels, seed=seed)
        self.layers = [synth.make_enc_layer_weights(dm, H, ffn, seed=seed, layer=l)
                       for l in range(L)]
        self.dstem = {k: dev(v, "bf16") for k, v in self.stem.items()}
        self.dlayers = [_dev_layer(w) for w in self.layers]


def _oracle_step(m, mel, state, W, H, sel=None, bf16=True):
    """One whole step on the oracle for the streams `sel` (state holds their
    caches, float64 rings per layer and positions; advanced in place)."""
    x = oracle.enc_stem_step(mel if sel is None else mel[sel], state["mc"], state["cc"],
                             m.stem["w1"], m.stem["b1"], m.stem["w2"], m.stem["b2"], bf16=bf16)
    for l, w in enumerate(m.layers):
        p = state["pos"].copy()
        x = oracle.enc_layer_step(x, w, state["rk"][l], state["rv"][l], p, W, H, bf16=bf16)
    state["pos"] += mel.shape[1] // 2
    return x


def _copy_state(st):
    return dict(mc=st["mc"].copy(), cc=st["cc"].copy(), rk=[a.copy() for a in st["rk"]],
                rv=[a.copy() for a in st["rv"]], pos=st["pos"].copy())


class _GpuState:
    """Device state of S streams: frame buffers, [L, ...] rings, positions."""

    def __init__(self, S, n, n_mels, dm, rk, rv, pos):
        import torch
        F = 2 * n + 2
        self.mel = torch.zeros((S, F, n_mels), dtype=torch.bfloat16, device="cuda")
        self.c1 = torch.zeros((S, F, dm), dtype=torch.bfloat16, device="cuda")
        self.rk, self.rv = rk, rv
        self.pin = pos
        self.pout = torch.empty_like(pos)

    def clone(self):
        c = _GpuState.__new__(_GpuState)
        c.mel, c.c1, c.rk, c.rv = self.mel.clone(), self.c1.clone(), self.rk.clone(), self.rv.clone()
        c.pin, c.pout = self.pin.clone(), self.pout.clone()
        return c

    def swap(self):
        self.pin, self.pout = self.pout, self.pin


def _whole_and_chained(m, A, B, mel, W, H, work):
    """One step on A with vx_enc_step and on B with the calls one by one.
    Returns (x of A, [GPU residual before each layer and after the last] of B)."""
    import torch
    A.mel[:, 2:] = dev(mel, "bf16")
    B.mel[:, 2:] = dev(mel, "bf16")
    xa = host(vx.enc_step(A.mel, A.c1, m.dstem, m.dlayers, A.rk, A.rv, A.pin, A.pout, window=W,
                          H=H, work=work))
    x = vx.enc_stem_step(B.mel, B.c1, m.dstem)
    xs = [host(x)]
    for l, w in enumerate(m.dlayers):
        vx.enc_layer_step(x, w, B.rk[l], B.rv[l], B.pin, B.pout, window=W, H=H, work=work)
        xs.append(host(x))
    assert np.array_equal(xa, xs[-1]), "whole step differs from the calls one by one"
    assert torch.equal(A.rk, B.rk) and torch.equal(A.rv, B.rv) and torch.equal(A.c1, B.c1)
    assert torch.equal(A.pout, B.pout)
    A.swap()
    B.swap()
    return xa, xs


def _teacher_forced(m, xs, tf, W, H, sel, what):
    """Each layer on the oracle from the GPU's input to it (tf: per-layer float64
    rings of the streams sel and positions, advanced in place)."""
    for l, w in enumerate(m.layers):
        p = tf["pos"].copy()
        want = oracle.enc_layer_step(xs[l][sel], w, tf["rk"][l], tf["rv"][l], p, W, H, bf16=True)
        _check_resid(xs[l + 1][sel], want, f"  {what} layer {l} (teacher forced)")
    tf["pos"] += xs[0].shape[1]


def test_enc_step_from_stream_start_matches_oracle():
    import torch
    L, S, n, H, dm, ffn, n_mels, W = 3, 2, 4, 2, 256, 512, 128, 12
    m = _Model(L, H, dm, ffn, n_mels, seed=[51])
    rk = torch.zeros((L, S, H, W, 64), dtype=torch.bfloat16, device="cuda")
    A = _GpuState(S, n, n_mels, dm, rk, torch.zeros_like(rk),
                  torch.zeros(S, dtype=torch.int64, device="cuda"))
    B = A.clone()
    state = dict(mc=np.zeros((S, 2, n_mels)), cc=np.zeros((S, 2, dm)),
                 rk=[np.zeros((S, H, W, 64)) for _ in range(L)],
                 rv=[np.zeros((S, H, W, 64)) for _ in range(L)], pos=np.zeros(S, dtype=np.int64))
    exact_state = _copy_state(state)
    tf = _copy_state(state)
    work = vx.enc_work(S, n, H, dm, ffn)
    sel = list(range(S))
    for step in range(6):
        mel = synth.make_mel(S, 2 * n, n_mels, seed=[51], step=step)
        say(f"enc step L{L} S{S} n{n} H{H} d_model {dm} W{W} step {step}")
        x, xs = _whole_and_chained(m, A, B, mel, W, H, work)
        _teacher_forced(m, xs, tf, W, H, sel, f"step {step}")
        want = _oracle_step(m, mel, state, W, H)
        exact = _oracle_step(m, mel, exact_state, W, H, bf16=False)
        _check_resid(x, want, f"  step {step} out (free running)", exact=exact)
        assert host(A.pin).tolist() == state["pos"].tolist()


def test_enc_step_full_workload_sampled_streams():
    """The bench configuration (64 streams x 4 frames, 32 layers, W 750,
    d_model 1280, FFN 5120) for two steps; every layer's rings start as the
    same seeded full-ring draw; the oracle runs streams 0, 29 and 63."""
    import torch
    c = synth.ENC_STEP
    S, n, H, dm, ffn, n_mels, L, W = (c[k] for k in ("S", "n", "H", "d_model", "ffn", "n_mels",
                                                      "L", "W"))
    m = _Model(L, H, dm, ffn, n_mels, seed=c["seed"])
    st = synth.make_stream_state(S, H, W, seed=[c["seed"], 1], pos_lo=c["pos_lo"],
                                 pos_hi=c["pos_hi"])
    rk = dev(st["ring_k"], "bf16").unsqueeze(0).repeat(L, 1, 1, 1, 1)
    rv = dev(st["ring_v"], "bf16").unsqueeze(0).repeat(L, 1, 1, 1, 1)
    A = _GpuState(S, n, n_mels, dm, rk, rv, torch.from_numpy(st["pos"].copy()).cuda())
    B = A.clone()
    sel = [0, 29, 63]
    state = dict(mc=np.zeros((3, 2, n_mels)), cc=np.zeros((3, 2, dm)),
                 rk=[st["ring_k"][sel].astype(np.float64) for _ in range(L)],
                 rv=[st["ring_v"][sel].astype(np.float64) for _ in range(L)],
                 pos=st["pos"][sel].copy())
    exact_state = _copy_state(state)
    tf = _copy_state(state)
    work = vx.enc_work(S, n, H, dm, ffn)
    for step in range(2):
        mel = synth.make_mel(S, 2 * n, n_mels, seed=c["seed"], step=step)
        say(f"enc step full workload L{L} S{S} n{n} H{H} d_model {dm} ffn {ffn} W{W} step {step}")
        x, xs = _whole_and_chained(m, A, B, mel, W, H, work)
        _teacher_forced(m, xs, tf, W, H, sel, f"step {step}")
        want = _oracle_step(m, mel, state, W, H, sel=sel)
        exact = _oracle_step(m, mel, exact_state, W, H, sel=sel, bf16=False)
        _check_resid(x[sel], want, f"  step {step} out (3 streams, free running)", exact=exact)
        assert host(A.pin).tolist() == (st["pos"] + n * (step + 1)).tolist()
    # the last layer's rings hold its new keys (teacher-forced oracle rings)
    _close_bf16(host(A.rk[L - 1][sel]), tf["rk"][L - 1], "  last layer ring_k (3 streams)")
