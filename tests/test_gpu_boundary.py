"""GPU tests of the boundary's semantics against the float64 oracle.

Per-batch positions (pos0 as a device array), the three sources of cos/sin
(a caller table, a table built in the workspace, cos/sin computed in the
kernel), and the loud failures: invalid positions and over-long streams give NaN outputs and leave
the streaming state alone instead of a silent partial result.
Tolerances are those of test_gpu_parity (bf16 contract: max |err| <= 2e-2,
relative RMS <= 1e-2).
"""
import numpy as np
import pytest

import oracle
import sliding_window_attention_vx_amd as vx
from sliding_window_attention_vx_amd import synth

pytestmark = pytest.mark.gpu

BF16_MAX = 2e-2
BF16_RRMS = 1e-2


def say(*a):
    print(*a, flush=True)


def dev(x, dtype="bf16"):
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


def positions(pos0, T):
    return np.asarray(pos0, dtype=np.int64)[:, None] + np.arange(T, dtype=np.int64)[None, :]


def pos_tensor(pos0):
    import torch
    return torch.tensor(pos0, dtype=torch.int64, device="cuda")


@pytest.mark.parametrize("source", ["table", "workspace", "kernel"])
def test_per_batch_positions(source):
    """B = 4 chunks at positions {0, 777, 12345, 19999}: each entry against
    oracle.prefill at its own positions, for each source of cos/sin."""
    pos0 = [0, 777, 12345, 19999]
    B, T, H, W = 4, 300, 8, 750
    say(f"per-batch pos0 {pos0}, B{B} T{T} H{H}, cos/sin from {source}")
    x = synth.make_prefill(B, T, H, seed=71, dtype="bf16", scale=0.5)
    q, k, v = (dev(x[n]) for n in ("q", "k", "v"))
    p0 = pos_tensor(pos0)
    if source == "table":
        table = vx.rope_table(0, 20400)
        o = vx.prefill(q, k, v, window=W, pos0=p0, table=table, table_p0=0)
    elif source == "workspace":
        ws = vx.prefill_workspace(B, T, H, W)
        o = vx.prefill(q, k, v, window=W, pos0=p0, workspace=ws)
    else:
        o = vx.prefill(q, k, v, window=W, pos0=p0)
    want = oracle.prefill(x["q"], x["k"], x["v"], W, pos=positions(pos0, T), bf16=True)
    got = host(o)
    for b in range(B):
        check_bf16(got[b], want[b], f"{source} entry {b} at {pos0[b]}")


def test_cos_sin_sources_agree_bitwise():
    """The same float64 angle gives the same cos/sin whatever its source, so
    the three paths produce identical bits on a grid where they run the same
    kernel shape (one block per wave, no split)."""
    import torch
    B, T, H, W = 2, 260, 4, 64
    x = synth.make_prefill(B, T, H, seed=72, dtype="bf16", scale=0.5)
    q, k, v = (dev(x[n]) for n in ("q", "k", "v"))
    p0 = pos_tensor([5, 70000])
    table = vx.rope_table(0, 70300)
    a = vx.prefill(q, k, v, window=W, pos0=p0, table=table)
    b = vx.prefill(q, k, v, window=W, pos0=p0, workspace=vx.prefill_workspace(B, T, H, W))
    c = vx.prefill(q, k, v, window=W, pos0=p0)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


def test_invalid_positions_are_loud():
    """An entry whose positions fall outside the given table, or whose pos0
    is negative, gets NaN in every output; the other entries are exact."""
    B, T, H, W = 3, 200, 4, 750
    x = synth.make_prefill(B, T, H, seed=73, dtype="bf16", scale=0.5)
    q, k, v = (dev(x[n]) for n in ("q", "k", "v"))
    table = vx.rope_table(12000, 2000)  # positions 12000 .. 13999
    pos0 = [12345, 13900, -5]  # entry 1 runs past the table, entry 2 is negative
    o = host(vx.prefill(q, k, v, window=W, pos0=pos_tensor(pos0), table=table, table_p0=12000))
    want = oracle.prefill(x["q"][:1], x["k"][:1], x["v"][:1], W, pos=12345, bf16=True)
    check_bf16(o[0], want[0], "valid entry")
    assert np.all(np.isnan(o[1])) and np.all(np.isnan(o[2]))
    # the same table without pos0 (positions 0 .. T-1) is refused on the host
    with pytest.raises(vx.VxError):
        vx.prefill(q, k, v, window=W, table=table, table_p0=12000)


def test_rope_qk_per_batch_positions_and_negative_entry():
    import torch
    B, T, H = 3, 50, 4
    x = synth.make_prefill(B, T, H, seed=74, dtype="bf16", scale=1.0)
    q, k = dev(x["q"]), dev(x["k"])
    pos0 = [0, 31337, -1]
    vx.rope_qk(q, k, pos0=pos_tensor(pos0))
    torch.cuda.synchronize()
    got = host(q)
    for b in range(2):
        want = oracle.rope(x["q"][b:b + 1], pos=positions(pos0[b:b + 1], T), bf16=True)
        err = np.abs(got[b:b + 1] - want)
        # float32 rotation against the float64 oracle: at most one bf16 step
        assert float(err.max()) <= 2.0 ** -7 * max(1.0, float(np.abs(want).max()))
    assert np.all(np.isnan(got[2])) and np.all(np.isnan(host(k)[2]))


def test_varlen_stream_longer_than_max_T_is_loud():
    """A stream longer than max_T: every output row of that stream is NaN, its
    ring and pos are untouched; the other streams are seeded and exact."""
    import torch
    lengths = [100, 160, 40]
    S, H, W, max_T = len(lengths), 4, 64, 128
    x = synth.make_first_chunks(S, H, lengths, seed=76)
    q, k, v = (dev(x[n]) for n in ("q", "k", "v"))
    cu = torch.from_numpy(x["cu"].astype(np.int32)).cuda()
    rk = torch.full((S, H, W, 64), 3.0, dtype=torch.bfloat16, device="cuda")
    rv = rk.clone()
    pos = torch.full((S,), -7, dtype=torch.int64, device="cuda")
    o = vx.prefill_varlen(q, k, v, cu, max_T, window=W, ring_k=rk, ring_v=rv, pos=pos)
    got = host(o)
    c0, c1 = int(x["cu"][1]), int(x["cu"][2])
    assert np.all(np.isnan(got[c0:c1])), "the over-long stream is not NaN"
    assert torch.all(rk[1] == 3.0) and torch.all(rv[1] == 3.0), "its ring was written"
    p = pos.cpu().numpy()
    assert p[1] == -7 and p[0] == 100 and p[2] == 40
    for s in (0, 2):
        a, b = int(x["cu"][s]), int(x["cu"][s + 1])
        want = oracle.prefill(x["q"][None, a:b], x["k"][None, a:b], x["v"][None, a:b], W,
                              bf16=True)[0]
        check_bf16(got[a:b], want, f"stream {s}")


@pytest.mark.parametrize("fused", [False, True])
def test_negative_stream_position_is_loud(fused):
    """A stream whose position is negative gets NaN outputs, no ring write and
    an unchanged position; the other streams step exactly as the oracle."""
    import torch
    S, n, H, W = 3, 4, 4, 64
    st = synth.make_stream_state(S, H, W, seed=77, pos_lo=64, pos_hi=500)
    fr = synth.make_stream_frames(S, n, H, seed=77, step=0)
    p_host = st["pos"].copy()
    p_host[1] = -3
    rk, rv = dev(st["ring_k"]), dev(st["ring_v"])
    rk0, rv0 = rk.clone(), rv.clone()
    pos = torch.from_numpy(p_host).cuda()
    q, k, v = (dev(fr[c]) for c in ("q", "k", "v"))
    if fused:
        pos_out = torch.empty_like(pos)
        o = vx.stream_step_append(q, k, v, rk, rv, pos, pos_out, window=W)
    else:
        o = vx.stream_step(q, k, v, rk, rv, pos, window=W)
        vx.ring_append(rk, rv, k, v, pos, window=W)
        pos_out = pos
    got = host(o)
    assert np.all(np.isnan(got[1]))
    assert torch.equal(rk[1], rk0[1]) and torch.equal(rv[1], rv0[1])
    po = pos_out.cpu().numpy()
    assert po[1] == -3
    for s in (0, 2):
        assert po[s] == p_host[s] + n
        want = oracle.stream_step(fr["q"][s:s + 1], fr["k"][s:s + 1], fr["v"][s:s + 1],
                                  st["ring_k"][s:s + 1], st["ring_v"][s:s + 1],
                                  p_host[s:s + 1], W, bf16=True)
        check_bf16(got[s:s + 1], want, f"stream {s}")
