"""GPU parity of the batched first-chunk prefill (vx_swa_attn_prefill_varlen):
streams of different lengths packed along the frame axis, optional ring
seeding, and continuation by the streaming step.

Tolerances as in test_gpu_parity: bf16 max |err| <= 2e-2 and relative RMS
<= 1e-2 against the bf16-contract oracle.  Seeded values are checked like
the ring append: values bit-exact, rotated keys within one bf16 rounding of
the float64 oracle's (a float32 rotation can round the other way at a tie).
"""
import numpy as np
import pytest

import oracle
import sliding_window_attention_vx_amd as vx
from sliding_window_attention_vx_amd import synth
from tests.test_gpu_parity import check_bf16, dev, host, say

pytestmark = pytest.mark.gpu


def _run(x, W, max_T, rings=None, fill=0.0, out_dtype="f32", rope_applied=False):
    import torch
    q, k, v = (dev(x[n], "bf16") for n in ("q", "k", "v"))
    cu = torch.from_numpy(x["cu"]).cuda()
    S, H = len(x["cu"]) - 1, q.shape[1]
    rk = rv = pos = None
    if rings:
        rk = torch.full((S, H, W, 64), fill, device="cuda").to(torch.bfloat16)
        rv = rk.clone()
        pos = torch.full((S,), -5, dtype=torch.int64, device="cuda")
    o = vx.prefill_varlen(q, k, v, cu, max_T, window=W, ring_k=rk, ring_v=rv, pos=pos,
                          out_dtype=out_dtype, rope_applied=rope_applied)
    return o, rk, rv, pos


def _check_rings(x, W, rk, rv, pos, fill):
    S, H = len(x["cu"]) - 1, x["q"].shape[1]
    rk_o = np.full((S, H, W, 64), fill, dtype=np.float64)
    rv_o = rk_o.copy()
    pos_o = np.zeros(S, dtype=np.int64)
    oracle.prefill_varlen(x["q"], x["k"], x["v"], x["cu"], W, ring_k=rk_o, ring_v=rv_o,
                          pos=pos_o, bf16=True)
    np.testing.assert_array_equal(host(pos.double()), pos_o)
    np.testing.assert_array_equal(host(rv), rv_o)
    gk = host(rk)
    # float32 rotation rounded to bf16 against float64 rotation rounded to
    # bf16: one bf16 ulp of the result, or the float32 rounding of the rotation
    # itself where x*c - y*s nearly cancels (the bound of the rope_qk test)
    assert np.all(np.abs(gk - rk_o) <= np.abs(rk_o) * 2.0 ** -7 + 4 * 2.0 ** -24 * 8.0)
    assert (gk != rk_o).mean() < 1e-3


@pytest.mark.parametrize("W", [750, 64])
def test_varlen_matches_oracle_and_seeds_rings(W):
    lengths = [156, 100, 1, 0, 64, 65, 130, 127, 33, 156]
    S, H = len(lengths), 4
    say(f"varlen W{W} lengths {lengths}")
    x = synth.make_first_chunks(S, H, lengths, seed=[61, W])
    o, rk, rv, pos = _run(x, W, 156, rings=True, fill=3.0)
    want = oracle.prefill_varlen(x["q"], x["k"], x["v"], x["cu"], W, bf16=True)
    check_bf16(host(o), want, f"varlen W{W}")
    # slots a stream did not fill keep their contents
    _check_rings(x, W, rk, rv, pos, fill=3.0)


@pytest.mark.parametrize("W", [750, 64])
def test_varlen_many_heads_match_oracle_and_seed_rings(W):
    """Chunks of up to 160 frames over 256 (stream, head) pairs (four-wave
    workgroups, two query tiles for the longer chunks): outputs against the
    oracle, the seeded rings and pos, and equality with the fixed-length
    prefill."""
    import torch
    lengths = [156, 129, 1, 0, 160, 140, 64, 130]
    S, H = len(lengths), 32
    say(f"varlen many heads W{W} lengths {lengths} H{H}")
    x = synth.make_first_chunks(S, H, lengths, seed=[64, W])
    o, rk, rv, pos = _run(x, W, max(lengths), rings=True, fill=3.0)
    got = host(o)
    cu = x["cu"]
    for s in (0, 1, 2, 4, 7):
        a, b = int(cu[s]), int(cu[s + 1])
        want = oracle.prefill(x["q"][None, a:b], x["k"][None, a:b], x["v"][None, a:b], W,
                              bf16=True)[0]
        check_bf16(got[a:b], want, f"many-heads stream {s} (T {b - a})")
    _check_rings(x, W, rk, rv, pos, fill=3.0)
    o16, _, _, _ = _run(x, W, max(lengths), out_dtype="bf16")
    for s in (0, 4):
        a, b = int(cu[s]), int(cu[s + 1])
        ref = fixed_prefill_128(x, a, b, W)
        assert torch.equal(o16[a:b], ref), f"stream {s} differs from the fixed-length prefill"


def fixed_prefill_128(x, a, b, W):
    """The fixed-length prefill of packed rows a..b-1 on a grid that runs
    128-query workgroups like the batched call (the stream copied into 16
    batch entries: at least 512 query tiles, more than 1.5 per CU), entry 0
    of its output."""
    import torch
    qs, ks, vs = (dev(x[n][a:b][None], "bf16").expand(16, -1, -1, -1).contiguous()
                  for n in ("q", "k", "v"))
    return vx.prefill(qs, ks, vs, window=W, out_dtype="bf16")[0]


def test_varlen_equals_fixed_prefill_bitwise():
    import torch
    lengths = [156, 77, 156, 10]
    S, H = len(lengths), 32
    x = synth.make_first_chunks(S, H, lengths, seed=62)
    o, _, _, _ = _run(x, 750, 156, out_dtype="bf16")
    cu = x["cu"]
    for s in range(S):
        a, b = int(cu[s]), int(cu[s + 1])
        ref = fixed_prefill_128(x, a, b, 750)
        assert torch.equal(o[a:b], ref), f"stream {s} differs from the fixed-length prefill"
        # a single-stream call runs the halves-split schedule: equal to rounding
        qs, ks, vs = (dev(x[n][a:b][None], "bf16") for n in ("q", "k", "v"))
        one = vx.prefill(qs, ks, vs, window=750, out_dtype="bf16")[0]
        assert float((one.float() - ref.float()).abs().max()) <= 2e-2


def test_varlen_layer_sized_chunks():
    c = synth.FIRST_CHUNK
    lengths = synth.first_chunk_lengths(c["S"], c["t_lo"], c["t_hi"], seed=c["seed"])
    x = synth.make_first_chunks(c["S"], c["H"], lengths, seed=c["seed"], scale=c["scale"])
    say(f"first-chunk workload: S {c['S']} H {c['H']} total {int(x['cu'][-1])}")
    o, rk, rv, pos = _run(x, c["W"], c["t_hi"], rings=True)
    # full check on a sample of streams (the oracle is per stream)
    for s in (0, 17, 63):
        a, b = int(x["cu"][s]), int(x["cu"][s + 1])
        want = oracle.prefill(x["q"][None, a:b], x["k"][None, a:b], x["v"][None, a:b], c["W"],
                              bf16=True)[0]
        check_bf16(host(o[a:b]), want, f"first chunk stream {s}")
    np.testing.assert_array_equal(host(pos.double()), lengths.astype(np.float64))


@pytest.mark.parametrize("W", [750, 40])
def test_seeded_ring_continues_like_prefill(W):
    """First chunk through the varlen prefill, then 4-frame streaming steps:
    the outputs equal one prefill over the whole sequence."""
    import torch
    S, H, T1, T2 = 3, 2, [156, 90, 120], 24
    x_all = synth.make_prefill(S, max(T1) + T2, H, seed=[63, W], dtype="bf16", scale=0.5)
    # stream s: first chunk = frames 0 .. T1[s]-1, then frames T1[s] .. T1[s]+T2-1
    chunks = [np.arange(T1[s]) for s in range(S)]
    cu = np.zeros(S + 1, dtype=np.int32)
    cu[1:] = np.cumsum(T1)
    x = {n: np.concatenate([x_all[n][s, chunks[s]] for s in range(S)]) for n in ("q", "k", "v")}
    x["cu"] = cu
    o1, rk, rv, pos = _run(x, W, max(T1), rings=True, fill=float("nan"))
    outs = []
    for step in range(T2 // 4):
        idx = [np.arange(T1[s] + 4 * step, T1[s] + 4 * step + 4) for s in range(S)]
        qn, kn, vn = (dev(np.stack([x_all[n][s, idx[s]] for s in range(S)]), "bf16")
                      for n in ("q", "k", "v"))
        outs.append(vx.stream_step(qn, kn, vn, rk, rv, pos, window=W, out_dtype="f32"))
        vx.ring_append(rk, rv, kn, vn, pos, window=W)
    o2 = host(torch.cat(outs, dim=1))
    for s in range(S):
        T = T1[s] + T2
        want = oracle.prefill(x_all["q"][None, s, :T], x_all["k"][None, s, :T],
                              x_all["v"][None, s, :T], W, bf16=True)[0]
        a, b = int(cu[s]), int(cu[s + 1])
        check_bf16(host(o1[a:b]), want[:T1[s]], f"stream {s} first chunk")
        check_bf16(o2[s], want[T1[s]:], f"stream {s} continuation")
