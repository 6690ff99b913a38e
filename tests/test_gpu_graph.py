"""HIP-graph capture of the library's calls.

The library allocates nothing and records no memsets, so its launches can be
captured in a graph (torch.cuda.CUDAGraph, which records the launches made on
torch's current stream) and replayed.  Each test replays the graph several
times, with eager work and synchronisations between the replays, and checks
every replay against the same calls made eagerly on copies of the state:
bit for bit, since the kernels are deterministic.
"""
import numpy as np
import pytest

import sliding_window_attention_vx_amd as vx
from sliding_window_attention_vx_amd import synth
from tests.test_gpu_parity import dev, say

pytestmark = pytest.mark.gpu


def _capture(fn):
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up launch outside the graph
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_prefill_graph_replays_match_eager():
    import torch
    say("graph: prefill B1 T1500 H32 W750 (fused RoPE)")
    x = synth.make_config("layer")
    q, k, v = (dev(x[n], "bf16") for n in ("q", "k", "v"))
    table = vx.rope_table(0, 1500)
    o = torch.empty_like(q)
    want = vx.prefill(q, k, v, window=750, table=table).clone()
    g = _capture(lambda: vx.prefill(q, k, v, window=750, table=table, out=o))
    for rep in range(3):
        o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, want), f"replay {rep} differs from the eager call"
        vx.prefill(q, k, v, window=750, table=table)  # eager work between replays


def test_stream_step_graph_replays_advance_state_like_eager():
    import torch
    S, n, H, W = 8, 4, 32, 750
    say(f"graph: fused streaming step S{S} n{n} H{H} W{W}, state advancing each replay")
    st = synth.make_stream_state(S, H, W, seed=[61, 1], pos_lo=W, pos_hi=20000)
    fr = synth.make_stream_frames(S, n, H, seed=61, step=0)
    qn, kn, vn = (dev(fr[c], "bf16") for c in ("q", "k", "v"))
    rk, rv = dev(st["ring_k"], "bf16"), dev(st["ring_v"], "bf16")
    p0 = torch.from_numpy(st["pos"].copy()).cuda()
    # the graph runs two steps, ping-ponging the position arrays, so each
    # replay starts where the previous one ended
    pa, pb = p0.clone(), torch.empty_like(p0)
    o1, o2 = torch.empty_like(qn), torch.empty_like(qn)
    gk, gv = rk.clone(), rv.clone()

    def two_steps():
        vx.stream_step_append(qn, kn, vn, gk, gv, pa, pb, window=W, out=o1)
        vx.stream_step_append(qn, kn, vn, gk, gv, pb, pa, window=W, out=o2)

    # capture on copies, then restore the starting state
    g = _capture(two_steps)
    gk.copy_(rk)
    gv.copy_(rv)
    pa.copy_(p0)
    ek, ev, epa, epb = rk.clone(), rv.clone(), p0.clone(), torch.empty_like(p0)
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        e1 = vx.stream_step_append(qn, kn, vn, ek, ev, epa, epb, window=W)
        e2 = vx.stream_step_append(qn, kn, vn, ek, ev, epb, epa, window=W)
        torch.cuda.synchronize()
        assert torch.equal(o1, e1) and torch.equal(o2, e2), f"replay {rep}: outputs differ"
        assert torch.equal(gk, ek) and torch.equal(gv, ev), f"replay {rep}: rings differ"
        assert torch.equal(pa, epa), f"replay {rep}: positions differ"
    assert (pa.cpu().numpy() == st["pos"] + 6 * n).all()


def test_encoder_step_graph_replays_match_eager():
    import torch
    L, S, n, H, dm, ffn, nm, W = 2, 2, 4, 2, 256, 512, 128, 16
    say(f"graph: whole encoder step L{L} S{S} n{n} H{H} d_model {dm} W{W}")
    sw = {k_: dev(v_, "bf16") for k_, v_ in synth.make_enc_stem_weights(dm, nm, seed=62).items()}
    lw = [{k_: dev(v_, "bf16") for k_, v_ in
           synth.make_enc_layer_weights(dm, H, ffn, seed=62, layer=l).items()} for l in range(L)]
    mel = [dev(synth.make_mel(S, 2 * n, nm, seed=62, step=i), "bf16") for i in range(4)]

    def state():
        return dict(mel=torch.zeros((S, 2 * n + 2, nm), dtype=torch.bfloat16, device="cuda"),
                    c1=torch.zeros((S, 2 * n + 2, dm), dtype=torch.bfloat16, device="cuda"),
                    rk=torch.zeros((L, S, H, W, 64), dtype=torch.bfloat16, device="cuda"),
                    rv=torch.zeros((L, S, H, W, 64), dtype=torch.bfloat16, device="cuda"),
                    pa=torch.zeros(S, dtype=torch.int64, device="cuda"),
                    pb=torch.zeros(S, dtype=torch.int64, device="cuda"),
                    x=torch.empty((S, n, dm), dtype=torch.float32, device="cuda"),
                    work=vx.enc_work(S, n, H, dm, ffn))

    G, E = state(), state()
    feed = torch.empty((S, 2 * n, nm), dtype=torch.bfloat16, device="cuda")

    def step(st, frames):
        # the new frames enter slots 2.. (a device copy, captured with the step)
        st["mel"][:, 2:].copy_(frames)
        vx.enc_step(st["mel"], st["c1"], sw, lw, st["rk"], st["rv"], st["pa"], st["pb"],
                    x=st["x"], window=W, H=H, work=st["work"])
        st["pa"].copy_(st["pb"])

    feed.copy_(mel[0])
    g = _capture(lambda: step(G, feed))
    # the warm-up and capture ran nothing into G's state that matters: reset it
    for key in ("mel", "c1", "rk", "rv", "pa", "pb"):
        G[key].zero_()
    for i in range(4):
        feed.copy_(mel[i])
        g.replay()
        step(E, mel[i])
        torch.cuda.synchronize()
        for key in ("x", "rk", "rv", "c1", "mel", "pa"):
            assert torch.equal(G[key], E[key]), f"step {i}: {key} differs from the eager step"
        say(f"  step {i}: graph replay equals the eager step (x rms "
            f"{float(np.sqrt(np.mean(G['x'].cpu().numpy() ** 2))):.3f})")
