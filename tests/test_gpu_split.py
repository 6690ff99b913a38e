"""GPU tests of the split walk of vx_swa_attn_prefill.

With VX_FLAG_SPLIT_WALK (force_split) and a workspace of
vx_swa_attn_prefill_workspace_size() bytes, grids of at most 1.5
four-wave (128-query) tiles per compute unit take the split walk instead of
the default halves-split workgroups: each query tile gets two workgroups,
one per half of its key band, and per wave the one that finishes second
merges the two softmax partials through the workspace.  Checked here,
through the C ABI:
- the outputs against the bf16-contract oracle, at the parity tests'
  tolerance, on the layer workload and on ragged and degenerate shapes (one
  key tile, so one half walks nothing; fewer than 8 (batch, head) pairs;
  W = 1; W above T; pre-rotated input; float32 output; per-entry positions);
- the split actually ran: the flag words, filled with a byte pattern before
  the call, read zero after it (each merge resets its flag); without the
  flag the workspace's flag region is left alone;
- run-to-run identical bits (the merge order does not depend on which half
  finishes first), also when the workspace starts out holding random bytes;
- graph replays equal to the eager call (the flags are zero again after
  every launch).
"""
import numpy as np
import pytest

import oracle
import sliding_window_attention_vx_amd as vx
from sliding_window_attention_vx_amd import synth
from tests.test_gpu_parity import check_bf16, dev, host, say

pytestmark = pytest.mark.gpu

PART_BYTES = 9 * 64 * 16  # one wave's partial result
N_CUS = 256


def split_layout(B, T, H, W, force):
    """(flag bytes, partial bytes) of the split walk, or None where it is not taken."""
    wg = -(-T // 128) * B * H
    if not (force and 2 * wg <= 3 * N_CUS):
        return None
    slots = wg * 4
    return (slots * 8 + 255) // 256 * 256, slots * 2 * PART_BYTES


def run(x, W, ws, pos0=None, table=None, table_p0=0, out_dtype=None, rope_applied=False,
        auto_table=True, force=True):
    q, k, v = (dev(x[n], "bf16") for n in ("q", "k", "v"))
    if rope_applied:
        vx.rope_qk(q, k, pos0=pos0)
    o = vx.prefill(q, k, v, window=W, pos0=pos0, table=table, table_p0=table_p0, workspace=ws,
                   out_dtype=out_dtype, rope_applied=rope_applied, auto_table=auto_table,
                   force_split=force)
    return o


def workspace(B, T, H, W, fill=0xA5, force=True):
    import torch
    n = vx.prefill_workspace_size(B, T, H, W, force_split=force)
    lay = split_layout(B, T, H, W, force)
    assert lay is not None and n >= sum(lay), "the shape should take the split walk"
    ws = torch.full(((n + 15) // 16 * 16,), fill, dtype=torch.uint8, device="cuda")
    return ws


def flags_zero(ws, off, B, T, H):
    import torch
    torch.cuda.synchronize()
    slots = -(-T // 128) * B * H * 4
    f = ws[off:off + slots * 8]
    return bool(torch.all(f == 0).item())


def test_split_layer_matches_oracle():
    c = synth.CONFIGS["layer"]
    x = synth.make_config("layer")
    say("split walk: layer B1 T1500 H32 W750, caller table")
    ws = workspace(c.B, c.T, c.H, c.W)
    table = vx.rope_table(0, c.T)
    got = run(x, c.W, ws, table=table)
    # with a caller table the split region starts at offset 0
    assert flags_zero(ws, 0, c.B, c.T, c.H), "flags not reset: the split walk did not run"
    want = oracle.prefill(x["q"], x["k"], x["v"], c.W, bf16=True)
    check_bf16(host(got), want, "split layer")


@pytest.mark.parametrize("B,T,H,W", [(1, 1, 4, 750), (1, 64, 3, 64), (1, 65, 2, 16),
                                     (2, 127, 4, 33), (1, 129, 8, 100), (2, 300, 4, 1),
                                     (1, 751, 5, 750), (3, 1000, 3, 97), (1, 1500, 4, 2000)])
def test_split_edge_shapes(B, T, H, W):
    say(f"split walk: B{B} T{T} H{H} W{W}")
    x = synth.make_prefill(B, T, H, seed=700 + T + W, dtype="bf16", scale=0.5)
    ws = workspace(B, T, H, W)
    got = host(run(x, W, ws, auto_table=False))  # the library builds a table in the workspace
    table_off = (B * T * 256 + 255) // 256 * 256
    assert flags_zero(ws, table_off, B, T, H)
    want = oracle.prefill(x["q"], x["k"], x["v"], W, bf16=True)
    check_bf16(got, want, f"split B{B} T{T} H{H} W{W}")
    # the unsplit walk (no workspace) agrees to rounding
    q, k, v = (dev(x[n], "bf16") for n in ("q", "k", "v"))
    ref = host(vx.prefill(q, k, v, window=W))
    assert np.max(np.abs(got - ref)) <= 2e-2


def test_split_positions_prerotated_and_f32_out():
    import torch
    B, T, H, W = 2, 700, 6, 750
    x = synth.make_prefill(B, T, H, seed=731, dtype="bf16", scale=0.5)
    p0 = torch.tensor([5, 40000], dtype=torch.int64, device="cuda")
    table = vx.rope_table(0, 41000)
    say("split walk: per-entry positions with a table, f32 out; pre-rotated input")
    ws = workspace(B, T, H, W)
    got = host(run(x, W, ws, pos0=p0, table=table, out_dtype="f32"))
    assert flags_zero(ws, 0, B, T, H)
    for b, p in enumerate((5, 40000)):
        sl = slice(b, b + 1)
        want = oracle.prefill(x["q"][sl], x["k"][sl], x["v"][sl], W, pos=p, bf16=True)
        check_bf16(got[sl], want, f"split pos0 {p}")
    ws2 = workspace(B, T, H, W)
    pre = host(run(x, W, ws2, pos0=p0, rope_applied=True))
    assert flags_zero(ws2, 0, B, T, H)
    for b, p in enumerate((5, 40000)):
        sl = slice(b, b + 1)
        want = oracle.prefill(x["q"][sl], x["k"][sl], x["v"][sl], W, pos=p, bf16=True)
        check_bf16(pre[sl], want, f"split pre-rotated pos0 {p}")


def test_split_deterministic_whatever_the_workspace_held():
    import torch
    B, T, H, W = 1, 1500, 32, 750
    x = synth.make_prefill(B, T, H, seed=741, dtype="bf16", scale=0.5)
    q, k, v = (dev(x[n], "bf16") for n in ("q", "k", "v"))
    table = vx.rope_table(0, T)
    say("split walk: repeated calls, zeroed and random workspaces")
    ws0 = workspace(B, T, H, W, fill=0)
    a = vx.prefill(q, k, v, window=W, table=table, workspace=ws0, force_split=True).clone()
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    ws1 = torch.randint(0, 256, ws0.shape, dtype=torch.uint8, device="cuda", generator=g)
    for rep in range(4):
        b = vx.prefill(q, k, v, window=W, table=table, workspace=ws1 if rep % 2 else ws0,
                       force_split=True)
        torch.cuda.synchronize()
        assert torch.equal(a, b), f"call {rep} differs"
    assert flags_zero(ws0, 0, B, T, H) and flags_zero(ws1, 0, B, T, H)


def test_split_graph_replays_match_eager():
    import torch
    from tests.test_gpu_graph import _capture
    c = synth.CONFIGS["layer"]
    x = synth.make_config("layer")
    say("split walk under graph replay: layer B1 T1500 H32 W750")
    q, k, v = (dev(x[n], "bf16") for n in ("q", "k", "v"))
    table = vx.rope_table(0, c.T)
    ws = workspace(c.B, c.T, c.H, c.W)
    o = torch.empty_like(q)
    want = vx.prefill(q, k, v, window=c.W, table=table, workspace=ws, force_split=True).clone()
    g = _capture(lambda: vx.prefill(q, k, v, window=c.W, table=table, out=o, workspace=ws,
                                    force_split=True))
    for rep in range(3):
        o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, want), f"replay {rep} differs from the eager call"
        vx.prefill(q, k, v, window=c.W, table=table, workspace=ws, force_split=True)  # eager work
    assert flags_zero(ws, 0, c.B, c.T, c.H)


def test_no_split_without_the_flag():
    """Without VX_FLAG_SPLIT_WALK a workspace holds the table only: the flag
    region of a workspace sized for the split is left alone, and the output
    equals the call without a workspace bit for bit (the halves-split
    schedule both times)."""
    import torch
    W = 750
    for T, H in ((1500, 16), (500, 32)):
        say(f"no split without the flag: B1 T{T} H{H}")
        x = synth.make_prefill(1, T, H, seed=760 + H, dtype="bf16", scale=0.5)
        table = vx.rope_table(0, T)
        assert vx.prefill_workspace_size(1, T, H, W) == T * 256
        ws = workspace(1, T, H, W)  # sized for the split (with the flag)
        got = run(x, W, ws, table=table, force=False)
        q, k, v = (dev(x[n_], "bf16") for n_ in ("q", "k", "v"))
        plain = vx.prefill(q, k, v, window=W, table=table)
        torch.cuda.synchronize()
        assert torch.equal(got, plain)
        assert bool(torch.all(ws[: 4 * -(-T // 128) * H * 8] == 0xA5).item())
        check_bf16(host(got), oracle.prefill(x["q"], x["k"], x["v"], W, bf16=True),
                   f"default schedule T{T} H{H}")
