"""GPU tests of the prefill with keys rotated ahead of the kernel.

On grids of at least 8 four-wave query tiles per compute unit (B8 T1024
H32 and up) and with a workspace of vx_swa_attn_prefill_workspace_size() bytes,
vx_swa_attn_prefill first rotates K once into the workspace, reading for
each frame the cos/sin row its own staging would read, and the kernel then
stages the rotated keys without rotating them again.  The rotation is the
same function on the same values, so the outputs must equal those of the
call without a workspace bit for bit; checked here with a caller table, per
entry positions and a table built in the workspace, float32 output and an
entry with an invalid position, and the rotated keys in the workspace
against vx_rope_qk.  Pre-rotated input (rope_applied) on such a grid takes
the same kernel mode and must equal the fused call bit for bit.
"""
import numpy as np
import pytest

import oracle
import sliding_window_attention_vx_amd as vx
from sliding_window_attention_vx_amd import synth
from tests.test_gpu_parity import check_bf16, dev, host, say

pytestmark = pytest.mark.gpu

B, T, H, W = 8, 2048, 32, 750
N_CUS = 256  # compute units of an MI355X


def inputs(seed):
    x = synth.make_prefill(B, T, H, seed=seed, dtype="bf16", scale=0.5)
    return x, tuple(dev(x[n], "bf16") for n in ("q", "k", "v"))


def workspace():
    import torch
    n = vx.prefill_workspace_size(B, T, H, W)
    assert n == B * T * 256 + B * T * H * 64 * 2, "the shape should rotate its keys ahead"
    return torch.zeros(((n + 15) // 16 * 16,), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_keys_rotated_ahead_equal_fused_with_a_table(out_dtype):
    import torch
    say(f"keys rotated ahead: B{B} T{T} H{H} W{W}, caller table, out {out_dtype}")
    x, (q, k, v) = inputs(901)
    table = vx.rope_table(0, T)
    ws = workspace()
    got = vx.prefill(q, k, v, window=W, table=table, workspace=ws, out_dtype=out_dtype)
    want = vx.prefill(q, k, v, window=W, table=table, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    # with a caller table the rotated keys sit at the start of the workspace
    k2 = k.clone()
    vx.rope_qk(None, k2)
    kws = ws[: B * T * H * 64 * 2].view(torch.bfloat16).view(B, T, H, 64)
    assert torch.equal(kws, k2), "the workspace does not hold the rotated keys"
    picks = [(0, 0), (7, 31), (2, 17)]
    sel = lambda a: np.stack([a[b_, :, h_] for b_, h_ in picks])[:, :, None]  # noqa: E731
    ref = oracle.prefill(sel(x["q"]), sel(x["k"]), sel(x["v"]), W, bf16=True)
    g = host(got)
    for i, (b_, h_) in enumerate(picks):
        check_bf16(g[b_, :, h_], ref[i, :, 0], f"rotated ahead b{b_} h{h_}")


def test_keys_rotated_ahead_positions_and_workspace_table():
    import torch
    pos = [0, 777, 12345, 19999, 5, 64, 300000, 3]
    say(f"keys rotated ahead: per-entry positions {pos}, caller table and workspace table")
    x, (q, k, v) = inputs(902)
    p0 = torch.tensor(pos, dtype=torch.int64, device="cuda")
    table = vx.rope_table(0, 302100)
    want = vx.prefill(q, k, v, window=W, pos0=p0, table=table)
    got = vx.prefill(q, k, v, window=W, pos0=p0, table=table, workspace=workspace())
    ws = workspace()
    got_ws = vx.prefill(q, k, v, window=W, pos0=p0, workspace=ws)  # table built in the workspace
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    assert torch.equal(got_ws, want)
    g = host(got)
    for b_, h_ in ((1, 5), (6, 30)):
        sl = (slice(b_, b_ + 1), slice(None), slice(h_, h_ + 1))
        ref = oracle.prefill(x["q"][sl], x["k"][sl], x["v"][sl], W, pos=pos[b_], bf16=True)
        check_bf16(g[sl], ref, f"rotated ahead pos0 {pos[b_]} h{h_}")


def test_keys_rotated_ahead_invalid_entry_is_loud():
    import torch
    say("keys rotated ahead: an entry with a negative position")
    _, (q, k, v) = inputs(903)
    p0 = torch.tensor([3, -5, 100, 7, 0, 1, 2, 9], dtype=torch.int64, device="cuda")
    table = vx.rope_table(0, T + 100)
    got = vx.prefill(q, k, v, window=W, pos0=p0, table=table, workspace=workspace())
    want = vx.prefill(q, k, v, window=W, pos0=p0, table=table)
    torch.cuda.synchronize()
    assert torch.isnan(got[1].float()).all()
    for b_ in (0, 2, 3, 4, 5, 6, 7):
        assert torch.equal(got[b_], want[b_])


def test_prerotated_input_on_a_large_grid_equals_fused():
    import torch
    say("pre-rotated input (no cos/sin staging) vs fused, B4 T1500 H32")
    x = synth.make_prefill(4, 1500, 32, seed=904, dtype="bf16", scale=0.5)
    q, k, v = (dev(x[n], "bf16") for n in ("q", "k", "v"))
    fused = vx.prefill(q, k, v, window=W)
    q2, k2 = q.clone(), k.clone()
    vx.rope_qk(q2, k2)
    pre = vx.prefill(q2, k2, v, window=W, rope_applied=True)
    torch.cuda.synchronize()
    assert torch.equal(fused, pre)


@pytest.mark.parametrize("B,T,H,W_", [(3, 1001, 32, 97), (2, 777, 64, 750), (1, 3001, 48, 1),
                                      (5, 450, 48, 2000)])
def test_prerotated_ragged_shapes_equal_fused_and_match_oracle(B, T, H, W_):
    """Grids of more than 1.5 four-wave query tiles per compute unit on
    pre-rotated input run the kernel on rotated keys, whose V tiles sit in
    compact swizzled 128-byte rows (four workgroups per CU); the fused call
    on the same grid runs the same schedule with padded V rows.  Ragged T
    (a partial last key tile), W from 1 to above T: the two agree bit for
    bit, and sampled (b, h) pairs match the oracle."""
    import torch
    from tests.test_gpu_parity import _check_picks
    wg4 = -(-T // 128) * H * B
    assert 2 * wg4 > 3 * N_CUS, "the shape should take 128-query workgroups"
    say(f"pre-rotated vs fused, 128-query workgroups: B{B} T{T} H{H} W{W_}")
    x = synth.make_prefill(B, T, H, seed=950 + T + W_, dtype="bf16", scale=0.5)
    q, k, v = (dev(x[n], "bf16") for n in ("q", "k", "v"))
    fused = vx.prefill(q, k, v, window=W_)
    q2, k2 = q.clone(), k.clone()
    vx.rope_qk(q2, k2)
    pre = vx.prefill(q2, k2, v, window=W_, rope_applied=True)
    torch.cuda.synchronize()
    assert torch.equal(fused, pre)
    picks = [(0, 0), (B - 1, H - 1), (B // 2, H // 2)]
    _check_picks(x, host(pre), picks, W_, f"pre-rotated B{B} T{T} H{H} W{W_}")
