"""GPU: every query tile of a prefill is computed, whatever order the grid
deals its tiles in.

The prefill deals each XCD's query tiles to its compute units in one of
three orders, chosen by how many of them fit at once (up to two, up to three
or more workgroups per CU).  These grids cover each order on a 256-CU
device (32 CUs per XCD), in both the halves-split schedule (64-query
workgroups) and the 128-query one.  The output buffer starts as NaN, so a
tile that no workgroup computed shows up as NaN; sampled heads are checked
against the float64 oracle (bf16 contract) to the parity bar
(max |err| <= 2e-2, relative RMS <= 1e-2).
"""
import numpy as np
import pytest

import oracle
import sliding_window_attention_vx_amd as vx
from sliding_window_attention_vx_amd import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda", torch.bfloat16)


# (B, T, H): per XCD, B*H/8 pairs x query tiles
CASES = [
    (1, 1500, 32),   # halves split, 96 tiles per XCD: three rounds
    (1, 1500, 24),   # halves split, 72: three rounds, the last one partial
    (1, 1500, 12),   # halves split, 48 (two rounds)
    (1, 3000, 24),   # 128-query tiles, 72: three rounds
    (3, 1500, 16),   # 128-query tiles, 72, three batch entries
    (4, 1500, 32),   # 128-query tiles, 192: more than fit at once
]


@pytest.mark.parametrize("B,T,H", CASES)
def test_every_tile_computed(B, T, H):
    import torch
    W = 750
    say(f"work order: B{B} T{T} H{H}")
    x = synth.make_prefill(B, T, H, seed=900 + B * 31 + H, dtype="bf16", scale=0.5)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    table = vx.rope_table(0, T)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    vx.prefill(q, k, v, window=W, table=table, out=out)
    torch.cuda.synchronize()
    n_nan = int(torch.isnan(out).sum().item())
    assert n_nan == 0, f"B{B} T{T} H{H}: {n_nan} outputs never written"
    rng = np.random.default_rng(B * 1000 + H)
    for b, h in {(int(rng.integers(B)), int(rng.integers(H))), (B - 1, H - 1)}:
        want = oracle.prefill(x["q"][b:b + 1, :, h:h + 1], x["k"][b:b + 1, :, h:h + 1],
                              x["v"][b:b + 1, :, h:h + 1], W, bf16=True)
        got = out[b:b + 1, :, h:h + 1].float().cpu().numpy().astype(np.float64)
        err = np.abs(got - want)
        mx = float(err.max())
        rrms = float(np.sqrt(np.mean(err ** 2)) / np.sqrt(np.mean(want ** 2)))
        say(f"  entry {b} head {h}: max|err| {mx:.3e}  rel-rms {rrms:.3e}")
        assert mx <= 2e-2 and rrms <= 1e-2
