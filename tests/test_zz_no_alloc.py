"""GPU test of the allocation-free prefill entry point through the C ABI.

vx_swa_attn_prefill_noalloc keeps the cos/sin rows of its positions in the
library's static device scratch instead of a caller table or workspace.  The
same float64 angle gives the same cos/sin wherever they are kept, so its
outputs must equal vx_swa_attn_prefill's (given a table of the same
positions) bit for bit.  Two calls in a row, the second smaller, check that
the shared scratch is fully rewritten by each call.
"""
import numpy as np
import pytest

import sliding_window_attention_vx_amd as vx
from sliding_window_attention_vx_amd import synth

pytestmark = pytest.mark.gpu


def dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda", torch.bfloat16)


def one_call(B, T, H, W, pos0, seed):
    import torch
    print(f"noalloc prefill B{B} T{T} H{H} W{W} pos0 {pos0}", flush=True)
    x = synth.make_prefill(B, T, H, seed=seed, dtype="bf16", scale=0.5)
    q, k, v = (dev(x[n]) for n in ("q", "k", "v"))
    p0 = torch.tensor(pos0, dtype=torch.int64, device="cuda")
    table = vx.rope_table(0, max(pos0) + T)
    want = vx.prefill(q, k, v, window=W, pos0=p0, table=table)
    got = vx.prefill_noalloc(q, k, v, window=W, pos0=p0)
    torch.cuda.synchronize()
    assert torch.equal(got, want), f"B{B} T{T}: differs from vx_swa_attn_prefill"
    # pre-rotated inputs use no scratch and give the same bits as well
    q2, k2 = q.clone(), k.clone()
    vx.rope_qk(q2, k2, pos0=p0)
    want2 = vx.prefill(q2, k2, v, window=W, rope_applied=True)
    got2 = vx.prefill_noalloc(q2, k2, v, window=W, rope_applied=True)
    torch.cuda.synchronize()
    assert torch.equal(got2, want2)
    assert torch.equal(got2, want), "pre-rotated and fused paths differ"


def test_noalloc_prefill_equals_prefill_on_two_calls():
    one_call(4, 1500, 32, 750, [0, 777, 12345, 19999], seed=81)
    one_call(2, 300, 8, 64, [5, 70000], seed=82)


def test_noalloc_prefill_rejects_more_rows_than_its_scratch():
    import torch
    q = torch.zeros((1, 65537, 1, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(vx.VxError, match="scratch"):
        vx.prefill_noalloc(q, q.clone(), q.clone())
