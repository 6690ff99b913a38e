"""Seeded synthetic inputs: determinism, shapes and the stated recipe."""
import numpy as np

from sliding_window_attention_vx_amd import synth


def test_same_seed_same_bytes():
    a = synth.make_prefill(1, 20, 2, seed=9, dtype="bf16", scale=0.5)
    b = synth.make_prefill(1, 20, 2, seed=9, dtype="bf16", scale=0.5)
    for key in ("q", "k", "v"):
        assert synth.sha256(a[key]) == synth.sha256(b[key])
    c = synth.make_prefill(1, 20, 2, seed=10, dtype="bf16", scale=0.5)
    assert synth.sha256(a["q"]) != synth.sha256(c["q"])


def test_bf16_inputs_are_representable():
    a = synth.make_prefill(2, 10, 3, seed=1, dtype="bf16")
    bits = a["q"].view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0)


def test_draw_order_and_scale():
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(7)))
    q = rng.standard_normal((1, 5, 2, 64), dtype=np.float32)
    k = rng.standard_normal((1, 5, 2, 64), dtype=np.float32)
    a = synth.make_prefill(1, 5, 2, seed=7, dtype="f32", scale=0.5)
    np.testing.assert_array_equal(a["q"], q * np.float32(0.5))
    np.testing.assert_array_equal(a["k"], k * np.float32(0.5))


def test_long_workload_stress_rows():
    # 1% of the 8*6000*32 key rows, chosen without replacement, scaled by 8 (exact).
    B, T, H = 8, 60, 32  # same recipe on a shorter sequence
    a = synth.make_prefill(B, T, H, seed=5, dtype="bf16", stress_frac=0.01, stress_mult=8.0)
    plain = synth.make_prefill(B, T, H, seed=5, dtype="bf16")
    rows = a["stressed_rows"]
    assert len(rows) == round(0.01 * B * T * H) and len(np.unique(rows)) == len(rows)
    kr, pr = a["k"].reshape(-1, 64), plain["k"].reshape(-1, 64)
    mask = np.zeros(len(kr), bool)
    mask[rows] = True
    np.testing.assert_array_equal(kr[~mask], pr[~mask])
    assert np.count_nonzero(synth.CONFIGS["long"].stress_frac * 8 * 6000 * 32) and \
        round(0.01 * 8 * 6000 * 32) == 15360


def test_stream_state_positions_in_range():
    st = synth.make_stream_state(64, 2, 750, seed=4, pos_lo=750, pos_hi=20000)
    assert st["pos"].dtype == np.int64
    assert st["pos"].min() >= 750 and st["pos"].max() <= 20000
    assert st["ring_k"].shape == (64, 2, 750, 64)
    f0 = synth.make_stream_frames(64, 4, 2, seed=4, step=0)
    f1 = synth.make_stream_frames(64, 4, 2, seed=4, step=1)
    assert synth.sha256(f0["q"]) != synth.sha256(f1["q"])


def test_band_pairs_counts():
    assert synth.band_pairs(64, 16) == 904
    assert synth.band_pairs(1500, 750) == 844125
    assert synth.band_pairs(6000, 750) == 4219125
    assert synth.band_pairs(5, 750) == 15
