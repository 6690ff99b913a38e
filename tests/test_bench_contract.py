"""Host checks of bench.py's contract (no GPU): refusal of several GPUs, the
algorithmic-byte and FLOP formulas, and whether every stored counter
measurement belongs to the kernel sources in the tree (bench.py reports no
traffic for a stale one)."""
import subprocess
import sys
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


@pytest.mark.parametrize("kind", sorted(bench.MEASURED_TRAFFIC))
def test_stored_counters_match_the_kernel_sources(kind):
    # bench.py reports traffic only for the sources the counters were taken
    # on (null otherwise); a skip here flags counters to take again
    if bench.measured_traffic(kind) is None:
        pytest.skip(f"the {kind} counters were taken on other sources: measure them again")
    files, _, nbytes = bench.MEASURED_TRAFFIC[kind]
    assert nbytes > 0 and files


def test_stream_step_bytes():
    # per (stream, head): 2 (W-1) ring rows, q/k/v in, o out, k/v appended; pos in and out
    S, n, H, W, row = 64, 4, 32, 750, 128
    per = 2 * (W - 1) * row + 3 * n * row + n * row + 2 * n * row
    assert bench.stream_bytes(S, n, H, W) == S * H * per + S * 16
    assert abs(bench.stream_bytes(S, n, H, W) - 399.0e6) < 0.1e6


def test_band_flops_of_the_layer_workload():
    # 4 * 64 FLOP per in-band (query, key) pair, W(W+1)/2 + (T-W) W pairs per head
    T, W = 1500, 750
    pairs = W * (W + 1) // 2 + (T - W) * W
    assert bench.band_flops(1, T, 32, W) == 4.0 * 64 * pairs * 32
    assert abs(bench.band_flops(1, T, 32, W) - 6.915e9) < 0.001e9
