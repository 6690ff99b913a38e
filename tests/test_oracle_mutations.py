"""The oracle pins must catch plausible mistakes.

Each case copies oracle.c, plants one mistake by text substitution, builds
the copy with gcc in a temporary directory and runs the pins against it: at
least one pin must fail.  The unmodified source, built the same way, must
pass them all.  Everything here runs on the CPU.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

PIN_CHECKS = [
    pins.test_bf16_round_ties_and_closed_forms,
    pins.test_rope_matches_complex_multiplication,
    pins.test_rope_frequencies_closed_form_theta_1e6,
    lambda: pins.test_prefill_matches_dense_brute_force(40, 7, 3, 16),
    lambda: pins.test_prefill_matches_dense_brute_force(64, 16, 4, 64),
    pins.test_prefill_full_causal_when_T_le_W,
    pins.test_window_locality,
    pins.test_constant_values_give_constant_output,
    pins.test_bf16_contract_rounds_rotated_qk,
    lambda: pins.test_streaming_equals_prefill([4, 1, 7, 3]),
    pins.test_streaming_equals_prefill_bf16_contract,
    pins.test_ring_holds_rotated_keys_at_position_mod_w,
    pins.test_stream_step_from_absolute_positions_matches_prefill_slice,
    lambda: pins.test_gqa_prefill_matches_dense_brute_force(48, 16, 8, 2, 128),
    pins.test_gqa_key_value_head_touches_only_its_group,
    lambda: pins.test_gqa_decode_equals_prefill_across_ring_wraps(1),
]

MUTATIONS = [
    ("window keeps W+1 keys", "t - W + 1 < 0 ? 0 : t - W + 1", "t - W < 0 ? 0 : t - W"),
    ("window keeps W-1 keys", "t - W + 1 < 0 ? 0 : t - W + 1", "t - W + 2 < 0 ? 0 : t - W + 2"),
    ("rotation sign flipped", "x[i] = x0 * c - x1 * s;", "x[i] = x0 * c + x1 * s;"),
    ("wrong rotation partner", "x1 = x[i + half];", "x1 = x[(i + 1) % D];"),
    ("frequency exponent halved", "-2.0 * (double)i / (double)D", "-1.0 * (double)i / (double)D"),
    ("scale dropped", "s[j] = scale * acc;", "s[j] = acc;"),
    ("weights not normalised", "double w = s[j] / l;", "double w = s[j];"),
    ("max not subtracted consistently", "s[j] = exp(s[j] - m);", "s[j] = exp(s[j] - m) + 1e-3;"),
    ("ring slot off by one", "int64_t slot = pp % W;", "int64_t slot = (pp + 1) % W;"),
    ("stream window off by one", "P + i - W + 1 < 0 ? 0 : P + i - W + 1", "P + i - W + 2 < 0 ? 0 : P + i - W + 2"),
    ("append rotates at the chunk start", "int64_t p = pos[s] + i;\n      int64_t slot", "int64_t p = pos[s];\n      int64_t slot"),
    ("bf16 ties away from zero", "double n = nearbyint(scaled);", "double n = round(scaled);"),
    ("bf16 truncates", "double n = nearbyint(scaled);", "double n = trunc(scaled);"),
    ("prefill key/value heads interleaved", "const int64_t hk = h / G;", "const int64_t hk = h % Hkv;"),
    ("decode key/value heads interleaved", "const int64_t kvh = h / G;", "const int64_t kvh = h % Hkv;"),
    ("new frames see the future", "for (int64_t jj = 0; jj <= i; ++jj, ++nk)", "for (int64_t jj = 0; jj < n; ++jj, ++nk)"),
]


def _build(src_text, tmp_path, tag):
    c = tmp_path / f"oracle_{tag}.c"
    so = tmp_path / f"liboracle_{tag}.so"
    c.write_text(src_text)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(so),
                    str(c), "-lm"], check=True, capture_output=True)
    return str(so)


def _failures_in_process(path):
    failed = []
    with oracle.using_library(path):
        for i, f in enumerate(PIN_CHECKS):
            try:
                with np.errstate(all="ignore"):
                    f()
            except (AssertionError, ValueError):
                failed.append(i)
    return failed


def _failures(path):
    """Run the pins against `path` in a child process; a crash counts as caught."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-m", "tests.test_oracle_mutations", path], cwd=root,
                       capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        return [f"child exited with {r.returncode}"]
    return [int(x) for x in r.stdout.split()[1:]]


def test_unmodified_source_passes_all_pins(tmp_path):
    assert _failures(_build(open(SRC).read(), tmp_path, "clean")) == []


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    failed = _failures(_build(src.replace(old, new), tmp_path, "mut"))
    assert failed, f"no pin caught the planted mistake: {name}"


if __name__ == "__main__":
    print("FAILED", *_failures_in_process(sys.argv[1]))
