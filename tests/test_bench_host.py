"""Host-side pieces of bench.py (no GPU): FLOP accounting and the --gpus guard."""
import subprocess
import sys

import numpy as np

import bench


def brute_pairs(sq, sk, causal):
    return sum(1 for i in range(sq) for j in range(sk) if not causal or j <= i + sk - sq)


def test_pairs_closed_form_matches_brute_force():
    rng = np.random.default_rng(0)
    cases = [(0, 0), (0, 5), (5, 0), (1, 1), (7, 7), (9, 4), (4, 9), (128, 100), (100, 128)]
    cases += [(int(rng.integers(0, 60)), int(rng.integers(0, 60))) for _ in range(60)]
    for sq, sk in cases:
        for causal in (False, True):
            assert bench.pairs_per_sequence(sq, sk, causal) == brute_pairs(sq, sk, causal), (sq, sk, causal)


def test_square_causal_pairs():
    assert bench.pairs_per_sequence(8192, 8192, True) == 8192 * 8193 // 2


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr
