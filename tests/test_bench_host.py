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


def test_key_offsets_shape_the_scores():
    """The key_offsets input recipe: q[..., 0] = 1 and k[j, :, 0] = offset_j / (scale log2 e), so
    scale * q.k * log2 e differs from the score without dimension 0 by offset_j (to bf16
    rounding of k[j, :, 0]); draws of the other dimensions are those of the plain recipe."""
    import math

    import fa_inputs

    offs = np.linspace(-5.0, 30.0, 70)
    w = fa_inputs.make(2, 3, 1, 5, 70, 64, causal=False, seed=7, key_offsets=offs)
    plain = fa_inputs.make(2, 3, 1, 5, 70, 64, causal=False, seed=7)
    q, k = w.q.double().numpy(), w.k.double().numpy()
    assert np.all(q[..., 0] == 1.0)
    assert np.array_equal(q[..., 1:], plain.q.double().numpy()[..., 1:])
    assert np.array_equal(k[..., 1:], plain.k.double().numpy()[..., 1:])
    got = k[:, 0, 0].reshape(2, 70) * w.softmax_scale * math.log2(math.e)
    assert np.allclose(got, offs[None, :], rtol=2 ** -8, atol=0)
    try:
        fa_inputs.make(1, 1, 1, 5, 70, 64, causal=False, seed=7, key_offsets=offs[:10])
    except ValueError:
        pass
    else:
        raise AssertionError("a key_offsets of the wrong length must be refused")
