"""CPU pin of exp2_poly, the FMA-pipe 2^x of the exp2 offload (fa_exp2_poly.h): the header is
compiled for the host (hipcc, host pass only) into a small driver that evaluates it over the
whole input range the softmax gives it; the values are checked here against exp2 in float64.

Claimed bound (header): relative error <= 7.5e-5 wherever 2^x is a normal float, exactly 0 at
-inf and below the clamp, NaN propagated."""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_forward_fa_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include <cstdlib>
#include <cmath>
#include "fa_exp2_poly.h"
// reads float bit patterns (hex) from stdin, writes exp2_poly of each as hex bits
int main() {
  unsigned u;
  while (std::scanf("%x", &u) == 1) {
    float x;
    __builtin_memcpy(&x, &u, 4);
    const float y = fa::exp2_poly(x);
    unsigned v;
    __builtin_memcpy(&v, &y, 4);
    std::printf("%08x\n", v);
  }
  return 0;
}
"""


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.fixture(scope="module")
def exp2_poly(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not found")
    d = tmp_path_factory.mktemp("exp2poly")
    src, exe = d / "drv.hip", d / "drv"
    src.write_text(DRIVER)
    subprocess.run([hipcc, "--offload-host-only", "-O2", "-std=c++17", "-I", CSRC, str(src),
                    "-o", str(exe)], check=True, capture_output=True)

    def run(x):
        x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
        inp = "\n".join(f"{b:08x}" for b in x.view(np.uint32).tolist()) + "\n"
        out = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True)
        return np.array([int(t, 16) for t in out.stdout.split()], dtype=np.uint32).view(np.float32)

    return run


def test_relative_error_on_the_reduced_range(exp2_poly):
    """f in [-1/2, 1/2] (the polynomial's own interval), 2^17 + 1 evenly spaced points."""
    x = np.linspace(-0.5, 0.5, (1 << 17) + 1).astype(np.float32)
    y = exp2_poly(x).astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    rel = np.abs(y - ref) / ref
    assert rel.max() <= 7.5e-5, rel.max()
    assert rel.max() >= 1e-5  # a degree-3 fit: a far smaller error would mean it is not what runs


def test_relative_error_over_the_normal_range(exp2_poly):
    """x in [-126, 8]: the exponents the softmax takes (scores against a maximum that is at most
    2^8 stale); the Cody-Waite reduction must not add error beyond the polynomial's."""
    x = np.concatenate([np.arange(-126.0, 8.0, 1.0 / 1024.0), [8.0, -0.5, 0.5, 0.0]]).astype(np.float32)
    y = exp2_poly(x).astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    rel = np.abs(y - ref) / ref
    assert rel.max() <= 7.5e-5, (rel.max(), x[np.argmax(rel)])


def test_subnormal_results(exp2_poly):
    """x in (-149, -126): the result is subnormal; error within the polynomial's relative bound
    plus half a subnormal step."""
    x = np.arange(-149.0, -126.0, 1.0 / 64.0).astype(np.float32)
    y = exp2_poly(x).astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    assert np.all(np.abs(y - ref) <= 7.5e-5 * ref + 2.0 ** -150)


def test_special_values(exp2_poly):
    """-inf (a masked score) and anything below the clamp give exactly 0; NaN propagates."""
    x = np.array([-np.inf, -1e30, -1000.0, -160.0, -150.5, np.nan], dtype=np.float32)
    y = exp2_poly(x)
    assert np.all(y[:5] == 0.0) and np.all(np.signbit(y[:5]) == False)  # noqa: E712
    assert np.isnan(y[5])
