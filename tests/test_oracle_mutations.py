"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that the pins catch every one of them.

Each mutation is a single textual edit of ``oracle/fa_oracle.c``; the broken
copy is compiled into a temporary directory and swapped in for the duration
of one test.  A mutation that no pin detects would mean the oracle could
carry that mistake unnoticed.
"""
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "fa_oracle.c")

MUTATIONS = {
    "causal_off_by_one": ("(int64_t)j > (int64_t)i + sk - sq", "(int64_t)j >= (int64_t)i + sk - sq"),
    "causal_top_left": ("(int64_t)j > (int64_t)i + sk - sq", "(int64_t)j > (int64_t)i"),
    "gqa_modulo_heads": ("const int g = h / (p->hq / p->hkv);", "const int g = h % p->hkv;"),
    "lse_drops_max": ("*lse = m + log(z);", "*lse = log(z);"),
    "scale_dropped": ("s[j] = p->scale * dot;", "s[j] = dot;"),
    "exp_sign_flipped": ("if (admissible(p, i, j, sq, sk)) z += exp(s[j] - m);",
                         "if (admissible(p, i, j, sq, sk)) z += exp(m - s[j]);"),
    "no_normalisation": ("const double pij = exp(s[j] - m) / z;", "const double pij = exp(s[j] - m);"),
    "masked_lse_zero": ("*lse = -INFINITY;\n    return;", "*lse = 0.0;\n    return;"),
    "v_stride_uses_d": ("const int64_t vbase = ((k0 + j) * p->hkv + g) * (int64_t)p->dv;",
                        "const int64_t vbase = ((k0 + j) * p->hkv + g) * (int64_t)p->d;"),
    "k_uses_query_head": ("const int64_t kbase = ((k0 + j) * p->hkv + g) * (int64_t)p->d;",
                          "const int64_t kbase = ((k0 + j) * p->hkv + (h % p->hkv)) * (int64_t)p->d;"),
    "key_range_short": ("for (int j = 0; j < sk; ++j) {\n    if (!admissible(p, i, j, sq, sk)) continue;\n    const int64_t kbase",
                        "for (int j = 0; j < sk - 1; ++j) {\n    if (!admissible(p, i, j, sq, sk)) continue;\n    const int64_t kbase"),
    "e4m3_bias_8": ("mag = ldexp(1.0 + (double)mant / 8.0, expo - 7);", "mag = ldexp(1.0 + (double)mant / 8.0, expo - 8);"),
    "e4m3_subnormal": ("mag = ldexp((double)mant / 8.0, 1 - 7);", "mag = ldexp((double)mant / 8.0, -7);"),
    "bf16_shift": ("uint32_t u = (uint32_t)bits << 16;", "uint32_t u = (uint32_t)bits << 15;"),
    "descale_v_uses_q": ("p->dvs = descales[2];", "p->dvs = descales[0];"),
    "varlen_k_offset": ("*k0 = p->cu[p->batch + 1 + b];", "*k0 = p->cu[b];"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutated = tmp_path / "fa_oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-o", str(lib),
                    str(mutated), "-lm"], check=True)
    handle = oracle.swap_library(str(lib))
    caught = []
    try:
        for pin in oracle_pins.ALL_PINS:
            try:
                pin()
            except (AssertionError, ValueError):
                caught.append(pin.__name__)
    finally:
        oracle.restore_library(handle)
    assert caught, f"no pin detects the planted mistake '{name}'"
