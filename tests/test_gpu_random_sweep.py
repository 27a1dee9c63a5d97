"""GPU parity on a seeded random sweep of shapes: batch, head ratio, fixed or packed
(varlen) lengths including empty sequences, head_dim, causal masking, bf16 or e4m3 inputs,
and the schedule (automatic or forced) and exp2 offload, drawn together, so that
combinations the hand-picked shapes leave out are checked against the fp64 oracle, whole
output, into NaN-filled buffers (an element never written fails)."""
import numpy as np
import pytest

import fa_inputs
from parity import check_written, compare, gpu_run, oracle_full, say

pytestmark = pytest.mark.gpu

N_CASES = 128


def draw_case(i: int):
    rng = np.random.default_rng(9000 + i)
    dtype = "e4m3" if rng.random() < 0.3 else "bf16"
    d = int(rng.choice([64, 128]))
    group = int(rng.choice([1, 2, 3, 4, 8]))
    hkv = int(rng.integers(1, 4))
    hq = group * hkv
    causal = bool(rng.random() < 0.5)
    if rng.random() < 0.4:  # packed varlen batch; a length may be 0
        nseq = int(rng.integers(1, 6))
        lengths = []
        for _ in range(nseq):
            sq = int(rng.integers(0, 601)) if rng.random() > 0.1 else 0
            sk = int(rng.integers(0, 701)) if rng.random() > 0.1 else 0
            lengths.append((sq, sk))
        if sum(a for a, _ in lengths) == 0:
            lengths[0] = (int(rng.integers(1, 300)), lengths[0][1])
        shape = dict(lengths=lengths)
        desc = f"varlen{lengths}"
    else:
        b = int(rng.integers(1, 4))
        sq, sk = int(rng.integers(1, 601)), int(rng.integers(1, 701))
        shape = dict(batch=b, seqlen_q=sq, seqlen_k=sk)
        desc = f"b{b}_sq{sq}_sk{sk}"
    schedule = int(rng.choice([0, 0, 1, 2, 3, 4, 5]))
    offload = int(rng.choice([0, 0, 0, 4, 8]))
    return dict(dtype=dtype, d=d, hq=hq, hkv=hkv, causal=causal, shape=shape, schedule=schedule,
                offload=offload, name=f"sweep{i}_{dtype}_d{d}_hq{hq}_hkv{hkv}_c{int(causal)}_"
                                      f"{desc}_s{schedule}_x{offload}")


@pytest.mark.parametrize("i", range(N_CASES), ids=[f"case{i}" for i in range(N_CASES)])
def test_random_sweep(i):
    import exact_attention_forward_fa_amd as fa

    c = draw_case(i)
    sh = c["shape"]
    if "lengths" in sh:
        w = fa_inputs.make(0, c["hq"], c["hkv"], 0, 0, c["d"], causal=c["causal"], seed=9000 + i,
                           dtype=c["dtype"], lengths=sh["lengths"], name=c["name"])
    else:
        w = fa_inputs.make(sh["batch"], c["hq"], c["hkv"], sh["seqlen_q"], sh["seqlen_k"], c["d"],
                           causal=c["causal"], seed=9000 + i, dtype=c["dtype"], name=c["name"])
    say(f"[sweep] {c['name']}")
    fa.fa_set_schedule(c["schedule"])
    fa.fa_set_exp2_offload(c["offload"])
    try:
        o, lse = gpu_run(w)
    finally:
        fa.fa_set_schedule(0)
        fa.fa_set_exp2_offload(0)
    check_written(w, o, lse)
    ro, rl = oracle_full(w)
    compare(o, lse, ro, rl, w.dtype, w.name)
