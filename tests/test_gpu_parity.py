"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.  bf16: max|dO| <= 2e-2, max|dLSE| <= 1e-3; fp8 e4m3:
5e-2 / 5e-3; rows with no admissible key exactly O = 0, LSE = -inf."""
import numpy as np
import pytest
import torch

import fa_inputs
from parity import (check_written, compare, gather_rows, gpu_run, nan_outputs, oracle_full,
                    oracle_rows, say, tile_rows, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(params=[1, 2, 3, 4, 5], ids=["sched1", "sched2", "sched3", "sched4", "sched5"])
def schedule(request):
    """Force each bf16 schedule (1: one query tile per wave; 2: two; 3: 8-wave ping-pong,
    where heads_q / heads_kv is even (two heads per workgroup) or 1 (two adjacent query tiles
    of one head); 4: decode, where heads_q / heads_kv * seqlen_q <= 32; 5: schedule 3's items
    on resident workgroups (persistent launch, next item's query rows prefetched), where 3
    applies; else 1) for the test."""
    import exact_attention_forward_fa_amd as fa

    fa.fa_set_schedule(request.param)
    yield request.param
    fa.fa_set_schedule(0)


def full_check(w):
    o, lse = gpu_run(w)
    ro, rl = oracle_full(w)
    return compare(o, lse, ro, rl, w.dtype, w.name)


def sampled_check(w):
    """Full-size workloads: the whole output is checked for unwritten elements (NaN pre-fill)
    and exact fully masked rows, and rows of every (sequence, head, query tile, 32-row slice)
    are compared with the oracle."""
    tensors = to_device(w)
    o, lse = gpu_run(w, tensors)
    check_written(w, o, lse)
    rows = tile_rows(w, seed=w.seed)
    say(f"[oracle] {len(rows)} rows of {w.name} (every tile and 32-row slice of every head)")
    ro, rl = oracle_rows(w, rows)
    og, lg = gather_rows(w, o, lse, rows)
    compare(og, lg, ro, rl, w.dtype, w.name + " (rows of every tile)")
    return o, lse


# ---------------------------------------------------------------- named workloads

def test_tiny_noncausal_d64():
    full_check(fa_inputs.workload("tiny_b1_h2_s256_d64"))


@pytest.mark.parametrize("name", ["mha_b4_h16_s1024_d128", "mha_causal_b4_h16_s1024_d128"])
def test_mha_1024(name, schedule):
    full_check(fa_inputs.workload(name))


def test_gqa_causal_8192_sampled():
    sampled_check(fa_inputs.workload("gqa_causal_b2_hq32_hkv8_s8192_d128"))


@pytest.mark.timeout(900)
def test_gqa_causal_8192_full_oracle():
    """The bench workload in the launch configuration bench.py times, every output element
    against the oracle (524 288 rows x 128 dims, about 1.1e12 fp64 flops: 1-2 minutes on the
    host's cores), in chunks of 32 768 rows with a progress line each."""
    w = fa_inputs.workload("gqa_causal_b2_hq32_hkv8_s8192_d128")
    o, lse = gpu_run(w)
    check_written(w, o, lse)
    rows = np.array([(b, h, i) for b in range(w.batch) for h in range(w.heads_q)
                     for i in range(w.seqlen_q)], dtype=np.int32)
    eo = el = 0.0
    chunk = 32768
    for c0 in range(0, rows.shape[0], chunk):
        part = rows[c0:c0 + chunk]
        ro, rl = oracle_rows(w, part)
        og, lg = gather_rows(w, o, lse, [tuple(r) for r in part])
        a, b = compare(og, lg, ro, rl, w.dtype, f"{w.name} rows {c0}..{c0 + part.shape[0] - 1}")
        eo, el = max(eo, a), max(el, b)
    say(f"[parity] {w.name} whole output: max|dO|={eo:.3e} max|dLSE|={el:.3e}")


def test_gqa_causal_8192_sampled_one_tile_per_wave():
    """The same workload through schedule 1 (the planner picks the ping-pong for it)."""
    import exact_attention_forward_fa_amd as fa

    w = fa_inputs.workload("gqa_causal_b2_hq32_hkv8_s8192_d128")
    fa.fa_set_schedule(1)
    try:
        sampled_check(w)
    finally:
        fa.fa_set_schedule(0)


def test_varlen_causal_sampled():
    """Every row that sees no key (sk < sq, i < sq - sk) exactly zero / -inf, every other row
    written, rows of every tile against the oracle."""
    w = fa_inputs.workload("varlen_causal_18seq_h16_d128")
    assert any(sk < sq for sq, sk in w.lengths)
    sampled_check(w)


@pytest.mark.parametrize("shape", [(3, 8, 4, 300, 300, True), (9, 2, 1, 200, 330, False),
                                   (1, 8, 1, 520, 520, True), (2, 4, 2, 130, 260, True)])
def test_grid_layouts(shape, schedule):
    """Pair counts that are not whole rounds of the 8 XCDs: 12 (one dealt round, 4 pairs spread),
    9 (one round, 1 spread), 1 and 4 (all spread), under every schedule."""
    b, hq, hkv, sq, sk, causal = shape
    w = fa_inputs.make(b, hq, hkv, sq, sk, 128, causal=causal, seed=sq + 3 * hq + 7 * b,
                       name=f"grid_b{b}_hq{hq}_hkv{hkv}_{sq}x{sk}_c{int(causal)}")
    full_check(w)


def test_varlen_equals_per_sequence_calls(schedule):
    """Packed varlen output equals separate fixed-length calls, bit for bit (same tiling)."""
    lens = [(300, 517), (1, 64), (129, 100), (64, 0), (0, 40), (255, 256), (70, 700)]
    w = fa_inputs.make(0, 4, 2, 0, 0, 128, causal=True, seed=50, lengths=lens, name="varlen_small")
    o, lse = gpu_run(w)
    ro, rl = oracle_full(w)
    compare(o, lse, ro, rl, "bf16", w.name)
    if schedule == 4:
        return  # decode applies per call: the (1, 64) call takes it, the packed call cannot
    cu = w.cu_seqlens
    nb = len(lens)
    for b, (sq, sk) in enumerate(lens):
        if sq == 0:
            continue
        q0, k0 = int(cu[b]), int(cu[nb + 1 + b])
        wb = fa_inputs.make(1, 4, 2, sq, sk, 128, causal=True, seed=50, name=f"seq{b}")
        wb.q, wb.k, wb.v = w.q[q0:q0 + sq], w.k[k0:k0 + sk], w.v[k0:k0 + sk]
        if sk == 0:
            wb.k = torch.zeros((0, 2, 128), dtype=torch.bfloat16)
            wb.v = torch.zeros((0, 2, 128), dtype=torch.bfloat16)
        ob, lb = gpu_run(wb)
        assert np.array_equal(ob, o[q0:q0 + sq]), f"sequence {b}: O differs from packed call"
        assert np.array_equal(lb, lse[:, q0:q0 + sq]), f"sequence {b}: LSE differs from packed call"


# ----------------------------------------------------------------- edge cases

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 4, 4, 300, 300), (1, 8, 2, 200, 517), (1, 4, 1, 517, 200),
                                   (3, 2, 2, 1, 1), (1, 2, 2, 1, 333), (1, 32, 1, 130, 130),
                                   (1, 2, 2, 600, 250), (2, 3, 3, 250, 640), (1, 6, 2, 300, 520)])
def test_ragged_shapes(shape, causal, d, schedule):
    b, hq, hkv, sq, sk = shape
    w = fa_inputs.make(b, hq, hkv, sq, sk, d, causal=causal, seed=sq * 7 + sk + d,
                       name=f"ragged_b{b}_hq{hq}_hkv{hkv}_sq{sq}_sk{sk}_d{d}_c{int(causal)}_s{schedule}")
    full_check(w)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 8, 2, 1, 1000), (1, 16, 4, 8, 777), (3, 16, 2, 4, 100),
                                   (1, 4, 2, 16, 33), (2, 2, 2, 32, 5), (1, 8, 8, 1, 4096)])
def test_decode_shapes(shape, causal, d):
    """The decode schedule (all (head, row) pairs of a KV group in one 32-column tile, the key
    range split over the waves) as the planner picks it: key counts that leave some waves with
    no block or a partial one, causal rows that see few keys, groups of 1 to 8."""
    import exact_attention_forward_fa_amd as fa

    b, hq, hkv, sq, sk = shape
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, b, hq, hkv, sq, sk, False, d, d, causal).schedule == 4
    w = fa_inputs.make(b, hq, hkv, sq, sk, d, causal=causal, seed=sq * 11 + sk + d,
                       name=f"decode_b{b}_hq{hq}_hkv{hkv}_sq{sq}_sk{sk}_d{d}_c{int(causal)}")
    full_check(w)


def test_decode_varlen():
    """Varlen decode: per-sequence query rows 0 .. 4 (group 4 x 4 rows = 16 columns), key counts
    from 0 to 3000, causal."""
    import exact_attention_forward_fa_amd as fa

    lens = [(1, 3000), (4, 37), (0, 500), (3, 0), (2, 1), (4, 2049)]
    w = fa_inputs.make(0, 8, 2, 0, 0, 128, causal=True, seed=70, lengths=lens, name="decode_varlen")
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, len(lens), 8, 2, 4, 3000, True, 128, 128,
                          True).schedule == 4
    full_check(w)


@pytest.mark.parametrize("every", [4, 8])
@pytest.mark.parametrize("shape", [(2, 4, 2, 300, 300, 128, True), (1, 8, 2, 200, 517, 64, False),
                                   (1, 4, 2, 517, 200, 128, True)])
def test_exp2_offload(shape, every):
    """Ping-pong schedule with every 4th / 8th exponential on the FMA polynomial: same
    tolerances against the oracle."""
    import exact_attention_forward_fa_amd as fa

    b, hq, hkv, sq, sk, d, causal = shape
    w = fa_inputs.make(b, hq, hkv, sq, sk, d, causal=causal, seed=sq + sk + every,
                       name=f"exp2_offload{every}_b{b}_hq{hq}_hkv{hkv}_sq{sq}_sk{sk}_d{d}")
    fa.fa_set_schedule(3)  # small grids default to schedule 1
    fa.fa_set_exp2_offload(every)
    try:
        assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, b, hq, hkv, sq, sk, False, d, d, causal).schedule == 3
        full_check(w)
    finally:
        fa.fa_set_exp2_offload(0)
        fa.fa_set_schedule(0)


def test_exp2_offload_large_q():
    """Peaked softmax rows (Q x 50): the polynomial's relative error must not show in LSE."""
    import exact_attention_forward_fa_amd as fa

    w = fa_inputs.make(1, 4, 2, 256, 256, 128, causal=True, seed=65, q_mult=50.0,
                       name="exp2_offload_q_x50")
    fa.fa_set_schedule(3)
    fa.fa_set_exp2_offload(4)
    try:
        full_check(w)
    finally:
        fa.fa_set_exp2_offload(0)
        fa.fa_set_schedule(0)


@pytest.mark.parametrize("shape", [(8, 8, 2, 1, 4096), (4, 16, 4, 3, 2500)])
def test_pingpong_short_steps_repeat(shape):
    """The ping-pong schedule on shapes whose steps are short (one or a few query rows, many
    key blocks): each step's K/V loads must be complete before the next step's barrier, or
    waves read half-written blocks.  Five calls, each against the oracle and all bit-identical."""
    import exact_attention_forward_fa_amd as fa

    b, hq, hkv, sq, sk = shape
    w = fa_inputs.make(b, hq, hkv, sq, sk, 128, causal=True, seed=sq + sk,
                       name=f"pp_short_b{b}_hq{hq}_hkv{hkv}_sq{sq}_sk{sk}")
    fa.fa_set_schedule(3)
    try:
        assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, b, hq, hkv, sq, sk, False, 128, 128,
                              True).schedule == 3
        t = to_device(w)
        ro, rl = oracle_full(w)
        first = None
        for rep in range(5):
            o, lse = gpu_run(w, t)
            compare(o, lse, ro, rl, "bf16", f"{w.name}_rep{rep}")
            if first is None:
                first = (o, lse)
            else:
                assert np.array_equal(o, first[0]) and np.array_equal(lse, first[1])
    finally:
        fa.fa_set_schedule(0)


def test_seqlen_k_zero():
    w = fa_inputs.make(2, 2, 2, 100, 0, 128, causal=False, seed=60, name="sk0")
    o, lse = gpu_run(w)
    assert np.all(o == 0.0) and np.all(lse == -np.inf)


def test_large_q_magnitude(schedule):
    w = fa_inputs.make(1, 4, 4, 256, 256, 128, causal=True, seed=61, q_mult=50.0, name="q_x50")
    full_check(w)


def key_offset_pattern(pattern: str, sk: int) -> np.ndarray:
    """Per-key score offsets in base-2 units.  Blocks of keys are visited from the last key
    to the first, so 'jumpG' raises the running maximum of every row that sees keys on both
    sides of sk/2 by G at once, 'rampA' by A every 64 keys, 'fall' lets it fall (scores of
    later-visited keys underflow), 'saw' alternates high and low 64-key blocks."""
    j = np.arange(sk, dtype=np.float64)
    kind, amount = pattern.rstrip("0123456789."), pattern[len(pattern.rstrip("0123456789.")):]
    a = float(amount) if amount else 0.0
    if kind == "jump":
        return np.where(j < sk // 2, a, 0.0)
    if kind == "ramp":
        return a * (sk - 1 - j) / 64.0
    if kind == "fall":
        return 6.0 * j / 64.0
    if kind == "saw":
        return np.where((j // 64) % 2 == 0, 12.0, 0.0)
    raise ValueError(pattern)


GROWTH_PATTERNS = ["jump3", "jump7.9", "jump8.1", "jump30", "ramp3", "ramp10", "fall", "saw"]


@pytest.mark.parametrize("pattern", GROWTH_PATTERNS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 4, 2, 520, 520), (1, 8, 2, 4, 1000)], ids=["prefill", "decode"])
def test_running_max_growth(shape, causal, pattern, schedule):
    """Scores whose row maximum grows by less than, about and more than the lazy-rescale bound
    (2^8) as key blocks are visited, in steps and ramps, or falls: the exponentials taken
    against a stale maximum must be redone against the block maximum exactly when needed."""
    b, hq, hkv, sq, sk = shape
    w = fa_inputs.make(b, hq, hkv, sq, sk, 128, causal=causal, seed=80 + GROWTH_PATTERNS.index(pattern),
                       key_offsets=key_offset_pattern(pattern, sk),
                       name=f"growth_{pattern}_sq{sq}_sk{sk}_c{int(causal)}")
    full_check(w)


# The fp8 matrix instruction sums the products of the score's dot product to about 14 bits
# relative to their magnitude (measured alike on the scaled f8f6f4 form the kernel uses and on
# the unscaled 32x32x16 fp8 form: the same 5.9e-3), so a row's LSE, which equals its largest
# scores, carries an error of about 1e-4 of them: inside the fp8 LSE tolerance (5e-3) up to
# scores of about 50.  The causal steep ramp reaches 58.7.
FP8_SCORE_PRECISION = ("fp8 MFMA accumulation keeps ~14 bits relative to the scores: LSE error "
                       "5.9e-3 at |LSE| = 58.7 (causal ramp10, 520 keys), above 5e-3; "
                       "fa_set_fp8_exact_scores(1) meets it (test_fp8_exact_scores_*)")


@pytest.mark.parametrize("pattern", GROWTH_PATTERNS)
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_running_max_growth(causal, pattern, request):
    """As above for e4m3, over 520 keys."""
    if causal and pattern == "ramp10":
        request.applymarker(pytest.mark.xfail(strict=True, reason=FP8_SCORE_PRECISION))
    s = 520
    w = fa_inputs.make(1, 4, 2, s, s, 128, causal=causal, seed=90 + GROWTH_PATTERNS.index(pattern),
                       dtype="e4m3", key_offsets=key_offset_pattern(pattern, s),
                       name=f"fp8_growth_{pattern}_s{s}_c{int(causal)}")
    full_check(w)


def test_fp8_large_q_magnitude():
    """e4m3 counterpart of test_large_q_magnitude: Q x 50 (the q descale grows 50-fold), rows
    dominated by one key."""
    w = fa_inputs.make(1, 4, 2, 256, 256, 128, causal=True, seed=61, q_mult=50.0, dtype="e4m3",
                       name="fp8_q_x50")
    full_check(w)


def test_fp8_moderately_peaked_rows():
    """e4m3 with Q x 20: rows whose weight is spread over a few keys, where the rounding of P to
    e4m3 (3 mantissa bits) for the P V product matters most."""
    w = fa_inputs.make(1, 4, 2, 512, 512, 128, causal=True, seed=62, q_mult=20.0, dtype="e4m3",
                       name="fp8_q_x20")
    full_check(w)


def test_gqa_equals_repeated_mha_on_gpu(schedule):
    w = fa_inputs.make(1, 8, 2, 257, 257, 128, causal=True, seed=62, name="gqa")
    o1, l1 = gpu_run(w)
    w2 = fa_inputs.make(1, 8, 2, 257, 257, 128, causal=True, seed=62, name="gqa_as_mha")
    w2.k = w.k.repeat_interleave(4, dim=1).contiguous()
    w2.v = w.v.repeat_interleave(4, dim=1).contiguous()
    w2.heads_kv = 8
    o2, l2 = gpu_run(w2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_deterministic(schedule):
    w = fa_inputs.make(2, 8, 2, 700, 700, 128, causal=True, seed=63, name="det")
    t = to_device(w)
    o1, l1 = gpu_run(w, t)
    o2, l2 = gpu_run(w, t)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_no_writes_outside_outputs(schedule):
    """Outputs carved from larger buffers filled with a sentinel: nothing past the ends changes."""
    import exact_attention_forward_fa_amd as fa

    lens = [(130, 70), (5, 300), (257, 257)]
    w = fa_inputs.make(0, 4, 2, 0, 0, 128, causal=True, seed=64, lengths=lens, name="canary")
    q, k, v, cu, _ = to_device(w)
    pad = 4096
    obuf = torch.full((w.total_q * 4 * 128 + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((4 * w.total_q + 2 * pad,), 7.0, dtype=torch.float32, device="cuda")
    o = obuf[pad:pad + w.total_q * 4 * 128].view(w.total_q, 4, 128)
    lse = lbuf[pad:pad + 4 * w.total_q].view(4, w.total_q)
    say("[gpu] fa_fwd canary")
    fa.forward(q, k, v, causal=True, softmax_scale=w.softmax_scale, cu_seqlens=cu,
               max_seqlen_q=w.seqlen_q, max_seqlen_k=w.seqlen_k, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(obuf[:pad] == 7.0) and torch.all(obuf[-pad:] == 7.0)
    assert torch.all(lbuf[:pad] == 7.0) and torch.all(lbuf[-pad:] == 7.0)
    ro, rl = oracle_full(w)
    compare(o.float().cpu().double().numpy(), lse.cpu().double().numpy(), ro, rl, "bf16", w.name)


# ------------------------------------------------------------------- fp8 e4m3

def test_fp8_causal_16384_sampled():
    sampled_check(fa_inputs.workload("fp8_causal_b1_h32_s16384_d128"))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 4, 4, 300, 300), (1, 8, 2, 200, 517), (1, 4, 1, 517, 200),
                                   (1, 2, 2, 1, 1)])
def test_fp8_ragged_shapes(shape, causal, d):
    b, hq, hkv, sq, sk = shape
    w = fa_inputs.make(b, hq, hkv, sq, sk, d, causal=causal, seed=sq * 5 + sk + d + 1, dtype="e4m3",
                       name=f"fp8_b{b}_hq{hq}_hkv{hkv}_sq{sq}_sk{sk}_d{d}_c{int(causal)}")
    full_check(w)


def test_fp8_varlen():
    lens = [(300, 517), (1, 64), (129, 100), (64, 0), (0, 40), (255, 256)]
    w = fa_inputs.make(0, 4, 2, 0, 0, 128, causal=True, seed=70, lengths=lens, dtype="e4m3",
                       name="fp8_varlen_small")
    full_check(w)


# ---------------------------------------- fp8 with exact scores (opt-in switch)


@pytest.fixture
def fp8_exact():
    """fa_set_fp8_exact_scores(1) for the test: Q K^T on the bf16 matrix instruction from Q and
    K widened exactly from e4m3."""
    import exact_attention_forward_fa_amd as fa

    fa.fa_set_fp8_exact_scores(1)
    yield
    fa.fa_set_fp8_exact_scores(0)


@pytest.mark.parametrize("pattern", GROWTH_PATTERNS)
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_exact_scores_running_max_growth(causal, pattern, fp8_exact):
    """The growth patterns of test_fp8_running_max_growth with exact scores: all within the
    fp8 tolerance, the causal steep ramp (|LSE| = 58.7) included."""
    s = 520
    w = fa_inputs.make(1, 4, 2, s, s, 128, causal=causal, seed=90 + GROWTH_PATTERNS.index(pattern),
                       dtype="e4m3", key_offsets=key_offset_pattern(pattern, s),
                       name=f"fp8x_growth_{pattern}_s{s}_c{int(causal)}")
    full_check(w)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 4, 4, 300, 300), (1, 8, 2, 200, 517), (1, 4, 1, 517, 200),
                                   (1, 2, 2, 1, 1)])
def test_fp8_exact_scores_ragged_shapes(shape, causal, d, fp8_exact):
    b, hq, hkv, sq, sk = shape
    w = fa_inputs.make(b, hq, hkv, sq, sk, d, causal=causal, seed=sq * 5 + sk + d + 1, dtype="e4m3",
                       name=f"fp8x_b{b}_hq{hq}_hkv{hkv}_sq{sq}_sk{sk}_d{d}_c{int(causal)}")
    full_check(w)


def test_fp8_exact_scores_large_q_and_varlen(fp8_exact):
    full_check(fa_inputs.make(1, 4, 2, 256, 256, 128, causal=True, seed=61, q_mult=50.0,
                              dtype="e4m3", name="fp8x_q_x50"))
    full_check(fa_inputs.make(1, 4, 2, 512, 512, 128, causal=True, seed=62, q_mult=20.0,
                              dtype="e4m3", name="fp8x_q_x20"))
    lens = [(300, 517), (1, 64), (129, 100), (64, 0), (0, 40), (255, 256)]
    full_check(fa_inputs.make(0, 4, 2, 0, 0, 128, causal=True, seed=70, lengths=lens,
                              dtype="e4m3", name="fp8x_varlen_small"))


def test_fp8_exact_scores_16384_sampled(fp8_exact):
    """The fp8 workload with exact scores, every tile sampled against the oracle."""
    sampled_check(fa_inputs.workload("fp8_causal_b1_h32_s16384_d128"))


# ------------------------------------------------------- KV cache (AppendKV)

def kvcache_check(case, name):
    """fa_fwd_kvcache against the oracle: the caches afterwards bit for bit, O/LSE to the
    tolerance of the input type."""
    import oracle

    import exact_attention_forward_fa_amd as fa

    def dev(t):
        return None if t is None else t.cuda()

    q, kc, vc, kn, vn = (dev(case.q), dev(case.k_cache), dev(case.v_cache), dev(case.k_new),
                         dev(case.v_new))
    lens = torch.from_numpy(case.cache_seqlens).cuda()
    ds = None if case.descales is None else torch.from_numpy(case.descales).cuda()
    say(f"[gpu] fa_fwd_kvcache {name}")
    b, sq, hq, d = case.q.shape
    o = torch.full((b * sq, hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((hq, b * sq), float("nan"), dtype=torch.float32, device="cuda")
    fa.forward_kvcache(q, kc, vc, lens, kn, vn, causal=case.causal,
                       softmax_scale=case.softmax_scale, descales=ds, out=o, lse=lse)
    torch.cuda.synchronize()
    dt = oracle.BF16 if case.dtype == "bf16" else oracle.E4M3
    ro, rl, rk, rv = oracle.attention_kvcache(case.q, case.k_cache, case.v_cache, case.k_new,
                                              case.v_new, case.cache_seqlens,
                                              softmax_scale=case.softmax_scale, causal=case.causal,
                                              descales=case.descales, dtype=dt)

    def bits(t):
        t = t.cpu()
        return t.view(torch.int16).numpy().view(np.uint16) if case.dtype == "bf16" else t.numpy()

    assert np.array_equal(bits(kc), rk), f"{name}: K cache after the append"
    assert np.array_equal(bits(vc), rv), f"{name}: V cache after the append"
    compare(o.float().cpu().double().numpy(), lse.cpu().double().numpy(), ro, rl, case.dtype, name)
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
def test_kvcache_decode_gqa(causal, schedule):
    """One new token per sequence, cache lengths from empty to exactly full."""
    case = fa_inputs.make_kvcache(4, 1, 1, 4096, [0, 1000, 4095, 2047], 8, 2, 128, causal=causal,
                                  seed=80)
    kvcache_check(case, f"kv_decode_c{int(causal)}_s{schedule}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_kvcache_prefill_chunk(causal, d, schedule):
    """A 300-row chunk appended behind a prefix; the second sequence overflows the cache, so
    its last new rows are dropped and its length clamps to the capacity."""
    case = fa_inputs.make_kvcache(2, 300, 300, 2048, [100, 1900], 4, 4, d, causal=causal,
                                  seed=81 + d)
    kvcache_check(case, f"kv_chunk_d{d}_c{int(causal)}_s{schedule}")


def test_kvcache_decode_bench_workload():
    """The KV-cache decode step bench.py times, at full size (32 sequences, 8192-row caches,
    32 query / 8 KV heads), in the configuration it times (the planner's decode schedule):
    caches bit for bit, every output row against the oracle."""
    import bench
    import exact_attention_forward_fa_amd as fa

    name = "kvcache_decode_b32_hq32_hkv8_c8192_d128"
    cfg = bench.KVCACHE_WORKLOADS[name]
    b, hq, hkv, cap, d = cfg["batch"], cfg["heads_q"], cfg["heads_kv"], cfg["capacity"], cfg["head_dim"]
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, b, hq, hkv, 1, cap, False, d, d, True).schedule == 4
    case = fa_inputs.make_kvcache(b, 1, 1, cap, [cap - 1] * b, hq, hkv, d, causal=True,
                                  seed=cfg["seed"])
    kvcache_check(case, name)


def test_kvcache_no_new_rows():
    case = fa_inputs.make_kvcache(3, 17, 0, 512, [0, 200, 512], 4, 1, 128, causal=True, seed=84)
    kvcache_check(case, "kv_no_new_rows")


def test_kvcache_equals_packed_varlen_call():
    """The cached forward reads exactly the appended prefix: same answer as fa_fwd on the
    packed (prefix + new) sequences, bit for bit."""
    import exact_attention_forward_fa_amd as fa

    case = fa_inputs.make_kvcache(3, 64, 64, 1024, [10, 500, 960], 8, 2, 128, causal=True, seed=85)
    o, lse = kvcache_check(case, "kv_vs_varlen")
    used = [min(int(n) + 64, 1024) for n in case.cache_seqlens]
    import oracle

    kc, vc, _ = oracle.append_kv(case.k_cache, case.v_cache, case.k_new, case.v_new,
                                 case.cache_seqlens)
    kp = torch.from_numpy(np.concatenate([kc[b, :used[b]] for b in range(3)])).view(torch.bfloat16)
    vp = torch.from_numpy(np.concatenate([vc[b, :used[b]] for b in range(3)])).view(torch.bfloat16)
    cu = np.concatenate([np.arange(4) * 64, np.concatenate([[0], np.cumsum(used)])]).astype(np.int32)
    o2, l2 = fa.forward(case.q.reshape(3 * 64, 8, 128).cuda(), kp.cuda(), vp.cuda(), causal=True,
                        softmax_scale=case.softmax_scale, cu_seqlens=torch.from_numpy(cu).cuda(),
                        max_seqlen_q=64, max_seqlen_k=max(used))
    torch.cuda.synchronize()
    assert torch.equal(o.cpu(), o2.cpu()) and torch.equal(lse.cpu(), l2.cpu())


def test_kvcache_fp8():
    case = fa_inputs.make_kvcache(2, 130, 70, 1024, [0, 400], 4, 2, 128, causal=True, seed=86,
                                  dtype="e4m3")
    kvcache_check(case, "kv_fp8")


def test_kvcache_fp8_exact_scores(fp8_exact):
    """The KV-cache entry point takes the fp8 exact-score switch as fa_fwd does."""
    case = fa_inputs.make_kvcache(2, 130, 70, 1024, [0, 400], 4, 2, 128, causal=True, seed=86,
                                  dtype="e4m3")
    kvcache_check(case, "kv_fp8_exact")


# ------------------------------------------------------------ graph capture

@pytest.mark.parametrize("case", ["gqa_pingpong", "mha_pairs", "varlen", "fp8", "decode"])
def test_graph_capture_replays(case):
    """fa_fwd allocates nothing and launches only kernels on the caller's stream, so it can be
    captured into a HIP graph: every replay (with other work on the device between replays)
    gives the eager call's O and LSE bit for bit."""
    import exact_attention_forward_fa_amd as fa

    if case == "gqa_pingpong":
        w = fa_inputs.make(2, 8, 2, 300, 517, 128, causal=True, seed=71, name="graph_gqa")
    elif case == "mha_pairs":
        w = fa_inputs.make(2, 3, 3, 600, 600, 64, causal=True, seed=72, name="graph_mha")
    elif case == "varlen":
        w = fa_inputs.make(0, 4, 2, 0, 0, 128, causal=True, seed=73,
                           lengths=[(300, 517), (1, 64), (129, 100), (255, 256)], name="graph_varlen")
    elif case == "fp8":
        w = fa_inputs.make(1, 4, 4, 260, 260, 128, causal=True, seed=74, dtype="e4m3", name="graph_fp8")
    else:
        w = fa_inputs.make(4, 16, 4, 1, 1000, 128, causal=True, seed=75, name="graph_decode")
    q, k, v, cu, ds = to_device(w)
    total_q = q.shape[0]
    hq, dv = w.heads_q, w.head_dim_v

    def call(o, lse):
        fa.fa_fwd(q, k, v, o, lse, w.batch, hq, w.heads_kv, w.seqlen_q, w.seqlen_k, cu,
                  w.head_dim, dv, w.softmax_scale, int(w.causal), ds)

    say(f"[gpu] graph capture {w.name}")
    o_ref = torch.empty(total_q, hq, dv, dtype=torch.bfloat16, device="cuda")
    lse_ref = torch.empty(hq, total_q, dtype=torch.float32, device="cuda")
    call(o_ref, lse_ref)
    o = torch.empty_like(o_ref)
    lse = torch.empty_like(lse_ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(o, lse)  # warm-up on the capture stream, as torch's capture expects
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(o, lse)
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()  # other work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), f"replay {rep}: O differs"
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32)), f"replay {rep}: LSE differs"


# ----------------------------------------------------------------- maximum sizes

def _repeat_keys(w, reps):
    """K and V of ``w`` (one sequence of P keys) repeated ``reps`` times along the keys, on
    the GPU.  Every key then occurs reps times with the same score, so the softmax weights
    are those over the P keys: O is unchanged and LSE grows by exactly ln(reps)."""
    return (w.k.to("cuda").repeat(reps, 1, 1).contiguous(),
            w.v.to("cuda").repeat(reps, 1, 1).contiguous())


@pytest.mark.parametrize("sq,causal", [(64, False), (1, True)])
def test_longest_supported_key_range(sq, causal, schedule):
    """One sequence whose K (and V) is just under the 2 GiB the kernels address per sequence:
    1 KV head, D = 128, bf16, 1021 x 8216 = 8 388 536 keys (the largest multiple of the
    1021-key period below 2^31 / 256).  The reference is the oracle over the 1021 keys, with
    LSE + ln(8216); causal with one query row (bottom-right) sees every key."""
    import exact_attention_forward_fa_amd as fa

    period, reps = 1021, 8216
    assert period * reps * 128 * 2 < (1 << 31) <= period * (reps + 1) * 128 * 2
    w = fa_inputs.make(1, 2, 1, sq, period, 128, causal=False, seed=70 + sq,
                       name=f"keys_{period}x{reps}_sq{sq}_c{int(causal)}_s{schedule}")
    ro, rl = oracle_full(w)
    q = w.q.to("cuda")
    k, v = _repeat_keys(w, reps)
    say(f"[gpu] fa_fwd {w.name}: hq=2 hkv=1 sq={sq} sk={period * reps} d=128 causal={causal}")
    o, lse = nan_outputs(w)
    fa.forward(q, k, v, causal=causal, softmax_scale=w.softmax_scale, max_seqlen_q=sq,
               max_seqlen_k=period * reps, batch=1, out=o, lse=lse)
    torch.cuda.synchronize()
    del k, v
    compare(o.float().cpu().double().numpy(), lse.cpu().double().numpy(), ro,
            rl + np.log(reps), "bf16", w.name)


def test_fp8_longest_supported_key_range():
    """As above for e4m3 (one byte per element): 1021 x 16 432 = 16 777 072 keys."""
    import exact_attention_forward_fa_amd as fa

    period, reps = 1021, 16432
    assert period * reps * 128 < (1 << 31) <= period * (reps + 1) * 128
    w = fa_inputs.make(1, 2, 1, 64, period, 128, causal=False, seed=72, dtype="e4m3",
                       name=f"fp8_keys_{period}x{reps}")
    ro, rl = oracle_full(w)
    q = w.q.to("cuda")
    k, v = _repeat_keys(w, reps)
    ds = torch.from_numpy(w.descales).to("cuda")
    say(f"[gpu] fa_fwd {w.name}: hq=2 hkv=1 sq=64 sk={period * reps} d=128 fp8")
    o, lse = nan_outputs(w)
    fa.forward(q, k, v, causal=False, softmax_scale=w.softmax_scale, max_seqlen_q=64,
               max_seqlen_k=period * reps, descales=ds, batch=1, out=o, lse=lse)
    torch.cuda.synchronize()
    del k, v
    compare(o.float().cpu().double().numpy(), lse.cpu().double().numpy(), ro,
            rl + np.log(reps), "e4m3", w.name)
