#!/usr/bin/env python3
"""Benchmark of the exact-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one forward pass (fa_fwd through the C ABI) over the whole
workload with inputs already resident in HBM.  Default workload: causal GQA,
batch 2, 32 query heads, 8 key/value heads, seqlen 8192, head_dim 128, bf16.
Prints ONE JSON line with the throughput in causal-adjusted TFLOPS
(FLOPs = 2 * (D + Dv) * Hq * admissible (query, key) pairs; softmax not
counted), the roofline of the kernel against the MI355X dense MFMA peak, and
the fp64 CPU oracle timed on a bounded row sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOPS (causal-adjusted) and % of bf16 MFMA peak, 1 MI355X"
DEFAULT_WORKLOAD = "gqa_causal_b2_hq32_hkv8_s8192_d128"
# MI355X published dense peaks (TFLOP/s): bf16 2.5 PFLOP/s, fp8 5.0 PFLOP/s.
PEAK_TFLOPS = {"bf16": 2500.0, "e4m3": 5000.0}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def pairs_per_sequence(sq: int, sk: int, causal: bool) -> int:
    """Admissible (query, key) pairs of one sequence.  Under bottom-right causal alignment row i
    sees min(max(i + sk - sq + 1, 0), sk) keys; the sum over rows is taken in closed form."""
    if not causal:
        return sq * sk

    def s(n: int) -> int:  # sum_{x=1..n} min(x, sk), n >= 0
        if n <= sk:
            return n * (n + 1) // 2
        return sk * (sk + 1) // 2 + (n - sk) * sk

    a = sk - sq + 1  # keys seen by row 0 (before clipping)
    b = a + sq - 1  # keys seen by row sq-1 (before clipping)
    return s(max(b, 0)) - s(max(a - 1, 0))


def workload_flops(w) -> int:
    pairs = sum(pairs_per_sequence(sq, sk, w.causal) for sq, sk in w.lengths)
    return 2 * (w.head_dim + w.head_dim_v) * w.heads_q * pairs


def row_flops(w, b: int, i: int) -> int:
    sq, sk = w.lengths[b]
    n = min(sk, i + sk - sq + 1) if w.causal else sk
    return 2 * (w.head_dim + w.head_dim_v) * max(n, 0)


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_attention_forward_fa_amd", "csrc")
    for fn in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, fn), "rb") as f:
            h.update(fn.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM traffic per launch from the committed rocprofv3 PMC summary, if it was taken on the
    current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"fa_fwd_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_digest") != kernel_source_digest():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(w, target_s: float):
    """The fp64 oracle on a random row sample of the workload; TFLOPS in the metric's unit."""
    import numpy as np

    import oracle

    rng = np.random.default_rng(1234)
    rows, flops = [], 0

    def draw(n):
        nonlocal flops
        out = []
        for _ in range(n):
            b = int(rng.integers(0, w.batch))
            sq = w.lengths[b][0]
            if sq == 0:
                continue
            i = int(rng.integers(0, sq))
            h = int(rng.integers(0, w.heads_q))
            out.append((b, h, i))
            flops += row_flops(w, b, i)
        return out

    dt = oracle.BF16 if w.dtype == "bf16" else oracle.E4M3
    kw = w.shape_kwargs()
    # calibrate on a sample large enough to keep every thread busy (a handful of rows
    # under-reports the rate: thread start-up and imbalance dominate), then draw rows until the
    # measured sample holds about target_s seconds of work
    cal = draw(64 * oracle.num_threads())
    t0 = time.perf_counter()
    oracle.attention_rows(w.q, w.k, w.v, cal, descales=w.descales, dtype=dt, **kw)
    t_cal = time.perf_counter() - t0
    rate = flops / max(t_cal, 1e-6)
    flops = 0
    rows = []
    while flops < rate * target_s and len(rows) < 2_000_000:
        rows += draw(256)
    t0 = time.perf_counter()
    oracle.attention_rows(w.q, w.k, w.v, rows, descales=w.descales, dtype=dt, **kw)
    sec = time.perf_counter() - t0
    return {"value": round(flops / sec / 1e12, 6), "unit": "TFLOPS", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{len(rows)} random (batch, head, query) rows of the same workload, "
                      f"{flops:.3e} causal-adjusted FLOPs in {sec:.1f} s (fp64)"}


def copy_calibration(nbytes: int) -> None:
    """A plain device-to-device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE
    counters of the attention kernel."""
    import torch

    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    log(f"copied {nbytes} bytes x3")


# KV-cache decode: one new token per sequence appended to a long cache, then attention of
# that token over the whole cache (bottom-right causal).  Bound by HBM: the cache is read once.
KVCACHE_WORKLOADS = {
    "kvcache_decode_b32_hq32_hkv8_c8192_d128": dict(batch=32, heads_q=32, heads_kv=8,
                                                    capacity=8192, head_dim=128, seed=90),
}
HBM_PEAK_GBPS = 8000.0


def run_kvcache(args, cfg) -> int:
    """One step = fa_fwd_kvcache appending 1 row per sequence at position capacity-1 (the same
    row every step) and attending over all `capacity` rows."""
    import torch

    import fa_inputs
    import exact_attention_forward_fa_amd as fa

    b, hq, hkv, cap, d = cfg["batch"], cfg["heads_q"], cfg["heads_kv"], cfg["capacity"], cfg["head_dim"]
    case = fa_inputs.make_kvcache(b, 1, 1, cap, [cap - 1] * b, hq, hkv, d, causal=True,
                                  seed=cfg["seed"])
    log(f"workload {args.workload}: KV-cache decode, batch={b} hq={hq} hkv={hkv} cache={cap} d={d}")
    q, kc, vc = case.q.cuda(), case.k_cache.cuda(), case.v_cache.cuda()
    kn, vn = case.k_new.cuda(), case.v_new.cuda()
    lens = torch.from_numpy(case.cache_seqlens).cuda()
    o = torch.empty((b, hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((hq, b), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        fa.fa_fwd_kvcache(q, kc, vc, kn, vn, o, lse, b, hq, hkv, 1, 1, cap, lens, d, d,
                          case.softmax_scale, 1, None, stream=stream.cuda_stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    flops = 2 * (d + d) * hq * b * cap  # each query row sees all `cap` keys
    # algorithmic bytes: the used cache rows of K and V read once, Q in, O and LSE out, the
    # appended K/V rows read and written
    hbm = 2 * b * cap * hkv * d * 2 + b * hq * d * 2 * 2 + b * hq * 4 + 2 * 2 * b * hkv * d * 2
    gbps = hbm / (step_ms * 1e-3) / 1e9
    value = flops / (ms_per_step * 1e-3) / 1e12
    log(f"step {step_ms:.4f} ms (events: append + attention), {gbps:.0f} GB/s = "
        f"{100 * gbps / HBM_PEAK_GBPS:.1f}% of {HBM_PEAK_GBPS:.0f} GB/s, {value:.2f} TFLOPS")
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_peak": round(100 * value / PEAK_TFLOPS["bf16"], 2),
        "config": {"workload": args.workload, "batch": b, "heads_q": hq, "heads_kv": hkv,
                   "seqlen_q": 1, "seqlen_new": 1, "cache_capacity": cap, "head_dim": d,
                   "causal": True, "flops_per_step": flops, "hbm_bytes_per_step": hbm},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel_ms": round(step_ms, 5)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    return 0


# The five configurations of the metric (the dense MHA one run causal and not); each gets its
# own entry in the "configs" list of the output line, timed like the headline workload.  An idle
# MI355X raises its shader clock over its first ~35 ms of load and lowers it again within tens of
# ms of idling (measured on the GQA causal 8192 workload: launches 0-4 at 1.61 ms, 5-24 at
# 0.97 ms, 0.915 ms from launch 30 on), so a run with a few warm-up launches, or one timed after
# the host has spent a while building inputs, times that ramp instead of the kernel.  Every
# workload's device inputs are therefore built before anything is timed, and the lines are timed
# back to back: a long one first (its warm-up launches take the clock through the ramp) and the
# headline workload's own line last, right before the headline's timed launches on the same
# inputs, so that each line and the headline see the clock the GPU holds under sustained load.
CONFIG_WORKLOADS = ["fp8_causal_b1_h32_s16384_d128", "varlen_causal_18seq_h16_d128",
                    "mha_b4_h16_s1024_d128", "mha_causal_b4_h16_s1024_d128",
                    "tiny_b1_h2_s256_d64", "gqa_causal_b2_hq32_hkv8_s8192_d128"]


def device_inputs(w):
    import torch

    q, k, v = w.q.cuda(), w.k.cuda(), w.v.cuda()
    cu = torch.from_numpy(w.cu_seqlens).cuda() if w.cu_seqlens is not None else None
    ds = torch.from_numpy(w.descales).cuda() if w.descales is not None else None
    o = torch.empty((w.total_q, w.heads_q, w.head_dim_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.heads_q, w.total_q), dtype=torch.float32, device="cuda")
    return q, k, v, cu, ds, o, lse


def timed_launches(w, tensors, warmup: int, steps: int):
    """Launch fa_fwd warmup + steps times back to back on torch's current stream; returns
    (kernel ms per launch from HIP events recorded on that stream, wall ms per launch)."""
    import torch

    import exact_attention_forward_fa_amd as fa

    q, k, v, cu, ds, o, lse = tensors
    stream = torch.cuda.current_stream()

    def step():
        fa.fa_fwd(q, k, v, o, lse, w.batch, w.heads_q, w.heads_kv, w.seqlen_q, w.seqlen_k, cu,
                  w.head_dim, w.head_dim_v, w.softmax_scale, int(w.causal), ds,
                  stream=stream.cuda_stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return ev0.elapsed_time(ev1) / steps, wall * 1e3 / steps


def config_lines(prepared, warmup: int, steps: int):
    """Every configuration of the metric: kernel time per launch (HIP events), TFLOPS and the
    fraction of its input type's dense MFMA peak, and the schedule the planner chose.
    `prepared`: (workload, device tensors) pairs in timing order."""
    import exact_attention_forward_fa_amd as fa

    out = []
    for w, tensors in prepared:
        kernel_ms, _ = timed_launches(w, tensors, warmup, steps)
        flops = workload_flops(w)
        peak = PEAK_TFLOPS[w.dtype]
        tf = flops / (kernel_ms * 1e-3) / 1e12
        plan = fa.fa_fwd_plan(fa.FA_DTYPE_BF16 if w.dtype == "bf16" else fa.FA_DTYPE_E4M3,
                              w.batch, w.heads_q, w.heads_kv, w.seqlen_q, w.seqlen_k,
                              w.cu_seqlens is not None, w.head_dim, w.head_dim_v, w.causal)
        line = {"workload": w.name, "dtype": w.dtype, "causal": w.causal, "flops": flops,
                "kernel_ms": round(kernel_ms, 5), "tflops": round(tf, 2), "peak": peak,
                "frac": round(tf / peak, 4), "schedule": int(plan.schedule)}
        log(f"config {w.name}: {kernel_ms:.4f} ms, {tf:.1f} TFLOPS = {100 * tf / peak:.1f}% of "
            f"{peak:.0f} (schedule {plan.schedule})")
        out.append(line)
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration lines (all five configurations of the metric)")
    ap.add_argument("--config-steps", type=int, default=100,
                    help="timed launches per configuration line (after as many warm-up launches)")
    ap.add_argument("--exp2-offload", type=int, default=0, choices=[0, 4, 8],
                    help="ping-pong schedule: every N-th exponential on the FMA polynomial "
                         "(0: off, the default)")
    ap.add_argument("--fp8-exact-scores", type=int, default=0, choices=[0, 1],
                    help="e4m3 workloads: scores on the bf16 MFMA from exactly widened Q and K "
                         "(1), or on the fp8 MFMA (0, the default)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a device copy of BYTES bytes (counter scaling) and exit")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported; the "
              "library runs the forward on one GPU and has no multi-GPU path.", file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return 0

    import torch

    import fa_inputs
    import exact_attention_forward_fa_amd as fa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.workload in KVCACHE_WORKLOADS:
        return run_kvcache(args, KVCACHE_WORKLOADS[args.workload])
    w = fa_inputs.workload(args.workload)
    fa.fa_set_exp2_offload(args.exp2_offload)
    fa.fa_set_fp8_exact_scores(args.fp8_exact_scores)
    log(f"workload {w.name}: batch={w.batch} hq={w.heads_q} hkv={w.heads_kv} sq={w.seqlen_q} "
        f"sk={w.seqlen_k} d={w.head_dim} causal={w.causal} dtype={w.dtype}")
    # every input on the device first, then the per-configuration lines back to back (see
    # CONFIG_WORKLOADS: they carry the GPU through its clock ramp), then exactly args.warmup
    # untimed and args.steps timed launches of the workload
    tensors = device_inputs(w)
    configs = None
    if not args.no_configs:
        order = [n for n in CONFIG_WORKLOADS if n != w.name] + \
                ([w.name] if w.name in CONFIG_WORKLOADS else [])
        prepared = []
        for n in order:
            wn = w if n == w.name else fa_inputs.workload(n)
            prepared.append((wn, tensors if n == w.name else device_inputs(wn)))
        torch.cuda.synchronize()
        configs = config_lines(prepared, args.config_steps, args.config_steps)
    # no host work between the last line and the headline's launches: a few ms of GPU idle
    # (freeing the other workloads' inputs, say) already lowers the clock (measured: 5 ms idle,
    # then 25 launches 6 % slower than under sustained load)
    kernel_ms, ms_per_step = timed_launches(w, tensors, args.warmup, args.steps)
    if not args.no_configs:
        del prepared
    del tensors
    flops = workload_flops(w)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    log(f"kernel {kernel_ms:.4f} ms/launch (events), wall {ms_per_step:.4f} ms/step, "
        f"{achieved:.1f} TFLOPS = {100 * achieved / peak:.1f}% of {peak:.0f}")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the fp64 CPU oracle on a row sample ...")
        cpu = cpu_baseline(w, args.cpu_seconds)
        log(f"oracle: {cpu}")

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "pct_of_peak": round(100 * value / peak, 2),
        "config": {"workload": w.name, "batch": w.batch, "heads_q": w.heads_q,
                   "heads_kv": w.heads_kv, "seqlen_q": w.seqlen_q, "seqlen_k": w.seqlen_k,
                   "head_dim": w.head_dim, "head_dim_v": w.head_dim_v, "causal": w.causal,
                   "flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": (None if args.exp2_offload or args.fp8_exact_scores
                                 else load_traffic(w.name)),
                     "kernel_ms": round(kernel_ms, 5)},
        "cpu_baseline": cpu,
        "configs": configs,
        "timed_after": ("the configs lines, back to back, the last on this workload's inputs "
                        "(about 0.6 s of launches: the GPU at its sustained-load clock)"
                        if configs is not None else "nothing: a cold GPU's clock ramp falls in "
                        "the first ~35 ms of launches"),
    }
    if args.exp2_offload:
        line["config"]["exp2_offload"] = args.exp2_offload
    if args.fp8_exact_scores:
        line["config"]["fp8_exact_scores"] = 1
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
