"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same seeded inputs, compare element by element."""
from __future__ import annotations

import sys

import numpy as np
import torch

import fa_inputs
import oracle

# Tolerances: max |dO| and max |dLSE| over rows that have an admissible key.
TOL = {"bf16": (2e-2, 1e-3), "e4m3": (5e-2, 5e-3)}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(w: fa_inputs.Workload):
    dev = "cuda"
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    cu = torch.from_numpy(w.cu_seqlens).to(dev) if w.cu_seqlens is not None else None
    ds = torch.from_numpy(w.descales).to(dev) if w.descales is not None else None
    return q, k, v, cu, ds


def nan_outputs(w: fa_inputs.Workload):
    """O and LSE buffers pre-filled with NaN, so that an element the kernel never writes cannot
    pass any check (every comparison below rejects NaN)."""
    o = torch.full((w.total_q, w.heads_q, w.head_dim_v), float("nan"), dtype=torch.bfloat16,
                   device="cuda")
    lse = torch.full((w.heads_q, w.total_q), float("nan"), dtype=torch.float32, device="cuda")
    return o, lse


def gpu_run(w: fa_inputs.Workload, tensors=None):
    """Forward on the GPU through the C ABI, into NaN-filled outputs.
    Returns (O [total_q,Hq,Dv], LSE [Hq,total_q]) as float64."""
    import exact_attention_forward_fa_amd as fa

    q, k, v, cu, ds = tensors if tensors is not None else to_device(w)
    say(f"[gpu] fa_fwd {w.name}: b={w.batch} hq={w.heads_q} hkv={w.heads_kv} sq={w.seqlen_q} "
        f"sk={w.seqlen_k} d={w.head_dim} causal={w.causal} dtype={w.dtype} seed={w.seed}")
    o, lse = nan_outputs(w)
    fa.forward(q, k, v, causal=w.causal, softmax_scale=w.softmax_scale, cu_seqlens=cu,
               max_seqlen_q=w.seqlen_q, max_seqlen_k=w.seqlen_k, descales=ds, batch=w.batch,
               out=o, lse=lse)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


def dead_rows(w: fa_inputs.Workload):
    """Boolean [Hq, total_q]: rows with no admissible key (bottom-right causal: i < sq - sk;
    any row of a sequence with no key), from the lengths alone."""
    dead = np.zeros((w.heads_q, w.total_q), dtype=bool)
    q0 = 0
    for sq, sk in w.lengths:
        n = sq if sk == 0 else (min(max(sq - sk, 0), sq) if w.causal else 0)
        dead[:, q0:q0 + n] = True
        q0 += sq
    return dead


def check_written(w: fa_inputs.Workload, o, lse):
    """Whole-output checks that need no reference: every element written (no NaN left from the
    pre-fill), every row with an admissible key has a finite LSE and a finite O, every row
    without one is exactly O = 0 and LSE = -inf."""
    dead = dead_rows(w)
    assert not np.isnan(lse).any(), f"{w.name}: {int(np.isnan(lse).sum())} LSE elements not written"
    assert not np.isnan(o).any(), f"{w.name}: {int(np.isnan(o).sum())} O elements not written"
    assert np.all(lse[dead] == -np.inf), f"{w.name}: a fully masked row has LSE != -inf"
    assert np.all(o[dead.T] == 0.0), f"{w.name}: a fully masked row has O != 0"
    assert np.all(np.isfinite(lse[~dead])), f"{w.name}: non-finite LSE on a row with keys"
    assert np.all(np.isfinite(o[~dead.T])), f"{w.name}: non-finite O on a row with keys"
    say(f"[written] {w.name}: all {o.size} O and {lse.size} LSE elements written; "
        f"{int(dead.sum())} fully masked rows exact")


def oracle_full(w: fa_inputs.Workload):
    dt = oracle.BF16 if w.dtype == "bf16" else oracle.E4M3
    return oracle.attention(w.q, w.k, w.v, descales=w.descales, dtype=dt, **w.shape_kwargs())


def oracle_rows(w: fa_inputs.Workload, rows):
    dt = oracle.BF16 if w.dtype == "bf16" else oracle.E4M3
    return oracle.attention_rows(w.q, w.k, w.v, rows, descales=w.descales, dtype=dt,
                                 **w.shape_kwargs())


def compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype: str, what: str):
    """Element-wise parity.  Rows whose reference LSE is -inf must be exactly O = 0, LSE = -inf."""
    tol_o, tol_l = TOL[dtype]
    assert o_gpu.shape == o_ref.shape and lse_gpu.shape == lse_ref.shape, what
    assert not np.isnan(o_gpu).any(), f"{what}: NaN in O"
    assert not np.isnan(lse_gpu).any(), f"{what}: NaN in LSE"
    dead = ~np.isfinite(lse_ref)  # [Hq, total_q] or [n]
    assert np.all(lse_gpu[dead] == -np.inf), f"{what}: fully masked rows must have LSE = -inf"
    live = ~dead
    assert np.all(np.isfinite(lse_gpu[live])), f"{what}: non-finite LSE on a live row"
    if o_ref.ndim == 3:  # [total_q, Hq, Dv] vs LSE [Hq, total_q]
        dead_o = dead.T
    else:  # rows
        dead_o = dead
    assert np.all(o_gpu[dead_o] == 0.0), f"{what}: fully masked rows must have O = 0"
    eo = float(np.max(np.abs(o_gpu[~dead_o] - o_ref[~dead_o]))) if (~dead_o).any() else 0.0
    el = float(np.max(np.abs(lse_gpu[live] - lse_ref[live]))) if live.any() else 0.0
    say(f"[parity] {what}: max|dO|={eo:.3e} (tol {tol_o}) max|dLSE|={el:.3e} (tol {tol_l}) "
        f"masked rows={int(dead.sum())}")
    assert eo <= tol_o, f"{what}: max|dO| {eo:.3e} > {tol_o}"
    assert el <= tol_l, f"{what}: max|dLSE| {el:.3e} > {tol_l}"
    return eo, el


def sample_rows(w: fa_inputs.Workload, n_random: int = 24, seed: int = 0):
    """(b, h, i) rows: tile edges, first/last rows, the first admissible rows of sequences with
    fewer keys than queries, and random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b, (sq, sk) in enumerate(w.lengths):
        if sq == 0:
            continue
        hs = {0, w.heads_q - 1, int(rng.integers(0, w.heads_q))}
        cand = {0, 1, sq - 1, min(127, sq - 1), min(128, sq - 1), sq // 2}
        if w.causal and sk < sq:
            cand |= {max(sq - sk - 1, 0), min(sq - sk, sq - 1)}
        for h in hs:
            for i in cand:
                rows.add((b, h, i))
    for _ in range(n_random):
        b = int(rng.integers(0, w.batch))
        sq = w.lengths[b][0]
        if sq:
            rows.add((b, int(rng.integers(0, w.heads_q)), int(rng.integers(0, sq))))
    return sorted(rows)


def tile_rows(w: fa_inputs.Workload, tile: int = 128, slice_rows: int = 32, seed: int = 0):
    """Rows (b, h, i) covering every (sequence, query head, 128-row query tile): the tile's
    first row, its last row inside the sequence and one random row of each of its 32-row
    slices (the rows one wave owns), so that every workgroup's and every wave's output is
    compared with the oracle; plus the edge rows of sample_rows."""
    rng = np.random.default_rng(seed)
    rows = set(sample_rows(w, n_random=0, seed=seed))
    for b, (sq, _) in enumerate(w.lengths):
        for m0 in range(0, sq, tile):
            last = min(m0 + tile, sq) - 1
            for h in range(w.heads_q):
                rows.add((b, h, m0))
                rows.add((b, h, last))
                for s0 in range(m0, last + 1, slice_rows):
                    rows.add((b, h, int(rng.integers(s0, min(s0 + slice_rows, last + 1)))))
    return sorted(rows)


def gather_rows(w: fa_inputs.Workload, o, lse, rows):
    """Pick rows (b, h, i) out of full GPU outputs."""
    q0 = [0] * w.batch
    if w.cu_seqlens is not None:
        q0 = [int(w.cu_seqlens[b]) for b in range(w.batch)]
    else:
        q0 = [b * w.seqlen_q for b in range(w.batch)]
    og = np.stack([o[q0[b] + i, h] for b, h, i in rows])
    lg = np.array([lse[h, q0[b] + i] for b, h, i in rows])
    return og, lg
