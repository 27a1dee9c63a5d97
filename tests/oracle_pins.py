"""Pins that tie the fp64 oracle to facts outside itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
something the mathematics or a library routine fixes independently: exact
decoders checked against torch's dtype casts over every bit pattern, closed
forms (two-key softmax, constant V, single admissible key), invariants (rows
of P sum to one, key shift, key permutation, key repetition), special cases that reduce to
``torch.nn.functional.scaled_dot_product_attention`` in float64, and an
independent one-pass online-softmax brute force (``oracle/online.py``).

They are plain functions so that ``test_oracle_mutations.py`` can run them
all against deliberately broken builds of the oracle and show that each
plausible mistake fails at least one of them.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import fa_inputs
import oracle
from oracle.online import online_attention

TIGHT = 1e-12


def _dec(w: fa_inputs.Workload):
    """Decode the workload's inputs with torch's casts (not the oracle's decoders)."""
    if w.dtype == "bf16":
        f = lambda t: t.to(torch.float64)
        return f(w.q), f(w.k), f(w.v)
    ds = [float(x) for x in w.descales]
    f = lambda t, d: t.view(torch.float8_e4m3fn).to(torch.float64) * d
    return f(w.q, ds[0]), f(w.k, ds[1]), f(w.v, ds[2])


def _run(w: fa_inputs.Workload):
    kw = w.shape_kwargs()
    dt = oracle.BF16 if w.dtype == "bf16" else oracle.E4M3
    return oracle.attention(w.q, w.k, w.v, descales=w.descales, dtype=dt, **kw)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), f"{what}: finiteness differs"
    assert np.array_equal(a[~fin], b[~fin]), f"{what}: non-finite values differ"
    err = float(np.max(np.abs(a[fin] - b[fin]))) if fin.any() else 0.0
    assert err <= tol, f"{what}: max error {err:.3e} > {tol:.1e}"


def _bf16_tensor(values, shape):
    t = torch.tensor(np.asarray(values, dtype=np.float32).reshape(shape)).to(torch.bfloat16)
    assert torch.equal(t.to(torch.float32), torch.tensor(np.asarray(values, dtype=np.float32).reshape(shape))), \
        "test values must be exact in bf16"
    return t


# ---------------------------------------------------------------- decoders

def pin_decode_bf16_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan), "bf16 NaN patterns differ"
    assert np.array_equal(ours[~nan], ref[~nan]), "bf16 decode differs from torch's cast"


def pin_decode_e4m3_exhaustive():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan), "e4m3 NaN patterns differ"
    assert np.array_equal(ours[~nan], ref[~nan]), "e4m3 decode differs from torch's cast"
    # From the OCP FP8 format definition: bias 7, max normal 448, smallest subnormal 2^-9.
    assert ours[0x38] == 1.0 and ours[0xB8] == -1.0
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])


# ------------------------------------------------------------ closed forms

def pin_two_key_closed_form():
    """One query, two keys: P = (1 - sigma(s), sigma(s)), LSE = log(1 + e^s)."""
    for scale in (0.5, 1.0, 2.0, 3.0):
        q = _bf16_tensor([1.0], (1, 1, 1))
        k = _bf16_tensor([0.0, 1.0], (2, 1, 1))
        v = _bf16_tensor([0.0, 1.0, 1.0, -2.0], (2, 1, 2))
        o, lse = oracle.attention(q, k, v, batch=1, heads_q=1, heads_kv=1, seqlen_q=1, seqlen_k=2,
                                  head_dim=1, head_dim_v=2, softmax_scale=scale, causal=False)
        sig = 1.0 / (1.0 + math.exp(-scale))
        _close(o[0, 0], [sig, (1 - sig) * 1.0 + sig * -2.0], TIGHT, "two-key O")
        _close(lse[0, 0], math.log1p(math.exp(scale)), TIGHT, "two-key LSE")


def pin_constant_v():
    """V equal to the same vector for every key gives O equal to that vector."""
    w = fa_inputs.make(2, 4, 2, 17, 23, 16, 8, causal=True, seed=11)
    const = np.array([0.5, -1.25, 3.0, 0.0, 2.0, -0.75, 1.0, 8.0], dtype=np.float32)
    w.v = _bf16_tensor(np.tile(const, w.total_k * w.heads_kv), (w.total_k, w.heads_kv, 8))
    o, lse = _run(w)
    valid = np.isfinite(lse.T)  # [total_q, Hq]
    assert valid.any()
    _close(o[valid], np.broadcast_to(const, o[valid].shape), TIGHT, "constant V")


def pin_causal_first_row():
    """Square causal: query 0 sees only key 0, so O[0] = V[0] and LSE[0] = scale * q0.k0."""
    w = fa_inputs.make(1, 2, 2, 9, 9, 8, causal=True, seed=12)
    o, lse = _run(w)
    qd, kd, vd = _dec(w)
    for h in range(2):
        _close(o[0, h], vd[0, h].numpy(), 0.0, "causal row 0 O")
        s00 = w.softmax_scale * float(torch.dot(qd[0, h], kd[0, h]))
        _close(lse[h, 0], s00, TIGHT, "causal row 0 LSE")


def pin_lse_unshifted_closed_form():
    """LSE_i = log sum_j exp(s_ij), evaluated without the max shift (small scores)."""
    w = fa_inputs.make(1, 3, 3, 6, 10, 4, causal=False, seed=13)
    o, lse = _run(w)
    qd, kd, _ = _dec(w)
    for h in range(3):
        for i in range(6):
            s = [w.softmax_scale * float(torch.dot(qd[i, h], kd[j, h])) for j in range(10)]
            _close(lse[h, i], math.log(math.fsum(math.exp(x) for x in s)), 1e-13, "unshifted LSE")


# --------------------------------------------------------------- invariants

def pin_rows_sum_to_one():
    for causal in (False, True):
        w = fa_inputs.make(1, 4, 2, 12, 19, 8, causal=causal, seed=14)
        kw = w.shape_kwargs()
        for h in range(4):
            for i in range(12):
                p, o, lse = oracle.probs_row(w.q, w.k, w.v, 0, h, i, **kw)
                assert (p >= 0).all()
                _close(p.sum(), 1.0, TIGHT, "sum of P")
                if causal:  # keys past i + sk - sq carry no weight
                    assert not p[i + 19 - 12 + 1:].any(), "masked keys carry weight"
                _, vd = _dec(w)[1:]
                _close(o, p @ vd[:, h // 2, :].numpy(), TIGHT, "O = P V")


def pin_key_shift_invariance():
    """Adding u to every key adds scale*q.u to LSE and leaves O unchanged."""
    rng = np.random.default_rng(15)
    sq, sk, d = 5, 7, 8
    qv = rng.integers(-8, 9, size=(sq, 1, d)) / 8.0
    kv = rng.integers(-8, 9, size=(sk, 1, d)) / 8.0
    u = rng.integers(-8, 9, size=(d,)) / 4.0
    vv = rng.standard_normal((sk, 1, d)).astype(np.float32)
    q, k, k2 = _bf16_tensor(qv, qv.shape), _bf16_tensor(kv, kv.shape), _bf16_tensor(kv + u, kv.shape)
    v = torch.from_numpy(vv).to(torch.bfloat16)
    kw = dict(batch=1, heads_q=1, heads_kv=1, seqlen_q=sq, seqlen_k=sk, head_dim=d, head_dim_v=d,
              softmax_scale=0.7, causal=False)
    o1, l1 = oracle.attention(q, k, v, **kw)
    o2, l2 = oracle.attention(q, k2, v, **kw)
    _close(o2, o1, 1e-13, "key shift O")
    _close(l2[0], l1[0] + 0.7 * (qv[:, 0, :] @ u), 1e-12, "key shift LSE")


def pin_key_permutation_invariance():
    w = fa_inputs.make(1, 2, 1, 6, 13, 8, causal=False, seed=16)
    o1, l1 = _run(w)
    perm = torch.from_numpy(np.random.default_rng(16).permutation(13))
    w.k, w.v = w.k[perm].contiguous(), w.v[perm].contiguous()
    o2, l2 = _run(w)
    _close(o2, o1, 1e-13, "key permutation O")
    _close(l2, l1, 1e-13, "key permutation LSE")


def pin_key_repetition():
    """Every key (with its value) present r times: each weight's numerator and the sum gain the
    factor r, so O is unchanged and LSE grows by ln r (the GPU maximum-size tests rely on it)."""
    w = fa_inputs.make(1, 2, 1, 6, 13, 8, causal=False, seed=17)
    o1, l1 = _run(w)
    r = 5
    w.k, w.v = w.k.repeat(r, 1, 1).contiguous(), w.v.repeat(r, 1, 1).contiguous()
    w.seqlen_k *= r
    o2, l2 = _run(w)
    _close(o2, o1, 1e-13, "key repetition O")
    _close(l2, l1 + math.log(r), 1e-13, "key repetition LSE")


# ----------------------------------------------------- library special cases

def _sdpa(qd, kd, vd, scale, causal):
    """torch SDPA in float64 on [S, H, D] tensors (MHA); LSE by torch.logsumexp."""
    q = qd.permute(1, 0, 2).contiguous()
    k = kd.permute(1, 0, 2).contiguous()
    v = vd.permute(1, 0, 2).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale)
    s = scale * torch.matmul(q, k.transpose(1, 2).contiguous())
    if causal:
        mask = torch.ones(s.shape[-2:], dtype=torch.bool).tril()
        s = s.masked_fill(~mask, -math.inf)
    return o.permute(1, 0, 2).numpy(), torch.logsumexp(s, dim=-1).numpy()


def pin_sdpa_library():
    for causal in (False, True):
        w = fa_inputs.make(1, 3, 3, 33, 33, 16, causal=causal, seed=17)
        o, lse = _run(w)
        ro, rl = _sdpa(*_dec(w), w.softmax_scale, causal)
        _close(o, ro, 1e-12, "SDPA O")
        _close(lse, rl, 1e-12, "SDPA LSE")


def pin_large_q_stable():
    """Q scaled by 50: max subtraction keeps everything finite and exact."""
    w = fa_inputs.make(1, 2, 2, 20, 20, 16, causal=True, seed=18, q_mult=50.0)
    o, lse = _run(w)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    ro, rl = _sdpa(*_dec(w), w.softmax_scale, True)
    _close(o, ro, 1e-11, "large-Q O")
    _close(lse, rl, 1e-10, "large-Q LSE")


def pin_gqa_equals_repeated_mha():
    w = fa_inputs.make(2, 8, 2, 11, 14, 8, causal=True, seed=19)
    o, lse = _run(w)
    w2 = fa_inputs.make(2, 8, 2, 11, 14, 8, causal=True, seed=19)
    w2.k = w.k.repeat_interleave(4, dim=1).contiguous()
    w2.v = w.v.repeat_interleave(4, dim=1).contiguous()
    w2.heads_kv = 8
    o2, l2 = _run(w2)
    _close(o, o2, 0.0, "GQA vs repeated MHA O")
    _close(lse, l2, 0.0, "GQA vs repeated MHA LSE")


def pin_varlen_equals_separate():
    lens = [(7, 9), (3, 3), (5, 2), (4, 0), (6, 11)]
    w = fa_inputs.make(0, 2, 1, 0, 0, 8, causal=True, seed=20, lengths=lens)
    o, lse = _run(w)
    cu = w.cu_seqlens
    nb = len(lens)
    for b, (sq, sk) in enumerate(lens):
        q0, k0 = int(cu[b]), int(cu[nb + 1 + b])
        ob, lb = oracle.attention(w.q[q0:q0 + sq], w.k[k0:k0 + sk], w.v[k0:k0 + sk], batch=1,
                                  heads_q=2, heads_kv=1, seqlen_q=sq, seqlen_k=sk, head_dim=8,
                                  head_dim_v=8, softmax_scale=w.softmax_scale, causal=True)
        _close(o[q0:q0 + sq], ob, 0.0, f"varlen seq {b} O")
        _close(lse[:, q0:q0 + sq], lb, 0.0, f"varlen seq {b} LSE")


def pin_masked_rows_exact():
    """Bottom-right causal with sq > sk: rows i < sq - sk see no key; sk = 0: no row sees one."""
    lens = [(9, 5), (4, 0)]
    w = fa_inputs.make(0, 2, 2, 0, 0, 8, causal=True, seed=21, lengths=lens)
    o, lse = _run(w)
    assert np.all(o[:4] == 0.0) and np.all(lse[:, :4] == -np.inf)
    assert np.all(np.isfinite(lse[:, 4:9])) and np.any(o[4:9] != 0.0)
    assert np.all(o[9:13] == 0.0) and np.all(lse[:, 9:13] == -np.inf)
    # row 4 of sequence 0 sees exactly key 0
    _close(o[4], w.v[0].to(torch.float64).numpy(), 0.0, "first admissible row")


def pin_online_bruteforce():
    """The one-pass exp2 online softmax over keys (reverse order) equals the full-row oracle."""
    cases = [
        dict(batch=1, heads_q=2, heads_kv=2, seqlen_q=13, seqlen_k=13, head_dim=8, head_dim_v=4, causal=False),
        dict(batch=2, heads_q=4, heads_kv=2, seqlen_q=7, seqlen_k=11, head_dim=8, head_dim_v=8, causal=True),
        dict(batch=1, heads_q=2, heads_kv=1, seqlen_q=9, seqlen_k=5, head_dim=4, head_dim_v=6, causal=True),
    ]
    for n, c in enumerate(cases):
        c = dict(c)
        w = fa_inputs.make(c.pop("batch"), c.pop("heads_q"), c.pop("heads_kv"), c.pop("seqlen_q"),
                           c.pop("seqlen_k"), c.pop("head_dim"), c.pop("head_dim_v"), seed=30 + n,
                           causal=c.pop("causal"))
        o, lse = _run(w)
        qd, kd, vd = _dec(w)
        bo, bl = online_attention(qd.numpy(), kd.numpy(), vd.numpy(), batch=w.batch, heads_q=w.heads_q,
                                  heads_kv=w.heads_kv, seqlen_q=w.seqlen_q, seqlen_k=w.seqlen_k,
                                  softmax_scale=w.softmax_scale, causal=w.causal)
        _close(o, bo, TIGHT, f"online case {n} O")
        _close(lse, bl, TIGHT, f"online case {n} LSE")
    lens = [(5, 7), (6, 0), (4, 3), (0, 3), (3, 9)]
    w = fa_inputs.make(0, 2, 2, 0, 0, 8, causal=True, seed=40, lengths=lens)
    o, lse = _run(w)
    qd, kd, vd = _dec(w)
    bo, bl = online_attention(qd.numpy(), kd.numpy(), vd.numpy(), batch=w.batch, heads_q=2, heads_kv=2,
                              seqlen_q=w.seqlen_q, seqlen_k=w.seqlen_k, softmax_scale=w.softmax_scale,
                              causal=True, cu_seqlens=w.cu_seqlens)
    _close(o, bo, TIGHT, "online varlen O")
    _close(lse, bl, TIGHT, "online varlen LSE")


# ---------------------------------------------------------------------- fp8

def pin_fp8_power_of_two_descales_equal_bf16():
    """e4m3 codes times power-of-two descales are exact in bf16: both input paths agree exactly."""
    w = fa_inputs.make(1, 2, 2, 10, 12, 16, causal=True, seed=22, dtype="e4m3")
    w.descales = np.array([0.25, 2.0, 0.5], dtype=np.float32)
    o8, l8 = _run(w)
    qd, kd, vd = _dec(w)
    wb = fa_inputs.make(1, 2, 2, 10, 12, 16, causal=True, seed=22)
    wb.q, wb.k, wb.v = qd.to(torch.bfloat16), kd.to(torch.bfloat16), vd.to(torch.bfloat16)
    assert torch.equal(wb.q.to(torch.float64), qd) and torch.equal(wb.v.to(torch.float64), vd)
    ob, lb = _run(wb)
    _close(o8, ob, 0.0, "fp8 vs bf16 O")
    _close(l8, lb, 0.0, "fp8 vs bf16 LSE")


def pin_fp8_sdpa():
    w = fa_inputs.make(1, 2, 2, 24, 24, 16, causal=True, seed=23, dtype="e4m3")
    o, lse = _run(w)
    ro, rl = _sdpa(*_dec(w), w.softmax_scale, True)
    _close(o, ro, 1e-12, "fp8 SDPA O")
    _close(lse, rl, 1e-12, "fp8 SDPA LSE")


def pin_rows_api_matches_full():
    w = fa_inputs.make(0, 4, 2, 0, 0, 8, causal=True, seed=24, lengths=[(6, 8), (5, 3)])
    o, lse = _run(w)
    rows = [(0, 0, 0), (0, 3, 5), (1, 1, 0), (1, 2, 4)]
    ro, rl = oracle.attention_rows(w.q, w.k, w.v, rows, **w.shape_kwargs())
    cu = w.cu_seqlens
    for n, (b, h, i) in enumerate(rows):
        _close(ro[n], o[int(cu[b]) + i, h], 0.0, "rows API O")
        _close(rl[n], lse[h, int(cu[b]) + i], 0.0, "rows API LSE")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
