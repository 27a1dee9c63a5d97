"""fp64 CPU oracle for exact attention forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  It shares no code with the GPU library
(``exact_attention_forward_fa_amd``) and never imports it.

``fa_oracle.c`` holds the arithmetic (plain definition of exact attention:
full score row, explicit softmax, natural-log LSE, zero output and -inf LSE
for rows with no admissible key); this module only builds it with gcc and
marshals numpy arrays through ctypes.  ``online.py`` holds an independent
one-pass online-softmax brute force (exp2 form) used to pin this oracle on
tiny inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BF16 = 0
E4M3 = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile fa_oracle.c into oracle/liboracle.so with gcc (IEEE doubles)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    shape = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, i32, i32, dbl, i32, vp]
    lib.oracle_fwd.argtypes = shape + [vp, vp]
    lib.oracle_fwd.restype = i32
    lib.oracle_fwd_rows.argtypes = shape + [vp, i64, vp, vp]
    lib.oracle_fwd_rows.restype = i32
    lib.oracle_probs_row.argtypes = shape + [i32, i32, i32, vp, vp, vp]
    lib.oracle_probs_row.restype = i32
    lib.oracle_decode_bf16.argtypes = [vp, vp, i64]
    lib.oracle_decode_e4m3.argtypes = [vp, vp, i64]
    lib.oracle_num_threads.restype = i32
    return lib


def swap_library(path):
    """Point this module at another build of fa_oracle.c (the mutation tests
    compile deliberately broken copies on the CPU).  Returns the previous
    handle; pass it back to ``restore_library``."""
    global _lib
    old = _load()
    _lib = _bind(ctypes.CDLL(path))
    return old


def restore_library(handle):
    global _lib
    _lib = handle


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _as_bits(x, dtype):
    """Raw input codes as a contiguous numpy array: uint16 (bf16) or uint8 (e4m3)."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            x = x.view(torch.int16 if dtype == BF16 else torch.uint8).numpy()
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    want = np.uint16 if dtype == BF16 else np.uint8
    return x.view(want) if x.dtype != want else x


def _common(q, k, v, dtype, cu_seqlens, descales):
    q = _as_bits(q, dtype)
    k = _as_bits(k, dtype)
    v = _as_bits(v, dtype)
    cu = None if cu_seqlens is None else np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    ds = None if descales is None else np.ascontiguousarray(np.asarray(descales, dtype=np.float64))
    return q, k, v, cu, ds


def attention(q, k, v, *, batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim, head_dim_v,
              softmax_scale, causal, cu_seqlens=None, descales=None, dtype=BF16):
    """Whole forward.  Returns (O [total_q, Hq, Dv] float64, LSE [Hq, total_q] float64)."""
    q, k, v, cu, ds = _common(q, k, v, dtype, cu_seqlens, descales)
    total_q = int(cu[batch]) if cu is not None else batch * seqlen_q
    o = np.zeros((total_q, heads_q, head_dim_v), dtype=np.float64)
    lse = np.zeros((heads_q, total_q), dtype=np.float64)
    rc = _load().oracle_fwd(_ptr(q), _ptr(k), _ptr(v), dtype, batch, heads_q, heads_kv, seqlen_q,
                            seqlen_k, _ptr(cu), head_dim, head_dim_v, float(softmax_scale),
                            int(bool(causal)), _ptr(ds), _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_fwd rejected the call")
    return o, lse


def attention_rows(q, k, v, rows, *, batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim,
                   head_dim_v, softmax_scale, causal, cu_seqlens=None, descales=None, dtype=BF16):
    """Selected rows (b, h, i).  Returns (O rows [n, Dv], LSE [n]) as float64."""
    q, k, v, cu, ds = _common(q, k, v, dtype, cu_seqlens, descales)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
    o = np.zeros((r.shape[0], head_dim_v), dtype=np.float64)
    lse = np.zeros((r.shape[0],), dtype=np.float64)
    rc = _load().oracle_fwd_rows(_ptr(q), _ptr(k), _ptr(v), dtype, batch, heads_q, heads_kv,
                                 seqlen_q, seqlen_k, _ptr(cu), head_dim, head_dim_v,
                                 float(softmax_scale), int(bool(causal)), _ptr(ds), _ptr(r),
                                 r.shape[0], _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_fwd_rows rejected the call")
    return o, lse


def probs_row(q, k, v, b, h, i, *, batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim,
              head_dim_v, softmax_scale, causal, cu_seqlens=None, descales=None, dtype=BF16):
    """Explicit softmax row P[i, :] of (b, h) plus its O row and LSE."""
    q, k, v, cu, ds = _common(q, k, v, dtype, cu_seqlens, descales)
    sk = seqlen_k if cu is None else int(cu[batch + 2 + b] - cu[batch + 1 + b])
    p = np.zeros((max(sk, 0),), dtype=np.float64)
    o = np.zeros((head_dim_v,), dtype=np.float64)
    lse = np.zeros((1,), dtype=np.float64)
    rc = _load().oracle_probs_row(_ptr(q), _ptr(k), _ptr(v), dtype, batch, heads_q, heads_kv,
                                  seqlen_q, seqlen_k, _ptr(cu), head_dim, head_dim_v,
                                  float(softmax_scale), int(bool(causal)), _ptr(ds), b, h, i,
                                  _ptr(p), _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_probs_row rejected the call")
    return p, o, float(lse[0])


def append_kv(k_cache, v_cache, k_new, v_new, cache_seqlens, *, dtype=BF16):
    """The append step of the KV-cache forward (the AppendKV branch of the forward-pass page's
    producer loop, read as the usual cached forward): copies of the caches in which row j of
    sequence b's new keys/values sits at position cache_seqlens[b] + j; positions outside
    [0, capacity) are dropped.  Caches [B, cap, Hkv, D], new rows [B, Snew, Hkv, D], as raw
    codes.  Returns (k_cache', v_cache', lengths) with lengths[b] = clamp(cache_seqlens[b] +
    Snew, 0, cap), the number of cache rows the attention step reads."""
    kc = _as_bits(k_cache, dtype).copy()
    vc = _as_bits(v_cache, dtype).copy()
    lens = np.asarray(cache_seqlens, dtype=np.int64).reshape(-1)
    cap = kc.shape[1]
    if k_new is not None:
        kn = _as_bits(k_new, dtype)
        vn = _as_bits(v_new, dtype)
        for b in range(kc.shape[0]):
            for j in range(kn.shape[1]):
                pos = int(lens[b]) + j
                if 0 <= pos < cap:
                    kc[b, pos] = kn[b, j]
                    vc[b, pos] = vn[b, j]
        snew = kn.shape[1]
    else:
        snew = 0
    used = np.clip(lens + snew, 0, cap)
    return kc, vc, used


def attention_kvcache(q, k_cache, v_cache, k_new, v_new, cache_seqlens, *, softmax_scale, causal,
                      descales=None, dtype=BF16):
    """KV-cache forward: append_kv, then the plain forward of sequence b's queries
    (q [B, Sq, Hq, D]) over the first lengths[b] rows of its cache, bottom-right causal.
    Returns (O [B*Sq, Hq, D], LSE [Hq, B*Sq], k_cache', v_cache') with O, LSE float64."""
    qb = _as_bits(q, dtype)
    kc, vc, used = append_kv(k_cache, v_cache, k_new, v_new, cache_seqlens, dtype=dtype)
    b, sq, hq, d = qb.shape
    hkv = kc.shape[2]
    # pack the used cache rows as a variable-length batch: [q offsets][k offsets]
    k_off = np.concatenate([[0], np.cumsum(used)]).astype(np.int32)
    q_off = (np.arange(b + 1) * sq).astype(np.int32)
    kp = np.concatenate([kc[i, :used[i]] for i in range(b)], axis=0) if used.sum() else \
        np.zeros((0, hkv, d), dtype=kc.dtype)
    vp = np.concatenate([vc[i, :used[i]] for i in range(b)], axis=0) if used.sum() else \
        np.zeros((0, hkv, d), dtype=vc.dtype)
    o, lse = attention(qb.reshape(b * sq, hq, d), kp, vp, batch=b, heads_q=hq, heads_kv=hkv,
                       seqlen_q=sq, seqlen_k=int(used.max()) if b else 0, head_dim=d,
                       head_dim_v=d, softmax_scale=softmax_scale, causal=causal,
                       cu_seqlens=np.concatenate([q_off, k_off]), descales=descales, dtype=dtype)
    return o, lse, kc, vc


def decode_bf16(bits):
    bits = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    out = np.empty(bits.shape, dtype=np.float64)
    _load().oracle_decode_bf16(_ptr(bits), _ptr(out), bits.size)
    return out


def decode_e4m3(codes):
    codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    out = np.empty(codes.shape, dtype=np.float64)
    _load().oracle_decode_e4m3(_ptr(codes), _ptr(out), codes.size)
    return out


def num_threads() -> int:
    return int(_load().oracle_num_threads())
