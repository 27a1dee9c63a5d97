"""Seeded synthetic inputs for exact attention forward.

The only module shared by the GPU path's tests/benchmark and the CPU oracle.
It draws random numbers and packs them into the layouts both sides read; it
holds none of the method's arithmetic.

Recipe (every workload):
  * q, k, v are drawn in that order from one CPU ``torch.Generator`` seeded
    with the workload's seed, ``randn`` in fp32, then rounded to bf16
    (round-to-nearest-even, torch's cast).
  * fp8 workloads draw x = randn * 0.5 and quantise per tensor:
    descale = max|x| / 448, code = e4m3fn(clamp(x / descale, -448, 448))
    (torch's round-to-nearest-even cast); descales travel as float32[3]
    in the order (q, k, v).
  * variable-length batches draw their lengths from
    ``numpy.random.default_rng(seed)`` and pack sequences back to back;
    ``cu_seqlens`` is int32[2*(batch+1)]: query offsets, then key offsets.
  * ``key_offsets`` (optional, one float per key position): dimension 0 of
    every query is set to 1 and dimension 0 of key j to
    key_offsets[j] / (softmax_scale * log2 e), before rounding or
    quantising, so every query's scaled score with key j gains about
    key_offsets[j] in base-2 units on top of the random part of the other
    dimensions: a controlled shape of the running row maximum.
  * KV-cache cases draw q, k_cache, v_cache, k_new, v_new in that order; the
    whole cache is filled (rows past the used length too); fp8 quantises the
    cache and the new rows of K (and of V) with one shared descale.

Layouts: Q [total_q][Hq][D], K [total_k][Hkv][D], V [total_k][Hkv][Dv];
KV cache [B][capacity][Hkv][D], new rows [B][Snew][Hkv][D].
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

E4M3_MAX = 448.0


@dataclass
class Workload:
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    seqlen_q: int  # maximum over sequences when cu_seqlens is set
    seqlen_k: int
    head_dim: int
    head_dim_v: int
    softmax_scale: float
    causal: bool
    dtype: str  # "bf16" or "e4m3"
    q: torch.Tensor  # CPU tensor: bfloat16, or uint8 e4m3 codes
    k: torch.Tensor
    v: torch.Tensor
    cu_seqlens: Optional[np.ndarray] = None  # int32[2*(batch+1)]
    descales: Optional[np.ndarray] = None  # float32[3] (q, k, v)
    seed: int = 0
    lengths: List[Tuple[int, int]] = field(default_factory=list)  # (sq, sk) per sequence

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens[self.batch]) if self.cu_seqlens is not None else self.batch * self.seqlen_q

    @property
    def total_k(self) -> int:
        if self.cu_seqlens is not None:
            return int(self.cu_seqlens[2 * self.batch + 1])
        return self.batch * self.seqlen_k

    def shape_kwargs(self) -> dict:
        return dict(batch=self.batch, heads_q=self.heads_q, heads_kv=self.heads_kv,
                    seqlen_q=self.seqlen_q, seqlen_k=self.seqlen_k, head_dim=self.head_dim,
                    head_dim_v=self.head_dim_v, softmax_scale=self.softmax_scale, causal=self.causal,
                    cu_seqlens=self.cu_seqlens)


def _randn(g: torch.Generator, shape, mult: float = 1.0) -> torch.Tensor:
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    return x * mult if mult != 1.0 else x


def _quant_e4m3(x: torch.Tensor) -> Tuple[torch.Tensor, float]:
    amax = float(x.abs().max())
    descale = amax / E4M3_MAX if amax > 0 else 1.0
    codes = (x / descale).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), descale


def make(batch: int, heads_q: int, heads_kv: int, seqlen_q: int, seqlen_k: int, head_dim: int,
         head_dim_v: Optional[int] = None, *, causal: bool, seed: int, dtype: str = "bf16",
         lengths: Optional[Sequence[Tuple[int, int]]] = None, softmax_scale: Optional[float] = None,
         q_mult: float = 1.0, fp8_mult: float = 0.5, key_offsets: Optional[Sequence[float]] = None,
         name: str = "custom") -> Workload:
    """Build one workload.  ``lengths`` (list of (sq, sk)) makes a packed varlen batch;
    ``key_offsets`` (seqlen_k values, fixed-length batches only) shapes the scores per key."""
    dv = head_dim if head_dim_v is None else head_dim_v
    scale = 1.0 / math.sqrt(head_dim) if softmax_scale is None else softmax_scale
    cu = None
    lens: List[Tuple[int, int]] = []
    if lengths is not None:
        lens = [(int(a), int(b)) for a, b in lengths]
        batch = len(lens)
        cq = np.concatenate([[0], np.cumsum([a for a, _ in lens])]).astype(np.int64)
        ck = np.concatenate([[0], np.cumsum([b for _, b in lens])]).astype(np.int64)
        cu = np.concatenate([cq, ck]).astype(np.int32)
        seqlen_q = max([a for a, _ in lens] + [0])
        seqlen_k = max([b for _, b in lens] + [0])
        total_q, total_k = int(cq[-1]), int(ck[-1])
    else:
        lens = [(seqlen_q, seqlen_k)] * batch
        total_q, total_k = batch * seqlen_q, batch * seqlen_k
    g = torch.Generator().manual_seed(seed)
    mult = 1.0 if dtype == "bf16" else fp8_mult
    xq = _randn(g, (total_q, heads_q, head_dim), mult * q_mult)
    xk = _randn(g, (total_k, heads_kv, head_dim), mult)
    xv = _randn(g, (total_k, heads_kv, dv), mult)
    if key_offsets is not None:
        offs = np.asarray(key_offsets, dtype=np.float64).reshape(-1)
        if lengths is not None or offs.shape[0] != seqlen_k:
            raise ValueError("key_offsets needs a fixed-length batch and one value per key")
        b0 = torch.from_numpy(offs / (scale * math.log2(math.e))).float()
        xq[:, :, 0] = 1.0
        xk[:, :, 0] = b0.repeat(batch)[:, None]
    if dtype == "bf16":
        q, k, v = (x.to(torch.bfloat16) for x in (xq, xk, xv))
        descales = None
    elif dtype == "e4m3":
        q, dq = _quant_e4m3(xq)
        k, dk = _quant_e4m3(xk)
        v, dvs = _quant_e4m3(xv)
        descales = np.array([dq, dk, dvs], dtype=np.float32)
    else:
        raise ValueError(dtype)
    return Workload(name=name, batch=batch, heads_q=heads_q, heads_kv=heads_kv, seqlen_q=seqlen_q,
                    seqlen_k=seqlen_k, head_dim=head_dim, head_dim_v=dv, softmax_scale=scale,
                    causal=causal, dtype=dtype, q=q, k=k, v=v, cu_seqlens=cu, descales=descales,
                    seed=seed, lengths=lens)


@dataclass
class KVCacheCase:
    """Inputs of one KV-cache forward: q [B, Sq, Hq, D], caches [B, cap, Hkv, D], new rows
    [B, Snew, Hkv, D] (None when Snew = 0), cache_seqlens int32[B]; raw codes (bf16, or e4m3
    uint8 with descales float32[3] shared by the cache and the new rows)."""
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    k_new: Optional[torch.Tensor]
    v_new: Optional[torch.Tensor]
    cache_seqlens: np.ndarray
    softmax_scale: float
    causal: bool
    dtype: str
    descales: Optional[np.ndarray] = None


def make_kvcache(batch: int, seqlen_q: int, seqlen_new: int, capacity: int, cache_seqlens,
                 heads_q: int, heads_kv: int, head_dim: int, *, causal: bool, seed: int,
                 dtype: str = "bf16", fp8_mult: float = 0.5) -> KVCacheCase:
    """Seeded KV-cache inputs, drawn in the order q, k_cache, v_cache, k_new, v_new.  The whole
    cache is filled with data (rows past cache_seqlens too), so a kernel that reads beyond
    the used length gives a wrong answer instead of a lucky zero.  fp8: one descale per
    tensor family, taken over the cache and the new rows together (a cache has one scale)."""
    g = torch.Generator().manual_seed(seed)
    scale = 1.0 / math.sqrt(head_dim)
    shp_q = (batch, seqlen_q, heads_q, head_dim)
    shp_c = (batch, capacity, heads_kv, head_dim)
    shp_n = (batch, seqlen_new, heads_kv, head_dim)
    lens = np.asarray(cache_seqlens, dtype=np.int32).reshape(batch)
    if dtype == "bf16":
        q = _randn(g, shp_q).to(torch.bfloat16)
        kc = _randn(g, shp_c).to(torch.bfloat16)
        vc = _randn(g, shp_c).to(torch.bfloat16)
        kn = _randn(g, shp_n).to(torch.bfloat16)
        vn = _randn(g, shp_n).to(torch.bfloat16)
        descales = None
    elif dtype == "e4m3":
        q, dq = _quant_e4m3(_randn(g, shp_q, fp8_mult))
        k_all, dk = _quant_e4m3(torch.cat([_randn(g, shp_c, fp8_mult).reshape(-1),
                                           _randn(g, shp_n, fp8_mult).reshape(-1)]))
        v_all, dvs = _quant_e4m3(torch.cat([_randn(g, shp_c, fp8_mult).reshape(-1),
                                            _randn(g, shp_n, fp8_mult).reshape(-1)]))
        nc = int(np.prod(shp_c))
        kc, kn = k_all[:nc].reshape(shp_c).contiguous(), k_all[nc:].reshape(shp_n).contiguous()
        vc, vn = v_all[:nc].reshape(shp_c).contiguous(), v_all[nc:].reshape(shp_n).contiguous()
        descales = np.array([dq, dk, dvs], dtype=np.float32)
    else:
        raise ValueError(dtype)
    if seqlen_new == 0:
        kn = vn = None
    return KVCacheCase(q=q, k_cache=kc, v_cache=vc, k_new=kn, v_new=vn, cache_seqlens=lens,
                       softmax_scale=scale, causal=causal, dtype=dtype, descales=descales)


def varlen_lengths(seed: int = 4, n_long_k: int = 16, n_short_k: int = 2) -> List[Tuple[int, int]]:
    """16 sequences with sq ~ U{128..4096}, sk = sq + U{0..512}; 2 with sk = sq - U{1..min(512, sq-1)}
    (their first rows see no key under bottom-right causal alignment); order shuffled."""
    rng = np.random.default_rng(seed)
    lens = []
    for _ in range(n_long_k):
        sq = int(rng.integers(128, 4097))
        lens.append((sq, sq + int(rng.integers(0, 513))))
    for _ in range(n_short_k):
        sq = int(rng.integers(128, 4097))
        lens.append((sq, sq - int(rng.integers(1, min(512, sq - 1) + 1))))
    order = rng.permutation(len(lens))
    return [lens[i] for i in order]


# The five named workloads (seeds 1..5).
WORKLOADS = {
    "tiny_b1_h2_s256_d64": dict(batch=1, heads_q=2, heads_kv=2, seqlen_q=256, seqlen_k=256,
                                head_dim=64, causal=False, seed=1),
    "mha_b4_h16_s1024_d128": dict(batch=4, heads_q=16, heads_kv=16, seqlen_q=1024, seqlen_k=1024,
                                  head_dim=128, causal=False, seed=2),
    "mha_causal_b4_h16_s1024_d128": dict(batch=4, heads_q=16, heads_kv=16, seqlen_q=1024,
                                         seqlen_k=1024, head_dim=128, causal=True, seed=2),
    "gqa_causal_b2_hq32_hkv8_s8192_d128": dict(batch=2, heads_q=32, heads_kv=8, seqlen_q=8192,
                                               seqlen_k=8192, head_dim=128, causal=True, seed=3),
    "varlen_causal_18seq_h16_d128": dict(batch=18, heads_q=16, heads_kv=16, seqlen_q=0, seqlen_k=0,
                                         head_dim=128, causal=True, seed=4, varlen=True),
    "fp8_causal_b1_h32_s16384_d128": dict(batch=1, heads_q=32, heads_kv=32, seqlen_q=16384,
                                          seqlen_k=16384, head_dim=128, causal=True, seed=5,
                                          dtype="e4m3"),
}


def workload(name: str) -> Workload:
    cfg = dict(WORKLOADS[name])
    varlen = cfg.pop("varlen", False)
    if varlen:
        lens = varlen_lengths(cfg["seed"])
        return make(cfg["batch"], cfg["heads_q"], cfg["heads_kv"], 0, 0, cfg["head_dim"],
                    causal=cfg["causal"], seed=cfg["seed"], lengths=lens, name=name)
    return make(name=name, **cfg)
