"""One-pass online-softmax brute force in exp2 form -- TEST INFRASTRUCTURE ONLY.

An independent second reading of the method, used to pin the fp64 oracle
(``fa_oracle.c``) on tiny inputs.  Where the oracle materialises a whole
score row and then normalises it, this walks the keys one at a time and
keeps a running maximum ``m`` (in base-2 units), a running sum ``l`` and an
unnormalised output accumulator, rescaling both by ``alpha = 2**(m_old -
m_new)`` whenever the maximum grows -- the streaming softmax of FlashAttention
(Dao et al. 2022) that the forward-pass page's consumer loop runs tile by tile
(``Softmax`` object with ``softmax_scale_log2``, ``row_sum`` handed to the
epilogue).  Keys are visited from the last to the first, the block order of
that loop (``n_block`` from ``n_block_max - 1`` down to ``n_block_min``), so the
association order differs from the oracle's.

Pure Python loops over float64 inputs that are already decoded; only for
tiny shapes.
"""
from __future__ import annotations

import math

import numpy as np

LOG2E = 1.0 / math.log(2.0)
LN2 = math.log(2.0)


def _seq(b, batch, seqlen_q, seqlen_k, cu):
    if cu is None:
        return b * seqlen_q, seqlen_q, b * seqlen_k, seqlen_k
    cu = [int(x) for x in cu]
    return cu[b], cu[b + 1] - cu[b], cu[batch + 1 + b], cu[batch + 2 + b] - cu[batch + 1 + b]


def online_attention(qd, kd, vd, *, batch, heads_q, heads_kv, seqlen_q, seqlen_k, softmax_scale,
                     causal, cu_seqlens=None, reverse=True):
    """qd [total_q, Hq, D], kd [total_k, Hkv, D], vd [total_k, Hkv, Dv] float64 (decoded).

    Returns (O [total_q, Hq, Dv], LSE [Hq, total_q]).
    """
    qd = np.asarray(qd, dtype=np.float64)
    kd = np.asarray(kd, dtype=np.float64)
    vd = np.asarray(vd, dtype=np.float64)
    total_q = qd.shape[0]
    dv = vd.shape[2]
    out = np.zeros((total_q, heads_q, dv))
    lse = np.zeros((heads_q, total_q))
    group = heads_q // heads_kv
    c = softmax_scale * LOG2E  # scores in base-2 units
    for b in range(batch):
        q0, sq, k0, sk = _seq(b, batch, seqlen_q, seqlen_k, cu_seqlens)
        for h in range(heads_q):
            g = h // group
            for i in range(sq):
                m = -math.inf
                l = 0.0
                acc = [0.0] * dv
                qrow = qd[q0 + i, h, :].tolist()
                keys = range(sk - 1, -1, -1) if reverse else range(sk)
                for j in keys:
                    if causal and j > i + sk - sq:
                        continue
                    krow = kd[k0 + j, g, :].tolist()
                    t = 0.0
                    for a, bb in zip(qrow, krow):
                        t += a * bb
                    t *= c
                    m_new = t if t > m else m
                    alpha = 0.0 if m == -math.inf else 2.0 ** (m - m_new)
                    p = 2.0 ** (t - m_new)
                    l = l * alpha + p
                    vrow = vd[k0 + j, g, :].tolist()
                    for e in range(dv):
                        acc[e] = acc[e] * alpha + p * vrow[e]
                    m = m_new
                if l == 0.0:
                    out[q0 + i, h, :] = 0.0
                    lse[h, q0 + i] = -math.inf
                else:
                    out[q0 + i, h, :] = [a / l for a in acc]
                    lse[h, q0 + i] = (m + math.log2(l)) * LN2
    return out, lse
