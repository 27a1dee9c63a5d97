"""Pins of the oracle's KV-cache forward (CPU only): the append step against its
definition, and the attention step reduced to the already pinned plain forward and to a
float64 SDPA written out for the bottom-right causal case."""
import numpy as np
import torch

import oracle


def _bf16(shape, gen):
    return torch.randn(*shape, generator=gen).to(torch.bfloat16)


def test_append_places_rows_and_drops_out_of_range():
    g = torch.Generator().manual_seed(11)
    kc, vc = _bf16((3, 6, 2, 64), g), _bf16((3, 6, 2, 64), g)
    kn, vn = _bf16((3, 3, 2, 64), g), _bf16((3, 3, 2, 64), g)
    lens = [0, 4, 6]
    k2, v2, used = oracle.append_kv(kc, vc, kn, vn, lens)
    bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    kcb, knb, vnb = bits(kc), bits(kn), bits(vn)
    # b = 0: rows 0..2 replaced; b = 1: rows 4, 5 replaced, the third new row dropped;
    # b = 2: full cache, every new row dropped
    assert np.array_equal(k2[0, :3], knb[0]) and np.array_equal(k2[0, 3:], kcb[0, 3:])
    assert np.array_equal(k2[1, 4:6], knb[1, :2]) and np.array_equal(k2[1, :4], kcb[1, :4])
    assert np.array_equal(k2[2], kcb[2])
    assert np.array_equal(v2[1, 4:6], vnb[1, :2])
    assert list(used) == [3, 6, 6]


def test_two_appends_equal_one():
    g = torch.Generator().manual_seed(12)
    kc, vc = _bf16((2, 16, 1, 64), g), _bf16((2, 16, 1, 64), g)
    kn, vn = _bf16((2, 5, 1, 64), g), _bf16((2, 5, 1, 64), g)
    lens = np.array([3, 9])
    ka, va, _ = oracle.append_kv(kc, vc, kn[:, :2].contiguous(), vn[:, :2].contiguous(), lens)
    kb, vb, used = oracle.append_kv(ka, va, kn[:, 2:].contiguous(), vn[:, 2:].contiguous(), lens + 2)
    k1, v1, used1 = oracle.append_kv(kc, vc, kn, vn, lens)
    assert np.array_equal(kb, k1) and np.array_equal(vb, v1) and list(used) == list(used1)


def test_full_cache_from_empty_is_the_plain_forward():
    """cache_seqlens = 0 and Snew = capacity: attention over exactly the new keys."""
    g = torch.Generator().manual_seed(13)
    b, sq, s, hq, hkv, d = 2, 7, 9, 4, 2, 64
    q = _bf16((b, sq, hq, d), g)
    kn, vn = _bf16((b, s, hkv, d), g), _bf16((b, s, hkv, d), g)
    kc = torch.zeros((b, s, hkv, d), dtype=torch.bfloat16)
    for causal in (False, True):
        o, lse, _, _ = oracle.attention_kvcache(q, kc, kc.clone(), kn, vn, [0, 0],
                                                softmax_scale=0.125, causal=causal)
        ro, rl = oracle.attention(q.reshape(b * sq, hq, d), kn.reshape(b * s, hkv, d),
                                  vn.reshape(b * s, hkv, d), batch=b, heads_q=hq, heads_kv=hkv,
                                  seqlen_q=sq, seqlen_k=s, head_dim=d, head_dim_v=d,
                                  softmax_scale=0.125, causal=causal)
        assert np.array_equal(o, ro) and np.array_equal(lse, rl)


def test_cached_prefix_against_float64_sdpa():
    """A cache with a prefix plus new rows, bottom-right causal: the last query row sees every
    used key, query i sees keys j <= i + (used - sq); written out with float64 SDPA."""
    g = torch.Generator().manual_seed(14)
    b, sq, cap, hq, d = 1, 4, 12, 2, 64
    q = _bf16((b, sq, hq, d), g)
    kc, vc = _bf16((b, cap, hq, d), g), _bf16((b, cap, hq, d), g)
    kn, vn = _bf16((b, 3, hq, d), g), _bf16((b, 3, hq, d), g)
    o, lse, k2, v2 = oracle.attention_kvcache(q, kc, vc, kn, vn, [5], softmax_scale=0.2, causal=True)
    used = 8
    kf = torch.cat([kc[0, :5], kn[0]]).double()          # [used, H, D]
    vf = torch.cat([vc[0, :5], vn[0]]).double()
    qf = q[0].double()                                    # [sq, H, D]
    allow = torch.arange(used)[None, :] <= torch.arange(sq)[:, None] + (used - sq)
    for h in range(hq):
        s = (qf[:, h] @ kf[:, h].T) * 0.2
        s = s.masked_fill(~allow, float("-inf"))
        ref = torch.softmax(s, dim=-1) @ vf[:, h]
        assert np.allclose(o[:, h], ref.numpy(), rtol=0, atol=1e-12)
        assert np.allclose(lse[h], torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)
    assert np.array_equal(k2[0, 5:8], kn[0].view(torch.int16).numpy().view(np.uint16))
