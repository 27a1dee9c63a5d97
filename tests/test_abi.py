"""Host-side checks of libfa_fwd.so (no GPU): exported symbols, argument
validation before any HIP call, the shared-memory screen against the page's
worked figures, and the planner."""
import ctypes
import json
import math
import os
import re

import pytest

import exact_attention_forward_fa_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KIB = 1024


def declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"fa_fwd", "fa_strerror", "fa_fwd_plan", "fa_smem_screen", "fa_gfx950_limits"} <= set(names)
    lib = ctypes.CDLL(fa.library_path())
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


def test_strerror_covers_codes():
    for code in (0, -1, -2, -3, -4):
        assert fa.fa_strerror(code) and "unknown" not in fa.fa_strerror(code)
    assert "unknown" in fa.fa_strerror(-99)


# Non-zero fake addresses: validation must reject these calls before touching them.
P = 0x1000


def call(**kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, batch=1, heads_q=4, heads_kv=2, seqlen_q=128,
                seqlen_k=128, cu_seqlens=None, head_dim=128, head_dim_v=128, softmax_scale=0.1,
                causal=0, descales=None, stream=0)
    args.update(kw)
    try:
        return fa.fa_fwd(**args)
    except fa.FaError as e:
        return e.code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), fa.FA_ERR_NULL),
    (dict(k=None), fa.FA_ERR_NULL),
    (dict(v=None), fa.FA_ERR_NULL),
    (dict(o=None), fa.FA_ERR_NULL),
    (dict(lse=None), fa.FA_ERR_NULL),
    (dict(batch=0), fa.FA_ERR_INVALID),
    (dict(heads_q=0), fa.FA_ERR_INVALID),
    (dict(heads_kv=0), fa.FA_ERR_INVALID),
    (dict(heads_q=6, heads_kv=4), fa.FA_ERR_INVALID),
    (dict(seqlen_q=-1), fa.FA_ERR_INVALID),
    (dict(seqlen_k=-5), fa.FA_ERR_INVALID),
    (dict(softmax_scale=0.0), fa.FA_ERR_INVALID),
    (dict(softmax_scale=-0.1), fa.FA_ERR_INVALID),
    (dict(softmax_scale=math.inf), fa.FA_ERR_INVALID),
    (dict(softmax_scale=math.nan), fa.FA_ERR_INVALID),
    (dict(causal=2), fa.FA_ERR_INVALID),
    (dict(head_dim=96, head_dim_v=96), fa.FA_ERR_UNSUPPORTED),
    (dict(head_dim=256, head_dim_v=256), fa.FA_ERR_UNSUPPORTED),
    (dict(head_dim=128, head_dim_v=64), fa.FA_ERR_UNSUPPORTED),
    (dict(head_dim=0), fa.FA_ERR_INVALID),
    # one sequence's K (or V) must stay below 2 GiB: bf16, 2 KV heads x 128 x 2 B per key
    (dict(seqlen_k=(1 << 31) // (2 * 128 * 2)), fa.FA_ERR_UNSUPPORTED),
    # fp8: one byte per element, so twice the keys
    (dict(seqlen_k=(1 << 31) // (2 * 128), descales=P), fa.FA_ERR_UNSUPPORTED),
    # fixed-length row offsets are 32-bit
    (dict(batch=2, seqlen_q=1 << 30), fa.FA_ERR_UNSUPPORTED),
])
def test_validation_before_any_hip_call(kw, code):
    assert call(**kw) == code


def test_empty_problem_is_a_no_op():
    # no query rows: nothing to launch, so no device is needed either
    assert call(q=None, o=None, lse=None, seqlen_q=0) == fa.FA_OK
    # the same for a packed batch whose longest query length is 0
    assert call(q=None, o=None, lse=None, seqlen_q=0, cu_seqlens=P) == fa.FA_OK


@pytest.mark.parametrize("varlen", [False, True])
def test_null_keys_only_without_keys(varlen):
    """K and V may be NULL exactly when the (largest) key length is 0, Q/O/LSE when the
    (largest) query length is 0: otherwise the call is refused before any HIP call.  (The
    accepted form is checked here without query rows, so that nothing is launched on these
    fake addresses; the GPU sweep runs a packed batch without keys on real buffers.)"""
    cu = P if varlen else None
    assert call(k=None, v=None, seqlen_k=1, cu_seqlens=cu) == fa.FA_ERR_NULL
    assert call(q=None, seqlen_q=1, cu_seqlens=cu) == fa.FA_ERR_NULL
    assert call(q=None, o=None, lse=None, k=None, v=None, seqlen_q=0, seqlen_k=0,
                cu_seqlens=cu) == fa.FA_OK


def _limits(name, fx):
    d = fx["devices"][name]
    L = fa.DeviceLimits()
    L.lds_bytes_per_block = d["per_block_kib"] * KIB
    L.lds_bytes_per_cu = d["per_sm_kib"] * KIB
    L.num_cus, L.simds_per_cu, L.regs_per_simd_lane, L.max_waves_per_simd = 1, 4, 512, 8
    return L


@pytest.fixture(scope="module")
def fixtures():
    with open(os.path.join(ROOT, "tests", "golden", "smem_screen_page_fixtures.json")) as f:
        return json.load(f)


def test_screen_reproduces_page_tile_figures(fixtures):
    for case in fixtures["tile_cases"]:
        cfg = fa.TileConfig(**case["cfg"])
        for dev, fits in case["fits"].items():
            s = fa.fa_smem_screen(cfg, _limits(dev, fixtures))
            assert s.smem_bytes == case["smem_kib"] * KIB
            assert bool(s.fits) == fits, (case, dev)


def _block_cfg(kib):
    # a configuration whose buffers total exactly `kib` KiB: Q (kib-2) KiB + K 1 KiB + V 1 KiB
    return fa.TileConfig(tile_m=kib - 2, tile_n=1, head_dim=1, head_dim_v=1, elem_bytes=KIB,
                         kv_stages=1, q_in_regs=0)


def test_screen_reproduces_page_block_examples(fixtures):
    for case in fixtures["block_cases"]:
        cfg = _block_cfg(case["block_kib"])
        for dev, fits in case["fits"].items():
            s = fa.fa_smem_screen(cfg, _limits(dev, fixtures))
            assert s.smem_bytes == case["block_kib"] * KIB
            assert bool(s.fits) == fits, (case, dev)
        for dev, n in case.get("blocks_per_sm", {}).items():
            assert fa.fa_smem_screen(cfg, _limits(dev, fixtures)).blocks_per_cu == n, (case, dev)


def test_screen_q_in_regs_takes_max_of_q_and_v():
    # Q and V buffers have disjoint lifetimes when Q lives in registers: K + max(Q, V)
    cfg = fa.TileConfig(tile_m=128, tile_n=128, head_dim=128, head_dim_v=128, elem_bytes=2,
                        kv_stages=1, q_in_regs=1)
    s = fa.fa_smem_screen(cfg, fa.fa_gfx950_limits())
    assert s.smem_bytes == 64 * KIB


def test_screen_gfx950_answers():
    g = fa.fa_gfx950_limits()
    assert g.lds_bytes_per_block == 160 * KIB and g.lds_bytes_per_cu == 160 * KIB
    one = fa.TileConfig(tile_m=128, tile_n=128, head_dim=128, head_dim_v=128, elem_bytes=2,
                        kv_stages=1, q_in_regs=0)
    two = fa.TileConfig(tile_m=128, tile_n=128, head_dim=128, head_dim_v=128, elem_bytes=2,
                        kv_stages=2, q_in_regs=0)
    s1, s2 = fa.fa_smem_screen(one, g), fa.fa_smem_screen(two, g)
    assert (s1.fits, s1.blocks_per_cu) == (1, 1)   # 96 KiB
    assert (s2.fits, s2.blocks_per_cu) == (1, 1)   # 160 KiB: exactly the gfx950 limit
    assert fa.fa_smem_screen(_block_cfg(72), g).blocks_per_cu == 2
    assert fa.fa_smem_screen(_block_cfg(161), g).fits == 0


def call_kv(**kw):
    args = dict(q=P, k_cache=P, v_cache=P, k_new=P, v_new=P, o=P, lse=P, batch=2, heads_q=4,
                heads_kv=2, seqlen_q=16, seqlen_new=4, cache_capacity=64, cache_seqlens=P,
                head_dim=128, head_dim_v=128, softmax_scale=0.1, causal=1, descales=None, stream=0)
    args.update(kw)
    try:
        return fa.fa_fwd_kvcache(**args)
    except fa.FaError as e:
        return e.code


@pytest.mark.parametrize("kw,code", [
    (dict(cache_seqlens=None), fa.FA_ERR_NULL),
    (dict(k_new=None), fa.FA_ERR_NULL),
    (dict(v_new=None), fa.FA_ERR_NULL),
    (dict(k_cache=None), fa.FA_ERR_NULL),
    (dict(v_cache=None), fa.FA_ERR_NULL),
    (dict(q=None), fa.FA_ERR_NULL),
    (dict(o=None), fa.FA_ERR_NULL),
    (dict(lse=None), fa.FA_ERR_NULL),
    (dict(seqlen_new=-1), fa.FA_ERR_INVALID),
    (dict(cache_capacity=-1), fa.FA_ERR_INVALID),
    (dict(batch=0), fa.FA_ERR_INVALID),
    (dict(heads_q=6, heads_kv=4), fa.FA_ERR_INVALID),
    (dict(softmax_scale=0.0), fa.FA_ERR_INVALID),
    (dict(causal=2), fa.FA_ERR_INVALID),
    (dict(head_dim=96, head_dim_v=96), fa.FA_ERR_UNSUPPORTED),
    # one sequence's cache must fit the 31-bit byte range of a buffer resource
    (dict(cache_capacity=(1 << 31) // (2 * 128 * 2)), fa.FA_ERR_UNSUPPORTED),
])
def test_kvcache_validation_before_any_hip_call(kw, code):
    assert call_kv(**kw) == code


def test_screen_rejects_bad_sizes():
    cfg = fa.TileConfig(tile_m=0, tile_n=64, head_dim=128, head_dim_v=128, elem_bytes=2,
                        kv_stages=1, q_in_regs=0)
    with pytest.raises(fa.FaError):
        fa.fa_smem_screen(cfg, fa.fa_gfx950_limits())


def test_plan_gfx950():
    # GQA with an even group: the ping-pong schedule, 8 waves holding 128 rows of two query
    # heads, one workgroup per CU (2 waves per SIMD at 256 registers)
    p = fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 2, 32, 8, 8192, 8192, False, 128, 128, True)
    assert (p.schedule, p.tile_m, p.tile_n, p.waves, p.kv_stages) == (3, 128, 64, 8, 2)
    assert (p.query_tiles, p.heads_per_workgroup, p.wg_per_cu, p.vgprs_per_lane) == (1, 2, 1, 256)
    assert p.lds_bytes == 64 * KIB
    # 16 (batch, kv-head) pairs = 2 rounds over 8 XCDs, x 64 tiles x 2 head pairs per kv-head
    assert p.m_tiles == 64 and p.num_workgroups == 2 * 8 * 64 * 2
    # MHA (heads_q / heads_kv = 1) with at least one workgroup per CU: still the ping-pong
    # schedule, its two groups on two adjacent 128-row tiles of one head (256 rows per
    # workgroup); 64 (batch, head) pairs = 8 rounds over the XCDs x 4 tile pairs
    pm = fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 4, 16, 16, 1024, 1024, False, 128, 128, True)
    assert (pm.schedule, pm.tile_m, pm.query_tiles, pm.wg_per_cu, pm.vgprs_per_lane) == \
        (3, 256, 1, 1, 256)
    assert (pm.waves, pm.heads_per_workgroup, pm.m_tiles, pm.num_workgroups) == (8, 1, 4, 8 * 8 * 4)
    # 2100 rows: 17 tiles of 128 rows = 9 tile pairs (the upper tile of the last pair is empty)
    p2100 = fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 4, 16, 16, 2100, 2100, False, 128, 128, False)
    assert (p2100.schedule, p2100.m_tiles, p2100.num_workgroups) == (3, 9, 8 * 8 * 9)
    # fewer ping-pong workgroups than CUs: schedule 1's finer grid (one query tile per wave);
    # 2 (batch, kv-head) pairs, fewer than the 8 XCDs: their 2 tiles x 1 head each are spread
    # over all XCDs (4 items, padded to 8) instead of being dealt to 2 of them
    p64 = fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 1, 2, 2, 256, 256, False, 64, 64, False)
    assert (p64.schedule, p64.tile_m, p64.query_tiles, p64.wg_per_cu, p64.vgprs_per_lane) == \
        (1, 128, 1, 2, 256)
    assert p64.m_tiles == 2 and p64.num_workgroups == 8 and p64.lds_bytes < p.lds_bytes
    # 12 pairs: one round of 8 dealt to the XCDs (8 x 8 tiles) after the 4 others' items
    # spread over all XCDs (4 x 8 tiles = 32, a multiple of 8)
    p12 = fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 3, 4, 4, 1024, 1024, False, 128, 128, True)
    assert (p12.schedule, p12.m_tiles, p12.num_workgroups) == (1, 8, 32 + 8 * 8)
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 1, 8, 2, 512, 512, False, 128, 128, True).schedule == 1
    # causal tile pairs over several rounds below 6144 rows: schedule 1; non-causal: pairs
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 4, 16, 16, 2048, 2048, False, 128, 128, True).schedule == 1
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 4, 16, 16, 4096, 4096, False, 128, 128, True).schedule == 1
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 2, 16, 16, 6144, 6144, False, 128, 128, True).schedule == 3
    # grids below one workgroup per CU: non-causal ones of more than half a round take the
    # ping-pong, causal ones schedule 1
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 1, 16, 16, 3072, 3072, False, 128, 128, False).schedule == 3
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 1, 16, 4, 3072, 3072, False, 128, 128, False).schedule == 3
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 1, 8, 8, 4096, 4096, False, 128, 128, False).schedule == 1
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 1, 16, 16, 3072, 3072, False, 128, 128, True).schedule == 1
    # head_dim 64: schedule 1 wherever the ping-pong would otherwise be taken
    for args in ((2, 32, 8, 8192, True), (2, 32, 8, 8192, False), (2, 16, 16, 8192, True),
                 (4, 16, 16, 4096, False), (2, 16, 16, 2048, False)):
        b_, hq, hkv, s_, c = args
        assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, b_, hq, hkv, s_, s_, False, 128, 128, c).schedule == 3
        assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, b_, hq, hkv, s_, s_, False, 64, 64, c).schedule == 1
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 4, 16, 16, 2048, 2048, False, 128, 128, False).schedule == 3
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 2, 24, 8, 8192, 8192, False, 128, 128, True).schedule == 3
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 4, 24, 8, 2048, 2048, False, 128, 128, True).schedule == 1
    # head pairs below 2048 rows over several rounds: schedule 1; one round or 2048+: ping-pong
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 8, 32, 8, 1024, 1024, False, 128, 128, True).schedule == 1
    # without causal masking from 1024 rows
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 8, 32, 8, 1024, 1024, False, 128, 128, False).schedule == 3
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 8, 16, 16, 1024, 1024, False, 128, 128, False).schedule == 3
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 32, 16, 16, 512, 512, False, 128, 128, False).schedule == 1
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 4, 32, 8, 2048, 2048, False, 128, 128, True).schedule == 3
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 2, 32, 8, 1024, 1024, False, 128, 128, True).schedule == 3
    # packed varlen MHA stays on schedule 1 (128-row tiles, two workgroups per CU)
    pv = fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 18, 16, 16, 4096, 4608, True, 128, 128, True)
    assert (pv.schedule, pv.tile_m, pv.wg_per_cu) == (1, 128, 2)
    # fp8 always uses schedule 1
    p8 = fa.fa_fwd_plan(fa.FA_DTYPE_E4M3, 1, 32, 8, 16384, 16384, False, 128, 128, True)
    assert (p8.schedule, p8.tile_m, p8.query_tiles, p8.lds_bytes) == (1, 128, 1, 32 * KIB)
    # decode: 4 query heads per KV head x 1 row fit one 32-column tile; one workgroup of 4
    # waves per (sequence, kv-head), a 2-slot ring of 32-key K and V blocks per wave in LDS
    pd = fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 32, 32, 8, 1, 8192, False, 128, 128, True)
    assert (pd.schedule, pd.tile_m, pd.tile_n, pd.waves, pd.kv_stages) == (4, 32, 32, 4, 2)
    assert (pd.num_workgroups, pd.heads_per_workgroup, pd.wg_per_cu, pd.vgprs_per_lane) == \
        (32 * 8, 4, 1, 512)
    assert pd.lds_bytes == 4 * (2 * 2 * 32 * 128 * 2)
    # 8 heads x 4 rows = 32 columns still fits; 8 x 5 does not
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 1, 8, 1, 4, 100, False, 64, 64, False).schedule == 4
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 1, 8, 1, 5, 100, False, 64, 64, False).schedule == 1
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 64, 8, 1, 5, 100, False, 128, 128, False).schedule == 3
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 64, 8, 1, 5, 100, False, 64, 64, False).schedule == 1
    # a single causal round over at most 8 (sequence, kv-head) pairs: schedule 1; 16 pairs: 3
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 1, 32, 8, 2048, 2048, False, 128, 128, True).schedule == 1
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 1, 32, 1, 2048, 2048, False, 128, 128, True).schedule == 1
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 2, 16, 8, 2048, 2048, False, 128, 128, True).schedule == 3
    assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 1, 32, 8, 2048, 2048, False, 128, 128, False).schedule == 3
    # fp8 never takes it
    assert fa.fa_fwd_plan(fa.FA_DTYPE_E4M3, 32, 32, 8, 1, 8192, False, 128, 128, True).schedule == 1


def test_schedule_override():
    args = (fa.FA_DTYPE_BF16, 2, 32, 8, 8192, 8192, False, 128, 128, True)
    try:
        fa.fa_set_schedule(1)
        p = fa.fa_fwd_plan(*args)
        assert (p.schedule, p.tile_m, p.waves, p.m_tiles, p.wg_per_cu) == (1, 128, 4, 64, 2)
        assert p.num_workgroups == 2 * 8 * 64 * 4
        fa.fa_set_schedule(2)
        p = fa.fa_fwd_plan(*args)
        assert (p.schedule, p.tile_m, p.query_tiles, p.m_tiles, p.wg_per_cu, p.vgprs_per_lane) == \
            (2, 256, 2, 32, 1, 512)
        assert p.num_workgroups == 2 * 8 * 32 * 4
        # schedule 3 with an odd heads_q / heads_kv: two adjacent query tiles of one head
        fa.fa_set_schedule(3)
        odd = fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 1, 3, 1, 300, 300, False, 64, 64, False)
        assert (odd.schedule, odd.waves, odd.heads_per_workgroup, odd.tile_m) == (3, 8, 1, 256)
        # one (batch, kv-head) pair: its 2 tile pairs x 3 heads spread over the XCDs, 6 -> 8
        assert (odd.m_tiles, odd.num_workgroups) == (2, 8)
        # ... but not for packed varlen batches: falls back to 1
        oddv = fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 1, 3, 1, 300, 300, True, 64, 64, False)
        assert (oddv.schedule, oddv.waves, oddv.heads_per_workgroup) == (1, 4, 1)
        # fp8 always uses 1
        p8 = fa.fa_fwd_plan(fa.FA_DTYPE_E4M3, 1, 2, 1, 300, 300, False, 64, 64, False)
        assert p8.schedule == 1
        # schedule 4 needs heads_q / heads_kv * seqlen_q <= 32: falls back to 1
        fa.fa_set_schedule(4)
        assert fa.fa_fwd_plan(*args).schedule == 1
        assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 2, 32, 8, 1, 8192, False, 128, 128,
                              True).schedule == 4
        # schedule 5: schedule 3's items on resident workgroups -- one per CU (a whole
        # number per XCD), at most one per item; the LDS holds a Q stage of 32 rows per wave
        fa.fa_set_schedule(5)
        p = fa.fa_fwd_plan(*args)
        assert (p.schedule, p.waves, p.tile_m, p.heads_per_workgroup, p.m_tiles) == (5, 8, 128, 2, 64)
        assert (p.num_workgroups, p.wg_per_cu) == (256, 1)
        assert p.lds_bytes == 4 * 64 * 128 * 2 + 8 * 32 * 128 * 2
        small = fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 1, 4, 2, 256, 256, False, 64, 64, True)
        assert (small.schedule, small.num_workgroups) == (5, 8)  # 2 pairs x 2 tiles, padded
        # where schedule 3 does not apply (fp8, odd groups in packed batches): 1
        assert fa.fa_fwd_plan(fa.FA_DTYPE_E4M3, 2, 32, 8, 8192, 8192, False, 128, 128,
                              True).schedule == 1
        assert fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 1, 3, 1, 300, 300, True, 64, 64,
                              False).schedule == 1
        # a device with fewer CUs than XCDs cannot hold a whole number per XCD
        lim = fa.fa_gfx950_limits()
        lim.num_cus = 4
        p4 = fa.fa_fwd_plan(*args, dev=lim)
        assert p4.schedule == 1
        for bad in (-1, 6):
            with pytest.raises(fa.FaError) as e:
                fa.fa_set_schedule(bad)
            assert e.value.code == fa.FA_ERR_INVALID
    finally:
        fa.fa_set_schedule(0)
    assert fa.fa_fwd_plan(*args).schedule == 3


def test_exp2_offload_setting():
    try:
        for ok in (4, 8, 0):
            fa.fa_set_exp2_offload(ok)
        for bad in (-1, 1, 2, 3, 5, 16):
            with pytest.raises(fa.FaError) as e:
                fa.fa_set_exp2_offload(bad)
            assert e.value.code == fa.FA_ERR_INVALID
    finally:
        fa.fa_set_exp2_offload(0)


def test_fp8_exact_scores_setting():
    try:
        for ok in (1, 0):
            fa.fa_set_fp8_exact_scores(ok)
        for bad in (-1, 2, 8):
            with pytest.raises(fa.FaError) as e:
                fa.fa_set_fp8_exact_scores(bad)
            assert e.value.code == fa.FA_ERR_INVALID
    finally:
        fa.fa_set_fp8_exact_scores(0)


def test_plan_reports_unsupported_when_nothing_fits():
    small = fa.DeviceLimits(lds_bytes_per_block=48 * KIB, lds_bytes_per_cu=48 * KIB, num_cus=1,
                            simds_per_cu=4, regs_per_simd_lane=512, max_waves_per_simd=8)
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 1, 4, 4, 1024, 1024, False, 128, 128, True, small)
    assert e.value.code == fa.FA_ERR_UNSUPPORTED


def test_one_hip_runtime_when_package_is_imported_before_torch():
    """Importing the package first must not leave two HIP runtimes in the process."""
    import subprocess
    import sys

    code = ("import exact_attention_forward_fa_amd, torch\n"
            "paths = set()\n"
            "for line in open('/proc/self/maps'):\n"
            "    if 'libamdhip64' in line:\n"
            "        paths.add(os.path.realpath(line.split()[-1]))\n"
            "print(len(paths), sorted(paths))\n")
    r = subprocess.run([sys.executable, "-c", "import os\n" + code], capture_output=True, text=True,
                       cwd=ROOT)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split()[0] == "1", r.stdout


# ---------------------------------------------------------------- cu_seqlens validator

def _cu(q_lens, k_lens):
    import numpy as np

    return np.concatenate([np.concatenate([[0], np.cumsum(q_lens)]),
                           np.concatenate([[0], np.cumsum(k_lens)])]).astype(np.int32)


def check_cu(cu, batch, sq, sk, rows_q, rows_k):
    try:
        fa.fa_check_cu_seqlens(cu, batch, sq, sk, rows_q, rows_k)
        return fa.FA_OK
    except fa.FaError as e:
        return e.code


def test_cu_seqlens_validator_accepts_packed_batches():
    cu = _cu([300, 1, 0, 129], [517, 64, 40, 0])
    assert check_cu(cu, 4, 300, 517, 430, 621) == fa.FA_OK
    assert check_cu(cu, 4, 300, 517, 430, 10_000) == fa.FA_OK  # K/V may be longer than used
    # the named varlen workload's offsets
    import fa_inputs

    lens = fa_inputs.varlen_lengths(4)
    cu = _cu([a for a, _ in lens], [b for _, b in lens])
    assert check_cu(cu, len(lens), max(a for a, _ in lens), max(b for _, b in lens),
                    int(cu[len(lens)]), int(cu[-1])) == fa.FA_OK


@pytest.mark.parametrize("case", ["q_start", "k_start", "q_decreasing", "k_decreasing", "q_over_max",
                                  "k_over_max", "rows_q_short", "rows_q_long", "rows_k_short",
                                  "wrong_length", "batch0"])
def test_cu_seqlens_validator_rejects(case):
    """Every condition of the contract has its own rejection (FA_ERR_INVALID), before anything is
    launched: offsets that do not start at 0, that decrease, lengths above the maxima, and a
    total that does not match the rows of Q (and of each LSE row) or exceeds the rows of K/V."""
    base = _cu([100, 50, 7], [120, 60, 7])
    cu, batch, sq, sk, rq, rk = base.copy(), 3, 100, 120, 157, 187
    if case == "q_start":
        cu[:4] += 1
        rq += 1
    elif case == "k_start":
        cu[4:] += 1
        rk += 1
    elif case == "q_decreasing":
        cu[2] = cu[1] - 1
    elif case == "k_decreasing":
        cu[6] = cu[5] - 1
    elif case == "q_over_max":
        sq = 99
    elif case == "k_over_max":
        sk = 119
    elif case == "rows_q_short":
        rq = 156
    elif case == "rows_q_long":
        rq = 158  # LSE rows are cu[batch] long: a padded q would stride LSE wrongly
    elif case == "rows_k_short":
        rk = 186
    elif case == "wrong_length":
        cu = cu[:-1]
    elif case == "batch0":
        batch = 0
        cu = cu[:2]
    assert check_cu(cu, batch, sq, sk, rq, rk) == fa.FA_ERR_INVALID


def test_cu_seqlens_validator_null():
    lib = ctypes.CDLL(fa.library_path())
    lib.fa_check_cu_seqlens.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int64, ctypes.c_int64]
    assert lib.fa_check_cu_seqlens(None, 1, 1, 1, 1, 1) == fa.FA_ERR_NULL
