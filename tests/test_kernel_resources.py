"""CPU pin of the kernels' resources against the planner (no GPU): the kernel source is
compiled for gfx950 (device pass only) with the compiler's kernel-resource-usage remarks, and
for every kernel instantiation the test asserts no scratch memory, no register spills and no
dynamic stack, a register count within the budget fa_fwd_plan assumes for its schedule, the
occupancy (waves per SIMD) the plan's workgroups per CU need, and an LDS size equal to the
plan's lds_bytes.  A compiler change that makes a kernel spill or lose occupancy fails here."""
import os
import re
import shutil
import subprocess

import pytest

import exact_attention_forward_fa_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "exact_attention_forward_fa_amd", "csrc", "fa_fwd_kernel.hip")


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.fixture(scope="module")
def usage(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not found")
    out = tmp_path_factory.mktemp("res") / "k.o"
    r = subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang",
                        "-target-feature", "-Xclang", "-packed-fp32-ops", "--offload-device-only",
                        "-I", os.path.join(ROOT, "include"), "-Rpass-analysis=kernel-resource-usage",
                        "-c", SRC, "-o", str(out)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?):\s+(\S+)\s+\[-Rpass", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    assert kernels, "no resource remarks parsed"
    return kernels


def _plan(schedule, d, dtype):
    """The planner's figures for a schedule, from a shape that schedule applies to."""
    fa.fa_set_schedule(schedule if dtype == fa.FA_DTYPE_BF16 else 0)
    try:
        if schedule == 4:
            p = fa.fa_fwd_plan(dtype, 32, 32, 8, 1, 8192, False, d, d, True)
        elif dtype == fa.FA_DTYPE_E4M3:
            p = fa.fa_fwd_plan(dtype, 1, 32, 32, 16384, 16384, False, d, d, True)
        else:
            p = fa.fa_fwd_plan(dtype, 2, 32, 8, 8192, 8192, False, d, d, True)
    finally:
        fa.fa_set_schedule(0)
    assert p.schedule == schedule
    return p


def _classify(name):
    """(schedule, head_dim, dtype) of a mangled kernel name, or None for non-attention kernels."""
    m = re.search(r"(fa_fwd_bf16_kernel|fa_fwd_bf16_pp_kernel|fa_fwd_bf16_pp_persist_kernel|"
                  r"fa_fwd_bf16_decode_kernel|fa_fwd_fp8_kernel)ILi(\d+)ELb([01])E(?:Li(\d+)E)?",
                  name)
    if not m:
        return None
    kind, d = m.group(1), int(m.group(2))
    extra = int(m.group(4)) if m.group(4) is not None else None
    if kind == "fa_fwd_bf16_kernel":
        return (1 if extra == 1 else 2), d, fa.FA_DTYPE_BF16
    if kind == "fa_fwd_bf16_pp_kernel":
        return 3, d, fa.FA_DTYPE_BF16
    if kind == "fa_fwd_bf16_pp_persist_kernel":
        return 5, d, fa.FA_DTYPE_BF16
    if kind == "fa_fwd_bf16_decode_kernel":
        return 4, d, fa.FA_DTYPE_BF16
    return 1, d, fa.FA_DTYPE_E4M3


# The non-causal 4-wave kernels (schedules 1 and 2) keep a few wave-uniform values (kernel
# arguments, sequence pointers) across the masked-tail loop in VGPR lanes (v_writelane /
# v_readlane in the prologue, at the loop transition and in the epilogue; no memory, nothing in
# the key-block loop).  The non-causal ping-pong kernels do the same since their steady loop
# runs in pairs of steps with constant buffer offsets (one or two v_readlane per step, measured
# faster than the unpaired loop without them).  The persistent ping-pong kernel (schedule 5, an
# opt-in) carries its item loop's state as well and reloads 20-30 such values per step.  The
# counts are pinned at what the current compiler does, so that an increase fails; every other
# kernel must have none.  Key: (kernel, head_dim, causal, queries per wave for the 4-wave
# kernels / exp2 offload for the ping-pong kernel / None for the persistent one).
SGPR_LANE_SPILLS = {("fa_fwd_bf16_kernel", 128, 0, 1): 21, ("fa_fwd_bf16_kernel", 64, 0, 1): 13,
                    ("fa_fwd_bf16_kernel", 128, 0, 2): 25, ("fa_fwd_bf16_kernel", 64, 0, 2): 16,
                    ("fa_fwd_bf16_pp_kernel", 128, 0, 0): 20, ("fa_fwd_bf16_pp_kernel", 128, 0, 4): 21,
                    ("fa_fwd_bf16_pp_kernel", 128, 0, 8): 21, ("fa_fwd_bf16_pp_kernel", 64, 0, 0): 14,
                    ("fa_fwd_bf16_pp_kernel", 64, 0, 4): 14, ("fa_fwd_bf16_pp_kernel", 64, 0, 8): 14}
# (head_dim, causal) of the persistent ping-pong kernel
PERSIST_LANE_SPILLS = {(128, 0): 62, (128, 1): 75, (64, 0): 63, (64, 1): 60}


def _sgpr_allowance(name):
    m = re.search(r"fa_fwd_bf16_pp_persist_kernelILi(\d+)ELb([01])E", name)
    if m:
        return PERSIST_LANE_SPILLS.get((int(m.group(1)), int(m.group(2))), 0)
    m = re.search(r"(fa_fwd_bf16_kernel|fa_fwd_bf16_pp_kernel)ILi(\d+)ELb([01])ELi(\d+)E", name)
    if not m:
        return 0
    return SGPR_LANE_SPILLS.get((m.group(1), int(m.group(2)), int(m.group(3)), int(m.group(4))), 0)


def test_every_kernel_has_no_scratch_or_spills(usage):
    for name, u in usage.items():
        assert u.get("ScratchSize [bytes/lane]") == "0", (name, u)
        assert u.get("VGPRs Spill") == "0", (name, u)
        assert int(u.get("SGPRs Spill")) <= _sgpr_allowance(name), (name, u)
        assert u.get("Dynamic Stack") == "False", (name, u)


def test_attention_kernels_match_their_plans(usage):
    seen = set()
    limits = fa.fa_gfx950_limits()
    for name, u in usage.items():
        c = _classify(name)
        if c is None:
            continue
        sched, d, dtype = c
        p = _plan(sched, d, dtype)
        regs = int(u["VGPRs"]) + int(u["AGPRs"])
        waves_per_simd = p.wg_per_cu * p.waves // limits.simds_per_cu
        assert regs <= p.vgprs_per_lane, (name, regs, p.vgprs_per_lane)
        assert int(u["Occupancy [waves/SIMD]"]) >= waves_per_simd, (name, u, waves_per_simd)
        assert int(u["LDS Size [bytes/block]"]) == p.lds_bytes, (name, u, p.lds_bytes)
        assert p.lds_bytes * p.wg_per_cu <= limits.lds_bytes_per_cu
        seen.add((sched, d, dtype))
    # every schedule of both head dims (bf16) and the fp8 kernels were found
    for d in (64, 128):
        for s in (1, 2, 3, 4, 5):
            assert (s, d, fa.FA_DTYPE_BF16) in seen, (s, d)
        assert (1, d, fa.FA_DTYPE_E4M3) in seen, d
