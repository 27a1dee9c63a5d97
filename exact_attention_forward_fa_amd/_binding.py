"""ctypes binding of libfa_fwd.so (argument marshalling only)."""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libfa_fwd.so")

FA_OK = 0
FA_ERR_NULL = -1
FA_ERR_INVALID = -2
FA_ERR_UNSUPPORTED = -3
FA_ERR_DEVICE = -4
FA_DTYPE_BF16 = 0
FA_DTYPE_E4M3 = 1


class FaError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {fa_strerror(code)} (code {code})")
        self.code = code


class DeviceLimits(ctypes.Structure):
    _fields_ = [("lds_bytes_per_block", ctypes.c_int64), ("lds_bytes_per_cu", ctypes.c_int64),
                ("num_cus", ctypes.c_int), ("simds_per_cu", ctypes.c_int),
                ("regs_per_simd_lane", ctypes.c_int), ("max_waves_per_simd", ctypes.c_int)]


class TileConfig(ctypes.Structure):
    _fields_ = [("tile_m", ctypes.c_int), ("tile_n", ctypes.c_int), ("head_dim", ctypes.c_int),
                ("head_dim_v", ctypes.c_int), ("elem_bytes", ctypes.c_int),
                ("kv_stages", ctypes.c_int), ("q_in_regs", ctypes.c_int)]


class Screen(ctypes.Structure):
    _fields_ = [("smem_bytes", ctypes.c_int64), ("fits", ctypes.c_int),
                ("blocks_per_cu", ctypes.c_int)]


class Plan(ctypes.Structure):
    _fields_ = [("tile_m", ctypes.c_int), ("tile_n", ctypes.c_int), ("waves", ctypes.c_int),
                ("kv_stages", ctypes.c_int), ("lds_bytes", ctypes.c_int64),
                ("wg_per_cu", ctypes.c_int), ("vgprs_per_lane", ctypes.c_int),
                ("num_workgroups", ctypes.c_int64), ("m_tiles", ctypes.c_int),
                ("kernel_variant", ctypes.c_int), ("query_tiles", ctypes.c_int),
                ("heads_per_workgroup", ctypes.c_int), ("schedule", ctypes.c_int)]


def library_path() -> str:
    return _LIB_PATH


def _load():
    # PyTorch for ROCm ships its own libamdhip64 and links it by the unversioned name, so a
    # HIP runtime that our library pulled in first (by its versioned SONAME) would not be
    # shared: torch would load a second runtime and its streams and allocations would be
    # foreign to ours.  Importing torch first makes our libamdhip64.so.7 dependency resolve to
    # the runtime torch already loaded, so both use one HIP runtime.
    import torch  # noqa: F401

    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python exact_attention_forward_fa_amd/build.py` "
            "(there is no CPU or PyTorch fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, i32, i32,
                           ctypes.c_float, i32, vp, vp]
    lib.fa_fwd.restype = i32
    lib.fa_strerror.argtypes = [i32]
    lib.fa_strerror.restype = ctypes.c_char_p
    lib.fa_smem_screen.argtypes = [ctypes.POINTER(TileConfig), ctypes.POINTER(DeviceLimits),
                                   ctypes.POINTER(Screen)]
    lib.fa_smem_screen.restype = i32
    lib.fa_gfx950_limits.argtypes = [ctypes.POINTER(DeviceLimits)]
    lib.fa_gfx950_limits.restype = i32
    lib.fa_fwd_plan.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                ctypes.POINTER(DeviceLimits), ctypes.POINTER(Plan)]
    lib.fa_fwd_plan.restype = i32
    lib.fa_version.restype = i32
    lib.fa_set_schedule.argtypes = [i32]
    lib.fa_set_schedule.restype = i32
    lib.fa_set_exp2_offload.argtypes = [i32]
    lib.fa_set_exp2_offload.restype = i32
    lib.fa_set_fp8_exact_scores.argtypes = [i32]
    lib.fa_set_fp8_exact_scores.restype = i32
    lib.fa_fwd_kvcache.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp,
                                   i32, i32, ctypes.c_float, i32, vp, vp]
    lib.fa_fwd_kvcache.restype = i32
    lib.fa_check_cu_seqlens.argtypes = [vp, i32, i32, i32, ctypes.c_int64, ctypes.c_int64]
    lib.fa_check_cu_seqlens.restype = i32
    return lib


_lib = _load()


def fa_strerror(code: int) -> str:
    return _lib.fa_strerror(int(code)).decode()


def fa_version() -> int:
    return int(_lib.fa_version())


def fa_set_schedule(schedule: int) -> None:
    """Tuning override of the planner: 0 automatic; 1 one query tile per wave; 2 two query tiles
    per wave (bf16); 3 the 8-wave ping-pong (bf16, even heads_q / heads_kv, or odd for fixed
    lengths); 4 decode (bf16, heads_q / heads_kv * seqlen_q <= 32); 5 the ping-pong's items
    walked by resident workgroups (persistent launch, where 3 applies)."""
    rc = _lib.fa_set_schedule(int(schedule))
    if rc != 0:
        raise FaError(rc, "fa_set_schedule")


def fa_set_exp2_offload(every: int) -> None:
    """exp2 offload in the ping-pong schedule: 0 off (default), or every 4th / 8th exponential
    on the FMA polynomial instead of the transcendental unit."""
    rc = _lib.fa_set_exp2_offload(int(every))
    if rc != 0:
        raise FaError(rc, "fa_set_exp2_offload")


def fa_set_fp8_exact_scores(on: int) -> None:
    """e4m3 inputs: 1 computes the scores on the bf16 matrix instruction from exactly widened Q
    and K (no loss of precision in the product), 0 (default) on the fp8 one."""
    rc = _lib.fa_set_fp8_exact_scores(int(on))
    if rc != 0:
        raise FaError(rc, "fa_set_fp8_exact_scores")


def fa_gfx950_limits() -> DeviceLimits:
    out = DeviceLimits()
    rc = _lib.fa_gfx950_limits(ctypes.byref(out))
    if rc:
        raise FaError(rc, "fa_gfx950_limits")
    return out


def fa_smem_screen(cfg: TileConfig, dev: DeviceLimits) -> Screen:
    out = Screen()
    rc = _lib.fa_smem_screen(ctypes.byref(cfg), ctypes.byref(dev), ctypes.byref(out))
    if rc:
        raise FaError(rc, "fa_smem_screen")
    return out


def fa_fwd_plan(dtype: int, batch: int, heads_q: int, heads_kv: int, seqlen_q: int,
                seqlen_k: int, varlen: bool, head_dim: int, head_dim_v: int, causal: bool,
                dev: Optional[DeviceLimits] = None) -> Plan:
    out = Plan()
    rc = _lib.fa_fwd_plan(int(dtype), int(batch), int(heads_q), int(heads_kv), int(seqlen_q),
                          int(seqlen_k), int(bool(varlen)), int(head_dim), int(head_dim_v),
                          int(bool(causal)), ctypes.byref(dev) if dev is not None else None,
                          ctypes.byref(out))
    if rc:
        raise FaError(rc, "fa_fwd_plan")
    return out


def fa_check_cu_seqlens(cu_host, batch: int, seqlen_q: int, seqlen_k: int, rows_q: int,
                        rows_k: int) -> None:
    """Check a host copy of a packed batch's offsets (int32[2*(batch+1)], numpy or CPU tensor)
    with the library's host-side validator; raises FaError(FA_ERR_INVALID) when the offsets
    do not start at 0, decrease, exceed the maxima or do not match the tensors' row counts."""
    import numpy as np

    if hasattr(cu_host, "detach"):
        cu_host = cu_host.detach().cpu().numpy()
    arr = np.ascontiguousarray(np.asarray(cu_host, dtype=np.int32))
    if arr.ndim != 1 or arr.shape[0] != 2 * (int(batch) + 1):
        raise FaError(FA_ERR_INVALID, "fa_check_cu_seqlens")
    rc = _lib.fa_check_cu_seqlens(arr.ctypes.data_as(ctypes.c_void_p), int(batch), int(seqlen_q),
                                  int(seqlen_k), int(rows_q), int(rows_k))
    if rc:
        raise FaError(rc, "fa_check_cu_seqlens")


def _ptr(x) -> Optional[int]:
    """A device pointer from a torch tensor, an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _current_stream() -> int:
    import torch

    return int(torch.cuda.current_stream().cuda_stream)


def fa_fwd(q, k, v, o, lse, batch: int, heads_q: int, heads_kv: int, seqlen_q: int,
           seqlen_k: int, cu_seqlens, head_dim: int, head_dim_v: int, softmax_scale: float,
           causal, descales, stream=None) -> int:
    """Call the C entry point.  Tensors are passed by device address; raises FaError on a
    non-zero return code.  ``stream`` is a hipStream_t address (default: torch's current)."""
    st = _current_stream() if stream is None else int(stream)
    rc = _lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(batch), int(heads_q),
                     int(heads_kv), int(seqlen_q), int(seqlen_k), _ptr(cu_seqlens), int(head_dim),
                     int(head_dim_v), ctypes.c_float(float(softmax_scale)), int(causal),
                     _ptr(descales), st)
    if rc:
        raise FaError(rc, "fa_fwd")
    return rc


def forward(q, k, v, *, causal: bool, softmax_scale: Optional[float] = None, cu_seqlens=None,
            max_seqlen_q: Optional[int] = None, max_seqlen_k: Optional[int] = None,
            descales=None, batch: Optional[int] = None, out=None, lse=None):
    """Allocate O (bf16) and LSE (fp32) and run the forward.

    q [total_q, Hq, D], k [total_k, Hkv, D], v [total_k, Hkv, Dv] on the GPU: bf16, or uint8 /
    float8_e4m3fn codes with ``descales`` (float32[3] on the GPU).  Without ``cu_seqlens`` the
    leading dimension is batch*seqlen with ``batch`` given (default 1).  With ``cu_seqlens``
    (int32[2*(batch+1)] on the GPU) ``max_seqlen_q`` / ``max_seqlen_k`` must be given; a host copy
    of the offsets is checked first (fa_check_cu_seqlens: starting at 0, non-decreasing, lengths
    within the maxima, cu[batch] == q.shape[0], cu[2*batch+1] <= k.shape[0]), which costs one
    device-to-host copy per call.  ``out`` / ``lse`` may be given (shapes as returned).
    Returns (O [total_q, Hq, Dv], LSE [Hq, total_q]).
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 3:
            raise ValueError(f"{name} must be a contiguous 3-d GPU tensor")
    fp8 = descales is not None
    want = (torch.uint8, torch.float8_e4m3fn) if fp8 else (torch.bfloat16,)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype not in want:
            raise ValueError(f"{name} has dtype {t.dtype}, expected one of {want}")
    total_q, hq, d = q.shape
    total_k, hkv, dk = k.shape
    dv = v.shape[2]
    if dk != d or v.shape[0] != total_k or v.shape[1] != hkv:
        raise ValueError(f"k {tuple(k.shape)} / v {tuple(v.shape)} do not match q {tuple(q.shape)}")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on one device")
    if cu_seqlens is not None:
        if max_seqlen_q is None or max_seqlen_k is None:
            raise ValueError("cu_seqlens needs max_seqlen_q and max_seqlen_k")
        if (cu_seqlens.dtype != torch.int32 or cu_seqlens.device != q.device
                or cu_seqlens.numel() % 2 or cu_seqlens.numel() < 4):
            raise ValueError("cu_seqlens must be int32[2*(batch+1)] on the device of q")
        nb = cu_seqlens.numel() // 2 - 1
        if batch is not None and batch != nb:
            raise ValueError("batch does not match cu_seqlens")
        batch, sq, sk = nb, int(max_seqlen_q), int(max_seqlen_k)
        # the kernels read the offsets on the device only; check a host copy of them first
        fa_check_cu_seqlens(cu_seqlens, batch, sq, sk, total_q, total_k)
    else:
        batch = 1 if batch is None else int(batch)
        if batch <= 0 or total_q % batch or total_k % batch:
            raise ValueError("leading dimensions are not divisible by batch")
        sq, sk = total_q // batch, total_k // batch
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if descales is not None and (descales.device != q.device or descales.dtype != torch.float32
                                 or descales.numel() != 3):
        raise ValueError("descales must be float32[3] on the device of q")
    if out is None:
        out = torch.empty((total_q, hq, dv), dtype=torch.bfloat16, device=q.device)
    elif (out.shape != (total_q, hq, dv) or out.dtype != torch.bfloat16 or not out.is_contiguous()
          or out.device != q.device):
        raise ValueError(f"out must be a contiguous bf16 tensor of shape {(total_q, hq, dv)}")
    if lse is None:
        lse = torch.empty((hq, total_q), dtype=torch.float32, device=q.device)
    elif (lse.shape != (hq, total_q) or lse.dtype != torch.float32 or not lse.is_contiguous()
          or lse.device != q.device):
        raise ValueError(f"lse must be a contiguous float32 tensor of shape {(hq, total_q)}")
    fa_fwd(q, k, v, out, lse, batch, hq, hkv, sq, sk, cu_seqlens, d, dv, softmax_scale,
           int(bool(causal)), descales)
    return out, lse


def fa_fwd_kvcache(q, k_cache, v_cache, k_new, v_new, o, lse, batch: int, heads_q: int,
                   heads_kv: int, seqlen_q: int, seqlen_new: int, cache_capacity: int,
                   cache_seqlens, head_dim: int, head_dim_v: int, softmax_scale: float, causal,
                   descales, stream=None) -> int:
    """Call the C entry point (append new K/V to the cache, then the forward over it)."""
    st = _current_stream() if stream is None else int(stream)
    rc = _lib.fa_fwd_kvcache(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
                             _ptr(o), _ptr(lse), int(batch), int(heads_q), int(heads_kv),
                             int(seqlen_q), int(seqlen_new), int(cache_capacity),
                             _ptr(cache_seqlens), int(head_dim), int(head_dim_v),
                             ctypes.c_float(float(softmax_scale)), int(causal), _ptr(descales), st)
    if rc:
        raise FaError(rc, "fa_fwd_kvcache")
    return rc


def forward_kvcache(q, k_cache, v_cache, cache_seqlens, k_new=None, v_new=None, *, causal: bool,
                    softmax_scale: Optional[float] = None, descales=None, out=None, lse=None):
    """Append (k_new, v_new) to the caches and attend over them.

    q [B, Sq, Hq, D]; k_cache / v_cache [B, capacity, Hkv, D] (updated in place); k_new / v_new
    [B, Snew, Hkv, D] or None; cache_seqlens int32[B] on the GPU (not advanced).  bf16, or e4m3
    codes with ``descales``.  Returns (O [B*Sq, Hq, D], LSE [Hq, B*Sq]).
    """
    import torch

    tensors = [("q", q), ("k_cache", k_cache), ("v_cache", v_cache)]
    if k_new is not None or v_new is not None:
        if k_new is None or v_new is None:
            raise ValueError("k_new and v_new go together")
        tensors += [("k_new", k_new), ("v_new", v_new)]
    fp8 = descales is not None
    want = (torch.uint8, torch.float8_e4m3fn) if fp8 else (torch.bfloat16,)
    for name, t in tensors:
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-d GPU tensor")
        if t.dtype not in want:
            raise ValueError(f"{name} has dtype {t.dtype}, expected one of {want}")
    b, sq, hq, d = q.shape
    _, cap, hkv, _ = k_cache.shape
    if k_cache.shape != (b, cap, hkv, d) or v_cache.shape != (b, cap, hkv, d):
        raise ValueError(f"caches must be [batch, capacity, heads_kv, head_dim] = {(b, cap, hkv, d)}")
    snew = 0 if k_new is None else k_new.shape[1]
    if k_new is not None and (k_new.shape != (b, snew, hkv, d) or v_new.shape != (b, snew, hkv, d)):
        raise ValueError(f"new rows must be [batch, seqlen_new, heads_kv, head_dim] = {(b, snew, hkv, d)}")
    for name, t in tensors:
        if t.device != q.device:
            raise ValueError(f"{name} is not on the device of q")
    if (cache_seqlens.dtype != torch.int32 or cache_seqlens.device != q.device
            or cache_seqlens.numel() != b):
        raise ValueError("cache_seqlens must be int32[batch] on the device of q")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if descales is not None and (descales.device != q.device or descales.dtype != torch.float32
                                 or descales.numel() != 3):
        raise ValueError("descales must be float32[3] on the device of q")
    if out is None:
        out = torch.empty((b * sq, hq, d), dtype=torch.bfloat16, device=q.device)
    elif (out.shape != (b * sq, hq, d) or out.dtype != torch.bfloat16 or not out.is_contiguous()
          or out.device != q.device):
        raise ValueError(f"out must be a contiguous bf16 tensor of shape {(b * sq, hq, d)}")
    if lse is None:
        lse = torch.empty((hq, b * sq), dtype=torch.float32, device=q.device)
    elif (lse.shape != (hq, b * sq) or lse.dtype != torch.float32 or not lse.is_contiguous()
          or lse.device != q.device):
        raise ValueError(f"lse must be a contiguous float32 tensor of shape {(hq, b * sq)}")
    fa_fwd_kvcache(q, k_cache, v_cache, k_new, v_new, out, lse, b, hq, hkv, sq, snew, cap,
                   cache_seqlens, d, d, softmax_scale, int(bool(causal)), descales)
    return out, lse
