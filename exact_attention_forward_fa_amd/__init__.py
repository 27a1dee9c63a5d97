"""MI355X (gfx950) exact attention forward: thin Python binding of libfa_fwd.so.

Every step of the forward pass runs in the HIP library; this module only
marshals arguments (torch tensors -> device pointers, the current HIP stream)
through ctypes.  The names mirror the C ABI in ``include/fa_fwd.h``:

    fa_fwd(q, k, v, o, lse, batch, heads_q, heads_kv, seqlen_q, seqlen_k,
           cu_seqlens, head_dim, head_dim_v, softmax_scale, causal, descales,
           stream=None)
    fa_fwd_plan(...), fa_smem_screen(...), fa_gfx950_limits(), fa_strerror(code),
    fa_set_schedule(n), fa_set_exp2_offload(every), fa_set_fp8_exact_scores(on),
    fa_check_cu_seqlens(cu_host, ...)

``forward(q, k, v, ...)`` is a convenience that allocates O and LSE with torch
and calls ``fa_fwd``.  There is no fallback: if the library is missing the
import of the binding raises.
"""
from ._binding import (  # noqa: F401
    FA_DTYPE_BF16,
    FA_DTYPE_E4M3,
    FA_ERR_DEVICE,
    FA_ERR_INVALID,
    FA_ERR_NULL,
    FA_ERR_UNSUPPORTED,
    FA_OK,
    FaError,
    DeviceLimits,
    Plan,
    Screen,
    TileConfig,
    fa_check_cu_seqlens,
    fa_fwd,
    fa_fwd_kvcache,
    fa_fwd_plan,
    fa_set_schedule,
    fa_set_exp2_offload,
    fa_set_fp8_exact_scores,
    fa_gfx950_limits,
    fa_smem_screen,
    fa_strerror,
    fa_version,
    forward,
    forward_kvcache,
    library_path,
)
