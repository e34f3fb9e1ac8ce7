"""Fused memory-bound LLM row operators for AMD MI355X (gfx950).

RMSNorm, LayerNorm, RoPE (interleaved and NeoX half-split), the fused
RMSNorm -> RoPE -> per-token FP8 (E4M3FN) quantisation and per-token /
per-group FP8 activation quantisation and per-head QK RMSNorm + RoPE, as
hand-written HIP
kernels behind a C ABI (include/qrw.h, libqrw.so).  The Python functions here
are a thin ctypes binding with the same names.
"""
from ._binding import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    PROBE_EXPORTS,
    PROBE_LIB_PATH,
    QrwError,
    act_quant_fp8_fwd,
    layernorm_fwd,
    ew_add_fwd,
    ew_scale_add_fwd,
    ew_scale_cast_fwd,
    load,
    load_probe,
    qk_norm_rope_fp8_kv_fwd,
    rmsnorm_rope_fp8_rounded_fwd,
    qk_norm_rope_fwd,
    rmsnorm_fwd,
    rmsnorm_rope_fp8_fwd,
    rope_apply_interleaved,
    rope_apply_neox,
)
