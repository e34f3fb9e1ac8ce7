"""ctypes binding of libqrw.so: argument marshalling only.

Each function takes torch tensors that live on a ROCm device, turns them into
the pointers, sizes and strides of the C ABI (include/qrw.h) and calls the
entry point of the same name on torch's current stream.  Every step of the
computation runs in the library's HIP kernels; nothing here computes, and
there is no fallback: if the library is missing or a call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch  # the library shares torch's HIP runtime: load torch first

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqrw.so")
PROBE_LIB_PATH = os.path.join(_HERE, "libqrw_probe.so")

F16, BF16, F32 = 1, 2, 3
_DTYPE = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}

STATUS = {
    0: "QRW_OK", -1: "QRW_ERR_NULL", -2: "QRW_ERR_DTYPE", -3: "QRW_ERR_SHAPE",
    -4: "QRW_ERR_STRIDE", -5: "QRW_ERR_ALIGN", -6: "QRW_ERR_ALIAS", -7: "QRW_ERR_LAUNCH",
    -8: "QRW_ERR_VALUE",
}

EXPORTS = ("rmsnorm_fwd", "layernorm_fwd", "rope_apply_interleaved", "rope_apply_neox",
           "rmsnorm_rope_fp8_fwd", "act_quant_fp8_fwd", "qk_norm_rope_fwd",
           "qk_norm_rope_fp8_kv_fwd", "rmsnorm_rope_fp8_rounded_fwd", "ew_add_fwd",
           "ew_scale_cast_fwd", "ew_scale_add_fwd",
           "qrw_status_string")


class QrwError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg})")
        self.status = status


_lib = None


def load():
    """Load libqrw.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m quant_row_workgroup_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    L.rmsnorm_fwd.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, f32, vp]
    L.layernorm_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32, f32, vp]
    rope_args = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, i32, vp]
    L.rope_apply_interleaved.argtypes = rope_args
    L.rope_apply_neox.argtypes = rope_args
    L.rmsnorm_rope_fp8_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                       i32, i32, i32, f32, vp]
    L.rmsnorm_rope_fp8_rounded_fwd.argtypes = L.rmsnorm_rope_fp8_fwd.argtypes
    L.act_quant_fp8_fwd.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i32, vp]
    L.qk_norm_rope_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, i32,
                                   i32, f32, vp]
    L.ew_add_fwd.argtypes = [vp, vp, vp, i64, i32, vp]
    L.ew_scale_cast_fwd.argtypes = [vp, vp, i64, f32, i32, i32, vp]
    L.ew_scale_add_fwd.argtypes = [vp, vp, vp, i64, f32, i32, vp]
    L.qk_norm_rope_fp8_kv_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64,
                                          i64, i64, i64, i64, i64, i32, i32, i32, f32, vp]
    for name in EXPORTS[:-1]:
        getattr(L, name).restype = i32
    L.qrw_status_string.argtypes = [i32]
    L.qrw_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


PROBE_EXPORTS = ("qrw_probe_copy_fused_traffic", "qrw_probe_copy_qk_traffic", "qrw_probe_empty",
                 "qrw_probe_fused_timeline", "qrw_probe_sweep", "qrw_probe_recip_values")

_probe = None


def load_probe():
    """Load libqrw_probe.so (include/qrw_probe.h): the benchmark's and the GPU
    tests' measurement and self-check kernels, not operators."""
    global _probe
    if _probe is not None:
        return _probe
    if not os.path.exists(PROBE_LIB_PATH):
        raise ImportError(f"{PROBE_LIB_PATH} is missing: build it with "
                          "`python -m quant_row_workgroup_amd.build`")
    L = ctypes.CDLL(PROBE_LIB_PATH)
    vp, i64, i32, u32, f32 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32,
                              ctypes.c_float)
    L.qrw_probe_copy_fused_traffic.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i32, vp]
    L.qrw_probe_copy_qk_traffic.argtypes = [vp] * 10 + [i64, i64, i32, vp]
    L.qrw_probe_empty.argtypes = [vp, i64, vp]
    L.qrw_probe_fused_timeline.argtypes = [vp, vp, vp, vp, vp, vp, i64, f32, vp, vp]
    L.qrw_probe_sweep.argtypes = [i32, u32, u32, u32, vp, i64, vp]
    L.qrw_probe_recip_values.argtypes = [vp, vp, vp, i64, vp]
    for name in PROBE_EXPORTS:
        getattr(L, name).restype = i32
    _probe = L
    return L


def _check(fn, status):
    if status != 0:
        raise QrwError(fn, status, load().qrw_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype(t):
    if t.dtype not in _DTYPE:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DTYPE[t.dtype]


def _on_device(t, name):
    """The tensor every other argument is checked against: on a ROCm device."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a tensor on a ROCm device")
    return t


def _same_device(t, like, name):
    if not isinstance(t, torch.Tensor) or t.device != like.device:
        raise ValueError(f"{name} must be a tensor on {like.device}")
    return t


def _exact(t, like, name, shape, dtype):
    """An output (or a fixed-size input) the kernel reads or writes in full:
    exactly this shape and dtype, on like's device."""
    _same_device(t, like, name)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} {tuple(shape)}, got {t.dtype} "
                         f"{tuple(t.shape)}")
    return t


def _tables(cos, sin, tokens, rope_dim, like):
    """cos and sin: packed [tokens, rope_dim/2], one dtype (float32 or like's)."""
    for t, nm in ((cos, "cos"), (sin, "sin")):
        _exact(t, like, nm, (tokens, rope_dim // 2), cos.dtype)
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be packed [tokens, rope_dim/2]")


def _rows(t, name):
    if t.dim() == 2 and t.shape[0] == 0:  # empty: strides carry no meaning
        return 0, t.shape[1], t.shape[1]
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with a unit last stride, got {tuple(t.shape)} "
                         f"strides {t.stride()}")
    return t.shape[0], t.shape[1], t.stride(0)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _vec(t, n, name, like):
    if t is None:
        return None
    _same_device(t, like, name)
    if t.dim() != 1 or t.shape[0] != n or not t.is_contiguous() or t.dtype != like.dtype:
        raise ValueError(f"{name} must be a packed {like.dtype} vector of length {n}")
    return t


# ------------------------------------------------------------------ entry points
def _new_rows(rows, n, like):
    """A [rows, n] output whose rows start 16-byte aligned (stride padded to 8)."""
    return torch.empty((rows, (n + 7) // 8 * 8), dtype=like.dtype, device=like.device)[:, :n]


def rmsnorm_fwd(x, weight=None, eps: float = 1e-6, out=None):
    """RMSNorm over the last dim of 2-D ``x``; returns ``out``."""
    rows, n, xs = _rows(_on_device(x, "x"), "x")
    out = _new_rows(rows, n, x) if out is None else _exact(out, x, "out", (rows, n), x.dtype)
    _, _, ys = _rows(out, "out")
    st = load().rmsnorm_fwd(_ptr(x), _ptr(_vec(weight, n, "weight", x)), _ptr(out), rows, n, xs,
                            ys, _dtype(x), eps, _stream(x))
    _check("rmsnorm_fwd", st)
    return out


def layernorm_fwd(x, gamma=None, beta=None, eps: float = 1e-5, out=None):
    rows, n, xs = _rows(_on_device(x, "x"), "x")
    out = _new_rows(rows, n, x) if out is None else _exact(out, x, "out", (rows, n), x.dtype)
    _, _, ys = _rows(out, "out")
    st = load().layernorm_fwd(_ptr(x), _ptr(_vec(gamma, n, "gamma", x)),
                              _ptr(_vec(beta, n, "beta", x)), _ptr(out), rows, n, xs, ys,
                              _dtype(x), eps, _stream(x))
    _check("layernorm_fwd", st)
    return out


def _rope(fn, x, cos, sin, heads, head_dim, rope_dim, out):
    tokens, n, xs = _rows(_on_device(x, "x"), "x")
    if heads * head_dim != n:
        raise ValueError("heads * head_dim must equal the row length")
    if out is None:
        out = torch.empty((tokens, n), dtype=x.dtype, device=x.device)
    _, _, ys = _rows(_exact(out, x, "out", (tokens, n), x.dtype), "out")
    _tables(cos, sin, tokens, rope_dim, x)
    st = getattr(load(), fn)(_ptr(x), _ptr(cos), _ptr(sin), _ptr(out), tokens, heads, head_dim,
                             rope_dim, xs, ys, _dtype(x), _dtype(cos), _stream(x))
    _check(fn, st)
    return out


def rope_apply_interleaved(x, cos, sin, heads: int, head_dim: int, rope_dim: int | None = None,
                           out=None):
    return _rope("rope_apply_interleaved", x, cos, sin, heads, head_dim,
                 head_dim if rope_dim is None else rope_dim, out)


def rope_apply_neox(x, cos, sin, heads: int, head_dim: int, rope_dim: int | None = None,
                    out=None):
    return _rope("rope_apply_neox", x, cos, sin, heads, head_dim,
                 head_dim if rope_dim is None else rope_dim, out)


def _fused(fname, x, weight, cos, sin, heads, head_dim, rope_dim, neox, eps, q, scales):
    tokens, n, xs = _rows(_on_device(x, "x"), "x")
    if heads * head_dim != n:
        raise ValueError("heads * head_dim must equal the row length")
    rd = head_dim if rope_dim is None else rope_dim
    if q is None:
        q = torch.empty((tokens, n), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((tokens,), dtype=torch.float32, device=x.device)
    _, _, qs = _rows(_exact(q, x, "q", (tokens, n), torch.uint8), "q")
    if not _exact(scales, x, "scales", (tokens,), torch.float32).is_contiguous():
        raise ValueError("scales must be packed")
    _tables(cos, sin, tokens, rd, x)
    st = getattr(load(), fname)(_ptr(x), _ptr(_vec(weight, n, "weight", x)), _ptr(cos), _ptr(sin),
                                _ptr(q), _ptr(scales), tokens, heads, head_dim, rd, xs, qs,
                                _dtype(x), _dtype(cos), int(bool(neox)), eps, _stream(x))
    _check(fname, st)
    return q, scales


def rmsnorm_rope_fp8_fwd(x, weight, cos, sin, heads: int, head_dim: int,
                         rope_dim: int | None = None, neox: bool = True, eps: float = 1e-6,
                         q=None, scales=None):
    """Returns (codes uint8 [tokens, n], scales float32 [tokens])."""
    return _fused("rmsnorm_rope_fp8_fwd", x, weight, cos, sin, heads, head_dim, rope_dim, neox,
                  eps, q, scales)


def rmsnorm_rope_fp8_rounded_fwd(x, weight, cos, sin, heads: int, head_dim: int,
                                 rope_dim: int | None = None, neox: bool = True,
                                 eps: float = 1e-6, q=None, scales=None):
    """The staged form (normalised and rotated values rounded to x's dtype)."""
    return _fused("rmsnorm_rope_fp8_rounded_fwd", x, weight, cos, sin, heads, head_dim,
                  rope_dim, neox, eps, q, scales)


def act_quant_fp8_fwd(x, group: int | None = None, q=None, scales=None):
    """E4M3FN codes of 2-D ``x`` with one scale per ``group`` channels (None: per
    row).  Returns (codes uint8 [rows, n], scales float32 [rows, n / group])."""
    rows, n, xs = _rows(_on_device(x, "x"), "x")
    g = n if group is None else group
    if g < 1:
        raise ValueError("group must be positive")
    if q is None:
        q = torch.empty((rows, n), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, max(n // g, 1)), dtype=torch.float32, device=x.device)
    _, _, qs = _rows(_exact(q, x, "q", (rows, n), torch.uint8), "q")
    if not _exact(scales, x, "scales", (rows, max(n // g, 1)), torch.float32).is_contiguous():
        raise ValueError("scales must be packed")
    st = load().act_quant_fp8_fwd(_ptr(x), _ptr(q), _ptr(scales), rows, n, g, xs, qs, _dtype(x),
                                  _stream(x))
    _check("act_quant_fp8_fwd", st)
    return q, scales


def qk_norm_rope_fwd(qkv, q_weight, k_weight, cos, sin, q_heads: int, kv_heads: int,
                     head_dim: int, rope_dim: int | None = None, neox: bool = True,
                     eps: float = 1e-6):
    """Per-head RMSNorm + RoPE on the q and k heads of 2-D ``qkv``, in place."""
    tokens, n, xs = _rows(_on_device(qkv, "qkv"), "qkv")
    if (q_heads + 2 * kv_heads) * head_dim != n:
        raise ValueError("(q_heads + 2 * kv_heads) * head_dim must equal the row length")
    rd = head_dim if rope_dim is None else rope_dim
    _tables(cos, sin, tokens, rd, qkv)
    st = load().qk_norm_rope_fwd(_ptr(qkv), _ptr(_vec(q_weight, head_dim, "q_weight", qkv)),
                                 _ptr(_vec(k_weight, head_dim, "k_weight", qkv)), _ptr(cos),
                                 _ptr(sin),
                                 tokens, q_heads, kv_heads, head_dim, rd, xs, _dtype(qkv),
                                 _dtype(cos), int(bool(neox)), eps, _stream(qkv))
    _check("qk_norm_rope_fwd", st)
    return qkv


def qk_norm_rope_fp8_kv_fwd(qkv, q_weight, k_weight, cos, sin, k_cache, v_cache, k_scales,
                            v_scales, q_heads: int, kv_heads: int, head_dim: int,
                            rope_dim: int | None = None, slots=None, neox: bool = True,
                            eps: float = 1e-6):
    """QK RMSNorm + RoPE with q written back into 2-D ``qkv`` and k/v cast to
    E4M3 into the cache rows ``slots`` (int64 per token; None: row t)."""
    tokens, n, xs = _rows(_on_device(qkv, "qkv"), "qkv")
    if (q_heads + 2 * kv_heads) * head_dim != n:
        raise ValueError("(q_heads + 2 * kv_heads) * head_dim must equal the row length")
    rd = head_dim if rope_dim is None else rope_dim
    _tables(cos, sin, tokens, rd, qkv)
    _same_device(k_cache, qkv, "k_cache")
    num_slots, kvn, cs = _rows(k_cache, "k_cache")
    if kvn != kv_heads * head_dim:
        raise ValueError("k_cache rows must hold kv_heads * head_dim codes")
    _exact(v_cache, qkv, "v_cache", (num_slots, kvn), torch.uint8)
    if v_cache.stride() != k_cache.stride():
        raise ValueError("v_cache must have k_cache's shape and strides")
    if k_cache.dtype != torch.uint8:
        raise ValueError("caches hold uint8 E4M3 codes")
    for t, nm in ((k_scales, "k_scales"), (v_scales, "v_scales")):
        if not _exact(t, qkv, nm, (num_slots, kv_heads), torch.float32).is_contiguous():
            raise ValueError(f"{nm} must be packed float32 [num_slots, kv_heads]")
    if slots is not None and not _exact(slots, qkv, "slots", (tokens,),
                                        torch.int64).is_contiguous():
        raise ValueError("slots must be packed int64 [tokens]")
    st = load().qk_norm_rope_fp8_kv_fwd(
        _ptr(qkv), _ptr(_vec(q_weight, head_dim, "q_weight", qkv)),
        _ptr(_vec(k_weight, head_dim, "k_weight", qkv)), _ptr(cos), _ptr(sin), _ptr(k_cache),
        _ptr(v_cache), _ptr(k_scales), _ptr(v_scales), _ptr(slots), num_slots, tokens, q_heads,
        kv_heads, head_dim, rd, xs, cs, _dtype(qkv), _dtype(cos), int(bool(neox)), eps,
        _stream(qkv))
    _check("qk_norm_rope_fp8_kv_fwd", st)
    return qkv


def _flat(t, name):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def ew_add_fwd(a, b, out=None):
    """out = a + b (same shape and dtype), one rounding from fp32."""
    _exact(b, _on_device(a, "a"), "b", a.shape, a.dtype)
    y = torch.empty_like(a) if out is None else _exact(out, a, "out", a.shape, a.dtype)
    st = load().ew_add_fwd(_ptr(_flat(a, "a")), _ptr(_flat(b, "b")), _ptr(_flat(y, "out")),
                           a.numel(), _dtype(a), _stream(a))
    _check("ew_add_fwd", st)
    return y


def ew_scale_cast_fwd(x, alpha: float, out_dtype=None, out=None):
    """out = (x * alpha) cast to ``out_dtype`` (default: x's dtype)."""
    _on_device(x, "x")
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    _exact(out, x, "out", x.shape, out.dtype if out_dtype is None else out_dtype)
    st = load().ew_scale_cast_fwd(_ptr(_flat(x, "x")), _ptr(_flat(out, "out")), x.numel(), alpha,
                                  _dtype(x), _dtype(out), _stream(x))
    _check("ew_scale_cast_fwd", st)
    return out


def ew_scale_add_fwd(x, b, alpha: float, out=None):
    """out = x * alpha + b (same shape and dtype)."""
    _exact(b, _on_device(x, "x"), "b", x.shape, x.dtype)
    y = torch.empty_like(x) if out is None else _exact(out, x, "out", x.shape, x.dtype)
    st = load().ew_scale_add_fwd(_ptr(_flat(x, "x")), _ptr(_flat(b, "b")), _ptr(_flat(y, "out")),
                                 x.numel(), alpha, _dtype(x), _stream(x))
    _check("ew_scale_add_fwd", st)
    return y
