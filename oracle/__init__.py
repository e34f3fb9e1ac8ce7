"""Python face of the fp64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and
the benchmark's CPU-baseline leg may import this module.  The product path
(the HIP library and its binding) never loads it, and it never loads them.

Every function takes and returns raw storage bits as numpy arrays:
``uint16`` for binary16 / bfloat16 tensors, ``float32`` for binary32 tables,
``uint8`` for E4M3FN codes.  Row-major 2-D arrays; ``n`` columns of each row
are used (a row may be wider than ``n``, which models a row stride).

The definitions followed are those of the page "TileLang tutorial, ch. 13:
elementwise, normalisation and RoPE operators": RMSNorm and LayerNorm from
its reference implementations (s3.2.1), the two RoPE pairings (s3.3.1,
s3.3.2), the per-token / per-group FP8 cast (s3.1.5) and the fused
norm/rotate/quantise operator (s3.3.4).  The C source states each step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

DTYPE_CODE = {"f16": 1, "bf16": 2, "f32": 3}
_STORAGE = {"f16": np.uint16, "bf16": np.uint16, "f32": np.float32}

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (no fast-math) into liboracle.so."""
    if force or not os.path.exists(_SO):
        cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
               "-o", _SO + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_SO + ".tmp", _SO)
    return _SO


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        build(force=True)
    L = ctypes.CDLL(_SO)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    L.oracle_decode_f16.argtypes = [ctypes.c_uint16]
    L.oracle_decode_f16.restype = ctypes.c_double
    L.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
    L.oracle_decode_bf16.restype = ctypes.c_double
    L.oracle_decode_e4m3.argtypes = [ctypes.c_uint8]
    L.oracle_decode_e4m3.restype = ctypes.c_double
    L.oracle_encode_f16.argtypes = [ctypes.c_double]
    L.oracle_encode_f16.restype = ctypes.c_uint16
    L.oracle_encode_bf16.argtypes = [ctypes.c_double]
    L.oracle_encode_bf16.restype = ctypes.c_uint16
    L.oracle_encode_e4m3.argtypes = [ctypes.c_double]
    L.oracle_encode_e4m3.restype = ctypes.c_uint8
    L.oracle_rmsnorm.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, f32, vp]
    L.oracle_rmsnorm.restype = None
    L.oracle_layernorm.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32, f32]
    L.oracle_layernorm.restype = None
    L.oracle_rope.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, i32, i32, vp]
    L.oracle_rope.restype = None
    L.oracle_rmsnorm_rope_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                          i64, i64, i32, i32, i32, f32, vp, i32]
    L.oracle_rmsnorm_rope_fp8.restype = None
    L.oracle_act_quant_fp8.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i32, i32]
    L.oracle_act_quant_fp8.restype = None
    L.oracle_qk_norm_rope.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64,
                                      i32, i32, i32, f32]
    L.oracle_qk_norm_rope.restype = None
    L.oracle_qk_norm_rope_fp8_kv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64,
                                             i64, i64, i64, i64, i64, i64, i64, i64, i32, i32,
                                             i32, f32]
    L.oracle_qk_norm_rope_fp8_kv.restype = None
    L.oracle_ew_scale_add.argtypes = [vp, vp, vp, i64, f32, i32, i32]
    L.oracle_ew_scale_add.restype = None
    _lib = L
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(a, dtype, name):
    if a is None:
        return None
    want = _STORAGE[dtype]
    if a.dtype != want:
        raise TypeError(f"{name}: expected {np.dtype(want)} storage for {dtype}, got {a.dtype}")
    if not a.flags.c_contiguous:
        raise ValueError(f"{name} must be C-contiguous")
    return a


# ---------------------------------------------------------------- scalars
def decode_f16(bits: int) -> float:
    return _load().oracle_decode_f16(int(bits))


def decode_bf16(bits: int) -> float:
    return _load().oracle_decode_bf16(int(bits))


def decode_e4m3(code: int) -> float:
    return _load().oracle_decode_e4m3(int(code))


def encode_f16(v: float) -> int:
    return _load().oracle_encode_f16(float(v))


def encode_bf16(v: float) -> int:
    return _load().oracle_encode_bf16(float(v))


def encode_e4m3(v: float) -> int:
    return _load().oracle_encode_e4m3(float(v))


# ---------------------------------------------------------------- operators
def rmsnorm(x, w, dtype: str, eps: float, n: int | None = None, y_stride: int | None = None,
            fill: int = 0, want_u: bool = False):
    """y[r, :n] = RMSNorm(x[r, :n]) * w, rounded once to ``dtype``.  With
    ``want_u`` also returns u = x * rstd * w in float64 before the rounding,
    [rows, n]."""
    L = _load()
    x = _check(x, dtype, "x")
    w = _check(w, dtype, "w")
    rows, xs = x.shape
    n = xs if n is None else n
    ys = n if y_stride is None else y_stride
    y = np.full((rows, ys), fill, dtype=_STORAGE[dtype])
    u = np.zeros((rows, n), dtype=np.float64) if want_u else None
    L.oracle_rmsnorm(_ptr(x), _ptr(w), _ptr(y), rows, n, xs, ys, DTYPE_CODE[dtype], eps, _ptr(u))
    return (y, u) if want_u else y


def layernorm(x, gamma, beta, dtype: str, eps: float, n: int | None = None,
              y_stride: int | None = None, fill: int = 0):
    """y[r, :n] = LayerNorm(x[r, :n]; gamma, beta), biased variance, one rounding."""
    L = _load()
    x = _check(x, dtype, "x")
    gamma = _check(gamma, dtype, "gamma")
    beta = _check(beta, dtype, "beta")
    rows, xs = x.shape
    n = xs if n is None else n
    ys = n if y_stride is None else y_stride
    y = np.full((rows, ys), fill, dtype=_STORAGE[dtype])
    L.oracle_layernorm(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), rows, n, xs, ys,
                       DTYPE_CODE[dtype], eps)
    return y


def rope(x, cos, sin, heads: int, head_dim: int, rope_dim: int, dtype: str, cs_dtype: str,
         neox: bool, y_stride: int | None = None, fill: int = 0, want_z: bool = False):
    """RoPE on each head's tail span.  x: [tokens, >= heads*head_dim];
    cos/sin: [tokens, rope_dim/2].  With ``want_z`` also returns every output
    in float64 before its rounding, [tokens, heads*head_dim]."""
    L = _load()
    x = _check(x, dtype, "x")
    cos = _check(cos, cs_dtype, "cos")
    sin = _check(sin, cs_dtype, "sin")
    tokens, xs = x.shape
    n = heads * head_dim
    assert cos.shape == (tokens, rope_dim // 2) and sin.shape == cos.shape
    ys = n if y_stride is None else y_stride
    y = np.full((tokens, ys), fill, dtype=_STORAGE[dtype])
    z = np.zeros((tokens, n), dtype=np.float64) if want_z else None
    L.oracle_rope(_ptr(x), _ptr(cos), _ptr(sin), _ptr(y), tokens, heads, head_dim, rope_dim,
                  xs, ys, DTYPE_CODE[dtype], DTYPE_CODE[cs_dtype], int(bool(neox)), _ptr(z))
    return (y, z) if want_z else y


def rmsnorm_rope_fp8(x, w, cos, sin, heads: int, head_dim: int, rope_dim: int, dtype: str,
                     cs_dtype: str, neox: bool, eps: float, q_stride: int | None = None,
                     want_z: bool = False, fill: int = 0, quotient64: bool = False):
    """Fused RMSNorm -> RoPE -> per-token E4M3FN.  Returns (codes, scales[, z]).
    ``quotient64`` (a diagnostic, not the parity reference) decides each code on
    the double quotient z / scale instead of the binary32 one."""
    L = _load()
    x = _check(x, dtype, "x")
    w = _check(w, dtype, "w")
    cos = _check(cos, cs_dtype, "cos")
    sin = _check(sin, cs_dtype, "sin")
    tokens, xs = x.shape
    n = heads * head_dim
    assert cos.shape == (tokens, rope_dim // 2) and sin.shape == cos.shape
    qs = n if q_stride is None else q_stride
    q = np.full((tokens, qs), fill, dtype=np.uint8)
    scales = np.zeros(tokens, dtype=np.float32)
    z = np.zeros((tokens, n), dtype=np.float64) if want_z else None
    L.oracle_rmsnorm_rope_fp8(_ptr(x), _ptr(w), _ptr(cos), _ptr(sin), _ptr(q), _ptr(scales),
                              tokens, heads, head_dim, rope_dim, xs, qs, DTYPE_CODE[dtype],
                              DTYPE_CODE[cs_dtype], int(bool(neox)), eps, _ptr(z),
                              int(bool(quotient64)))
    return (q, scales, z) if want_z else (q, scales)


def act_quant_fp8(x, dtype: str, group: int | None = None, n: int | None = None,
                  q_stride: int | None = None, fill: int = 0, quotient64: bool = False):
    """E4M3FN codes and scales of x[:, :n] with one scale per ``group`` channels
    (None: one per row).  Returns (codes [rows, q_stride], scales [rows, n/group]).
    ``quotient64``: see rmsnorm_rope_fp8."""
    L = _load()
    x = _check(x, dtype, "x")
    rows, xs = x.shape
    n = xs if n is None else n
    g = n if group is None else group
    assert n % g == 0
    qs = n if q_stride is None else q_stride
    q = np.full((rows, qs), fill, dtype=np.uint8)
    scales = np.zeros((rows, n // g), dtype=np.float32)
    L.oracle_act_quant_fp8(_ptr(x), _ptr(q), _ptr(scales), rows, n, g, xs, qs, DTYPE_CODE[dtype],
                           int(bool(quotient64)))
    return q, scales


def qk_norm_rope(x, q_weight, k_weight, cos, sin, q_heads: int, kv_heads: int, head_dim: int,
                 rope_dim: int, dtype: str, cs_dtype: str, neox: bool, eps: float,
                 y_stride: int | None = None, fill: int = 0):
    """Per-head RMSNorm (weights of length head_dim) then RoPE on the q and k heads
    of x [tokens, (q_heads + 2 kv_heads) * head_dim]; v heads are copied."""
    L = _load()
    x = _check(x, dtype, "x")
    q_weight = _check(q_weight, dtype, "q_weight")
    k_weight = _check(k_weight, dtype, "k_weight")
    cos = _check(cos, cs_dtype, "cos")
    sin = _check(sin, cs_dtype, "sin")
    tokens, xs = x.shape
    n = (q_heads + 2 * kv_heads) * head_dim
    assert cos.shape == (tokens, rope_dim // 2) and sin.shape == cos.shape
    ys = n if y_stride is None else y_stride
    y = np.full((tokens, ys), fill, dtype=_STORAGE[dtype])
    L.oracle_qk_norm_rope(_ptr(x), _ptr(q_weight), _ptr(k_weight), _ptr(cos), _ptr(sin), _ptr(y),
                          tokens, q_heads, kv_heads, head_dim, rope_dim, xs, ys,
                          DTYPE_CODE[dtype], DTYPE_CODE[cs_dtype], int(bool(neox)), eps)
    return y


def qk_norm_rope_fp8_kv(x, q_weight, k_weight, cos, sin, q_heads: int, kv_heads: int,
                        head_dim: int, rope_dim: int, dtype: str, cs_dtype: str, neox: bool,
                        eps: float, slots=None, num_slots: int | None = None,
                        cache_stride: int | None = None, fill: int = 0):
    """QK RMSNorm + RoPE with the FP8 KV-cache write.  Returns (q_out [tokens,
    q_heads*head_dim], k_cache, v_cache [num_slots, cache_stride] uint8, k_scales,
    v_scales [num_slots, kv_heads] float32).  Cache rows no token maps to keep
    ``fill`` (codes) and NaN (scales)."""
    L = _load()
    x = _check(x, dtype, "x")
    q_weight = _check(q_weight, dtype, "q_weight")
    k_weight = _check(k_weight, dtype, "k_weight")
    cos = _check(cos, cs_dtype, "cos")
    sin = _check(sin, cs_dtype, "sin")
    tokens, xs = x.shape
    assert cos.shape == (tokens, rope_dim // 2) and sin.shape == cos.shape
    ns = tokens if num_slots is None else num_slots
    cst = kv_heads * head_dim if cache_stride is None else cache_stride
    if slots is not None:
        slots = np.ascontiguousarray(slots, dtype=np.int64)
        assert slots.shape == (tokens,)
    qs = q_heads * head_dim
    q = np.full((tokens, qs), fill, dtype=_STORAGE[dtype])
    kc = np.full((ns, cst), fill, dtype=np.uint8)
    vc = np.full((ns, cst), fill, dtype=np.uint8)
    ksc = np.full((ns, kv_heads), np.nan, dtype=np.float32)
    vsc = np.full((ns, kv_heads), np.nan, dtype=np.float32)
    L.oracle_qk_norm_rope_fp8_kv(_ptr(x), _ptr(q_weight), _ptr(k_weight), _ptr(cos), _ptr(sin),
                                 _ptr(q), _ptr(kc), _ptr(vc), _ptr(ksc), _ptr(vsc), _ptr(slots),
                                 ns, tokens, q_heads, kv_heads, head_dim, rope_dim, xs, qs, cst,
                                 DTYPE_CODE[dtype], DTYPE_CODE[cs_dtype], int(bool(neox)), eps)
    return q, kc, vc, ksc, vsc


def ew_scale_add(x, b, alpha: float, x_dtype: str, y_dtype: str | None = None):
    """y = round(x * alpha + b) elementwise over flat arrays (b may be None)."""
    L = _load()
    x = _check(np.ascontiguousarray(x), x_dtype, "x")
    b = None if b is None else _check(np.ascontiguousarray(b), x_dtype, "b")
    if b is not None:
        assert b.shape == x.shape
    yd = x_dtype if y_dtype is None else y_dtype
    y = np.zeros(x.shape, dtype=_STORAGE[yd])
    L.oracle_ew_scale_add(_ptr(x), _ptr(b), _ptr(y), x.size, alpha, DTYPE_CODE[x_dtype],
                          DTYPE_CODE[yd])
    return y


def rmsnorm_rope_fp8_rounded(x, w, cos, sin, heads: int, head_dim: int, rope_dim: int,
                             dtype: str, cs_dtype: str, neox: bool, eps: float,
                             want_intermediates: bool = False):
    """The staged form of the fused operator ("TileLang tutorial, ch. 13", s3.3.4:
    the normalised row is written back in x's dtype and rotated there): RMSNorm
    rounded once to ``dtype``, RoPE of those values rounded once to ``dtype``, then
    the per-token cast (s3.1.5) of the result.  That is the composition of the
    three operators above; returns (codes [tokens, n], scales [tokens]).  With
    ``want_intermediates`` also returns a dict of the stored intermediates and
    their unrounded values: u (bits), u_exact, z (bits), z_exact."""
    n = heads * head_dim
    u, u_exact = rmsnorm(x, w, dtype, eps, n=n, want_u=True)
    z, z_exact = rope(u, cos, sin, heads, head_dim, rope_dim, dtype, cs_dtype, neox, want_z=True)
    q, scales = act_quant_fp8(z, dtype, None)
    if want_intermediates:
        return q, scales[:, 0].copy(), {"u": u, "u_exact": u_exact, "z": z, "z_exact": z_exact}
    return q, scales[:, 0].copy()
