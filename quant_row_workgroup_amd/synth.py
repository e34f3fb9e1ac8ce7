"""Seeded synthetic inputs for the row operators.

This module only draws random numbers and stores them in a tensor format; it
holds none of the operators' arithmetic.  Both the HIP path (through the
binding) and the CPU checker consume exactly the bits produced here.

Recipe (the workloads of the byte-ledger table in "TileLang tutorial, ch. 13:
elementwise, normalisation and RoPE operators", s1.2, made concrete):

* generator: ``numpy.random.Generator(PCG64(seed))``, values drawn in float64;
* ``N(mean, std)`` means normal with that mean and standard deviation;
* "outliers" multiply an independent Bernoulli(frac) subset by a factor;
* storage: binary16 by numpy's float64 -> float16 cast; bfloat16 by a float64
  -> float32 -> bfloat16 cast (torch, nearest-even); float32 by numpy.
  How an input is rounded does not matter for parity: both sides read the
  same stored bits.
* RoPE tables: theta(t, p) = t * base^(-2p/R) for positions t = 0..T-1 and
  pair p = 0..R/2-1, cos and sin evaluated in float64 and stored in the table
  dtype.  The pages leave the angle formula to the caller (the kernel only
  reads the table), so this is the common RoFormer choice.

Arrays are returned as numpy storage bits: ``uint16`` for f16/bf16, ``float32``
for f32.
"""
from __future__ import annotations

import numpy as np

STORAGE = {"f16": np.uint16, "bf16": np.uint16, "f32": np.float32}


def to_storage(v64: np.ndarray, dtype: str) -> np.ndarray:
    """Store float64 values in ``dtype`` (returns storage bits)."""
    v64 = np.ascontiguousarray(v64, dtype=np.float64)
    if dtype == "f16":
        return v64.astype(np.float16).view(np.uint16)
    if dtype == "f32":
        return v64.astype(np.float32)
    if dtype == "bf16":
        import torch

        t = torch.from_numpy(v64.astype(np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dtype)


def storage_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of stored bits (for generators and test checks)."""
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "f32":
        return bits.astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def normal(seed: int, shape, mean: float, std: float, dtype: str,
           outlier_frac: float = 0.0, outlier_mul: float = 1.0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    v = rng.normal(mean, std, size=shape)
    if outlier_frac > 0.0:
        mask = rng.random(size=shape) < outlier_frac
        v = np.where(mask, v * outlier_mul, v)
    return to_storage(v, dtype)


def rope_table(tokens: int, rope_dim: int, dtype: str, base: float = 10000.0):
    """(cos, sin) tables of shape [tokens, rope_dim/2]."""
    half = rope_dim // 2
    t = np.arange(tokens, dtype=np.float64)[:, None]
    p = np.arange(half, dtype=np.float64)[None, :]
    theta = t * np.power(base, -2.0 * p / rope_dim)
    return to_storage(np.cos(theta), dtype), to_storage(np.sin(theta), dtype)


def cache_slots(seed: int, tokens: int, num_slots: int) -> np.ndarray:
    """Distinct cache rows for ``tokens`` tokens, drawn uniformly without
    replacement from ``num_slots`` (a paged cache's scattered free slots)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.choice(num_slots, size=tokens, replace=False).astype(np.int64)


# ------------------------------------------------------------------ workloads
# The five configurations, named by what they are.
WORKLOADS = {
    "scale_add_1M_f32": dict(op="ew", kind="scale_add", n=1 << 20, dtype="f32", alpha=0.5,
                             seed=10),
    "add_16M_bf16": dict(op="ew", kind="add", n=1 << 24, dtype="bf16", seed=11),
    "scale_cast_16M_f32_to_f16": dict(op="ew", kind="scale_cast", n=1 << 24, dtype="f32",
                                      y_dtype="f16", alpha=0.5, seed=12),
    "rmsnorm_256x1024_f16": dict(op="rmsnorm", rows=256, n=1024, dtype="f16", eps=1e-6, seed=1),
    "rmsnorm_4096x4096_f16": dict(op="rmsnorm", rows=4096, n=4096, dtype="f16", eps=1e-6, seed=2),
    "rmsnorm_1024x32768_bf16": dict(op="rmsnorm", rows=1024, n=32768, dtype="bf16", eps=1e-6,
                                    seed=13),
    "rmsnorm_256x131072_bf16_splitk": dict(op="rmsnorm", rows=256, n=131072, dtype="bf16",
                                           eps=1e-6, x_passes=2, seed=14),
    "rmsnorm_4096x4095_bf16_ragged": dict(op="rmsnorm", rows=4096, n=4095, dtype="bf16", eps=1e-6,
                                          seed=16),
    "layernorm_1024x32768_bf16": dict(op="layernorm", rows=1024, n=32768, dtype="bf16", eps=1e-5,
                                      seed=15),
    "layernorm_4096x4096_bf16": dict(op="layernorm", rows=4096, n=4096, dtype="bf16", eps=1e-5,
                                     seed=3),
    "rope_4096x32x128_f16": dict(op="rope", tokens=4096, heads=32, head_dim=128, rope_dim=128,
                                 dtype="f16", cs_dtype="f32", seed=4),
    "rope_4096x32x128_f16_interleaved": dict(op="rope", tokens=4096, heads=32, head_dim=128,
                                             rope_dim=128, dtype="f16", cs_dtype="f32",
                                             neox=False, seed=4),
    "act_quant_4096x4096_bf16_g128": dict(op="act_quant", rows=4096, n=4096, group=128,
                                          dtype="bf16", seed=6),
    "act_quant_4096x4096_bf16_token": dict(op="act_quant", rows=4096, n=4096, group=None,
                                           dtype="bf16", seed=7),
    "qk_norm_rope_4096_q32_kv8_d128_bf16": dict(op="qk_norm_rope", tokens=4096, q_heads=32,
                                                kv_heads=8, head_dim=128, rope_dim=128,
                                                dtype="bf16", cs_dtype="bf16", eps=1e-6,
                                                neox=True, seed=8),
    "qk_norm_rope_fp8_kv_4096_q32_kv8_d128_bf16": dict(op="qk_kv", tokens=4096, q_heads=32,
                                                       kv_heads=8, head_dim=128, rope_dim=128,
                                                       dtype="bf16", cs_dtype="bf16", eps=1e-6,
                                                       neox=True, num_slots=16384, seed=9),
    "rmsnorm_rope_fp8_4096x4096_bf16_staged": dict(op="fused", tokens=4096, heads=32,
                                                   head_dim=128, rope_dim=128, dtype="bf16",
                                                   cs_dtype="bf16", eps=1e-6, neox=True,
                                                   staged=True, seed=5),
    "rmsnorm_rope_fp8_4096x4096_bf16_onehead": dict(op="fused", tokens=4096, heads=1,
                                                    head_dim=4096, rope_dim=128, dtype="bf16",
                                                    cs_dtype="bf16", eps=1e-6, neox=True, seed=5),
    "rmsnorm_rope_fp8_4096x4096_bf16": dict(op="fused", tokens=4096, heads=32, head_dim=128,
                                            rope_dim=128, dtype="bf16", cs_dtype="bf16",
                                            eps=1e-6, neox=True, seed=5),
}


def make_inputs(name: str, seed: int | None = None, rows: int | None = None) -> dict:
    """Inputs of a named workload (optionally with another seed or row count)."""
    cfg = dict(WORKLOADS[name])
    s = cfg["seed"] if seed is None else seed
    op = cfg["op"]
    if op == "rmsnorm":
        R = cfg["rows"] if rows is None else rows
        n, dt = cfg["n"], cfg["dtype"]
        x = normal(s, (R, n), 0.0, 1.0, dt)
        w = normal(s + 1000, (n,), 1.0, 0.1, dt)
        return dict(cfg, rows=R, x=x, w=w)
    if op == "layernorm":
        R = cfg["rows"] if rows is None else rows
        n, dt = cfg["n"], cfg["dtype"]
        x = normal(s, (R, n), 0.5, 2.0, dt)
        g = normal(s + 1000, (n,), 1.0, 0.1, dt)
        b = normal(s + 2000, (n,), 0.0, 0.1, dt)
        return dict(cfg, rows=R, x=x, gamma=g, beta=b)
    if op == "rope":
        T = cfg["tokens"] if rows is None else rows
        n = cfg["heads"] * cfg["head_dim"]
        x = normal(s, (T, n), 0.0, 1.0, cfg["dtype"])
        c, sn = rope_table(T, cfg["rope_dim"], cfg["cs_dtype"])
        return dict(cfg, tokens=T, x=x, cos=c, sin=sn)
    if op == "act_quant":
        R = cfg["rows"] if rows is None else rows
        x = normal(s, (R, cfg["n"]), 0.0, 3.0, cfg["dtype"], outlier_frac=0.01,
                   outlier_mul=10.0)
        return dict(cfg, rows=R, x=x)
    if op == "qk_norm_rope":
        T = cfg["tokens"] if rows is None else rows
        D = cfg["head_dim"]
        n = (cfg["q_heads"] + 2 * cfg["kv_heads"]) * D
        x = normal(s, (T, n), 0.0, 1.0, cfg["dtype"])
        qw = normal(s + 1000, (D,), 1.0, 0.1, cfg["dtype"])
        kw = normal(s + 2000, (D,), 1.0, 0.1, cfg["dtype"])
        c, sn = rope_table(T, cfg["rope_dim"], cfg["cs_dtype"])
        return dict(cfg, tokens=T, x=x, q_weight=qw, k_weight=kw, cos=c, sin=sn)
    if op == "ew":
        n = cfg["n"] if rows is None else rows
        x = normal(s, (n,), 0.0, 1.0, cfg["dtype"])
        out = dict(cfg, n=n, x=x)
        if cfg["kind"] != "scale_cast":
            out["b"] = normal(s + 1000, (n,), 0.0, 1.0, cfg["dtype"])
        return out
    if op == "qk_kv":
        T = cfg["tokens"] if rows is None else rows
        D = cfg["head_dim"]
        n = (cfg["q_heads"] + 2 * cfg["kv_heads"]) * D
        x = normal(s, (T, n), 0.0, 1.0, cfg["dtype"])
        qw = normal(s + 1000, (D,), 1.0, 0.1, cfg["dtype"])
        kw = normal(s + 2000, (D,), 1.0, 0.1, cfg["dtype"])
        c, sn = rope_table(T, cfg["rope_dim"], cfg["cs_dtype"])
        slots = cache_slots(s + 3000, T, cfg["num_slots"])
        return dict(cfg, tokens=T, x=x, q_weight=qw, k_weight=kw, cos=c, sin=sn, slots=slots)
    if op == "fused":
        T = cfg["tokens"] if rows is None else rows
        n = cfg["heads"] * cfg["head_dim"]
        x = normal(s, (T, n), 0.0, 3.0, cfg["dtype"], outlier_frac=0.01, outlier_mul=10.0)
        w = normal(s + 1000, (n,), 1.0, 0.1, cfg["dtype"])
        c, sn = rope_table(T, cfg["rope_dim"], cfg["cs_dtype"])
        return dict(cfg, tokens=T, x=x, w=w, cos=c, sin=sn)
    raise ValueError(op)
