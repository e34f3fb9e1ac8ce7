"""Exact-arithmetic checkers used to pin the CPU oracle.

Nothing here calls the oracle or the HIP library.  Values are carried as
``decimal.Decimal`` at 400 significant digits (every binary16/bfloat16/binary32
input and every product of two of them is exact at that precision), and each
result is rounded to a storage format by searching the format's sorted value
table for the nearest representable value, ties to the even code.  The value
tables come from independent decoders: numpy's float16, the bfloat16 layout
(top half of a binary32) read through numpy's float32, and torch's
``float8_e4m3fn``.
"""
from __future__ import annotations

import bisect
from decimal import Decimal, getcontext

import numpy as np

getcontext().prec = 400


class CodeTable:
    """Non-negative finite values of a sign-magnitude format, indexed by code."""

    def __init__(self, mags: np.ndarray, sign_bit: int, overflow_code: int):
        # mags[c] = value of code c for c = 0 .. max finite magnitude code
        assert np.all(np.diff(mags) > 0), "values must increase with the code"
        self.vals = [Decimal(float(v)) for v in mags]
        self.sign_bit = sign_bit
        self.overflow_code = overflow_code

    def nearest(self, v: Decimal) -> int:
        neg = v.is_signed()
        m = abs(v)
        vals = self.vals
        top = vals[-1]
        if m > top:
            # beyond the largest finite value: RNE keeps it only below the
            # midpoint to the next (non-representable) step
            step = top - vals[-2]
            mid = top + step / 2
            top_even = (len(vals) - 1) % 2 == 0
            if m < mid or (m == mid and top_even):
                c = len(vals) - 1
            else:
                c = self.overflow_code
        else:
            i = bisect.bisect_right(vals, m) - 1  # vals[i] <= m
            if i == len(vals) - 1 or vals[i] == m:
                c = i
            else:
                lo, hi = vals[i], vals[i + 1]
                dl, dh = m - lo, hi - m
                if dl < dh:
                    c = i
                elif dh < dl:
                    c = i + 1
                else:
                    c = i if i % 2 == 0 else i + 1
        return (self.sign_bit | c) if neg else c


def _f16_table():
    codes = np.arange(0, 0x7C00, dtype=np.uint16)
    return CodeTable(codes.view(np.float16).astype(np.float64), 0x8000, 0x7C00)


def _bf16_table():
    codes = np.arange(0, 0x7F80, dtype=np.uint32)
    return CodeTable((codes << 16).view(np.float32).astype(np.float64), 0x8000, 0x7F80)


def _e4m3_table():
    import torch

    codes = torch.arange(0, 0x7F, dtype=torch.uint8)
    vals = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return CodeTable(vals, 0x80, 0x7F)


_TABLES = {}


def table(fmt: str) -> CodeTable:
    if fmt not in _TABLES:
        _TABLES[fmt] = {"f16": _f16_table, "bf16": _bf16_table, "e4m3": _e4m3_table}[fmt]()
    return _TABLES[fmt]


def dec(bits: int, fmt: str) -> Decimal:
    """Exact value of one stored element."""
    if fmt == "f16":
        return Decimal(float(np.array([bits], dtype=np.uint16).view(np.float16)[0]))
    if fmt == "bf16":
        return Decimal(float(np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0]))
    if fmt == "f32":
        return Decimal(float(np.float32(bits)))
    if fmt == "e4m3":
        import torch

        return Decimal(float(torch.tensor([bits], dtype=torch.uint8)
                             .view(torch.float8_e4m3fn).to(torch.float64)[0]))
    raise ValueError(fmt)


def round_to(v: Decimal, fmt: str) -> int:
    return table(fmt).nearest(v)


def round_f32(v: Decimal) -> float:
    """Nearest binary32 to ``v`` (ties to even), by checking the neighbours."""
    f = np.float32(float(v))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = None
    for c in cands:
        d = abs(Decimal(float(c)) - v)
        even = (int(np.array([c], dtype=np.float32).view(np.uint32)[0]) & 1) == 0
        key = (d, 0 if even else 1)
        if best is None or key < best[0]:
            best = (key, c)
    return float(best[1])


def sqrt(v: Decimal) -> Decimal:
    return v.sqrt()


# ----------------------------------------------------------------- references
def rmsnorm_values(xrow, wrow, fmt, eps32):
    """Exact RMSNorm of one row before its rounding (Decimal values)."""
    xs = [dec(b, fmt) for b in xrow]
    ws = [dec(b, fmt) for b in wrow] if wrow is not None else [Decimal(1)] * len(xs)
    n = len(xs)
    ms = sum(x * x for x in xs) / n
    r = 1 / sqrt(ms + Decimal(float(np.float32(eps32))))
    return [x * r * w for x, w in zip(xs, ws)]


def rmsnorm_ref(xrow, wrow, fmt, eps32):
    """Exact RMSNorm of one row; returns output codes."""
    return [round_to(v, fmt) for v in rmsnorm_values(xrow, wrow, fmt, eps32)]


def layernorm_ref(xrow, grow, brow, fmt, eps32):
    xs = [dec(b, fmt) for b in xrow]
    n = len(xs)
    gs = [dec(b, fmt) for b in grow] if grow is not None else [Decimal(1)] * n
    bs = [dec(b, fmt) for b in brow] if brow is not None else [Decimal(0)] * n
    mu = sum(xs) / n
    var = sum((x - mu) * (x - mu) for x in xs) / n
    r = 1 / sqrt(var + Decimal(float(np.float32(eps32))))
    return [round_to((x - mu) * r * g + b, fmt) for x, g, b in zip(xs, gs, bs)]


def rope_pairs(rope_dim, neox):
    half = rope_dim // 2
    if neox:
        return [(p, p, p + half) for p in range(half)]
    return [(p, 2 * p, 2 * p + 1) for p in range(half)]


def rope_values(vals, cos_row, sin_row, heads, head_dim, rope_dim, neox):
    """Rotate exact values (list of Decimal, one token) on each head's tail span."""
    out = list(vals)
    start = head_dim - rope_dim
    for h in range(heads):
        base = h * head_dim + start
        for p, a, b in rope_pairs(rope_dim, neox):
            c, s = cos_row[p], sin_row[p]
            xa, xb = vals[base + a], vals[base + b]
            out[base + a] = xa * c - xb * s
            out[base + b] = xa * s + xb * c
    return out


def rope_ref(xrow, crow, srow, heads, head_dim, rope_dim, fmt, cs_fmt, neox):
    xs = [dec(b, fmt) for b in xrow]
    cs = [dec(b, cs_fmt) for b in crow]
    ss = [dec(b, cs_fmt) for b in srow]
    z = rope_values(xs, cs, ss, heads, head_dim, rope_dim, neox)
    start = head_dim - rope_dim
    out = []
    for j, v in enumerate(z):
        if (j % head_dim) < start:
            out.append(int(xrow[j]))  # pass-through channel: the same bits
        else:
            out.append(round_to(v, fmt))
    return out


def fused_ref(xrow, wrow, crow, srow, heads, head_dim, rope_dim, fmt, cs_fmt, neox, eps32):
    """Exact fused op of one token; returns (codes, scale, z values)."""
    xs = [dec(b, fmt) for b in xrow]
    n = len(xs)
    ws = [dec(b, fmt) for b in wrow] if wrow is not None else [Decimal(1)] * n
    ms = sum(x * x for x in xs) / n
    r = 1 / sqrt(ms + Decimal(float(np.float32(eps32))))
    normed = [x * r * w for x, w in zip(xs, ws)]
    cs = [dec(b, cs_fmt) for b in crow]
    ss = [dec(b, cs_fmt) for b in srow]
    z = rope_values(normed, cs, ss, heads, head_dim, rope_dim, neox)
    amax = max(abs(v) for v in z)
    floor = Decimal(float(np.float32(1e-4)))
    scale = round_f32(max(amax, floor) / 448)
    S = Decimal(scale)
    codes = []
    for v in z:
        q = Decimal(round_f32(v / S))  # the code is decided on the binary32 quotient
        q = min(max(q, Decimal(-448)), Decimal(448))
        codes.append(round_to(q, "e4m3"))
    return codes, scale, z


def act_quant_ref(xrow, fmt, group):
    """Exact per-group E4M3 quantisation of one row; returns (codes, scales)."""
    xs = [dec(b, fmt) for b in xrow]
    floor = Decimal(float(np.float32(1e-4)))
    codes, scales = [], []
    for k in range(0, len(xs), group):
        grp = xs[k:k + group]
        scale = round_f32(max(max(abs(v) for v in grp), floor) / 448)
        scales.append(scale)
        S = Decimal(scale)
        for v in grp:
            q = Decimal(round_f32(v / S))  # the code is decided on the binary32 quotient
            codes.append(round_to(min(max(q, Decimal(-448)), Decimal(448)), "e4m3"))
    return codes, scales


def qk_norm_rope_ref(xrow, qw, kw, crow, srow, q_heads, kv_heads, head_dim, rope_dim, fmt,
                     cs_fmt, neox, eps32):
    """Exact per-head RMSNorm + RoPE of one token row; returns output codes."""
    cs = [dec(b, cs_fmt) for b in crow]
    ss = [dec(b, cs_fmt) for b in srow]
    out = [int(b) for b in xrow]
    eps = Decimal(float(np.float32(eps32)))
    for h in range(q_heads + kv_heads):
        wrow = qw if h < q_heads else kw
        base = h * head_dim
        xs = [dec(b, fmt) for b in xrow[base:base + head_dim]]
        ws = [dec(b, fmt) for b in wrow] if wrow is not None else [Decimal(1)] * head_dim
        r = 1 / sqrt(sum(v * v for v in xs) / head_dim + eps)
        normed = [a * r * b for a, b in zip(xs, ws)]
        z = rope_values(normed, cs, ss, 1, head_dim, rope_dim, neox)
        for j, v in enumerate(z):
            out[base + j] = round_to(v, fmt)
    return out


def _quant_values(vals):
    """E4M3 codes and scale of a group of exact values (per-token cast, one group)."""
    floor = Decimal(float(np.float32(1e-4)))
    scale = round_f32(max(max(abs(v) for v in vals), floor) / 448)
    S = Decimal(scale)
    codes = []
    for v in vals:
        q = Decimal(round_f32(v / S))  # the code is decided on the binary32 quotient
        codes.append(round_to(min(max(q, Decimal(-448)), Decimal(448)), "e4m3"))
    return codes, scale


def qk_kv_ref(xrow, qw, kw, crow, srow, q_heads, kv_heads, head_dim, rope_dim, fmt, cs_fmt,
              neox, eps32):
    """Exact QK RMSNorm + RoPE with the FP8 KV write, one token row.  Returns
    (q output codes, k codes, k scales, v codes, v scales); k/v codes are the
    concatenation of the heads."""
    cs = [dec(b, cs_fmt) for b in crow]
    ss = [dec(b, cs_fmt) for b in srow]
    eps = Decimal(float(np.float32(eps32)))
    q, kc, ks, vc, vs = [], [], [], [], []
    for h in range(q_heads + 2 * kv_heads):
        base = h * head_dim
        xs = [dec(b, fmt) for b in xrow[base:base + head_dim]]
        if h >= q_heads + kv_heads:
            c, s = _quant_values(xs)
            vc += c
            vs.append(s)
            continue
        wrow = qw if h < q_heads else kw
        ws = [dec(b, fmt) for b in wrow] if wrow is not None else [Decimal(1)] * head_dim
        r = 1 / sqrt(sum(v * v for v in xs) / head_dim + eps)
        z = rope_values([a * r * b for a, b in zip(xs, ws)], cs, ss, 1, head_dim, rope_dim, neox)
        if h < q_heads:
            q += [round_to(v, fmt) for v in z]
        else:
            c, s = _quant_values(z)
            kc += c
            ks.append(s)
    return q, kc, ks, vc, vs
