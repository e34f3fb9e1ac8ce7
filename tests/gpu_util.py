"""Helpers for the GPU parity tests: move storage bits between numpy and
torch device tensors, and compare outputs with the tolerances of the
parity bar: FP8 codes equal on >= 99.9% of elements and never more than one
E4M3 step apart; per-token scales within 1e-6 relative; 16-bit outputs
within 2 ulp of the oracle's rounded result.  (For bfloat16 values of
magnitude 2 or more one ulp already exceeds 1e-2, so the 1e-2 absolute bound
that accompanies the ulp bound caps only the cancellation allowance below.)

For 16-bit outputs that are the sum of terms of opposite sign (LayerNorm's
(x - mu) * rstd * gamma + beta, RoPE's x_a c - x_b s), binary32 arithmetic
resolves the result only to a few binary32 ulps of the largest term, which
near a cancellation is many ulps of the result's own format.  There the ulp
is taken at the magnitude of the largest term (``term_scale``, computed here
in float64 from the inputs), and the difference must also stay within 1e-2;
elsewhere it is the ulp of the result."""
from __future__ import annotations

import numpy as np
import torch

from quant_row_workgroup_amd import synth

TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def dev(bits: np.ndarray, dtype: str, device="cuda"):
    """numpy storage bits -> device tensor of ``dtype``."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(bits)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(TORCH_DT[dtype]).to(device)


def host(t) -> np.ndarray:
    """device tensor -> numpy storage bits."""
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.uint8:
        return t.numpy()
    return t.numpy()


def ord16(bits):
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ord8(codes):
    b = codes.astype(np.int64)
    mag = b & 0x7F
    return np.where(b & 0x80, -mag, mag)


def ulp_at(mag, dtype):
    """Spacing of the 16-bit format at magnitude ``mag``."""
    mbits, emin = (10, -14) if dtype == "f16" else (7, -126)
    a = np.maximum(np.abs(mag), 2.0 ** emin)
    return 2.0 ** (np.floor(np.log2(a)) - mbits)


def assert_close16(got, want, dtype, max_ulp=2, max_abs=1e-2, term_scale=None, what=""):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (got.shape, want.shape)
    d = np.abs(ord16(got) - ord16(want))
    gv, wv = synth.storage_to_f64(got, dtype), synth.storage_to_f64(want, dtype)
    dv = np.abs(gv - wv)
    ok = d <= max_ulp
    if term_scale is not None:
        relaxed = max_ulp * ulp_at(np.maximum(np.abs(wv), term_scale), dtype)
        ok |= dv <= np.minimum(relaxed, max_abs)
    if d.size and not ok.all():
        i = np.unravel_index(np.argmin(ok), ok.shape)
        raise AssertionError(f"{what}: {int(d[i])} ulp apart at {i}: got {gv[i]!r} want {wv[i]!r}"
                             + ("" if term_scale is None else f" term scale {term_scale[i]!r}"))
    return {"max_ulp_of_result": int(d.max()) if d.size else 0,
            "within_2ulp_of_result": float((d <= 2).mean()) if d.size else 1.0,
            "exact_frac": float((d == 0).mean()) if d.size else 1.0}


def layernorm_terms(x, gamma, beta, dtype, eps):
    """|(x - mu) * rstd * gamma| and |beta|, elementwise max (float64)."""
    xv = synth.storage_to_f64(x, dtype)
    mu = xv.mean(axis=1, keepdims=True)
    rstd = 1.0 / np.sqrt(((xv - mu) ** 2).mean(axis=1, keepdims=True) + float(np.float32(eps)))
    g = 1.0 if gamma is None else synth.storage_to_f64(gamma, dtype)[None, :]
    b = 0.0 if beta is None else synth.storage_to_f64(beta, dtype)[None, :]
    return np.maximum(np.abs((xv - mu) * rstd * g), np.abs(b) + 0 * xv)


def rope_terms(x, cos, sin, heads, head_dim, rope_dim, dtype, cs_dtype, neox):
    """For each output channel of a rotated pair, max(|x_a c|, |x_b s|) (float64);
    pass-through channels get 0."""
    T = x.shape[0]
    xv = synth.storage_to_f64(x, dtype)[:, : heads * head_dim].reshape(T, heads, head_dim)
    return _pair_terms(xv, cos, sin, rope_dim, cs_dtype, neox).reshape(T, heads * head_dim)


def _pair_terms(xv, cos, sin, rope_dim, cs_dtype, neox):
    head_dim = xv.shape[-1]
    c = synth.storage_to_f64(cos, cs_dtype)[:, None, :]
    s = synth.storage_to_f64(sin, cs_dtype)[:, None, :]
    half = rope_dim // 2
    start = head_dim - rope_dim
    p = np.arange(half)
    a = start + (p if neox else 2 * p)
    b = start + (p + half if neox else 2 * p + 1)
    xa, xb = xv[..., a], xv[..., b]
    m = np.maximum(np.maximum(np.abs(xa * c), np.abs(xb * s)),
                   np.maximum(np.abs(xa * s), np.abs(xb * c)))
    out = np.zeros_like(xv)
    out[..., a] = m
    out[..., b] = m
    return out


def qk_terms(x, q_weight, k_weight, cos, sin, q_heads, kv_heads, head_dim, rope_dim, dtype,
             cs_dtype, neox, eps):
    """rope_terms of u = x * w for the q/k heads, times each head's rstd (float64);
    shape [tokens, (q_heads + kv_heads) * head_dim]."""
    T = x.shape[0]
    H = q_heads + kv_heads
    xv = synth.storage_to_f64(x, dtype)[:, : H * head_dim].reshape(T, H, head_dim)
    rstd = 1.0 / np.sqrt((xv ** 2).mean(axis=2, keepdims=True) + float(np.float32(eps)))
    w = np.ones((H, head_dim))
    if q_weight is not None:
        w[:q_heads] = synth.storage_to_f64(q_weight, dtype)
    if k_weight is not None:
        w[q_heads:] = synth.storage_to_f64(k_weight, dtype)
    terms = _pair_terms(xv * w[None], cos, sin, rope_dim, cs_dtype, neox) * rstd
    return terms.reshape(T, H * head_dim)


def assert_codes(got, want, min_exact=0.999, max_step=1, what=""):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape
    d = np.abs(ord8(got) - ord8(want))
    exact = float((d == 0).mean()) if d.size else 1.0
    worst = int(d.max()) if d.size else 0
    assert worst <= max_step, f"{what}: codes {worst} steps apart"
    assert exact >= min_exact, f"{what}: only {exact:.6f} of codes bit-exact"
    return {"max_step": worst, "exact_frac": exact}


def assert_scales(got, want, rtol=1e-6, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    rel = np.abs(got - want) / np.abs(want)
    assert rel.max() <= rtol, f"{what}: scale rel err {rel.max():.3e}"
    return float(rel.max())


def e4m3_boundaries():
    """Decision boundaries of round-to-nearest into E4M3FN: the midpoints between
    consecutive non-negative finite values (float64)."""
    v = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    v = np.unique(v.numpy())
    return (v[1:] + v[:-1]) / 2


def assert_codes_away_from_ties(got, want, quotient, rel=2.0 ** -20, what=""):
    """FP8 codes equal wherever the exact quotient z / scale lies farther than
    ``rel`` (relative) from an E4M3 rounding boundary; within that distance of a
    boundary either neighbour is a correct rounding at the precision the binary32
    row statistics resolve.  Never more than one step apart."""
    got = np.asarray(got)
    want = np.asarray(want)
    d = np.abs(ord8(got) - ord8(want))
    assert d.max() <= 1 if d.size else True, f"{what}: codes {int(d.max())} steps apart"
    b = e4m3_boundaries()
    q = np.abs(np.asarray(quotient, dtype=np.float64))
    i = np.clip(np.searchsorted(b, q), 1, len(b) - 1)
    gap = np.minimum(np.abs(q - b[i - 1]), np.abs(q - b[i]))
    near = gap <= rel * np.maximum(q, 2.0 ** -9)
    bad = (d != 0) & ~near
    assert not bad.any(), (f"{what}: {int(bad.sum())} codes differ away from a rounding "
                           f"boundary, e.g. at {np.argwhere(bad)[0]}")
    return {"exact_frac": float((d == 0).mean()), "near_tie_frac": float(near.mean()),
            "max_step": int(d.max()) if d.size else 0}
