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
    """Elementwise max (float64) of |(x - mu) * rstd * gamma|, |beta|, and the
    scale at which 2 ulp of the 16-bit format cover the binary32 mean's own
    rounding carried through x - mu: a mean of n values summed in binary32
    is within (ceil(log2 n) + 2) * 2^-24 * mean|x| of the exact one, and an
    output whose x - mu cancels below that bound cannot be resolved by any
    binary32 evaluation (2 * ulp_at(t) >= t * 2^-mbits, so t = e * 2^mbits)."""
    xv = synth.storage_to_f64(x, dtype)
    n = xv.shape[1]
    mu = xv.mean(axis=1, keepdims=True)
    rstd = 1.0 / np.sqrt(((xv - mu) ** 2).mean(axis=1, keepdims=True) + float(np.float32(eps)))
    g = 1.0 if gamma is None else synth.storage_to_f64(gamma, dtype)[None, :]
    b = 0.0 if beta is None else synth.storage_to_f64(beta, dtype)[None, :]
    mbits = 10 if dtype == "f16" else 7
    e_mu = (np.ceil(np.log2(max(n, 2))) + 2) * 2.0 ** -24 * np.abs(xv).mean(axis=1, keepdims=True)
    mu_term = e_mu * rstd * np.abs(g) * 2.0 ** mbits
    return np.maximum(np.maximum(np.abs((xv - mu) * rstd * g), np.abs(b) + 0 * xv), mu_term)


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


def rotation_terms(x, w, cos, sin, heads, head_dim, rope_dim, dtype, cs_dtype, neox, eps):
    """For each channel of the fused operator's output, an upper bound on the
    sum of the two products its rotation adds, |y_a c| + |y_b s| with
    y = x * w * rstd over the whole row (float64): twice the larger product.
    Pass-through channels get 0."""
    T = x.shape[0]
    n = heads * head_dim
    xv = synth.storage_to_f64(x, dtype)[:, :n]
    rstd = 1.0 / np.sqrt((xv ** 2).mean(axis=1, keepdims=True) + float(np.float32(eps)))
    wv = np.ones(n) if w is None else synth.storage_to_f64(w, dtype)[:n]
    y = (xv * wv[None] * rstd).reshape(T, heads, head_dim)
    return 2.0 * _pair_terms(y, cos, sin, rope_dim, cs_dtype, neox).reshape(T, n)


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


def assert_codes_away_from_ties(got, want, quotient, rel=2.0 ** -20, what="", magnitude=None):
    """FP8 codes equal wherever the exact quotient z / scale lies farther than
    ``rel`` times its magnitude from an E4M3 rounding boundary; within that
    distance of a boundary either neighbour is a correct rounding at the
    precision the binary32 row statistics resolve.  Never more than one step
    apart.  The magnitude is |z / scale|, or the larger of it and ``magnitude``
    where given: a rotated value is a sum of two products, and its binary32
    error is relative to those products, not to the sum, which cancellation
    can make far smaller (``rotation_terms``)."""
    got = np.asarray(got)
    want = np.asarray(want)
    d = np.abs(ord8(got) - ord8(want))
    assert d.max() <= 1 if d.size else True, f"{what}: codes {int(d.max())} steps apart"
    b = e4m3_boundaries()
    q = np.abs(np.asarray(quotient, dtype=np.float64))
    i = np.clip(np.searchsorted(b, q), 1, len(b) - 1)
    gap = np.minimum(np.abs(q - b[i - 1]), np.abs(q - b[i]))
    m = q if magnitude is None else np.maximum(q, np.asarray(magnitude, dtype=np.float64))
    near = gap <= rel * np.maximum(m, 2.0 ** -9)
    bad = (d != 0) & ~near
    assert not bad.any(), (f"{what}: {int(bad.sum())} codes differ away from a rounding "
                           f"boundary, e.g. at {np.argwhere(bad)[0]}")
    return {"exact_frac": float((d == 0).mean()), "near_tie_frac": float(near.mean()),
            "max_step": int(d.max()) if d.size else 0}


# ------------------------------------------------------------ staged fused form
def rn16_bits(v, dtype):
    """float64 values -> 16-bit storage bits, rounded to nearest, ties to even.
    binary16: numpy's direct float64 -> float16 conversion.  bfloat16: the value
    is first rounded to odd at binary32 precision, then to bfloat16 with ties to
    even, which together round once (24 >= 8 + 2 bits)."""
    v = np.asarray(v, dtype=np.float64)
    if dtype == "f16":
        with np.errstate(over="ignore"):
            return v.astype(np.float16).view(np.uint16)
    with np.errstate(over="ignore"):
        f = v.astype(np.float32)
    b = f.view(np.uint32).copy()
    inexact = (f.astype(np.float64) != v) & np.isfinite(v)
    even = (b & 1) == 0
    toward = np.where((f.astype(np.float64) < v) == (f >= 0), 1, -1).astype(np.int64)
    b = np.where(inexact & even, (b.astype(np.int64) + toward).astype(np.uint32), b)
    return ((b.astype(np.uint64) + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def _e4m3_of_f32(q):
    """binary32 values (clamped to +-448) -> E4M3FN codes, ties to even."""
    q = np.clip(np.asarray(q, dtype=np.float32), -448.0, 448.0)
    return torch.from_numpy(np.ascontiguousarray(q)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def _pair_layout(T, H, D, R, neox):
    """Per output channel of [T, H*D]: is it rotated, its role (first or second
    of its pair) and its pair index p; in the rotated span partner(j) is the
    other member of j's pair."""
    start = D - R
    half = R // 2
    k = np.arange(D)
    rot = k >= start
    local = np.where(rot, k - start, 0)
    if neox:
        first = local < half
        p = np.where(first, local, local - half)
        partner = np.where(first, local + half, local - half) + start
    else:
        first = local % 2 == 0
        p = local // 2
        partner = np.where(first, local + 1, local - 1) + start
    partner = np.where(rot, partner, k)
    return rot, first, p, partner


# Bound on the relative error of the kernels' binary32 rstd, as a multiple of
# 2^-24: a sum of n <= 8192 squares with at most 16 serial additions per lane
# slot (two roundings per packed dot), a 3-level slot tree and a 6-level wave
# reduction (<= 25 roundings of non-negative terms), the mean (one rounding
# unless n is a power of two) and eps (one), then a correctly rounded sqrt
# (half the argument's error plus one) and reciprocal (one):
# 27/2 + 2 = 15.5 -> 16.  The normalised product x*w*rstd is rounded once
# more to binary32 before its 16-bit rounding (one more).
STAGED_U_REL = 17.0 * 2.0 ** -24
# A rotated output is one binary32 fma of u_a*c and a binary32 product u_b*s
# (exact for 16-bit tables): at most 2^-24 of the product's magnitude plus
# 2^-24 of the result's, both within 2^-23 of |u_a c| + |u_b s|.
STAGED_Z_REL = 2.0 ** -23


def staged_intervals(x, w, c, s, H, D, R, dt, cs, neox, eps):
    """For the staged fused form, the interval of each stored 16-bit value that a
    binary32 evaluation within the bounds above can produce: returns the
    oracle's codes and scales and dicts of float64 interval ends for the
    normalised values u and the rotated values z ([T, H*D] each)."""
    import oracle

    T = x.shape[0]
    q_o, sc_o, it = oracle.rmsnorm_rope_fp8_rounded(x, w, c, s, H, D, R, dt, cs, neox, eps,
                                                    want_intermediates=True)
    ue = it["u_exact"]
    eta = np.abs(ue) * STAGED_U_REL
    u_lo_bits, u_hi_bits = rn16_bits(ue - eta, dt), rn16_bits(ue + eta, dt)
    u_lo = synth.storage_to_f64(u_lo_bits, dt)
    u_hi = synth.storage_to_f64(u_hi_bits, dt)
    assert np.all(u_lo <= u_hi)
    # the exact rotation at the four corners of each pair's (u_a, u_b) box
    rot, first, p, partner = _pair_layout(T, H, D, R, neox)
    rot_n, first_n = np.tile(rot, H), np.tile(first, H)
    corners = []
    for a_hi in (False, True):
        for b_hi in (False, True):
            pick = np.where(first_n, a_hi, b_hi)[None, :] & rot_n[None, :]
            ub = np.where(pick, u_hi_bits, u_lo_bits)
            _, ze = oracle.rope(np.ascontiguousarray(ub), c, s, H, D, R, dt, cs, neox,
                                want_z=True)
            corners.append(ze)
    corners = np.stack(corners)
    # magnitude of the two products of each rotated output
    cv = synth.storage_to_f64(c, cs)
    sv = synth.storage_to_f64(s, cs)
    pp = np.tile(p, H)
    part = (np.arange(H)[:, None] * D + partner[None, :]).reshape(-1)
    umax = np.maximum(np.abs(u_lo), np.abs(u_hi))
    terms = umax * np.abs(cv[:, pp]) + umax[:, part] * np.abs(sv[:, pp])
    dz = np.where(rot_n[None, :], terms * STAGED_Z_REL, 0.0)
    z_lo = np.where(rot_n[None, :], corners.min(axis=0) - dz, u_lo)
    z_hi = np.where(rot_n[None, :], corners.max(axis=0) + dz, u_hi)
    z_lo = synth.storage_to_f64(rn16_bits(z_lo, dt), dt)
    z_hi = synth.storage_to_f64(rn16_bits(z_hi, dt), dt)
    return q_o, sc_o, {"u": (u_lo, u_hi), "z": (z_lo, z_hi)}


def assert_staged_consistent(q, sc, x, w, c, s, H, D, R, dt, cs, neox, eps=1e-6, what=""):
    """The staged form's bar.  Each stored intermediate may be either 16-bit
    neighbour only where the oracle's unrounded value lies within the kernel's
    binary32 error bound of a rounding boundary (staged_intervals); a row's
    scale must follow from a possible row maximum, and each code must be the
    E4M3 rounding of a possible stored value divided by the kernel's own scale.
    Wherever the intervals hold one value, codes and scales are therefore
    bit-exact.  Returns the oracle's codes and some statistics."""
    q = np.asarray(q)
    sc = np.asarray(sc, dtype=np.float32)
    q_o, sc_o, iv = staged_intervals(x, w, c, s, H, D, R, dt, cs, neox, eps)
    z_lo, z_hi = iv["z"]
    amag_lo = np.where((z_lo <= 0) & (z_hi >= 0), 0.0, np.minimum(np.abs(z_lo), np.abs(z_hi)))
    amag_hi = np.maximum(np.abs(z_lo), np.abs(z_hi))
    floor = float(np.float32(1e-4))
    a_lo = np.maximum(amag_lo.max(axis=1), floor)
    a_hi = np.maximum(amag_hi.max(axis=1), floor)
    s_lo = (a_lo / 448.0).astype(np.float32)
    s_hi = (a_hi / 448.0).astype(np.float32)
    bad = (sc < s_lo) | (sc > s_hi)
    assert not bad.any(), (f"{what}: scale of row {int(np.argmax(bad))} outside what the "
                           f"possible row maxima give: {sc[bad][0]!r} not in "
                           f"[{s_lo[bad][0]!r}, {s_hi[bad][0]!r}]")
    S = sc.astype(np.float64)[:, None]
    c_lo = ord8(_e4m3_of_f32((z_lo / S).astype(np.float32)))
    c_hi = ord8(_e4m3_of_f32((z_hi / S).astype(np.float32)))
    got = ord8(q)
    badc = (got < c_lo) | (got > c_hi)
    assert not badc.any(), (f"{what}: {int(badc.sum())} codes outside the codes of their "
                            f"possible stored values, e.g. at {np.argwhere(badc)[0]}")
    d = np.abs(got - ord8(q_o))
    amb = (z_lo != z_hi)
    return {"exact_frac": float((d == 0).mean()) if d.size else 1.0,
            "max_step": int(d.max()) if d.size else 0,
            "ambiguous_frac": float(amb.mean()) if amb.size else 0.0,
            "scale_rel": float(np.max(np.abs(sc.astype(np.float64) - sc_o) / sc_o))
            if sc.size else 0.0}
