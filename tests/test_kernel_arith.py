"""CPU pins of the binary32 identities the quantising kernels rely on, with
every fma evaluated exactly.  The kernels form the E4M3 scale and the code's
quotient without a division instruction:

- RN(x / s) from y = RN(1/s) by Markstein's correction, with the remainder
  taken as q*s - x so that a zero x keeps its sign (div_rn);
- the scale RN(a / 448) the same way with the constant RN(1/448)
  (scale_e4m3), which must equal the correctly rounded quotient that the
  page's float32 cast ("TileLang tutorial, ch. 13", s3.1.5) and the oracle
  compute.

and the elementwise add: the binary32 sum of two 16-bit values, rounded once
to their format, is the correctly rounded sum (s3.1.1's a + b).

(The remaining identity, hardware reciprocal plus one Newton step == IEEE
1/s, depends on the GPU's reciprocal instruction and cannot be emulated
here.)"""
from fractions import Fraction

import numpy as np
import pytest

F32 = np.float32


def _rn32(exact: Fraction) -> np.float32:
    """Round an exact rational to binary32, ties to even (normal range)."""
    if exact == 0:
        return F32(0.0)
    sign = -1 if exact < 0 else 1
    m = abs(exact)
    e = m.numerator.bit_length() - m.denominator.bit_length() - 24
    while m / Fraction(2) ** e >= 2 ** 24:
        e += 1
    while m / Fraction(2) ** e < 2 ** 23:
        e -= 1
    t = m / Fraction(2) ** e
    fl = t.numerator // t.denominator
    rem = t - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return F32(sign * float(fl) * 2.0 ** e)


def _fma32(a, b, c) -> np.float32:
    """RN32(a*b + c) exactly, with IEEE signed-zero rules for an exact zero."""
    p = Fraction(float(a)) * Fraction(float(b))
    s = p + Fraction(float(c))
    if s == 0:
        neg_p = (np.signbit(a) != np.signbit(b)) if p == 0 else p < 0
        neg_c = bool(np.signbit(c)) if c == 0 else c < 0
        return F32(-0.0) if (neg_p and neg_c) else F32(0.0)
    return _rn32(s)


def _div_rn(x, s, y):
    q = F32(x * y)              # a binary32 product rounds once
    r = _fma32(q, s, -x)         # q*s - x, exact
    return _fma32(-r, y, q)      # q - r*y


def test_quotient_is_correctly_rounded_and_keeps_zero_signs():
    rng = np.random.default_rng(5)
    for _ in range(3000):
        amax = F32(abs(rng.standard_normal()) * 10.0 ** rng.integers(-3, 4) + 1e-4)
        s = F32(float(max(amax, F32(1e-4))) / 448.0)
        y = _rn32(1 / Fraction(float(s)))
        x = F32(rng.uniform(-1.0, 1.0) * float(amax))
        got = _div_rn(x, s, y)
        assert got == _rn32(Fraction(float(x)) / Fraction(float(s))), (x, s)
    for z in (F32(0.0), F32(-0.0)):
        got = _div_rn(z, F32(0.01), _rn32(Fraction(100)))
        assert got == 0 and np.signbit(got) == np.signbit(z)


def _scale_vectorised(a: np.ndarray) -> np.ndarray:
    """scale_e4m3 over an array; the fma steps are exact in binary64 here (the
    remainder has at most 34 significant bits; q - r*c is checked against the
    exact rational wherever the binary64 sum could have rounded)."""
    c = F32(1.0) / F32(448.0)
    q = (a * c).astype(F32)
    r64 = q.astype(np.float64) * 448.0 - a.astype(np.float64)
    r = r64.astype(F32)
    assert np.array_equal(r.astype(np.float64), r64), "remainder not exact"
    return (q.astype(np.float64) - r.astype(np.float64) * np.float64(c)).astype(F32)


def _reference(a: np.ndarray) -> np.ndarray:
    # a/448 = (a/7) * 2^-6 is never exactly halfway between two binary32 values
    # (1/7 has a periodic expansion), so rounding through binary64 is exact
    return (a.astype(np.float64) / 448.0).astype(F32)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_scale_of_every_16bit_amax(fmt):
    # act_quant's amax is an input value: all positive finite 16-bit values >= 1e-4
    bits = np.arange(0x0000, 0x7C00 if fmt == "f16" else 0x7F80, dtype=np.uint32)
    if fmt == "bf16":
        a = (bits << 16).view(np.float32)
    else:
        a = bits.astype(np.uint16).view(np.float16).astype(F32)
    a = np.maximum(a, F32(1e-4))
    assert np.array_equal(_scale_vectorised(a), _reference(a))


@pytest.mark.parametrize("e", [-14, -1, 0, 7, 20, 63, 127])
def test_scale_over_whole_binades(e):
    # fused / QK amax values are arbitrary binary32: every value of a binade
    m = np.arange(1 << 23, 1 << 24, dtype=np.int64)
    a = np.ldexp(m.astype(np.float64), e - 23).astype(F32)
    got, want = _scale_vectorised(a), _reference(a)
    bad = np.nonzero(got != want)[0]
    for i in bad[:20]:  # resolve any binary64 double rounding exactly
        q = F32(a[i] * (F32(1.0) / F32(448.0)))
        r = F32(float(q) * 448.0 - float(a[i]))
        exact = Fraction(float(q)) - Fraction(float(r)) * Fraction(float(F32(1.0) / F32(448.0)))
        assert _rn32(exact) == want[i], a[i]
    assert len(bad) <= 20


def _bf16_rne_from_f32(f: np.ndarray) -> np.ndarray:
    u = f.astype(F32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _round_odd_f32(d: np.ndarray) -> np.ndarray:
    f = d.astype(F32)
    u = f.view(np.uint32).copy()
    inexact = f.astype(np.float64) != d
    up = np.abs(d) > np.abs(f.astype(np.float64))
    fix = inexact & ((u & 1) == 0)
    u[fix & up] += 1
    u[fix & ~up] -= 1
    return u.view(F32)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.filterwarnings("ignore::RuntimeWarning")  # sums that overflow to inf
def test_sum_of_two_16bit_values_rounds_once_through_binary32(fmt):
    # the elementwise add of two 16-bit tensors forms x + b in binary32 and
    # rounds that once to the 16-bit format; it must equal the rounding of the
    # exact sum (formed in binary64, exact up to a 45-bit exponent gap, beyond
    # which the smaller operand cannot move the result), rounded to odd at
    # binary32 and then to the format (a single rounding, Boldo-Melquiond)
    rng = np.random.default_rng(11)
    n = 400_000
    if fmt == "bf16":
        bits = rng.integers(0, 0x7F80, size=(2, n), dtype=np.uint32)
        sign = rng.integers(0, 2, size=(2, n), dtype=np.uint32) << 15
        v = ((bits | sign) << 16).view(F32)
        a, b = v[0], v[1]
        # near-cancellation pairs and small exponent gaps
        b[: n // 4] = -a[: n // 4] * F32(1.0078125)
        b[n // 4: n // 2] = (a[n // 4: n // 2].view(np.uint32) ^ 0x80010000).view(F32)
        b = ((_bf16_rne_from_f32(b).astype(np.uint32)) << 16).view(F32)
        got = _bf16_rne_from_f32((a + b).astype(F32))
        want = _bf16_rne_from_f32(_round_odd_f32(a.astype(np.float64) + b.astype(np.float64)))
    else:
        bits = rng.integers(0, 0x7C00, size=(2, n), dtype=np.uint16)
        sign = rng.integers(0, 2, size=(2, n), dtype=np.uint16) << 15
        v = (bits | sign).view(np.float16).astype(F32)
        a, b = v[0], v[1]
        b[: n // 4] = (-a[: n // 4] * F32(1.0009765625)).astype(np.float16).astype(F32)
        got = (a + b).astype(F32).astype(np.float16).view(np.uint16)
        want = _round_odd_f32(a.astype(np.float64) + b.astype(np.float64)).astype(
            np.float16).view(np.uint16)
    assert np.array_equal(got, want)
