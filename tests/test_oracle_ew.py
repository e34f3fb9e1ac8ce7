"""Pins of the oracle's elementwise add / scale / cast ("TileLang tutorial, ch.
13", s3.1.1 reference semantics a + b and (x * alpha) cast to the output
dtype; s1.2's scale+add scenario y = x * a + b): one rounding from the exact
value."""
from decimal import Decimal

import numpy as np
import pytest

import oracle
from quant_row_workgroup_amd import synth
from tests import exact

FMTS = ["f16", "bf16", "f32"]


def _exact_round(v: Decimal, fmt: str) -> int:
    if fmt == "f32":
        return int(np.float32(exact.round_f32(v)).view(np.uint32))
    return exact.round_to(v, fmt)


def _bits(y, fmt):
    return y.view(np.uint32) if fmt == "f32" else y


def _dec(v, fmt):
    if fmt == "f32":
        return Decimal(float(v))
    return exact.dec(int(v), fmt)


@pytest.mark.parametrize("xf", FMTS)
@pytest.mark.parametrize("yf", FMTS)
@pytest.mark.parametrize("with_b", [True, False])
def test_brute_force_exact(xf, yf, with_b):
    if with_b and yf != xf:
        pytest.skip("scale+add keeps the input dtype")
    x = synth.normal(61, (257,), 0.0, 3.0, xf, outlier_frac=0.05, outlier_mul=1e3)
    b = synth.normal(62, (257,), 0.0, 3.0, xf) if with_b else None
    alpha = float(np.float32(0.7071067811865476))
    y = oracle.ew_scale_add(x, b, alpha, xf, yf)
    A = Decimal(alpha)
    for i in range(x.size):
        v = _dec(x[i], xf) * A + (_dec(b[i], xf) if with_b else 0)
        assert int(_bits(y, yf)[i]) == _exact_round(v, yf), i


def test_sum_is_rounded_once_not_twice():
    # x * alpha = (1 + 2^-18)(1 - 2^-18) 2^-7 = 2^-7 - 2^-43 and b = 2^17 + 2^-6 (odd last
    # bit): the exact sum lies just below the binary32 midpoint b + 2^-7, so it rounds to
    # b; a double sum would land on the midpoint and tie to the even neighbour b + 2^-6
    x = np.array([1 + 2.0 ** -18], np.float32)
    alpha = (1 - 2.0 ** -18) * 2.0 ** -7
    assert float(np.float32(alpha)) == alpha
    b = np.array([2.0 ** 17 + 2.0 ** -6], np.float32)
    y = oracle.ew_scale_add(x, b, alpha, "f32")
    assert y[0] == b[0]
    # the mirrored case rounds up
    y = oracle.ew_scale_add(-x, -b, alpha, "f32")
    assert y[0] == -b[0]
    x2 = np.array([1 + 2.0 ** -18], np.float32)
    y = oracle.ew_scale_add(x2, b, float(np.float32((1 + 2.0 ** -18) * 2.0 ** -7)), "f32")
    # 2^-7 + 2^-24 + 2^-43 above b: past the midpoint, so b + 2^-6
    assert y[0] == np.float32(2.0 ** 17 + 2.0 ** -5)


@pytest.mark.parametrize("xf,yf", [("f32", "f16"), ("f32", "bf16"), ("f16", "f32"),
                                   ("bf16", "f32"), ("f16", "bf16")])
def test_pure_cast_matches_the_format_conversion(xf, yf):
    # alpha = 1, no b: a plain dtype conversion (numpy / torch nearest-even casts)
    x = synth.normal(63, (4099,), 0.0, 50.0, xf, outlier_frac=0.01, outlier_mul=1e2)
    y = oracle.ew_scale_add(x, None, 1.0, xf, yf)
    want = synth.to_storage(synth.storage_to_f64(x, xf), yf)
    assert np.array_equal(_bits(y, yf), _bits(want, yf))


@pytest.mark.parametrize("fmt", FMTS)
def test_power_of_two_scale_is_exact_and_add_of_negation_is_zero(fmt):
    x = synth.normal(64, (1000,), 0.0, 1.0, fmt)
    y = oracle.ew_scale_add(x, None, 0.25, fmt, fmt)
    assert np.array_equal(synth.storage_to_f64(y, fmt), synth.storage_to_f64(x, fmt) * 0.25)
    neg = synth.to_storage(-synth.storage_to_f64(x, fmt), fmt)
    z = oracle.ew_scale_add(x, neg, 1.0, fmt)
    assert np.all(synth.storage_to_f64(z, fmt) == 0.0)
    two = oracle.ew_scale_add(x, x, 1.0, fmt)
    assert np.array_equal(synth.storage_to_f64(two, fmt), 2 * synth.storage_to_f64(x, fmt))


def test_overflow_saturates_to_infinity_and_empty_is_fine():
    x = np.array([60000.0, -60000.0], np.float32)
    y = oracle.ew_scale_add(x, None, 2.0, "f32", "f16")
    assert list(y) == [0x7C00, 0xFC00]  # binary16 overflow rounds to +-inf
    assert oracle.ew_scale_add(np.zeros(0, np.float32), None, 1.0, "f32").size == 0
