"""Pins of the oracle's format encoders/decoders against the format definitions
and independent library decoders (numpy float16, numpy float32 for bfloat16,
torch float8_e4m3fn), by brute force over every code."""
import numpy as np
import pytest
from decimal import Decimal

import oracle
from tests import exact


def test_spot_values_from_format_definitions():
    # OCP E4M3FN: max finite 448 = S.1111.110, 1.0 = exponent 7 = 0x38
    assert oracle.encode_e4m3(448.0) == 0x7E
    assert oracle.encode_e4m3(-448.0) == 0xFE
    assert oracle.encode_e4m3(1.0) == 0x38
    assert oracle.encode_e4m3(0.5) == 0x30
    assert oracle.encode_e4m3(2.0 ** -9) == 0x01          # smallest subnormal
    assert oracle.encode_e4m3(2.0 ** -10) == 0x00         # tie between 0 and 2^-9 -> even
    assert oracle.encode_e4m3(3 * 2.0 ** -10) == 0x02     # tie between 1 and 2 (x2^-9) -> even
    assert oracle.encode_e4m3(1.0625) == 0x38             # tie 1.0 / 1.125 -> even (1.0)
    assert oracle.encode_e4m3(1.1875) == 0x3A             # tie 1.125 / 1.25 -> even (1.25)
    assert oracle.encode_e4m3(2.0 ** -6) == 0x08          # smallest normal
    assert oracle.encode_e4m3(-0.0) == 0x80
    assert oracle.encode_e4m3(-1e-30) == 0x80             # tiny negative -> -0
    assert oracle.encode_e4m3(463.99) == 0x7E             # below the 448/480 midpoint
    assert oracle.encode_e4m3(464.0) == 0x7E              # the 448/480 midpoint ties to even 448
    assert oracle.encode_e4m3(464.5) == 0x7F              # above it: rounds past 448 -> NaN
    assert oracle.encode_f16(1.0) == 0x3C00
    assert oracle.encode_f16(65504.0) == 0x7BFF
    assert oracle.encode_f16(65520.0) == 0x7C00           # midpoint rounds to even = inf
    assert oracle.encode_f16(2.0 ** -24) == 0x0001
    assert oracle.encode_bf16(1.0) == 0x3F80
    assert oracle.encode_bf16(-2.0) == 0xC000
    assert oracle.decode_e4m3(0x7E) == 448.0
    assert np.isnan(oracle.decode_e4m3(0x7F)) and np.isnan(oracle.decode_e4m3(0xFF))


def test_decoders_match_library_decoders_on_every_code():
    import torch

    f16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    lib = f16.view(np.float16).astype(np.float64)
    mine = np.array([oracle.decode_f16(int(c)) for c in f16])
    fin = np.isfinite(lib)
    assert np.array_equal(mine[fin], lib[fin])
    assert np.array_equal(np.isnan(mine), np.isnan(lib))
    bf = np.arange(65536, dtype=np.uint32)
    lib = (bf << 16).view(np.float32).astype(np.float64)
    mine = np.array([oracle.decode_bf16(int(c)) for c in bf])
    fin = np.isfinite(lib)
    assert np.array_equal(mine[fin], lib[fin])
    assert np.array_equal(np.isnan(mine), np.isnan(lib))
    e = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = e.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([oracle.decode_e4m3(int(c)) for c in range(256)])
    fin = np.isfinite(lib)
    assert np.array_equal(mine[fin], lib[fin])
    assert np.array_equal(np.isnan(mine), np.isnan(lib))


def test_round_trip_every_finite_code():
    for c in range(65536):
        v = oracle.decode_f16(c)
        if np.isfinite(v):
            assert oracle.encode_f16(v) == c
        v = oracle.decode_bf16(c)
        if np.isfinite(v):
            assert oracle.encode_bf16(v) == c
    for c in range(256):
        v = oracle.decode_e4m3(c)
        if np.isfinite(v):
            assert oracle.encode_e4m3(v) == c


def _probe_values(rng, scale_lo, scale_hi, count):
    mags = np.exp(rng.uniform(np.log(scale_lo), np.log(scale_hi), size=count))
    sign = np.where(rng.random(count) < 0.5, -1.0, 1.0)
    return mags * sign


def _midpoints(codes_vals):
    v = np.sort(codes_vals[np.isfinite(codes_vals) & (codes_vals >= 0)])
    return (v[:-1] + v[1:]) / 2.0   # exact in float64 for these formats


def test_f16_encoder_matches_numpy_and_brute_force():
    rng = np.random.default_rng(11)
    vals = np.concatenate([
        _probe_values(rng, 1e-9, 7e4, 4000),
        _midpoints(np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64))[::37],
    ])
    for v in vals:
        lib = int(np.array([v]).astype(np.float16).view(np.uint16)[0])
        assert oracle.encode_f16(v) == lib, v
    for v in vals[::8]:
        assert oracle.encode_f16(v) == exact.round_to(Decimal(float(v)), "f16"), v


def test_bf16_encoder_matches_brute_force():
    rng = np.random.default_rng(12)
    mids = _midpoints((np.arange(0, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
                      .astype(np.float64))
    vals = np.concatenate([_probe_values(rng, 1e-40, 1e38, 3000), mids[::53], -mids[::97]])
    for v in vals:
        assert oracle.encode_bf16(v) == exact.round_to(Decimal(float(v)), "bf16"), v


def test_e4m3_encoder_matches_brute_force_and_torch():
    import torch

    rng = np.random.default_rng(13)
    allv = np.array([oracle.decode_e4m3(c) for c in range(0x7F)])
    mids = _midpoints(allv)
    vals = np.concatenate([_probe_values(rng, 1e-5, 463.0, 5000), mids, -mids,
                           np.nextafter(mids, 0), np.nextafter(mids, 1e9)])
    for v in vals:
        assert oracle.encode_e4m3(v) == exact.round_to(Decimal(float(v)), "e4m3"), v
    # torch's float32 -> float8_e4m3fn conversion is round-to-nearest-even; check
    # it on values exactly representable in float32
    v32 = vals.astype(np.float32)
    t = torch.from_numpy(v32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = np.array([oracle.encode_e4m3(float(v)) for v in v32])
    assert np.array_equal(mine, t)


@pytest.mark.parametrize("fmt,enc", [("f16", oracle.encode_f16), ("bf16", oracle.encode_bf16)])
def test_signed_zero_and_overflow(fmt, enc):
    assert enc(0.0) == 0
    assert enc(-0.0) == 0x8000
    assert enc(float("inf")) == (0x7C00 if fmt == "f16" else 0x7F80)
    assert enc(-float("inf")) == (0xFC00 if fmt == "f16" else 0xFF80)
