"""Pins of the oracle's RoPE ("TileLang tutorial, ch. 13", s3.3.1 pairing
conventions and partial rotation, s3.3.2 reference, s5.3 self-check)."""
from decimal import Decimal

import numpy as np
import pytest

import oracle
from quant_row_workgroup_amd import synth
from tests import exact


def _x(seed, tokens, n, fmt):
    return synth.normal(seed, (tokens, n), 0.0, 1.0, fmt)


def _const_table(tokens, half, value, cs_fmt):
    return synth.to_storage(np.full((tokens, half), value), cs_fmt)


CASES = [("f16", "f32"), ("bf16", "bf16"), ("f16", "f16"), ("bf16", "f32")]


@pytest.mark.parametrize("fmt,cs", CASES)
@pytest.mark.parametrize("neox", [True, False])
def test_identity_rotation_returns_x(fmt, cs, neox):
    # the page's self-check: c = 1, s = 0 must give x back unchanged
    x = _x(1, 5, 4 * 64, fmt)
    c = _const_table(5, 32, 1.0, cs)
    s = _const_table(5, 32, 0.0, cs)
    y = oracle.rope(x, c, s, heads=4, head_dim=64, rope_dim=64, dtype=fmt, cs_dtype=cs, neox=neox)
    assert np.array_equal(y, x)


@pytest.mark.parametrize("fmt,cs", CASES)
def test_quarter_turn_pairs_and_conventions_differ(fmt, cs):
    # c = 0, s = 1: interleaved gives (-x[2p+1], x[2p]); NeoX gives (-x[p+H], x[p]);
    # and the two conventions must disagree
    T, H, D = 3, 2, 32
    x = _x(2, T, H * D, fmt)
    c = _const_table(T, D // 2, 0.0, cs)
    s = _const_table(T, D // 2, 1.0, cs)
    yi = oracle.rope(x, c, s, H, D, D, fmt, cs, neox=False)
    yn = oracle.rope(x, c, s, H, D, D, fmt, cs, neox=True)
    neg = np.uint16(0x8000)
    xh = x.reshape(T, H, D)
    want_i = np.empty_like(xh)
    want_i[..., 0::2] = xh[..., 1::2] ^ neg
    want_i[..., 1::2] = xh[..., 0::2]
    want_n = np.empty_like(xh)
    want_n[..., : D // 2] = xh[..., D // 2:] ^ neg
    want_n[..., D // 2:] = xh[..., : D // 2]
    # 0 * x in the other term leaves a signed zero that the sum absorbs: -x + 0 = -x
    assert np.array_equal(yi.reshape(T, H, D), want_i)
    assert np.array_equal(yn.reshape(T, H, D), want_n)
    assert not np.array_equal(yi, yn)


@pytest.mark.parametrize("fmt,cs", CASES)
def test_neox_is_interleaved_conjugated_by_the_pair_permutation(fmt, cs):
    # NeoX(x) = P^T Interleaved(P x), with P taking (p, p+H) to (2p, 2p+1), bit-exactly
    T, H, D, R = 4, 3, 48, 32
    x = _x(3, T, H * D, fmt)
    c, s = synth.rope_table(T, R, cs)
    start = D - R
    perm = np.arange(H * D).reshape(H, D)
    span = perm[:, start:].copy()
    inter = np.empty_like(span)
    inter[:, 0::2] = span[:, : R // 2]
    inter[:, 1::2] = span[:, R // 2:]
    perm[:, start:] = inter
    perm = perm.reshape(-1)           # position j of P x holds x[perm[j]]
    px = np.ascontiguousarray(x[:, perm])
    yi = oracle.rope(px, c, s, H, D, R, fmt, cs, neox=False)
    back = np.empty_like(yi)
    back[:, perm] = yi
    yn = oracle.rope(x, c, s, H, D, R, fmt, cs, neox=True)
    assert np.array_equal(back, yn)


@pytest.mark.parametrize("fmt,cs", CASES)
@pytest.mark.parametrize("neox", [True, False])
def test_brute_force_small(fmt, cs, neox):
    # 4 tokens x (2 heads x 8), full rotation; then a partial span (rope 8 of 24)
    for (H, D, R) in [(2, 8, 8), (2, 24, 8)]:
        x = _x(4, 4, H * D, fmt)
        c, s = synth.rope_table(4, R, cs, base=3.0)  # large angles exercise both terms
        y = oracle.rope(x, c, s, H, D, R, fmt, cs, neox=neox)
        for t in range(4):
            want = exact.rope_ref(x[t], c[t], s[t], H, D, R, fmt, cs, neox)
            assert [int(v) for v in y[t]] == want, (H, D, R, t)


@pytest.mark.parametrize("neox", [True, False])
def test_pass_through_channels_are_copied_and_strides_respected(neox):
    T, H, D, R = 3, 4, 64, 16
    x = _x(5, T, H * D, "bf16")
    wide = np.full((T, H * D + 40), 0x7777, dtype=np.uint16)
    wide[:, : H * D] = x
    c, s = synth.rope_table(T, R, "f32")
    y = oracle.rope(wide, c, s, H, D, R, "bf16", "f32", neox=neox, y_stride=H * D + 8,
                    fill=0x4242)
    yh = y[:, : H * D].reshape(T, H, D)
    assert np.array_equal(yh[..., : D - R], x.reshape(T, H, D)[..., : D - R])
    assert np.all(y[:, H * D:] == 0x4242)
    assert np.array_equal(y[:, : H * D], oracle.rope(x, c, s, H, D, R, "bf16", "f32", neox))


def test_rotation_preserves_pair_norm():
    # with exact unit (c, s) the pair norm is kept; with float64 inputs the
    # check is to rounding of the output format
    T, H, D = 6, 2, 64
    x = _x(6, T, H * D, "f16")
    c, s = synth.rope_table(T, D, "f32")
    for neox in (True, False):
        y = synth.storage_to_f64(oracle.rope(x, c, s, H, D, D, "f16", "f32", neox), "f16")
        xv = synth.storage_to_f64(x, "f16")
        pairs = exact.rope_pairs(D, neox)
        a = np.array([p[1] for p in pairs])
        b = np.array([p[2] for p in pairs])
        xh, yh = xv.reshape(T, H, D), y.reshape(T, H, D)
        nx = np.hypot(xh[..., a], xh[..., b])
        ny = np.hypot(yh[..., a], yh[..., b])
        cv, sv = c.astype(np.float64), s.astype(np.float64)
        unit = np.sqrt(cv ** 2 + sv ** 2)[:, None, :]
        assert np.all(np.abs(ny - nx * unit) <= 2.0 ** -10 * nx + 1e-7)


@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("fmt,cs", [("bf16", "bf16"), ("f16", "f32")])
def test_unrounded_output_is_the_exact_rotation(fmt, cs, neox):
    # the optional float64 output carries each rotated value before its
    # rounding (pass-through channels: x itself)
    T, H, D, R = 3, 2, 24, 16
    x = synth.normal(51, (T, H * D), 0.0, 2.0, fmt)
    c, s = synth.rope_table(T, R, cs, base=7.0)
    y, z = oracle.rope(x, c, s, H, D, R, fmt, cs, neox, want_z=True)
    for t in range(T):
        xs = [exact.dec(b, fmt) for b in x[t]]
        ex = exact.rope_values(xs, [exact.dec(b, cs) for b in c[t]],
                               [exact.dec(b, cs) for b in s[t]], H, D, R, neox)
        for j, v in enumerate(ex):
            assert abs(Decimal(float(z[t, j])) - v) <= abs(v) * Decimal(2) ** -50, (t, j)
            assert exact.round_to(Decimal(float(z[t, j])), fmt) == int(y[t, j])
