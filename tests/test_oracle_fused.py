"""Pins of the oracle's fused RMSNorm -> RoPE -> per-token E4M3FN operator
("TileLang tutorial, ch. 13", s3.3.4 dataflow, s3.1.5 per-token cast)."""
import numpy as np
import pytest
from decimal import Decimal

import oracle
from quant_row_workgroup_amd import synth
from tests import exact


def _inputs(seed, T, H, D, R, fmt, cs, outliers=True, base=10000.0):
    x = synth.normal(seed, (T, H * D), 0.0, 3.0, fmt,
                     outlier_frac=0.01 if outliers else 0.0, outlier_mul=10.0)
    w = synth.normal(seed + 1, (H * D,), 1.0, 0.1, fmt)
    c, s = synth.rope_table(T, R, cs, base=base)
    return x, w, c, s


def _mag(code):
    return np.asarray(code) & 0x7F


@pytest.mark.parametrize("fmt,cs", [("bf16", "bf16"), ("f16", "f32")])
@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("shape", [(1, 8, 8), (2, 16, 8), (1, 24, 16)])
def test_brute_force_small(fmt, cs, neox, shape):
    H, D, R = shape
    x, w, c, s = _inputs(7, 4, H, D, R, fmt, cs, base=3.0)
    q, sc = oracle.rmsnorm_rope_fp8(x, w, c, s, H, D, R, fmt, cs, neox, 1e-6)
    for t in range(4):
        codes, scale, _ = exact.fused_ref(x[t], w, c[t], s[t], H, D, R, fmt, cs, neox, 1e-6)
        assert float(sc[t]) == scale, t
        assert [int(v) for v in q[t]] == codes, t


def test_z_matches_exact_composition():
    # the unrounded intermediate: RoPE(x * rstd * w) evaluated exactly
    H, D, R = 2, 32, 32
    x, w, c, s = _inputs(8, 3, H, D, R, "bf16", "bf16")
    _, _, z = oracle.rmsnorm_rope_fp8(x, w, c, s, H, D, R, "bf16", "bf16", True, 1e-6,
                                      want_z=True)
    for t in range(3):
        _, _, zt = exact.fused_ref(x[t], w, c[t], s[t], H, D, R, "bf16", "bf16", True, 1e-6)
        zt = np.array([float(v) for v in zt])
        assert np.all(np.abs(z[t] - zt) <= 1e-14 * np.abs(zt).max())


def test_codes_are_the_quantised_z_and_the_scale_is_amax_over_448():
    H, D, R = 32, 128, 128
    x, w, c, s = _inputs(9, 16, H, D, R, "bf16", "bf16")
    q, sc, z = oracle.rmsnorm_rope_fp8(x, w, c, s, H, D, R, "bf16", "bf16", True, 1e-6,
                                       want_z=True)
    amax = np.abs(z).max(axis=1)
    for t in range(16):
        assert float(sc[t]) == exact.round_f32(Decimal(float(amax[t])) / 448)
        # the binary32 quotient (numpy's float64 quotient rounds innocuously to float32)
        v = np.clip((z[t] / np.float64(sc[t])).astype(np.float32).astype(np.float64), -448, 448)
        want = [exact.round_to(Decimal(float(e)), "e4m3") for e in v[::61]]
        assert [int(e) for e in q[t, ::61]] == want
    # the largest magnitude of every row maps to the largest finite code
    assert np.all(_mag(q).max(axis=1) == 0x7E)


def test_dequantised_error_within_half_an_e4m3_step():
    H, D, R = 8, 128, 64
    x, w, c, s = _inputs(10, 32, H, D, R, "bf16", "bf16")
    q, sc, z = oracle.rmsnorm_rope_fp8(x, w, c, s, H, D, R, "bf16", "bf16", True, 1e-6,
                                       want_z=True)
    import torch

    deq = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    v = z / sc.astype(np.float64)[:, None]
    a = np.maximum(np.abs(v), 2.0 ** -6)
    step = 2.0 ** (np.floor(np.log2(a)) - 3)
    # half a step, plus the binary32 rounding of the quotient the code is decided on
    assert np.all(np.abs(deq - v) <= 0.5 * step * (1 + 1e-12) + np.abs(v) * 2.0 ** -24)


def test_zero_row_gives_zero_codes_and_the_floor_scale():
    H, D, R = 4, 64, 64
    x, w, c, s = _inputs(11, 3, H, D, R, "bf16", "bf16")
    x[1] = 0
    q, sc = oracle.rmsnorm_rope_fp8(x, w, c, s, H, D, R, "bf16", "bf16", True, 1e-6)
    assert np.all(q[1] == 0)
    assert sc[1] == np.float32(1e-4) / np.float32(448)


@pytest.mark.parametrize("neox", [True, False])
def test_identity_rotation_reduces_to_quantised_rmsnorm(neox):
    # c = 1, s = 0: the rotation is the identity, so the op is quant(RMSNorm(x))
    H, D, R = 2, 16, 16
    x, w, _, _ = _inputs(12, 4, H, D, R, "bf16", "bf16")
    c = synth.to_storage(np.ones((4, R // 2)), "bf16")
    s = synth.to_storage(np.zeros((4, R // 2)), "bf16")
    q, sc = oracle.rmsnorm_rope_fp8(x, w, c, s, H, D, R, "bf16", "bf16", neox, 1e-6)
    for t in range(4):
        xs = [exact.dec(b, "bf16") for b in x[t]]
        ws = [exact.dec(b, "bf16") for b in w]
        r = 1 / (sum(v * v for v in xs) / len(xs) + Decimal(float(np.float32(1e-6)))).sqrt()
        zn = [a * r * b for a, b in zip(xs, ws)]
        scale = exact.round_f32(max(abs(v) for v in zn) / 448)
        assert float(sc[t]) == scale
        want = [exact.round_to(Decimal(exact.round_f32(v / Decimal(scale))), "e4m3") for v in zn]
        assert [int(v) for v in q[t]] == want


def test_partial_rotation_leaves_the_head_prefix_as_plain_quantised_norm():
    # the pages' own reading of the fused op: one 4096-wide head, rotating its last 128
    H, D, R = 1, 4096, 128
    x, w, c, s = _inputs(13, 4, H, D, R, "bf16", "bf16")
    q, sc, z = oracle.rmsnorm_rope_fp8(x, w, c, s, H, D, R, "bf16", "bf16", True, 1e-6,
                                       want_z=True)
    xv = synth.storage_to_f64(x, "bf16")
    wv = synth.storage_to_f64(w, "bf16")
    rstd = 1.0 / np.sqrt((xv ** 2).mean(axis=1) + np.float64(np.float32(1e-6)))
    plain = xv * rstd[:, None] * wv[None, :]
    assert np.allclose(z[:, : D - R], plain[:, : D - R], rtol=1e-14, atol=0)
    assert not np.allclose(z[:, D - R:], plain[:, D - R:], rtol=1e-6, atol=0)


@pytest.mark.parametrize("neox", [True, False])
def test_staged_form_brute_force(neox):
    # s3.3.4's dataflow: round to the dtype after the norm and after the rotation
    H, D, R = 2, 8, 8
    x, w, c, s = _inputs(21, 3, H, D, R, "bf16", "bf16", base=3.0)
    q, sc = oracle.rmsnorm_rope_fp8_rounded(x, w, c, s, H, D, R, "bf16", "bf16", neox, 1e-6)
    for t in range(3):
        u = exact.rmsnorm_ref(x[t], w, "bf16", 1e-6)
        z = exact.rope_ref(np.array(u, np.uint16), c[t], s[t], H, D, R, "bf16", "bf16", neox)
        codes, scales = exact.act_quant_ref(np.array(z, np.uint16), "bf16", H * D)
        assert [int(v) for v in q[t]] == codes, t
        assert float(sc[t]) == scales[0], t


def test_staged_form_differs_from_the_exact_one_on_a_few_codes():
    # the intermediate roundings (relative 2^-9 of each bfloat16 value) move a few
    # percent of the codes by one step; only near a RoPE cancellation, where that
    # absolute error spans several of the fine steps of small codes, by more
    import torch

    H, D, R = 32, 128, 128
    x, w, c, s = _inputs(22, 64, H, D, R, "bf16", "bf16")
    q1, s1 = oracle.rmsnorm_rope_fp8(x, w, c, s, H, D, R, "bf16", "bf16", True, 1e-6)
    q2, s2 = oracle.rmsnorm_rope_fp8_rounded(x, w, c, s, H, D, R, "bf16", "bf16", True, 1e-6)
    frac = float((q1 != q2).mean())
    assert 1e-3 < frac < 0.2, frac
    signed = lambda q: (q & 0x7F).astype(int) * np.where(q & 0x80, -1, 1)
    steps = np.abs(signed(q1) - signed(q2))
    value = lambda q: torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    far = steps > 1
    assert far.mean() < 0.01
    # codes in units of scale: several steps apart only below 4 (of 448)
    assert np.all(np.maximum(np.abs(value(q1)), np.abs(value(q2)))[far] < 4)
    assert np.all(np.abs(s1.astype(np.float64) / s2 - 1) < 2.0 ** -7)
