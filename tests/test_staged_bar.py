"""CPU checks of the staged fused form's parity bar (tests/gpu_util.py,
assert_staged_consistent): it accepts every result a binary32 evaluation
within its stated error bounds can produce, and rejects a result that is off
anywhere the oracle's intermediates are not within those bounds of a 16-bit
rounding boundary.

The "binary32 evaluation" here is an emulation in numpy float32 of the staged
dataflow ("TileLang tutorial, ch. 13", s3.3.4: the normalised row is stored in
x's dtype and rotated there, then cast per token, s3.1.5): rstd from a float32
sum of squares (optionally perturbed within the bound), u = RN16(RN32(x*w*rstd)),
z = RN16(RN32(u_a*c - RN32(u_b*s))), scale = RN32(max|z|/448) and codes
E4M3(RN32(z/scale)).  Nothing here needs a GPU."""
import numpy as np
import pytest

import oracle
from quant_row_workgroup_amd import synth
from tests import gpu_util as gu

CASES = [(6, 4, 64, 32, "bf16", "bf16", True), (5, 2, 128, 128, "f16", "f32", False),
         (4, 8, 64, 64, "bf16", "f32", True), (3, 1, 512, 128, "f16", "f16", True)]


def _inputs(T, H, D, R, dt, cs, seed, weight=True):
    x = synth.normal(seed, (T, H * D), 0.0, 3.0, dt, outlier_frac=0.01, outlier_mul=10.0)
    w = synth.normal(seed + 1, (H * D,), 1.0, 0.1, dt) if weight else None
    c, s = synth.rope_table(T, R, cs, base=7.0)
    return x, w, c, s


def _emulate(x, w, c, s, H, D, R, dt, cs, neox, eps, rstd_rel=0.0):
    """The staged dataflow in binary32 (see the module docstring); rstd is
    multiplied by (1 + rstd_rel)."""
    T, n = x.shape
    xv = synth.storage_to_f64(x, dt).astype(np.float32)
    wv = np.ones(n, np.float32) if w is None else synth.storage_to_f64(w, dt).astype(np.float32)
    ss = (xv * xv).sum(axis=1, dtype=np.float32)
    rstd = (np.float32(1) / np.sqrt(ss / np.float32(n) + np.float32(eps))).astype(np.float64)
    rstd = (rstd * (1.0 + rstd_rel)).astype(np.float32)
    u32 = ((xv * wv[None, :]) * rstd[:, None]).astype(np.float32)
    u = synth.storage_to_f64(gu.rn16_bits(u32.astype(np.float64), dt), dt)
    cv = synth.storage_to_f64(c, cs)
    sv = synth.storage_to_f64(s, cs)
    rot, first, p, partner = gu._pair_layout(T, H, D, R, neox)
    rot_n, first_n, pp = np.tile(rot, H), np.tile(first, H), np.tile(p, H)
    part = (np.arange(H)[:, None] * D + partner[None, :]).reshape(-1)
    ua, ub = u, u[:, part]
    cc, sn = cv[:, pp], sv[:, pp]
    sgn = np.where(first_n, -1.0, 1.0)[None, :]
    prod = (ub.astype(np.float32) * (sgn * sn).astype(np.float32)).astype(np.float64)
    v32 = (ua * cc + prod).astype(np.float32)  # u_a*c exact in binary64, one rounding
    z = np.where(rot_n[None, :], synth.storage_to_f64(gu.rn16_bits(v32, dt), dt), u)
    amax = np.maximum(np.abs(z).max(axis=1), float(np.float32(1e-4)))
    scale = (amax / 448.0).astype(np.float32)
    qv = (z / scale.astype(np.float64)[:, None]).astype(np.float32)
    return gu._e4m3_of_f32(qv), scale


def test_rn16_bits_matches_the_oracle_encoders():
    rng = np.random.default_rng(3)
    v = rng.standard_normal(4000) * 10.0 ** rng.uniform(-5, 4, 4000)
    # and every midpoint between consecutive bf16 / f16 values in one binade
    mids16 = (np.arange(0x3C00, 0x3FFF).astype(np.uint16).view(np.float16).astype(np.float64)
              + 2.0 ** -11)
    midsb = (np.arange(0x3F80, 0x3FFF).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64) + 2.0 ** -8
    for dt, enc, extra in (("bf16", oracle.encode_bf16, midsb), ("f16", oracle.encode_f16, mids16)):
        vals = np.concatenate([v, extra, -extra])
        got = gu.rn16_bits(vals, dt)
        want = np.array([enc(float(t)) for t in vals], dtype=np.uint16)
        assert np.array_equal(got, want), dt


@pytest.mark.parametrize("case", CASES)
def test_the_oracle_itself_passes(case):
    T, H, D, R, dt, cs, neox = case
    x, w, c, s = _inputs(T, H, D, R, dt, cs, 61)
    q, sc = oracle.rmsnorm_rope_fp8_rounded(x, w, c, s, H, D, R, dt, cs, neox, 1e-6)
    st = gu.assert_staged_consistent(q, sc, x, w, c, s, H, D, R, dt, cs, neox, 1e-6)
    assert st["exact_frac"] == 1.0 and st["ambiguous_frac"] < 0.02


@pytest.mark.parametrize("rel", [0.0, 12 * 2.0 ** -24, -12 * 2.0 ** -24])
@pytest.mark.parametrize("case", CASES)
def test_binary32_evaluations_pass(case, rel):
    T, H, D, R, dt, cs, neox = case
    for weight in (True, False):
        x, w, c, s = _inputs(T, H, D, R, dt, cs, 71, weight)
        q, sc = _emulate(x, w, c, s, H, D, R, dt, cs, neox, 1e-6, rel)
        gu.assert_staged_consistent(q, sc, x, w, c, s, H, D, R, dt, cs, neox, 1e-6)


def test_planted_mistakes_fail():
    T, H, D, R, dt, cs, neox = CASES[0]
    x, w, c, s = _inputs(T, H, D, R, dt, cs, 81)
    q, sc = oracle.rmsnorm_rope_fp8_rounded(x, w, c, s, H, D, R, dt, cs, neox, 1e-6)
    _, _, iv = gu.staged_intervals(x, w, c, s, H, D, R, dt, cs, neox, 1e-6)
    z_lo, z_hi = iv["z"]
    # one code one step off where its stored value is unambiguous
    t, j = np.argwhere((z_lo == z_hi) & (np.abs(z_lo) > 0.1))[0]
    bad = q.copy()
    bad[t, j] = bad[t, j] + 1 if (bad[t, j] & 0x7F) < 0x7E else bad[t, j] - 1
    with pytest.raises(AssertionError):
        gu.assert_staged_consistent(bad, sc, x, w, c, s, H, D, R, dt, cs, neox, 1e-6)
    # one scale two binary32 ulps off
    sbad = sc.copy()
    sbad[2] = np.nextafter(np.nextafter(sbad[2], np.float32(1)), np.float32(1))
    with pytest.raises(AssertionError):
        gu.assert_staged_consistent(q, sbad, x, w, c, s, H, D, R, dt, cs, neox, 1e-6)
    # an rstd far outside the bound (2^-10 relative)
    q2, sc2 = _emulate(x, w, c, s, H, D, R, dt, cs, neox, 1e-6, 2.0 ** -10)
    with pytest.raises(AssertionError):
        gu.assert_staged_consistent(q2, sc2, x, w, c, s, H, D, R, dt, cs, neox, 1e-6)


def test_oracle_composition_is_the_staged_oracle():
    # the staged oracle is the three pinned operators composed
    T, H, D = 8, 4, 64
    x = synth.normal(9, (T, H * D), 0.0, 2.0, "f16")
    w = synth.normal(10, (H * D,), 1.0, 0.1, "f16")
    c, s = synth.rope_table(T, D, "f32")
    q, sc = oracle.rmsnorm_rope_fp8_rounded(x, w, c, s, H, D, D, "f16", "f32", False, 1e-6)
    u = oracle.rmsnorm(x, w, "f16", 1e-6)
    z = oracle.rope(u, c, s, H, D, D, "f16", "f32", False)
    q2, s2 = oracle.act_quant_fp8(z, "f16", None)
    assert np.array_equal(q, q2) and np.array_equal(sc, s2[:, 0])
