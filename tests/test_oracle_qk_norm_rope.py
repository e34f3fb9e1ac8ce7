"""Pins of the oracle's per-head QK RMSNorm + RoPE ("TileLang tutorial, ch.
13", s2.4: the cross-module fusion of a weighted RMSNorm and RoPE on the q/k
columns, v untouched)."""
import numpy as np
import pytest

import oracle
from quant_row_workgroup_amd import synth
from tests import exact


def _inputs(seed, T, Hq, Hk, D, R, fmt, cs, base=10000.0):
    n = (Hq + 2 * Hk) * D
    x = synth.normal(seed, (T, n), 0.0, 2.0, fmt)
    qw = synth.normal(seed + 1, (D,), 1.0, 0.2, fmt)
    kw = synth.normal(seed + 2, (D,), 1.0, 0.2, fmt)
    c, s = synth.rope_table(T, R, cs, base=base)
    return x, qw, kw, c, s


@pytest.mark.parametrize("fmt,cs", [("bf16", "bf16"), ("f16", "f32")])
@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("shape", [(2, 1, 8, 8), (1, 1, 16, 8), (3, 2, 16, 16)])
def test_brute_force_small(fmt, cs, neox, shape):
    Hq, Hk, D, R = shape
    x, qw, kw, c, s = _inputs(41, 3, Hq, Hk, D, R, fmt, cs, base=3.0)
    y = oracle.qk_norm_rope(x, qw, kw, c, s, Hq, Hk, D, R, fmt, cs, neox, 1e-6)
    for t in range(3):
        want = exact.qk_norm_rope_ref(x[t], qw, kw, c[t], s[t], Hq, Hk, D, R, fmt, cs, neox, 1e-6)
        assert [int(v) for v in y[t]] == want, t


def test_value_heads_are_untouched_and_heads_independent():
    Hq, Hk, D, R = 4, 2, 64, 64
    x, qw, kw, c, s = _inputs(42, 5, Hq, Hk, D, R, "bf16", "bf16")
    y = oracle.qk_norm_rope(x, qw, kw, c, s, Hq, Hk, D, R, "bf16", "bf16", True, 1e-6)
    assert np.array_equal(y[:, (Hq + Hk) * D:], x[:, (Hq + Hk) * D:])
    # each q head equals the fused single-head op written back in the activation dtype:
    # rmsnorm per head then rope == oracle.rmsnorm over that head then oracle.rope without
    # intermediate rounding, checked on a head whose rotation is the identity (t = 0)
    y0 = oracle.rmsnorm(np.ascontiguousarray(x[:1, :D]), qw, "bf16", 1e-6)
    assert np.array_equal(y[:1, :D], y0)


def test_identity_rotation_is_per_head_rmsnorm():
    Hq, Hk, D, R = 2, 1, 32, 32
    x, qw, kw, _, _ = _inputs(43, 4, Hq, Hk, D, R, "f16", "f16")
    c = synth.to_storage(np.ones((4, R // 2)), "f16")
    s = synth.to_storage(np.zeros((4, R // 2)), "f16")
    y = oracle.qk_norm_rope(x, qw, kw, c, s, Hq, Hk, D, R, "f16", "f16", True, 1e-6)
    for h in range(Hq + Hk):
        w = qw if h < Hq else kw
        want = oracle.rmsnorm(np.ascontiguousarray(x[:, h * D:(h + 1) * D]), w, "f16", 1e-6)
        assert np.array_equal(y[:, h * D:(h + 1) * D], want)


def test_quarter_turn_and_partial_span():
    # c = 0, s = 1 on a partial span: the prefix is the plain per-head RMSNorm, the
    # span is the quarter-turn of the normalised values
    Hq, Hk, D, R = 1, 1, 32, 16
    x, qw, kw, _, _ = _inputs(44, 2, Hq, Hk, D, R, "bf16", "bf16")
    c = synth.to_storage(np.zeros((2, R // 2)), "bf16")
    s = synth.to_storage(np.ones((2, R // 2)), "bf16")
    y = oracle.qk_norm_rope(x, qw, kw, c, s, Hq, Hk, D, R, "bf16", "bf16", True, 1e-6)
    for h, w in ((0, qw), (1, kw)):
        plain = oracle.rmsnorm(np.ascontiguousarray(x[:, h * D:(h + 1) * D]), w, "bf16", 1e-6)
        seg = y[:, h * D:(h + 1) * D]
        assert np.array_equal(seg[:, :D - R], plain[:, :D - R])
        lo, hi = plain[:, D - R:D - R // 2], plain[:, D - R // 2:]
        assert np.array_equal(seg[:, D - R:D - R // 2], hi ^ np.uint16(0x8000))
        assert np.array_equal(seg[:, D - R // 2:], lo)
