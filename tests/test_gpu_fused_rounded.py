"""GPU parity of rmsnorm_rope_fp8_rounded_fwd (the staged form of the fused
operator, "TileLang tutorial, ch. 13", s3.3.4: the normalised row is rounded to
x's dtype and rotated there, then cast per token) against the oracle's
composition of RMSNorm, RoPE and the per-token cast, through the C ABI.

Bar (tests/gpu_util.py, assert_staged_consistent).  The kernel evaluates in
binary32: its rstd is within a stated bound of the exact one, and each stored
16-bit intermediate is rounded from a binary32 value.  So a stored value may
be either 16-bit neighbour only where the oracle's unrounded value lies within
that bound of a rounding boundary; there the scale and codes must follow from
one of the possible stored values, with the kernel's own scale.  Everywhere
else codes and scales are bit-exact with the oracle's."""
import numpy as np
import pytest

import quant_row_workgroup_amd as qrw
from quant_row_workgroup_amd import synth
from tests.gpu_util import assert_staged_consistent, dev, host, ord8, staged_intervals

pytestmark = pytest.mark.gpu


def _check(x, w, c, s, H, D, R, dt, cs, neox, what, eps=1e-6):
    q, sc = qrw.rmsnorm_rope_fp8_rounded_fwd(dev(x, dt), None if w is None else dev(w, dt),
                                             dev(c, cs), dev(s, cs), H, D, R, neox=neox, eps=eps)
    return assert_staged_consistent(host(q), host(sc), x, w, c, s, H, D, R, dt, cs, neox, eps,
                                    what=what)


def test_rounded_workload_shape():
    # the benchmark's staged workload, at full size and in bench.py's launch form
    name = "rmsnorm_rope_fp8_4096x4096_bf16_staged"
    inp = synth.make_inputs(name)
    st = _check(inp["x"], inp["w"], inp["cos"], inp["sin"], inp["heads"], inp["head_dim"],
                inp["rope_dim"], inp["dtype"], inp["cs_dtype"], inp["neox"], name, inp["eps"])
    print(name, "staged", st)
    assert st["exact_frac"] >= 0.999


@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("dt,cs", [("bf16", "bf16"), ("f16", "f32")])
@pytest.mark.parametrize("T,H,D,R", [(64, 32, 128, 128), (16, 8, 128, 64), (9, 3, 48, 32),
                                     (7, 1, 1000, 16), (1, 1, 16, 16), (12, 1, 8192, 512),
                                     (8, 1, 4096, 128), (5, 4, 256, 128), (10, 20, 128, 128),
                                     (9, 48, 64, 64), (13, 40, 128, 128), (7, 64, 128, 128),
                                     (5, 24, 128, 64), (7, 40, 128, 64)])
def test_rounded_shapes(neox, dt, cs, T, H, D, R):
    x = synth.normal(T + H + D + R, (T, H * D), 0.0, 3.0, dt, outlier_frac=0.01,
                     outlier_mul=10.0)
    w = synth.normal(T + H + D + R + 1, (H * D,), 1.0, 0.1, dt)
    c, s = synth.rope_table(T, R, cs, base=10000.0 if T < 10 else 5.0)
    _check(x, w, c, s, H, D, R, dt, cs, neox, f"staged {T}x{H}x{D}/{R}")
    _check(x, None, c, s, H, D, R, dt, cs, neox, f"staged {T}x{H}x{D}/{R} no weight")


def test_rounded_equals_the_three_operators_in_sequence():
    # rmsnorm_fwd, rope_apply_neox and act_quant_fp8_fwd (one group per row) on
    # the GPU compute the same composition: both results meet the bar, and in
    # rows whose scales agree their codes are bit-identical wherever the stored
    # value is unambiguous
    T, H, D = 256, 32, 128
    x = synth.normal(3, (T, H * D), 0.0, 3.0, "bf16", outlier_frac=0.01, outlier_mul=10.0)
    w = synth.normal(4, (H * D,), 1.0, 0.1, "bf16")
    c, s = synth.rope_table(T, D, "bf16")
    xd, wd, cd, sd = dev(x, "bf16"), dev(w, "bf16"), dev(c, "bf16"), dev(s, "bf16")
    u = qrw.rmsnorm_fwd(xd, wd, 1e-6)
    z = qrw.rope_apply_neox(u, cd, sd, H, D, D)
    q3, s3 = qrw.act_quant_fp8_fwd(z)
    q1, s1 = qrw.rmsnorm_rope_fp8_rounded_fwd(xd, wd, cd, sd, H, D, D, neox=True, eps=1e-6)
    q1, s1, q3, s3 = host(q1), host(s1), host(q3), host(s3)[:, 0]
    for q, sc, what in ((q1, s1, "staged"), (q3, s3, "chain")):
        assert_staged_consistent(q, sc, x, w, c, s, H, D, D, "bf16", "bf16", True, 1e-6,
                                 what=what)
    # rows with equal scales: codes equal wherever the stored value is unambiguous
    _, _, iv = staged_intervals(x, w, c, s, H, D, D, "bf16", "bf16", True, 1e-6)
    same = s1 == s3
    assert same.mean() > 0.9
    clear = (iv["z"][0] == iv["z"][1]) & same[:, None]
    assert np.array_equal(ord8(q1)[clear], ord8(q3)[clear])
