"""GPU parity of rmsnorm_rope_fp8_rounded_fwd (the staged form of the fused
operator, "TileLang tutorial, ch. 13", s3.3.4: the normalised row is rounded to
x's dtype and rotated there, then cast per token) against the oracle's
composition of RMSNorm, RoPE and the per-token cast, through the C ABI.

Bar.  A stored intermediate can land one 16-bit ulp away from the oracle's (the
binary32 product is rounded once more on its way to the 16-bit format).  So:
- a row's scale is within 1e-6 of the oracle's, or, where its largest stored
  value was such an intermediate, within one 16-bit ulp of it (2^-10 relative
  in f16, 2^-7 in bf16), in at most max(1, 1%) of the rows;
- codes more than one step apart must be small, below 4 in units of the
  scale (of 448): a moved intermediate near a RoPE cancellation can move a
  small code by several of its fine steps;
- in the rows whose scale matches, codes are bit-exact on all but at most
  max(1, 0.1%) of them (in a row whose scale moved, codes near an E4M3
  rounding boundary move by a step)."""
import numpy as np
import pytest
import torch

import oracle
import quant_row_workgroup_amd as qrw
from quant_row_workgroup_amd import synth
from tests.gpu_util import assert_codes, assert_scales, dev, host, ord8

pytestmark = pytest.mark.gpu


def _value(q):
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def assert_staged(q, sc, wq, wsc, dt, what):
    """The staged form's bar (see the module docstring) on codes [T, n] and
    scales [T]."""
    rel = np.abs(sc.astype(np.float64) - wsc.astype(np.float64)) / wsc.astype(np.float64)
    ulp = 2.0 ** (-10 if dt == "f16" else -7)
    assert np.all(rel <= ulp), f"{what}: scale rel err {rel.max():.3e}"
    moved = rel > 1e-6
    assert int(moved.sum()) <= max(1, moved.size // 100), f"{what}: {int(moved.sum())} scales moved"
    steps = np.abs(ord8(q) - ord8(wq))
    far = steps > 1
    assert np.all(np.maximum(np.abs(_value(q)), np.abs(_value(wq)))[far] < 4), what
    kept = steps[~moved]
    differ = int((kept != 0).sum())
    assert differ <= max(1, kept.size // 1000), f"{what}: {differ} codes differ"
    return {"max_step": int(steps.max()) if steps.size else 0,
            "exact_frac": float((steps == 0).mean()) if steps.size else 1.0,
            "scale_rel": float(rel.max()) if rel.size else 0.0, "scales_moved": int(moved.sum()),
            "far": int(far.sum())}


def _check(x, w, c, s, H, D, R, dt, cs, neox, what, eps=1e-6):
    q, sc = qrw.rmsnorm_rope_fp8_rounded_fwd(dev(x, dt), None if w is None else dev(w, dt),
                                             dev(c, cs), dev(s, cs), H, D, R, neox=neox, eps=eps)
    q, sc = host(q), host(sc)
    wq, wsc = oracle.rmsnorm_rope_fp8_rounded(x, w, c, s, H, D, R, dt, cs, neox, eps)
    return assert_staged(q, sc, wq, wsc, dt, what)


def test_rounded_workload_shape():
    # the benchmark's staged workload, at full size and in bench.py's launch form
    name = "rmsnorm_rope_fp8_4096x4096_bf16_staged"
    inp = synth.make_inputs(name)
    st = _check(inp["x"], inp["w"], inp["cos"], inp["sin"], inp["heads"], inp["head_dim"],
                inp["rope_dim"], inp["dtype"], inp["cs_dtype"], inp["neox"], name, inp["eps"])
    print(name, "staged", st)


@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("dt,cs", [("bf16", "bf16"), ("f16", "f32")])
@pytest.mark.parametrize("T,H,D,R", [(64, 32, 128, 128), (16, 8, 128, 64), (9, 3, 48, 32),
                                     (7, 1, 1000, 16), (1, 1, 16, 16), (12, 1, 8192, 512),
                                     (8, 1, 4096, 128), (5, 4, 256, 128)])
def test_rounded_shapes(neox, dt, cs, T, H, D, R):
    x = synth.normal(T + H + D + R, (T, H * D), 0.0, 3.0, dt, outlier_frac=0.01,
                     outlier_mul=10.0)
    w = synth.normal(T + H + D + R + 1, (H * D,), 1.0, 0.1, dt)
    c, s = synth.rope_table(T, R, cs, base=10000.0 if T < 10 else 5.0)
    _check(x, w, c, s, H, D, R, dt, cs, neox, f"staged {T}x{H}x{D}/{R}")


def test_rounded_equals_the_three_operators_in_sequence():
    # rmsnorm_fwd, rope_apply_neox, act_quant_fp8_fwd (one group per row) on the GPU
    T, H, D = 256, 32, 128
    x = synth.normal(3, (T, H * D), 0.0, 3.0, "bf16", outlier_frac=0.01, outlier_mul=10.0)
    w = synth.normal(4, (H * D,), 1.0, 0.1, "bf16")
    c, s = synth.rope_table(T, D, "bf16")
    xd, wd, cd, sd = dev(x, "bf16"), dev(w, "bf16"), dev(c, "bf16"), dev(s, "bf16")
    u = qrw.rmsnorm_fwd(xd, wd, 1e-6)
    z = qrw.rope_apply_neox(u, cd, sd, H, D, D)
    q3, s3 = qrw.act_quant_fp8_fwd(z)
    q1, s1 = qrw.rmsnorm_rope_fp8_rounded_fwd(xd, wd, cd, sd, H, D, D, neox=True, eps=1e-6)
    assert_scales(host(s1), host(s3)[:, 0], what="staged vs chain")
    assert_codes(host(q1), host(q3), max_step=64, what="staged vs chain")
