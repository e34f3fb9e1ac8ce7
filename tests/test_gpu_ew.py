"""GPU parity of the elementwise family (ew_add_fwd, ew_scale_cast_fwd,
ew_scale_add_fwd; "TileLang tutorial, ch. 13", s3.1.1 and s1.2's scale+add)
against the oracle's single rounding of the exact value, through the C ABI:
the benchmark workloads, every dtype pairing, lengths that are not multiples
of the vector width (the ragged tail), both launch shapes, in-place calls.
Both sides round the exact value once (the kernel: a binary32 fma for fp32
outputs; a binary64 fma rounded to odd, then one cast, for 16-bit outputs), so
outputs are compared bit for bit.  (With fp32 inputs and a 16-bit output, the
binary64 fma is itself inexact when the addend is far below the product; it
could then differ from the exact rounding only if the binary64 value fell
exactly on a 16-bit midpoint, a case random inputs do not produce.)"""
import numpy as np
import pytest
import torch

import oracle
import quant_row_workgroup_amd as qrw
from quant_row_workgroup_amd import synth
from tests.gpu_util import TORCH_DT, assert_close16, dev, host

pytestmark = pytest.mark.gpu


def _compare(got, want, fmt, what):
    if fmt == "f32":
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), what
        return
    assert_close16(got, want, fmt, max_ulp=0, what=what)


def _run(kind, x, b, alpha, xf, yf):
    xd = dev(x, xf)
    if kind == "add":
        return host(qrw.ew_add_fwd(xd, dev(b, xf)))
    if kind == "scale_add":
        return host(qrw.ew_scale_add_fwd(xd, dev(b, xf), alpha))
    return host(qrw.ew_scale_cast_fwd(xd, alpha, TORCH_DT[yf]))


@pytest.mark.parametrize("name", ["scale_add_1M_f32", "add_16M_bf16",
                                  "scale_cast_16M_f32_to_f16"])
def test_ew_workload(name):
    inp = synth.make_inputs(name)
    xf, yf = inp["dtype"], inp.get("y_dtype", inp["dtype"])
    alpha = 1.0 if inp["kind"] == "add" else inp["alpha"]
    got = _run(inp["kind"], inp["x"], inp.get("b"), alpha, xf, yf)
    want = oracle.ew_scale_add(inp["x"], inp.get("b"), alpha, xf, yf)
    _compare(got, want, yf, name)


LENGTHS = [1, 7, 8, 9, 255, 256, 1000, 4099, 65539, (1 << 22) + 5, (1 << 23) + 3]


@pytest.mark.parametrize("n", LENGTHS)
@pytest.mark.parametrize("fmt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("kind", ["add", "scale_add"])
def test_ew_same_dtype(kind, fmt, n):
    x = synth.normal(n % 977 + 3, (n,), 0.0, 2.0, fmt, outlier_frac=0.01, outlier_mul=50.0)
    b = synth.normal(n % 977 + 4, (n,), 0.0, 2.0, fmt)
    alpha = 1.0 if kind == "add" else float(np.float32(-0.3183098861837907))
    got = _run(kind, x, b, alpha, fmt, fmt)
    _compare(got, oracle.ew_scale_add(x, b, alpha, fmt, fmt), fmt, f"{kind} {fmt} n={n}")


@pytest.mark.parametrize("n", [5, 1000, 65539, (1 << 22) + 7])
@pytest.mark.parametrize("xf", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("yf", ["f16", "bf16", "f32"])
def test_ew_scale_cast(xf, yf, n):
    x = synth.normal(n % 991 + 5, (n,), 0.0, 20.0, xf, outlier_frac=0.01, outlier_mul=50.0)
    alpha = float(np.float32(0.5)) if n % 2 else float(np.float32(1.7320508075688772))
    got = _run("scale_cast", x, None, alpha, xf, yf)
    _compare(got, oracle.ew_scale_add(x, None, alpha, xf, yf), yf, f"cast {xf}->{yf} n={n}")


def test_ew_in_place_and_views():
    n = 3 * 4096 + 5
    x = synth.normal(31, (n,), 0.0, 1.0, "bf16")
    b = synth.normal(32, (n,), 0.0, 1.0, "bf16")
    xd, bd = dev(x, "bf16"), dev(b, "bf16")
    qrw.ew_scale_add_fwd(xd, bd, 2.0, out=xd)   # x <- 2x + b
    _compare(host(xd), oracle.ew_scale_add(x, b, 2.0, "bf16"), "bf16", "in place on x")
    xd = dev(x, "bf16")
    qrw.ew_add_fwd(xd, bd, out=bd)              # b <- x + b
    _compare(host(bd), oracle.ew_scale_add(x, b, 1.0, "bf16"), "bf16", "in place on b")
    # a 2-D contiguous tensor is a flat array of its elements
    m = synth.normal(33, (64, 1000), 0.0, 1.0, "f16")
    got = host(qrw.ew_scale_cast_fwd(dev(m, "f16"), 0.25, torch.float32))
    assert np.array_equal(got, synth.storage_to_f64(m, "f16").astype(np.float32) * np.float32(0.25))


def test_ew_empty():
    z = torch.empty(0, dtype=torch.float32, device="cuda")
    assert qrw.ew_add_fwd(z, z).numel() == 0
    assert qrw.ew_scale_cast_fwd(z, 2.0, torch.float16).numel() == 0
