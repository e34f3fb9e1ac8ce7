"""GPU parity of rmsnorm_fwd / layernorm_fwd against the fp64 oracle, through
the C ABI, on the same seeded inputs: the benchmark configurations in full,
plus ragged rows, the size limits, strides, in-place calls, degenerate rows,
determinism and batch invariance."""
import numpy as np
import pytest
import torch

import oracle
import quant_row_workgroup_amd as qrw
from quant_row_workgroup_amd import synth
from tests.gpu_util import assert_close16, dev, host, layernorm_terms

pytestmark = pytest.mark.gpu


def _rms_case(rows, n, dtype, seed, with_w=True, eps=1e-6):
    x = synth.normal(seed, (rows, n), 0.0, 1.0, dtype)
    w = synth.normal(seed + 1, (n,), 1.0, 0.1, dtype) if with_w else None
    got = host(qrw.rmsnorm_fwd(dev(x, dtype), None if w is None else dev(w, dtype), eps))
    want = oracle.rmsnorm(x, w, dtype, eps)
    return assert_close16(got, want, dtype, what=f"rmsnorm {rows}x{n} {dtype}")


@pytest.mark.parametrize("name", ["rmsnorm_256x1024_f16", "rmsnorm_4096x4096_f16"])
def test_rmsnorm_workloads(name):
    inp = synth.make_inputs(name)
    dt = inp["dtype"]
    got = host(qrw.rmsnorm_fwd(dev(inp["x"], dt), dev(inp["w"], dt), inp["eps"]))
    want = oracle.rmsnorm(inp["x"], inp["w"], dt, inp["eps"])
    st = assert_close16(got, want, dt, what=name)
    print(name, st)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("rows,n", [(1, 8), (3, 16), (5, 1000), (7, 520), (33, 4096),
                                    (9, 4104), (4, 8192), (2, 8184), (17, 64), (6, 1024),
                                    (130, 2048)])
def test_rmsnorm_shapes(dtype, rows, n):
    _rms_case(rows, n, dtype, seed=rows * 31 + n)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_rmsnorm_without_weight(dtype):
    _rms_case(64, 1000, dtype, seed=5, with_w=False)


def test_rmsnorm_strides_and_in_place():
    dt = "bf16"
    rows, n, xs, ys = 37, 1000, 1032, 1008
    xw = synth.normal(41, (rows, xs), 0.0, 1.0, dt)
    w = synth.normal(42, (n,), 1.0, 0.1, dt)
    xt = dev(xw, dt)
    out = torch.full((rows, ys), 3.0, dtype=torch.bfloat16, device="cuda")
    qrw.rmsnorm_fwd(xt[:, :n], dev(w, dt), 1e-6, out=out[:, :n])
    want = oracle.rmsnorm(xw, w, dt, 1e-6, n=n)
    got = host(out)
    assert_close16(got[:, :n], want, dt, what="strided")
    assert np.all(got[:, n:] == host(torch.full((1,), 3.0, dtype=torch.bfloat16))[0])
    # in place
    xi = dev(xw, dt)
    qrw.rmsnorm_fwd(xi[:, :n], dev(w, dt), 1e-6, out=xi[:, :n])
    gi = host(xi)
    assert np.array_equal(gi[:, :n], got[:, :n])
    assert np.array_equal(gi[:, n:], xw[:, n:])  # the pad of each row is untouched


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_rmsnorm_degenerate_rows(dtype):
    n = 4096
    w = synth.normal(7, (n,), 1.0, 0.1, dtype)
    x = synth.to_storage(np.stack([np.full(n, 2.5), np.full(n, -1.0), np.zeros(n)]), dtype)
    got = host(qrw.rmsnorm_fwd(dev(x, dtype), dev(w, dtype), 1e-6))
    assert np.array_equal(got[0], w)                       # constant row -> w, bit-exact
    assert np.array_equal(got[1], w ^ np.uint16(0x8000))   # negative constant -> -w
    assert np.all((got[2] & 0x7FFF) == 0)                  # zero row -> (signed) zeros
    assert np.array_equal(got, oracle.rmsnorm(x, w, dtype, 1e-6))


def test_rmsnorm_empty_and_deterministic_and_batch_invariant():
    dt = "f16"
    x = synth.normal(9, (300, 4096), 0.0, 1.0, dt)
    w = synth.normal(10, (4096,), 1.0, 0.1, dt)
    xt, wt = dev(x, dt), dev(w, dt)
    empty = qrw.rmsnorm_fwd(xt[:0], wt, 1e-6)
    assert empty.shape == (0, 4096)
    a = host(qrw.rmsnorm_fwd(xt, wt, 1e-6))
    b = host(qrw.rmsnorm_fwd(xt, wt, 1e-6))
    assert np.array_equal(a, b)
    for r in (0, 77, 299):
        one = host(qrw.rmsnorm_fwd(xt[r:r + 1], wt, 1e-6))
        assert np.array_equal(one[0], a[r])


# ------------------------------------------------------------------ LayerNorm
def test_layernorm_workload():
    name = "layernorm_4096x4096_bf16"
    inp = synth.make_inputs(name)
    dt = inp["dtype"]
    got = host(qrw.layernorm_fwd(dev(inp["x"], dt), dev(inp["gamma"], dt), dev(inp["beta"], dt),
                                 inp["eps"]))
    want = oracle.layernorm(inp["x"], inp["gamma"], inp["beta"], dt, inp["eps"])
    ts = layernorm_terms(inp["x"], inp["gamma"], inp["beta"], dt, inp["eps"])
    st = assert_close16(got, want, dt, term_scale=ts, what=name)
    print(name, st)
    assert st["within_2ulp_of_result"] >= 0.9999


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("rows,n,affine", [(1, 8, True), (5, 1000, True), (3, 8192, True),
                                           (11, 4096, False), (64, 1536, True), (2, 24, False)])
def test_layernorm_shapes(dtype, rows, n, affine):
    x = synth.normal(rows + n, (rows, n), 0.5, 2.0, dtype)
    g = synth.normal(rows + n + 1, (n,), 1.0, 0.1, dtype) if affine else None
    b = synth.normal(rows + n + 2, (n,), 0.0, 0.1, dtype) if affine else None
    got = host(qrw.layernorm_fwd(dev(x, dtype), None if g is None else dev(g, dtype),
                                 None if b is None else dev(b, dtype), 1e-5))
    assert_close16(got, oracle.layernorm(x, g, b, dtype, 1e-5), dtype,
                   term_scale=layernorm_terms(x, g, b, dtype, 1e-5), what=f"layernorm {rows}x{n}")


# bf16 rows of 512 * k elements (k = 1, 2, 4, 8) with gamma and beta take the
# one-wave kernel with Chan statistics; the same rows without them, or in
# f16, the two-part mean.  Both meet the bar, and a row is the same alone and
# in a batch.
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("rows,n", [(3, 512), (1000, 1024), (37, 2048), (513, 4096)])
def test_layernorm_whole_rows(dtype, rows, n):
    x = synth.normal(rows * 3 + n, (rows, n), 0.5, 2.0, dtype)
    g = synth.normal(n + 1, (n,), 1.0, 0.1, dtype)
    b = synth.normal(n + 2, (n,), 0.0, 0.1, dtype)
    xt, gt, bt = dev(x, dtype), dev(g, dtype), dev(b, dtype)
    got = host(qrw.layernorm_fwd(xt, gt, bt, 1e-5))
    st = assert_close16(got, oracle.layernorm(x, g, b, dtype, 1e-5), dtype,
                        term_scale=layernorm_terms(x, g, b, dtype, 1e-5),
                        what=f"layernorm {rows}x{n} {dtype}")
    assert st["within_2ulp_of_result"] >= 0.9999
    for r in (0, rows - 1):
        assert np.array_equal(host(qrw.layernorm_fwd(xt[r:r + 1], gt, bt, 1e-5))[0], got[r])


# Whole rows of 64 * {3, 5, 6, 7, 10, 12, 14} granules (hidden sizes 1536 ...
# 7168) have one-wave instances of their own; RMSNorm with the weight read at
# output time (4 or more workgroups per CU) keeps the rounded-up instance, so
# a row must come out the same alone (exact instance) and in a large batch.
EXACT_WIDTHS = [1536, 2560, 3072, 3584, 5120, 6144, 7168]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("n", EXACT_WIDTHS)
def test_norms_exact_width_rows(dtype, n):
    rows = 37
    st = _rms_case(rows, n, dtype, seed=n + 7)
    assert st["within_2ulp_of_result"] >= 0.9999
    _rms_case(rows, n, dtype, seed=n + 8, with_w=False)
    x = synth.normal(n + 9, (rows, n), 0.5, 2.0, dtype)
    g = synth.normal(n + 10, (n,), 1.0, 0.1, dtype)
    b = synth.normal(n + 11, (n,), 0.0, 0.1, dtype)
    xt, gt, bt = dev(x, dtype), dev(g, dtype), dev(b, dtype)
    got = host(qrw.layernorm_fwd(xt, gt, bt, 1e-5))
    st = assert_close16(got, oracle.layernorm(x, g, b, dtype, 1e-5), dtype,
                        term_scale=layernorm_terms(x, g, b, dtype, 1e-5),
                        what=f"layernorm {rows}x{n} {dtype}")
    assert st["within_2ulp_of_result"] >= 0.9999
    assert np.array_equal(host(qrw.layernorm_fwd(xt[5:6], gt, bt, 1e-5))[0], got[5])


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_rmsnorm_exact_width_batch_invariant(dtype):
    rows, n = 4100, 5120  # over 4 workgroups per CU: the late-weight form
    x = synth.normal(41, (rows, n), 0.0, 1.0, dtype)
    w = synth.normal(42, (n,), 1.0, 0.1, dtype)
    xt, wt = dev(x, dtype), dev(w, dtype)
    got = host(qrw.rmsnorm_fwd(xt, wt, 1e-6))
    st = assert_close16(got, oracle.rmsnorm(x, w, dtype, 1e-6), dtype,
                        what=f"rmsnorm {rows}x{n} {dtype}")
    assert st["within_2ulp_of_result"] >= 0.9999
    for r in (0, 2049, rows - 1):
        assert np.array_equal(host(qrw.rmsnorm_fwd(xt[r:r + 1], wt, 1e-6))[0], got[r])
    part = host(qrw.rmsnorm_fwd(xt[:300], wt, 1e-6))
    assert np.array_equal(part, got[:300])


def test_layernorm_constant_row_gives_beta_and_in_place():
    dt = "bf16"
    n = 4096
    g = synth.normal(3, (n,), 1.0, 0.1, dt)
    b = synth.normal(4, (n,), 0.0, 0.1, dt)
    x = synth.to_storage(np.stack([np.full(n, 0.75), np.full(n, -3.0)]), dt)
    got = host(qrw.layernorm_fwd(dev(x, dt), dev(g, dt), dev(b, dt), 1e-5))
    assert np.array_equal(got, np.stack([b, b]))
    xr = synth.normal(5, (19, n), 0.5, 2.0, dt)
    xt = dev(xr, dt)
    ref = host(qrw.layernorm_fwd(xt, dev(g, dt), dev(b, dt), 1e-5))
    qrw.layernorm_fwd(xt, dev(g, dt), dev(b, dt), 1e-5, out=xt)
    assert np.array_equal(host(xt), ref)
