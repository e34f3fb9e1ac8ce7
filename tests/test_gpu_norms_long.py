"""GPU parity of rmsnorm_fwd / layernorm_fwd on ragged and long rows against the
fp64 oracle, through the C ABI ("TileLang tutorial, ch. 13", s5.4: a row whose
length is not a multiple of the vector width; s3.2.3 and s3.2.4: rows longer
than one wave's registers, including the pipelined kernels whose workgroups
walk several rows, and the two-pass split-K RMSNorm with its
reversed second pass).  Rows are stored padded (stride a multiple of 8); the padding
columns of y must come back untouched."""
import numpy as np
import pytest
import torch

import oracle
import quant_row_workgroup_amd as qrw
from quant_row_workgroup_amd import synth
from tests.gpu_util import TORCH_DT, assert_close16, dev, host, layernorm_terms

pytestmark = pytest.mark.gpu

FILL = 0x3C01  # a sentinel in both 16-bit formats


def _padded(bits, dt, stride):
    rows, n = bits.shape
    wide = torch.full((rows, stride), 0, dtype=torch.int16, device="cuda").view(TORCH_DT[dt])
    wide.view(torch.int16).fill_(FILL)
    wide[:, :n] = dev(bits, dt)
    return wide


def _stride(n, extra=8):
    return (n + 7) // 8 * 8 + extra


def _rms(rows, n, dt, seed, with_w=True, in_place=False):
    x = synth.normal(seed, (rows, n), 0.0, 1.0, dt, outlier_frac=0.01, outlier_mul=10.0)
    w = synth.normal(seed + 1, (n,), 1.0, 0.1, dt) if with_w else None
    xs = _stride(n)
    xw = _padded(x, dt, xs)
    yw = xw if in_place else _padded(np.zeros((rows, n), np.uint16), dt, _stride(n, 16))
    qrw.rmsnorm_fwd(xw[:, :n], None if w is None else dev(w, dt), 1e-6, out=yw[:, :n])
    got = host(yw)
    want = oracle.rmsnorm(x, w, dt, 1e-6)
    st = assert_close16(got[:, :n], want, dt, what=f"rmsnorm {rows}x{n} {dt}")
    assert np.all(got[:, n:] == FILL), "padding columns were written"
    return st


def _ln(rows, n, dt, seed, affine=True, in_place=False):
    x = synth.normal(seed, (rows, n), 0.5, 2.0, dt)
    g = synth.normal(seed + 1, (n,), 1.0, 0.1, dt) if affine else None
    b = synth.normal(seed + 2, (n,), 0.0, 0.1, dt) if affine else None
    xw = _padded(x, dt, _stride(n))
    yw = xw if in_place else _padded(np.zeros((rows, n), np.uint16), dt, _stride(n, 24))
    qrw.layernorm_fwd(xw[:, :n], None if g is None else dev(g, dt),
                      None if b is None else dev(b, dt), 1e-5, out=yw[:, :n])
    got = host(yw)
    want = oracle.layernorm(x, g, b, dt, 1e-5)
    st = assert_close16(got[:, :n], want, dt, term_scale=layernorm_terms(x, g, b, dt, 1e-5),
                        what=f"layernorm {rows}x{n} {dt}")
    assert np.all(got[:, n:] == FILL), "padding columns were written"
    return st


RAGGED = [1, 3, 7, 10, 13, 14, 100, 513, 1001, 2050, 4095, 4099, 4102, 8191]  # n % 8: every value 1-7


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("n", RAGGED)
def test_ragged_rmsnorm(dt, n):
    _rms(5, n, dt, seed=n + 1)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("n", RAGGED)
def test_ragged_layernorm(dt, n):
    _ln(5, n, dt, seed=n + 2)


def test_ragged_without_weights_and_in_place():
    _rms(9, 1001, "bf16", seed=3, with_w=False)
    _rms(9, 1001, "f16", seed=4, in_place=True)
    _ln(9, 4099, "bf16", seed=5, affine=False)
    _ln(9, 13, "f16", seed=6, in_place=True)


# one workgroup of several waves per row (8192 < n <= 65536)
ROWBLOCK = [8200, 12288, 12289, 12294, 16386, 16391, 32768, 40000, 65533, 65536]
# the two-pass kernel (n > 65536, RMSNorm only)
SPLITK = [65537, 131072, 262147, 1 << 20]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("n", ROWBLOCK + SPLITK)
def test_long_rmsnorm(dt, n):
    _rms(3, n, dt, seed=n % 1009)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("n", ROWBLOCK)
def test_long_layernorm(dt, n):
    _ln(3, n, dt, seed=n % 1013)


def test_long_rows_in_place_and_without_weights():
    _rms(4, 40000, "bf16", seed=7, in_place=True)
    _rms(2, 262147, "f16", seed=8, in_place=True, with_w=False)
    _ln(4, 16391, "f16", seed=9, in_place=True, affine=False)


# RMSNorm rows of exactly 8 granules per thread of 4, 8 or 16 waves (16384,
# 32768, 65536 elements) take the pipelined kernel when there are 1.5 to 4 rows
# per resident workgroup; its workgroups then walk several rows.  Fewer or
# more rows go to the row-block kernel.  On MI355X 1024, 512 and 256
# workgroups are resident for the three lengths: the cases walk 2-4 rows per
# workgroup, with and without weights, in place, and fall back on both sides.
@pytest.mark.parametrize("rows,n,dt,with_w,in_place", [
    (3000, 16384, "bf16", True, False), (1500, 32768, "f16", True, False),
    (1500, 32768, "bf16", False, True), (700, 65536, "bf16", True, False),
    (1000, 65536, "f16", False, False), (1100, 65536, "bf16", True, False),
    (2100, 32768, "f16", True, True), (1, 32768, "bf16", True, False),
    (768, 32768, "bf16", True, False), (700, 32768, "f16", False, True)])
def test_pipelined_rmsnorm_rows(rows, n, dt, with_w, in_place):
    st = _rms(rows, n, dt, seed=rows + n, with_w=with_w, in_place=in_place)
    assert st["within_2ulp_of_result"] >= 0.9999


# LayerNorm with gamma and beta takes the pipelined kernel on the same rows
# and row counts; without them, or outside the window, the row-block kernel.
@pytest.mark.parametrize("rows,n,dt,affine,in_place", [
    (3000, 16384, "bf16", True, False), (1500, 32768, "f16", True, True),
    (1024, 32768, "bf16", True, False), (700, 65536, "bf16", True, False),
    (768, 32768, "bf16", True, False), (1100, 65536, "f16", True, False),
    (2100, 32768, "bf16", True, True), (700, 32768, "f16", False, False)])
def test_pipelined_layernorm_rows(rows, n, dt, affine, in_place):
    st = _ln(rows, n, dt, seed=rows + n + 1, affine=affine, in_place=in_place)
    assert st["within_2ulp_of_result"] >= 0.9999


# Which kernel normalises a row depends on how many rows share the call, so
# the pipelined kernels must reproduce the row-block kernel's sums bit for
# bit ("The TileLang kernel DSL in DeepSeek-V4", batch invariance): every row
# of a batch that takes the pipelined kernel equals the same row normalised
# in batches of 128, which the row-block kernel takes.
@pytest.mark.parametrize("op", ["rmsnorm", "rmsnorm_now", "layernorm"])
@pytest.mark.parametrize("rows,n,dt", [(1536, 16384, "bf16"), (1024, 32768, "bf16"),
                                       (1024, 32768, "f16"), (512, 65536, "bf16")])
def test_pipelined_rows_are_batch_invariant(op, rows, n, dt):
    x = dev(synth.normal(rows + n, (rows, n), 0.5, 2.0, dt, outlier_frac=0.01,
                         outlier_mul=10.0), dt)
    g = dev(synth.normal(5, (n,), 1.0, 0.1, dt), dt)
    b = dev(synth.normal(6, (n,), 0.0, 0.1, dt), dt)
    if op == "layernorm":
        f = lambda t: qrw.layernorm_fwd(t, g, b, 1e-5)
    else:
        f = lambda t: qrw.rmsnorm_fwd(t, g if op == "rmsnorm" else None, 1e-6)
    whole = host(f(x))
    chunked = np.concatenate([host(f(x[r:r + 128])) for r in range(0, rows, 128)])
    diff = np.flatnonzero((whole != chunked).any(axis=1))
    assert diff.size == 0, f"{diff.size} rows differ, first {diff[:5]}"


# The whole-granule LayerNorm rows (16384, 32768, 65536 elements) take Chan's
# pairwise statistics in both kernels: a constant row must still give beta
# bit for bit (its per-thread means are exact and every merge adds zero), and
# rows far from zero mean must stay within the bar.  Small batches take the
# row-block kernel, 1.5-4 rows per resident workgroup the pipelined one.
@pytest.mark.parametrize("rows,n", [(3, 16384), (1536, 16384), (3, 32768), (1024, 32768),
                                    (2, 65536), (512, 65536)])
def test_whole_layernorm_rows_constant_and_offset(rows, n):
    dt = "bf16"
    g = synth.normal(3, (n,), 1.0, 0.1, dt)
    b = synth.normal(4, (n,), 0.0, 0.1, dt)
    # rows far from zero mean (x ~ N(300, 4), 2 ulps of bf16 there), the first
    # and last constant
    x = synth.normal(rows + 5, (rows, n), 300.0, 4.0, dt)
    const = [0, rows - 1]
    x[0] = synth.to_storage(np.full(n, 0.75), dt)
    x[rows - 1] = synth.to_storage(np.full(n, -3.0), dt)
    mid = slice(1, rows - 1)
    got = host(qrw.layernorm_fwd(dev(x, dt), dev(g, dt), dev(b, dt), 1e-5))
    for r in const:
        assert np.array_equal(got[r], b), f"constant row {r}"
    if rows > 2:
        xm = x[mid]
        st = assert_close16(got[mid], oracle.layernorm(xm, g, b, dt, 1e-5), dt,
                            term_scale=layernorm_terms(xm, g, b, dt, 1e-5),
                            what=f"offset layernorm {rows}x{n}")
        assert st["within_2ulp_of_result"] >= 0.9999


@pytest.mark.parametrize("n,dt,with_w", [(1 << 26, "bf16", True), ((1 << 26) - 3, "f16", False)])
def test_longest_rmsnorm_rows(n, dt, with_w):
    # the longest row the split-K kernel accepts (QRW_MAX_ROW_SPLIT = 2^26
    # elements, 128 MiB of bf16), whole and ragged
    _rms(1, n, dt, seed=13, with_w=with_w)


@pytest.mark.parametrize("n", [16391, 32768, 262147])
def test_long_rows_are_batch_invariant(n):
    # a row's output does not depend on which other rows share the launch
    x = synth.normal(11, (6, n), 0.0, 1.0, "bf16")
    w = dev(synth.normal(12, (n,), 1.0, 0.1, "bf16"), "bf16")
    xs = _padded(x, "bf16", _stride(n))[:, :n]
    all_rows = host(qrw.rmsnorm_fwd(xs, w, 1e-6))
    for r in (0, 5):
        one = host(qrw.rmsnorm_fwd(xs[r:r + 1], w, 1e-6))
        assert np.array_equal(one[0], all_rows[r])


@pytest.mark.parametrize("name", ["rmsnorm_1024x32768_bf16", "rmsnorm_256x131072_bf16_splitk",
                                  "rmsnorm_4096x4095_bf16_ragged", "layernorm_1024x32768_bf16"])
def test_long_and_ragged_workloads(name):
    inp = synth.make_inputs(name)
    dt, n = inp["dtype"], inp["n"]
    xw = _padded(inp["x"], dt, (n + 7) // 8 * 8)[:, :n]
    if inp["op"] == "rmsnorm":
        got = host(qrw.rmsnorm_fwd(xw, dev(inp["w"], dt), inp["eps"]))
        want = oracle.rmsnorm(inp["x"], inp["w"], dt, inp["eps"])
        ts = None
    else:
        got = host(qrw.layernorm_fwd(xw, dev(inp["gamma"], dt), dev(inp["beta"], dt), inp["eps"]))
        want = oracle.layernorm(inp["x"], inp["gamma"], inp["beta"], dt, inp["eps"])
        ts = layernorm_terms(inp["x"], inp["gamma"], inp["beta"], dt, inp["eps"])
    st = assert_close16(got, want, dt, term_scale=ts, what=name)
    print(name, st)
    assert st["within_2ulp_of_result"] >= 0.9999
