"""GPU parity of act_quant_fp8_fwd (per-token and per-group E4M3 activation
quantisation) against the fp64 oracle through the C ABI: the benchmark
workloads in full, every group size, ragged rows, strides, zero groups,
determinism and batch invariance.  Bar: scales within 1e-6 relative; codes
bit-exact on >= 99.9% and never more than one E4M3 step apart."""
import numpy as np
import pytest
import torch

import oracle
import quant_row_workgroup_amd as qrw
from quant_row_workgroup_amd import synth
from tests.gpu_util import assert_codes, assert_scales, dev, host

pytestmark = pytest.mark.gpu


def _check(x, dt, group, what):
    q, sc = qrw.act_quant_fp8_fwd(dev(x, dt), group)
    q, sc = host(q), host(sc)
    wq, wsc = oracle.act_quant_fp8(x, dt, group)
    rel = assert_scales(sc, wsc, what=what)
    st = assert_codes(q, wq, what=what)
    return q, sc, dict(st, scale_rel=rel)


@pytest.mark.parametrize("name", ["act_quant_4096x4096_bf16_g128", "act_quant_4096x4096_bf16_token"])
def test_act_quant_workloads(name):
    inp = synth.make_inputs(name)
    _, _, st = _check(inp["x"], inp["dtype"], inp["group"], name)
    print(name, st)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("rows,n,group", [
    (5, 4096, 128), (3, 4096, 8), (3, 4096, 16), (3, 4096, 32), (3, 4096, 64), (3, 4096, 256),
    (3, 4096, 512), (7, 1024, None), (2, 8192, 128), (2, 8192, None), (9, 640, 128),
    (4, 1000, None), (6, 1000, 8), (1, 8, None), (1, 8, 8), (33, 512, 512), (65, 2048, 64),
])
def test_act_quant_shapes(dt, rows, n, group):
    x = synth.normal(rows * 7 + n + (group or 0), (rows, n), 0.0, 2.0, dt, outlier_frac=0.02,
                     outlier_mul=20.0)
    _check(x, dt, group, f"act_quant {rows}x{n}/{group}")


# Whole rows of 64 * e granules, e not a power of two: per token, one-wave
# instances of their own; per group, waves on 128-, 256- or 512-granule
# segments when the row splits into them (else the one-wave kernel).
@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("n", [1536, 2560, 3072, 3584, 5120, 6144, 7168])
@pytest.mark.parametrize("group", [None, 128, 32])
def test_act_quant_exact_widths(dt, n, group):
    rows = 37
    x = synth.normal(rows * 13 + n + (group or 0), (rows, n), 0.0, 2.0, dt, outlier_frac=0.02,
                     outlier_mul=20.0)
    q, sc, _ = _check(x, dt, group, f"act_quant {rows}x{n}/{group}")
    q1, s1 = qrw.act_quant_fp8_fwd(dev(x[7:8], dt), group)
    assert np.array_equal(host(q1)[0], q[7]) and np.array_equal(host(s1)[0], sc[7])


# Rows longer than one wave holds (8192 channels, up to 65536): per group,
# waves on whole 4096- or 2048-channel segments, or 4096-channel segments with
# a shorter last one; per token, one workgroup of 16 waves per row.
@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("rows,n,group", [
    (3, 8200, None), (3, 8200, 8), (5, 14336, 128), (5, 14336, None), (4, 18432, 128),
    (4, 18432, None), (3, 16384, 128), (3, 16384, None), (2, 65536, 512), (2, 65536, None),
    (3, 12296, 8), (7, 20480, 64), (2, 10240, 32),
])
def test_act_quant_long_rows(dt, rows, n, group):
    x = synth.normal(rows * 11 + n + (group or 0), (rows, n), 0.0, 2.0, dt, outlier_frac=0.02,
                     outlier_mul=20.0)
    q, sc, _ = _check(x, dt, group, f"act_quant {rows}x{n}/{group}")
    q1, s1 = qrw.act_quant_fp8_fwd(dev(x[rows - 1:], dt), group)
    assert np.array_equal(host(q1)[0], q[rows - 1])
    assert np.array_equal(host(s1)[0], sc[rows - 1])


@pytest.mark.parametrize("group", [128, None])
def test_act_quant_long_rows_strided(group):
    n, rows = 14336, 6
    x = synth.normal(77 + (group or 0), (rows, n), 0.0, 3.0, "bf16")
    x[2, 1024:1152] = 0
    xw = np.zeros((rows, n + 64), dtype=np.uint16)
    xw[:, :n] = x
    qbuf = torch.full((rows, n + 16), 0x5A, dtype=torch.uint8, device="cuda")
    q, sc = qrw.act_quant_fp8_fwd(dev(xw, "bf16")[:, :n], group, q=qbuf[:, :n])
    qa = host(qbuf)
    assert np.all(qa[:, n:] == 0x5A)
    wq, wsc = oracle.act_quant_fp8(x, "bf16", group)
    assert_codes(qa[:, :n], wq)
    assert_scales(host(sc), wsc)


def test_act_quant_zero_groups_strides_determinism_batch_invariance():
    n = 4096
    x = synth.normal(40, (64, n), 0.0, 3.0, "bf16")
    x[3, 256:384] = 0
    x[9] = 0
    xw = np.zeros((64, n + 32), dtype=np.uint16)
    xw[:, :n] = x
    xt = dev(xw, "bf16")[:, :n]
    qbuf = torch.full((64, n + 8), 0x5A, dtype=torch.uint8, device="cuda")
    q, sc = qrw.act_quant_fp8_fwd(xt, 128, q=qbuf[:, :n])
    qa, sa = host(qbuf), host(sc)
    assert np.all(qa[:, n:] == 0x5A)
    wq, wsc = oracle.act_quant_fp8(x, "bf16", 128)
    assert_codes(qa[:, :n], wq)
    assert_scales(sa, wsc)
    floor = np.float32(1e-4) / np.float32(448)
    assert sa[3, 2] == floor and np.all(sa[9] == floor)
    assert np.all(qa[3, 256:384] == 0) and np.all(qa[9, :n] == 0)
    q2, s2 = qrw.act_quant_fp8_fwd(xt, 128)
    assert np.array_equal(host(q2), qa[:, :n]) and np.array_equal(host(s2), sa)
    for r in (0, 31, 63):
        q1, s1 = qrw.act_quant_fp8_fwd(xt[r:r + 1], 128)
        assert np.array_equal(host(q1)[0], qa[r, :n]) and np.array_equal(host(s1)[0], sa[r])
    qe, se = qrw.act_quant_fp8_fwd(xt[:0], 128)
    assert qe.shape == (0, n)


def test_act_quant_scales_are_exact():
    # amax is exact in binary32, so the scale max(amax, 1e-4)/448 is the oracle's bit for bit
    inp = synth.make_inputs("act_quant_4096x4096_bf16_g128", rows=256)
    q, sc = qrw.act_quant_fp8_fwd(dev(inp["x"], "bf16"), 128)
    _, wsc = oracle.act_quant_fp8(inp["x"], "bf16", 128)
    assert np.array_equal(host(sc), wsc)
