"""A NaN or an infinity in the input leaves its outputs unspecified, but
nothing else: rows (tokens) are independent in the norms, the fused operator
and the activation quant; groups in the per-group quant; heads in the QK
norm; rotation pairs in RoPE; elements in the elementwise family.  Each test
plants non-finite values in a few places and checks every other output
against the oracle on the same input, at the usual bars; the long-row
(workgroup per row), pipelined (1024 rows of 32768: a workgroup walks two
rows) and split-K paths are included, where the rows of a batch share no
reduction."""
import numpy as np
import pytest

import oracle
import quant_row_workgroup_amd as qrw
from quant_row_workgroup_amd import synth
from tests import test_gpu_ew, test_gpu_fused, test_gpu_qk_norm_rope
from tests.gpu_util import assert_close16, dev, host, layernorm_terms, rope_terms

pytestmark = pytest.mark.gpu

NAN = {"f16": 0x7E00, "bf16": 0x7FC0}
INF = {"f16": 0x7C00, "bf16": 0x7F80}
NINF = {"f16": 0xFC00, "bf16": 0xFF80}


def _plant(x, dt, spots):
    """x with NaN, +inf and -inf at the given (row, column) places, in turn."""
    x = x.copy()
    for k, (r, c) in enumerate(spots):
        x[r, c] = (NAN, INF, NINF)[k % 3][dt]
    return x


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("rows,n", [(8, 4096), (7, 1000), (6, 16384), (5, 40000), (3, 100000),
                                    (1024, 32768)])
def test_rmsnorm_rows_stay_independent(dt, rows, n):
    x = _plant(synth.normal(rows + n, (rows, n), 0.0, 1.0, dt), dt,
               [(1, 7), (rows - 1, n - 1), (rows - 1, 0)])
    w = synth.normal(2, (n,), 1.0, 0.1, dt)
    got = host(qrw.rmsnorm_fwd(dev(x, dt), dev(w, dt), 1e-6))
    keep = [r for r in range(rows) if r not in (1, rows - 1)]
    assert_close16(got[keep], oracle.rmsnorm(x[keep], w, dt, 1e-6), dt,
                   what=f"rmsnorm {rows}x{n}")


@pytest.mark.parametrize("rows,n", [(8, 4096), (6, 16384), (4, 65536), (1024, 32768)])
def test_layernorm_rows_stay_independent(rows, n):
    dt = "bf16"
    x = _plant(synth.normal(rows + n, (rows, n), 0.5, 2.0, dt), dt, [(0, 3), (rows - 2, n // 2)])
    g = synth.normal(2, (n,), 1.0, 0.1, dt)
    b = synth.normal(3, (n,), 0.0, 0.1, dt)
    got = host(qrw.layernorm_fwd(dev(x, dt), dev(g, dt), dev(b, dt), 1e-5))
    keep = [r for r in range(rows) if r not in (0, rows - 2)]
    xk = x[keep]
    assert_close16(got[keep], oracle.layernorm(xk, g, b, dt, 1e-5), dt,
                   term_scale=layernorm_terms(xk, g, b, dt, 1e-5), what=f"layernorm {rows}x{n}")


@pytest.mark.parametrize("neox", [True, False])
def test_rope_pairs_stay_independent(neox):
    dt, cs, T, H, D, R = "f16", "f32", 6, 4, 128, 64
    x = synth.normal(5, (T, H * D), 0.0, 1.0, dt)
    # one bad element in the rotated span of (token 1, head 2), one in the
    # pass-through part of (token 4, head 0)
    spots = [(1, 2 * D + (D - R) + 5), (4, 3)]
    x = _plant(x, dt, spots)
    c, s = synth.rope_table(T, R, cs)
    fn = qrw.rope_apply_neox if neox else qrw.rope_apply_interleaved
    got = host(fn(dev(x, dt), dev(c, cs), dev(s, cs), H, D, R))
    want = oracle.rope(x, c, s, H, D, R, dt, cs, neox)
    ts = rope_terms(x, c, s, H, D, R, dt, cs, neox)
    mask = np.ones((T, H * D), bool)
    j = 5  # the bad element's position in the span, and its partner's
    partner = (j + R // 2) % R if neox else j ^ 1
    mask[1, 2 * D + (D - R) + j] = mask[1, 2 * D + (D - R) + partner] = False
    mask[4, 3] = False
    assert_close16(got[mask], want[mask], dt, term_scale=ts[mask], what="rope")


def test_fused_tokens_stay_independent():
    dt, cs, T, H, D = "bf16", "bf16", 8, 32, 128
    x = synth.normal(6, (T, H * D), 0.0, 3.0, dt, outlier_frac=0.01, outlier_mul=10.0)
    x = _plant(x, dt, [(2, 100), (5, 4095), (5, 0)])
    w = synth.normal(7, (H * D,), 1.0, 0.1, dt)
    c, s = synth.rope_table(T, D, cs)
    q, sc = qrw.rmsnorm_rope_fp8_fwd(dev(x, dt), dev(w, dt), dev(c, cs), dev(s, cs), H, D)
    keep = [t for t in range(T) if t not in (2, 5)]
    # the finite tokens of this batch give the codes of a batch without the bad
    # ones, which in turn match the oracle
    q2, sc2 = qrw.rmsnorm_rope_fp8_fwd(dev(x[keep], dt), dev(w, dt), dev(c[keep], cs),
                                       dev(s[keep], cs), H, D)
    assert np.array_equal(host(q)[keep], host(q2)) and np.array_equal(host(sc)[keep], host(sc2))
    test_gpu_fused._check_ties(x[keep], w, c[keep], s[keep], H, D, D, dt, cs, True,
                               what="fused, finite tokens")


@pytest.mark.parametrize("group", [None, 128])
def test_act_quant_rows_and_groups_stay_independent(group):
    dt, rows, n = "bf16", 6, 4096
    x = _plant(synth.normal(8, (rows, n), 0.0, 1.0, dt), dt, [(1, 300), (4, 4000)])
    q, sc = qrw.act_quant_fp8_fwd(dev(x, dt), group)
    q, sc = host(q), host(sc)
    wq, wsc = oracle.act_quant_fp8(x, dt, group)
    g = n if group is None else group
    ok = np.ones((rows, n // g), bool)
    ok[1, 300 // g] = ok[4, 4000 // g] = False
    codes_ok = np.repeat(ok, g, axis=1)
    assert np.array_equal(sc.view(np.uint32)[ok], wsc.view(np.uint32)[ok])
    assert np.array_equal(q[codes_ok], wq[codes_ok])


def test_qk_heads_stay_independent():
    dt, cs, T, Hq, Hk, D = "bf16", "bf16", 5, 6, 2, 128
    x = synth.normal(9, (T, (Hq + 2 * Hk) * D), 0.0, 2.0, dt)
    x = _plant(x, dt, [(1, 3 * D + 17), (3, (Hq + 1) * D + 2)])  # a q head, a k head
    qw = synth.normal(10, (D,), 1.0, 0.2, dt)
    kw = synth.normal(11, (D,), 1.0, 0.2, dt)
    c, s = synth.rope_table(T, D, cs)
    got, _ = test_gpu_qk_norm_rope._run(x, qw, kw, c, s, Hq, Hk, D, D, dt, cs, True, 1e-6)
    want = oracle.qk_norm_rope(x, qw, kw, c, s, Hq, Hk, D, D, dt, cs, True, 1e-6)
    ok = np.ones((T, Hq + 2 * Hk), bool)
    ok[1, 3] = ok[3, Hq + 1] = False
    okc = np.repeat(ok, D, axis=1)
    m = (Hq + Hk) * D
    assert np.array_equal(got[:, m:], x[:, m:])  # value heads are never written
    assert_close16(got[:, :m][okc[:, :m]], want[:, :m][okc[:, :m]], dt, what="qk, finite heads")


@pytest.mark.parametrize("fmt", ["f16", "bf16", "f32"])
def test_elementwise_elements_stay_independent(fmt):
    n = 10007
    x = synth.normal(12, (n,), 0.0, 4.0, fmt)
    b = synth.normal(13, (n,), 0.0, 4.0, fmt)
    bad = [3, 4096, n - 1]
    if fmt == "f32":
        x = x.copy()
        x[bad] = np.array([np.nan, np.inf, -np.inf], np.float32)
    else:
        x = _plant(x.reshape(1, n), fmt, [(0, k) for k in bad]).reshape(n)
    got = test_gpu_ew._run("scale_add", x, b, 0.75, fmt, fmt)
    want = oracle.ew_scale_add(x, b, 0.75, fmt, fmt)
    ok = np.ones(n, bool)
    ok[bad] = False
    bits = np.uint32 if fmt == "f32" else np.uint16
    assert np.array_equal(got.view(bits)[ok], want.view(bits)[ok])
