"""Seeded random shapes aimed at the dispatch paths that rows of wide or
non-power-of-two widths take, against the fp64 oracle through the C ABI:
rows of 3 to 16 blocks of 512 channels in heads of 64 or 128 (the fused
operator's contiguous and two-waves-per-token kernels, the contiguous RoPE
kernel and, for partly rotated NeoX heads, the item kernels), one-wave norm
and activation-quant rows of 64 * e granules, and activation-quant rows up
to 65536 channels (segmented per group, one workgroup per token).  Bars as
in the hand-written tests of each operator."""
import numpy as np
import pytest

import oracle
import quant_row_workgroup_amd as qrw
from quant_row_workgroup_amd import synth
from tests import test_gpu_fused, test_gpu_fused_rounded
from tests.gpu_util import assert_close16, dev, host, layernorm_terms, rope_terms

pytestmark = pytest.mark.gpu

N_CASES = 256
BLOCKS = [3, 5, 6, 7, 10, 12, 14, 16]


def _rng(op, i):
    return np.random.default_rng(90000 + 1000 * ["fused", "rope", "norm", "aq"].index(op) + i)


def _wide_heads(r):
    """Heads of 64 or 128 on a row of 512 * blocks channels; the whole head
    rotates, or its tail."""
    D = [64, 128][int(r.integers(0, 2))]
    blocks = BLOCKS[int(r.integers(0, len(BLOCKS)))]
    H = 512 * blocks // D
    R = D if r.integers(0, 3) else [16, 32, D // 2][int(r.integers(0, 3))]
    return H, D, R


def _tokens(r):
    return int(r.integers(1, 40))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_wide_fused(i):
    r = _rng("fused", i)
    dt = ["f16", "bf16"][int(r.integers(0, 2))]
    cs = ["f32", dt][int(r.integers(0, 2))]
    neox = bool(r.integers(0, 2))
    H, D, R = _wide_heads(r)
    T = _tokens(r)
    x = synth.normal(i, (T, H * D), 0.0, 2.0, dt, outlier_frac=0.01, outlier_mul=10.0)
    w = synth.normal(i + 1, (H * D,), 1.0, 0.1, dt) if r.integers(0, 3) else None
    c, s = synth.rope_table(T, R, cs, base=7.0)
    what = f"fused {T}x{H}x{D}/{R} {dt}/{cs} {'neox' if neox else 'interleaved'}"
    st = test_gpu_fused._check_ties(x, w, c, s, H, D, R, dt, cs, neox, what=what)
    # the tie-aware bar of test_random_fused (test_gpu_random_shapes) decides
    if r.integers(0, 3) == 0:  # the staged form on the same shape
        test_gpu_fused_rounded._check(x, w, c, s, H, D, R, dt, cs, neox, what="staged " + what)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_wide_rope(i):
    r = _rng("rope", i)
    dt = ["f16", "bf16"][int(r.integers(0, 2))]
    cs = ["f32", dt][int(r.integers(0, 2))]
    neox = bool(r.integers(0, 2))
    H, D, R = _wide_heads(r)
    T = _tokens(r)
    x = synth.normal(i, (T, H * D), 0.0, 1.0, dt)
    c, s = synth.rope_table(T, R, cs, base=7.0)
    fn = qrw.rope_apply_neox if neox else qrw.rope_apply_interleaved
    got = host(fn(dev(x, dt), dev(c, cs), dev(s, cs), H, D, R))
    assert_close16(got, oracle.rope(x, c, s, H, D, R, dt, cs, neox), dt,
                   term_scale=rope_terms(x, c, s, H, D, R, dt, cs, neox),
                   what=f"rope {T}x{H}x{D}/{R} {dt}/{cs} {'neox' if neox else 'interleaved'}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_wide_norms(i):
    r = _rng("norm", i)
    dt = ["f16", "bf16"][int(r.integers(0, 2))]
    n = 512 * [3, 5, 6, 7, 10, 12, 14][int(r.integers(0, 7))]
    rows = int(r.integers(1, 300))
    x = synth.normal(i, (rows, n), 0.3, 1.5, dt, outlier_frac=0.01, outlier_mul=8.0)
    w = synth.normal(i + 1, (n,), 1.0, 0.1, dt) if r.integers(0, 4) else None
    got = host(qrw.rmsnorm_fwd(dev(x, dt), None if w is None else dev(w, dt), 1e-6))
    assert_close16(got, oracle.rmsnorm(x, w, dt, 1e-6), dt, what=f"rmsnorm {rows}x{n} {dt}")
    g = synth.normal(i + 2, (n,), 1.0, 0.1, dt) if r.integers(0, 4) else None
    b = synth.normal(i + 3, (n,), 0.0, 0.1, dt) if r.integers(0, 4) else None
    got = host(qrw.layernorm_fwd(dev(x, dt), None if g is None else dev(g, dt),
                                 None if b is None else dev(b, dt), 1e-5))
    assert_close16(got, oracle.layernorm(x, g, b, dt, 1e-5), dt,
                   term_scale=layernorm_terms(x, g, b, dt, 1e-5), what=f"layernorm {rows}x{n}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_wide_act_quant(i):
    r = _rng("aq", i)
    dt = ["f16", "bf16"][int(r.integers(0, 2))]
    group = [None, 8, 16, 32, 64, 128, 256, 512][int(r.integers(0, 8))]
    unit = group or 8
    if r.integers(0, 2):  # a whole row of 64 * e granules
        n = 512 * [3, 5, 6, 7, 10, 12, 14][int(r.integers(0, 7))]
    else:                 # longer than one wave holds
        n = int(r.integers(8193, 65537)) // unit * unit
    n = max(n // unit * unit, unit)
    rows = int(r.integers(1, 24))
    x = synth.normal(i, (rows, n), 0.0, 1.0, dt, outlier_frac=0.01, outlier_mul=20.0)
    q, sc = qrw.act_quant_fp8_fwd(dev(x, dt), group)
    wq, wsc = oracle.act_quant_fp8(x, dt, group)
    assert np.array_equal(host(sc).view(np.uint32), wsc.view(np.uint32)), (rows, n, group)
    assert np.array_equal(host(q), wq), (rows, n, group)
