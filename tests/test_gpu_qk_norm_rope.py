"""GPU parity of qk_norm_rope_fwd (per-head QK RMSNorm + RoPE in place on a
packed QKV activation, "TileLang tutorial, ch. 13", s2.4) against the fp64
oracle through the C ABI: the benchmark configuration, head sizes 64/128/256,
full and partial rotation, both pair conventions, table dtypes, ragged wave
chunks, absent weights, padded rows; value heads and row padding must come
back bit-identical."""
import numpy as np
import pytest

import oracle
import quant_row_workgroup_amd as qrw
from quant_row_workgroup_amd import synth
from tests.gpu_util import assert_close16, dev, host, qk_terms

pytestmark = pytest.mark.gpu


def _run(x, qw, kw, c, s, Hq, Hk, D, R, dt, cs, neox, eps, pad=0):
    T, n = x.shape
    xd = dev(x, dt)
    if pad:
        wide = dev(synth.normal(99, (T, n + pad), 0.0, 1.0, dt), dt)
        wide[:, :n] = xd
        xd = wide[:, :n]
    qrw.qk_norm_rope_fwd(xd, None if qw is None else dev(qw, dt),
                         None if kw is None else dev(kw, dt), dev(c, cs), dev(s, cs), Hq, Hk,
                         D, R, neox, eps)
    if pad:
        return host(xd), host(wide)
    return host(xd), None


def _check(x, got, qw, kw, c, s, Hq, Hk, D, R, dt, cs, neox, eps, what):
    want = oracle.qk_norm_rope(x, qw, kw, c, s, Hq, Hk, D, R, dt, cs, neox, eps)
    m = (Hq + Hk) * D
    # value heads are never written
    assert np.array_equal(got[:, m:], x[:, m:]), what
    ts = qk_terms(x, qw, kw, c, s, Hq, Hk, D, R, dt, cs, neox, eps)
    st = assert_close16(got[:, :m], want[:, :m], dt, term_scale=ts, what=what)
    # channels outside the rotated span are single products: 2 ulp of the result
    P = D - R
    if P:
        T = x.shape[0]
        g = got[:, :m].reshape(T, Hq + Hk, D)[..., :P]
        w = want[:, :m].reshape(T, Hq + Hk, D)[..., :P]
        assert_close16(g, w, dt, what=what + " (unrotated)")
    return st


@pytest.mark.parametrize("neox", [True, False])
def test_qk_norm_rope_workload(neox):
    name = "qk_norm_rope_4096_q32_kv8_d128_bf16"
    inp = synth.make_inputs(name)
    a = (inp["q_heads"], inp["kv_heads"], inp["head_dim"], inp["rope_dim"], inp["dtype"],
         inp["cs_dtype"], neox, inp["eps"])
    got, _ = _run(inp["x"], inp["q_weight"], inp["k_weight"], inp["cos"], inp["sin"], *a)
    st = _check(inp["x"], got, inp["q_weight"], inp["k_weight"], inp["cos"], inp["sin"], *a,
                what=name)
    print(name, "neox" if neox else "interleaved", st)
    assert st["within_2ulp_of_result"] >= 0.9999


SHAPES = [
    # tokens, q_heads, kv_heads, head_dim, rope_dim
    (5, 32, 8, 128, 128),
    (3, 8, 2, 128, 64),     # partial span
    (7, 4, 4, 64, 64),
    (4, 2, 1, 64, 16),      # one-granule half span
    (3, 16, 4, 256, 256),   # head of 32 lanes, partner 16 lanes away
    (2, 16, 2, 256, 128),
    (6, 1, 0, 128, 128),    # no key/value heads
    (9, 3, 1, 128, 32),     # q/k part smaller than one wave chunk
    (5, 5, 1, 64, 32),      # 48 granules: ragged first chunk
    (3, 7, 3, 256, 64),     # 320 granules: 2.5 chunks
    (2, 64, 8, 128, 128),   # 9 chunks per token
]


@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("dt,cs", [("bf16", "bf16"), ("f16", "f32"), ("bf16", "f32"),
                                   ("f16", "f16")])
@pytest.mark.parametrize("T,Hq,Hk,D,R", SHAPES)
def test_qk_norm_rope_shapes(neox, dt, cs, T, Hq, Hk, D, R):
    seed = T * 11 + Hq * 3 + Hk + D + R
    n = (Hq + 2 * Hk) * D
    x = synth.normal(seed, (T, n), 0.0, 2.0, dt, outlier_frac=0.02, outlier_mul=8.0)
    qw = synth.normal(seed + 1, (D,), 1.0, 0.2, dt)
    kw = synth.normal(seed + 2, (D,), 1.0, 0.2, dt)
    c, s = synth.rope_table(T, R, cs, base=10000.0 if T < 6 else 5.0)
    got, _ = _run(x, qw, kw, c, s, Hq, Hk, D, R, dt, cs, neox, 1e-6)
    _check(x, got, qw, kw, c, s, Hq, Hk, D, R, dt, cs, neox, 1e-6,
           what=f"qk {T}x({Hq}+{Hk}+{Hk})x{D}/{R} {dt}/{cs}")


@pytest.mark.parametrize("neox", [True, False])
def test_qk_norm_rope_without_weights_and_with_padded_rows(neox):
    T, Hq, Hk, D, R = 33, 8, 2, 128, 64
    n = (Hq + 2 * Hk) * D
    x = synth.normal(5, (T, n), 0.0, 1.0, "bf16")
    c, s = synth.rope_table(T, R, "bf16")
    got, wide = _run(x, None, None, c, s, Hq, Hk, D, R, "bf16", "bf16", neox, 1e-5, pad=24)
    _check(x, got, None, None, c, s, Hq, Hk, D, R, "bf16", "bf16", neox, 1e-5, what="no weights")
    pad = host(dev(synth.normal(99, (T, n + 24), 0.0, 1.0, "bf16"), "bf16"))[:, n:]
    assert np.array_equal(wide[:, n:], pad)
    # one weight only
    kw = synth.normal(6, (D,), 1.0, 0.2, "bf16")
    got, _ = _run(x, None, kw, c, s, Hq, Hk, D, R, "bf16", "bf16", neox, 1e-5)
    _check(x, got, None, kw, c, s, Hq, Hk, D, R, "bf16", "bf16", neox, 1e-5, what="k weight only")


def test_qk_norm_rope_identity_rotation_is_per_head_rmsnorm():
    # c = 1, s = 0: every q/k head becomes its weighted RMSNorm, which the oracle's
    # plain RMSNorm over rows of head_dim gives exactly
    T, Hq, Hk, D = 4, 4, 2, 128
    n = (Hq + 2 * Hk) * D
    x = synth.normal(8, (T, n), 0.0, 1.0, "bf16")
    w = synth.normal(9, (D,), 1.0, 0.1, "bf16")
    one = synth.to_storage(np.ones((T, D // 2)), "bf16")
    zero = synth.to_storage(np.zeros((T, D // 2)), "bf16")
    got, _ = _run(x, w, w, one, zero, Hq, Hk, D, D, "bf16", "bf16", True, 1e-6)
    heads = np.ascontiguousarray(x[:, : (Hq + Hk) * D].reshape(-1, D))
    want = oracle.rmsnorm(heads, w, "bf16", 1e-6).reshape(T, (Hq + Hk) * D)
    assert_close16(got[:, : (Hq + Hk) * D], want, "bf16", what="identity rotation")


def test_qk_norm_rope_empty():
    x = dev(np.zeros((0, 6 * 64), np.uint16), "bf16")
    c = dev(np.zeros((0, 32), np.uint16), "bf16")
    qrw.qk_norm_rope_fwd(x, None, None, c, c, 4, 1, 64)
