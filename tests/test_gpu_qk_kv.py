"""GPU parity of qk_norm_rope_fp8_kv_fwd (QK RMSNorm + RoPE with the FP8
KV-cache write, "TileLang tutorial, ch. 13", s2.4's cross-module fusion with
s3.1.5's cast per (token, head)) against the fp64 oracle through the C ABI:
the benchmark configuration with scattered cache slots, head sizes, partial
rotation, both pair conventions, table dtypes, slot maps with padding and
out-of-range entries, padded cache rows.  q as 16-bit outputs (2 ulp, with the
cancellation allowance), k codes by the FP8 bar, v codes and scales bit-exact
(v is quantised as stored), untouched cache rows and qkv's k/v columns
bit-identical."""
import numpy as np
import pytest
import torch

import oracle
import quant_row_workgroup_amd as qrw
from quant_row_workgroup_amd import synth
from tests.gpu_util import (assert_close16, assert_codes, assert_codes_away_from_ties,
                            assert_scales, dev, host, qk_terms, rotation_terms)

pytestmark = pytest.mark.gpu

FILL = 0xAB


def _run(x, qw, kw, c, s, Hq, Hk, D, R, dt, cs, neox, eps, slots, ns, cst):
    xd = dev(x, dt)
    kc = torch.full((ns, cst), FILL, dtype=torch.uint8, device="cuda")
    vc = torch.full((ns, cst), FILL, dtype=torch.uint8, device="cuda")
    ks = torch.full((ns, Hk), float("nan"), dtype=torch.float32, device="cuda")
    vs = torch.full((ns, Hk), float("nan"), dtype=torch.float32, device="cuda")
    sl = None if slots is None else torch.from_numpy(slots).cuda()
    qrw.qk_norm_rope_fp8_kv_fwd(xd, None if qw is None else dev(qw, dt),
                                None if kw is None else dev(kw, dt), dev(c, cs), dev(s, cs),
                                kc[:, : Hk * D], vc[:, : Hk * D], ks, vs, Hq, Hk, D, R,
                                slots=sl, neox=neox, eps=eps)
    return host(xd), host(kc), host(vc), host(ks), host(vs)


def _k_quotients(x, kw, c, s, Hq, Hk, D, R, dt, cs, neox, eps, k_scales):
    """z / scale of every k head, [tokens, Hk*D], and the rotation's products
    on the same scale: a k head is normalised and rotated as one 1-head row of
    the fused operator, whose oracle returns the unrounded z; the scales are the
    KV oracle's own."""
    T = x.shape[0]
    kx = np.ascontiguousarray(x[:, Hq * D:(Hq + Hk) * D]).reshape(T * Hk, D)
    kc, ks = np.repeat(c, Hk, axis=0), np.repeat(s, Hk, axis=0)
    _, _, z = oracle.rmsnorm_rope_fp8(kx, kw, kc, ks, 1, D, R, dt, cs, neox, eps, want_z=True)
    sd = k_scales.reshape(T * Hk, 1).astype(np.float64)
    terms = rotation_terms(kx, kw, kc, ks, 1, D, R, dt, cs, neox, eps)
    return (z / sd).reshape(T, Hk * D), (terms / sd).reshape(T, Hk * D)


def _check(x, qw, kw, c, s, Hq, Hk, D, R, dt, cs, neox, eps, slots=None, ns=None, pad=0,
           what="", ties=False):
    """``ties``: k codes exact wherever the quotient is clear of an E4M3
    rounding boundary (for small random cases, where the 99.9% bar would not
    tolerate a single boundary case)."""
    T = x.shape[0]
    ns = T if ns is None else ns
    cst = Hk * D + pad
    got = _run(x, qw, kw, c, s, Hq, Hk, D, R, dt, cs, neox, eps, slots, ns, cst)
    want = oracle.qk_norm_rope_fp8_kv(x, qw, kw, c, s, Hq, Hk, D, R, dt, cs, neox, eps,
                                      slots=slots, num_slots=ns, cache_stride=cst, fill=FILL)
    gx, gkc, gvc, gks, gvs = got
    wq, wkc, wvc, wks, wvs = want
    # k and v columns of qkv are only read
    assert np.array_equal(gx[:, Hq * D:], x[:, Hq * D:]), what
    ts = qk_terms(x, qw, kw, c, s, Hq, 0, D, R, dt, cs, neox, eps)
    st = {"q": assert_close16(gx[:, : Hq * D], wq, dt, term_scale=ts, what=what + " q")}
    # rows no token maps to (and cache row padding) keep their contents
    rows = np.zeros(ns, bool)
    sl = np.arange(T) if slots is None else slots
    rows[sl[(sl >= 0) & (sl < ns)]] = True
    for g, w in ((gkc, wkc), (gvc, wvc)):
        assert np.array_equal(g[~rows], w[~rows]), what
        assert np.all(g[:, Hk * D:] == FILL), what
    for g in (gks, gvs):
        assert np.all(np.isnan(g[~rows])), what
    if rows.any():
        if ties:
            kept = (sl >= 0) & (sl < ns)
            zq, mag = _k_quotients(x[kept], kw, c[kept], s[kept], Hq, Hk, D, R, dt, cs, neox,
                                   eps, wks[sl[kept]])
            st["k"] = assert_codes_away_from_ties(gkc[sl[kept], : Hk * D],
                                                  wkc[sl[kept], : Hk * D], zq, what=what + " k",
                                                  magnitude=mag)
        else:
            st["k"] = assert_codes(gkc[rows, : Hk * D], wkc[rows, : Hk * D], what=what + " k")
        assert_scales(gks[rows], wks[rows], what=what + " k scales")
        assert np.array_equal(gvc[rows], wvc[rows]), what + " v codes"
        assert np.array_equal(gvs[rows], wvs[rows]), what + " v scales"
    return st


@pytest.mark.parametrize("neox", [True, False])
def test_qk_kv_workload(neox):
    name = "qk_norm_rope_fp8_kv_4096_q32_kv8_d128_bf16"
    inp = synth.make_inputs(name)
    st = _check(inp["x"], inp["q_weight"], inp["k_weight"], inp["cos"], inp["sin"],
                inp["q_heads"], inp["kv_heads"], inp["head_dim"], inp["rope_dim"], inp["dtype"],
                inp["cs_dtype"], neox, inp["eps"], slots=inp["slots"], ns=inp["num_slots"],
                what=name)
    print(name, "neox" if neox else "interleaved", st)
    assert st["q"]["within_2ulp_of_result"] >= 0.9999


SHAPES = [
    # tokens, q_heads, kv_heads, head_dim, rope_dim
    (5, 32, 8, 128, 128),
    (3, 8, 2, 128, 64),
    (7, 4, 4, 64, 64),
    (4, 2, 1, 64, 16),
    (3, 16, 4, 256, 256),
    (2, 16, 2, 256, 128),
    (9, 3, 1, 128, 32),     # 80 granules: one ragged chunk
    (3, 7, 3, 256, 64),     # 416 granules
    (2, 64, 8, 128, 128),   # 10 chunks per token
]


@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("dt,cs", [("bf16", "bf16"), ("f16", "f32"), ("bf16", "f32"),
                                   ("f16", "f16")])
@pytest.mark.parametrize("T,Hq,Hk,D,R", SHAPES)
def test_qk_kv_shapes(neox, dt, cs, T, Hq, Hk, D, R):
    seed = T * 13 + Hq * 5 + Hk + D + R
    n = (Hq + 2 * Hk) * D
    x = synth.normal(seed, (T, n), 0.0, 2.0, dt, outlier_frac=0.02, outlier_mul=8.0)
    qw = synth.normal(seed + 1, (D,), 1.0, 0.2, dt)
    kw = synth.normal(seed + 2, (D,), 1.0, 0.2, dt)
    c, s = synth.rope_table(T, R, cs, base=10000.0 if T < 6 else 5.0)
    slots = synth.cache_slots(seed + 3, T, 2 * T + 3)
    _check(x, qw, kw, c, s, Hq, Hk, D, R, dt, cs, neox, 1e-6, slots=slots, ns=2 * T + 3,
           what=f"qk_kv {T}x({Hq}+{Hk}+{Hk})x{D}/{R} {dt}/{cs}")


@pytest.mark.parametrize("neox", [True, False])
def test_qk_kv_padding_slots_no_weights_and_padded_cache_rows(neox):
    T, Hq, Hk, D, R = 12, 8, 2, 128, 64
    n = (Hq + 2 * Hk) * D
    x = synth.normal(21, (T, n), 0.0, 1.0, "bf16")
    x[3, (Hq + Hk) * D:(Hq + Hk + 1) * D] = 0  # a zero v head: floor scale, zero codes
    c, s = synth.rope_table(T, R, "bf16")
    slots = np.array([5, -1, 0, 17, 2, 40, 9, 1, -7, 3, 11, 16], dtype=np.int64)
    _check(x, None, None, c, s, Hq, Hk, D, R, "bf16", "bf16", neox, 1e-5, slots=slots, ns=18,
           pad=32, what="padding slots")
    kw = synth.normal(22, (D,), 1.0, 0.2, "bf16")
    _check(x, None, kw, c, s, Hq, Hk, D, R, "bf16", "bf16", neox, 1e-5, what="identity slots")


def test_qk_kv_empty():
    x = dev(np.zeros((0, 6 * 64), np.uint16), "bf16")
    c = dev(np.zeros((0, 32), np.uint16), "bf16")
    kc = torch.zeros((0, 64), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((0, 1), dtype=torch.float32, device="cuda")
    qrw.qk_norm_rope_fp8_kv_fwd(x, None, None, c, c, kc, kc.clone(), ks, ks.clone(), 4, 1, 64)
