"""Pins of the oracle's QK RMSNorm + RoPE with the FP8 KV-cache write ("TileLang
tutorial, ch. 13", s2.4: the cross-module fusion of Q/K RMSNorm, RoPE and the
quantised KV-cache write; the quantisation is the per-token cast of s3.1.5
with one scale per (token, head))."""
import numpy as np
import pytest

import oracle
from quant_row_workgroup_amd import synth
from tests import exact


def _inputs(seed, T, Hq, Hk, D, R, fmt, cs, base=10000.0):
    n = (Hq + 2 * Hk) * D
    x = synth.normal(seed, (T, n), 0.0, 2.0, fmt, outlier_frac=0.02, outlier_mul=8.0)
    qw = synth.normal(seed + 1, (D,), 1.0, 0.2, fmt)
    kw = synth.normal(seed + 2, (D,), 1.0, 0.2, fmt)
    c, s = synth.rope_table(T, R, cs, base=base)
    return x, qw, kw, c, s


@pytest.mark.parametrize("fmt,cs", [("bf16", "bf16"), ("f16", "f32")])
@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("shape", [(2, 1, 8, 8), (1, 2, 16, 8), (3, 1, 16, 16)])
def test_brute_force_small(fmt, cs, neox, shape):
    Hq, Hk, D, R = shape
    T = 3
    x, qw, kw, c, s = _inputs(51, T, Hq, Hk, D, R, fmt, cs, base=3.0)
    q, kc, vc, ks, vs = oracle.qk_norm_rope_fp8_kv(x, qw, kw, c, s, Hq, Hk, D, R, fmt, cs, neox,
                                                   1e-6)
    for t in range(T):
        wq, wkc, wks, wvc, wvs = exact.qk_kv_ref(x[t], qw, kw, c[t], s[t], Hq, Hk, D, R, fmt, cs,
                                                 neox, 1e-6)
        assert [int(v) for v in q[t]] == wq, t
        assert [int(v) for v in kc[t]] == wkc, t
        assert [int(v) for v in vc[t]] == wvc, t
        assert [float(v) for v in ks[t]] == wks, t
        assert [float(v) for v in vs[t]] == wvs, t


def test_q_matches_qk_norm_rope_and_v_matches_group_quant():
    # q is the (separately pinned) QK-norm operator's q columns; v is the (separately
    # pinned) activation cast with a group of head_dim over the v columns
    Hq, Hk, D, R = 8, 2, 128, 64
    x, qw, kw, c, s = _inputs(52, 6, Hq, Hk, D, R, "bf16", "bf16")
    q, kc, vc, ks, vs = oracle.qk_norm_rope_fp8_kv(x, qw, kw, c, s, Hq, Hk, D, R, "bf16", "bf16",
                                                   True, 1e-6)
    y = oracle.qk_norm_rope(x, qw, kw, c, s, Hq, Hk, D, R, "bf16", "bf16", True, 1e-6)
    assert np.array_equal(q, y[:, : Hq * D])
    v = np.ascontiguousarray(x[:, (Hq + Hk) * D:])
    codes, scales = oracle.act_quant_fp8(v, "bf16", D)
    assert np.array_equal(vc, codes)
    assert np.array_equal(vs, scales)


def test_k_cache_is_the_quantised_normed_rotated_k():
    # every k head's largest magnitude maps to the largest finite code, and
    # dequantised codes are within half an E4M3 step of the unrounded value
    Hq, Hk, D, R = 4, 4, 64, 64
    x, qw, kw, c, s = _inputs(53, 5, Hq, Hk, D, R, "bf16", "bf16")
    _, kc, _, ks, _ = oracle.qk_norm_rope_fp8_kv(x, qw, kw, c, s, Hq, Hk, D, R, "bf16", "bf16",
                                                 False, 1e-6)
    codes = kc.reshape(5, Hk, D)
    assert np.all((codes & 0x7F).max(axis=2) == 0x7E)
    for t in range(5):
        _, wkc, wks, _, _ = exact.qk_kv_ref(x[t], qw, kw, c[t], s[t], Hq, Hk, D, R, "bf16",
                                            "bf16", False, 1e-6)
        assert [int(v) for v in kc[t]] == wkc
        assert [float(v) for v in ks[t]] == wks


def test_slots_place_rows_and_out_of_range_slots_write_nothing():
    Hq, Hk, D, R = 2, 2, 64, 32
    T = 6
    x, qw, kw, c, s = _inputs(54, T, Hq, Hk, D, R, "f16", "f32")
    base = oracle.qk_norm_rope_fp8_kv(x, qw, kw, c, s, Hq, Hk, D, R, "f16", "f32", True, 1e-6)
    slots = np.array([7, 2, -1, 0, 9, 4], dtype=np.int64)   # 9 >= num_slots, -1 negative
    q, kc, vc, ks, vs = oracle.qk_norm_rope_fp8_kv(x, qw, kw, c, s, Hq, Hk, D, R, "f16", "f32",
                                                   True, 1e-6, slots=slots, num_slots=8,
                                                   cache_stride=Hk * D + 32, fill=0xAB)
    assert np.array_equal(q, base[0])  # q never depends on the slot
    for t, sl in enumerate(slots):
        if 0 <= sl < 8:
            assert np.array_equal(kc[sl, : Hk * D], base[1][t])
            assert np.array_equal(vc[sl, : Hk * D], base[2][t])
            assert np.array_equal(ks[sl], base[3][t]) and np.array_equal(vs[sl], base[4][t])
    untouched = [r for r in range(8) if r not in set(slots.tolist())]
    assert untouched == [1, 3, 5, 6]
    for r in untouched:
        assert np.all(kc[r] == 0xAB) and np.all(vc[r] == 0xAB)
        assert np.all(np.isnan(ks[r])) and np.all(np.isnan(vs[r]))
    assert np.all(kc[:, Hk * D:] == 0xAB)  # row padding of the cache is never written


def test_zero_heads_give_zero_codes_and_the_floor_scale():
    Hq, Hk, D, R = 1, 1, 64, 64
    x, qw, kw, c, s = _inputs(55, 2, Hq, Hk, D, R, "bf16", "bf16")
    x[1] = 0
    q, kc, vc, ks, vs = oracle.qk_norm_rope_fp8_kv(x, qw, kw, c, s, Hq, Hk, D, R, "bf16", "bf16",
                                                   True, 1e-6)
    floor = np.float32(1e-4) / np.float32(448)
    assert np.all(q[1] & 0x7FFF == 0)
    assert np.all(kc[1] & 0x7F == 0) and np.all(vc[1] == 0)
    assert ks[1, 0] == floor and vs[1, 0] == floor
