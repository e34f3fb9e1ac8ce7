"""Pins of the oracle's activation quantisation ("TileLang tutorial, ch. 13",
s3.1.5: per-token / per-group amax -> scale -> clamp -> E4M3 cast)."""
import numpy as np
import pytest
import torch

import oracle
from quant_row_workgroup_amd import synth
from tests import exact


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("group", [8, 16, None])
def test_brute_force_small(fmt, group):
    x = synth.normal(31, (4, 32), 0.0, 2.0, fmt, outlier_frac=0.05, outlier_mul=10.0)
    q, sc = oracle.act_quant_fp8(x, fmt, group)
    g = 32 if group is None else group
    for r in range(4):
        codes, scales = exact.act_quant_ref(x[r], fmt, g)
        assert [int(v) for v in q[r]] == codes
        assert [float(v) for v in sc[r]] == scales


@pytest.mark.parametrize("group", [128, None])
def test_each_group_reaches_the_largest_code_and_dequantises_within_half_a_step(group):
    x = synth.normal(32, (16, 4096), 0.0, 3.0, "bf16", outlier_frac=0.01, outlier_mul=10.0)
    q, sc = oracle.act_quant_fp8(x, "bf16", group)
    g = 4096 if group is None else group
    mags = (q & 0x7F).reshape(16, -1, g).max(axis=2)
    assert np.all(mags == 0x7E)
    deq = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    v = synth.storage_to_f64(x, "bf16") / np.repeat(sc.astype(np.float64), g, axis=1)
    step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6))) - 3)
    assert np.all(np.abs(deq - v) <= 0.5 * step * (1 + 1e-12) + np.abs(v) * 2.0 ** -24)


def test_per_token_is_the_group_of_the_whole_row_and_groups_are_independent():
    x = synth.normal(33, (8, 512), 0.0, 1.0, "f16")
    q1, s1 = oracle.act_quant_fp8(x, "f16", None)
    q2, s2 = oracle.act_quant_fp8(x, "f16", 512)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)
    # quantising the 128-wide slices separately gives the per-128 result
    qg, sg = oracle.act_quant_fp8(x, "f16", 128)
    for k in range(4):
        qk, sk = oracle.act_quant_fp8(np.ascontiguousarray(x[:, 128 * k:128 * (k + 1)]), "f16")
        assert np.array_equal(qg[:, 128 * k:128 * (k + 1)], qk)
        assert np.array_equal(sg[:, k], sk[:, 0])


def test_zero_group_gives_floor_scale_and_zero_codes():
    x = synth.normal(34, (2, 256), 0.0, 1.0, "bf16")
    x[1, 128:] = 0
    q, sc = oracle.act_quant_fp8(x, "bf16", 128)
    assert sc[1, 1] == np.float32(1e-4) / np.float32(448)
    assert np.all(q[1, 128:] == 0)


def test_scale_invariance_by_powers_of_two():
    # scaling x by 2^k scales every scale by 2^k and leaves the codes unchanged
    x = synth.normal(35, (4, 256), 0.0, 1.0, "bf16")
    q0, s0 = oracle.act_quant_fp8(x, "bf16", 64)
    xs = synth.to_storage(synth.storage_to_f64(x, "bf16") * 8.0, "bf16")
    q1, s1 = oracle.act_quant_fp8(xs, "bf16", 64)
    assert np.array_equal(q0, q1)
    assert np.array_equal(s1, s0 * np.float32(8.0))


def test_codes_are_decided_on_the_binary32_quotient():
    # bf16 x over scale = amax/448 often lands exactly on an E4M3 midpoint in binary32;
    # the code must be the nearest-even E4M3 of that binary32 quotient
    x = synth.normal(36, (32, 128), 0.0, 1.0, "bf16")
    q, sc = oracle.act_quant_fp8(x, "bf16", 128)
    xv = synth.storage_to_f64(x, "bf16")
    quot = (xv / sc.astype(np.float64)).astype(np.float32)
    want = torch.from_numpy(np.clip(quot, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, want)
