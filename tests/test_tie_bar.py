"""The tie-aware FP8 code bar on the CPU: the rotation's products bound every
rotated value the oracle returns (a sum of two products never exceeds their
magnitudes' sum) and vanish on pass-through channels; a one-step code
difference is accepted only within 2^-20 of the magnitude from an E4M3
rounding boundary, and never two steps."""
import numpy as np
import pytest

import oracle
from quant_row_workgroup_amd import synth
from tests.gpu_util import assert_codes_away_from_ties, e4m3_boundaries, rotation_terms


@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("weighted", [True, False])
def test_rotation_terms_bound_the_rotated_values(neox, weighted):
    T, H, D, R = 5, 3, 64, 32
    x = synth.normal(7, (T, H * D), 0.0, 2.0, "bf16")
    w = synth.normal(8, (H * D,), 1.0, 0.2, "bf16") if weighted else None
    c, s = synth.rope_table(T, R, "f32", base=7.0)
    _, _, z = oracle.rmsnorm_rope_fp8(x, w, c, s, H, D, R, "bf16", "f32", neox, 1e-6,
                                      want_z=True)
    t = rotation_terms(x, w, c, s, H, D, R, "bf16", "f32", neox, 1e-6).reshape(T, H, D)
    z = z.reshape(T, H, D)
    assert np.all(t[..., : D - R] == 0)
    assert np.all(np.abs(z[..., D - R:]) <= t[..., D - R:] * (1 + 2.0 ** -40))
    # and not loosely: the bound is within a factor of two of |a c| + |b s|,
    # which some channel nearly reaches when its two products share a sign
    assert np.max(np.abs(z[..., D - R:]) / t[..., D - R:]) > 0.4


def _codes_near(q):
    """The E4M3 codes of q and of its upper neighbour (as bytes)."""
    import torch

    a = torch.tensor([q], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).item()
    return np.array([a], np.uint8), np.array([a + 1], np.uint8)


def test_band_accepts_a_step_only_within_the_magnitude():
    b = e4m3_boundaries()
    edge = float(b[np.searchsorted(b, 0.0146)])  # a rounding boundary near 0.0146
    q = edge * (1 - 2.0 ** -15)                   # 2^-15 below it (relative)
    lo, hi = _codes_near(q)
    quot = np.array([q])
    with pytest.raises(AssertionError, match="away from a rounding"):
        assert_codes_away_from_ties(hi, lo, quot)
    with pytest.raises(AssertionError, match="away from a rounding"):
        assert_codes_away_from_ties(hi, lo, quot, magnitude=np.array([8.0 * q]))
    st = assert_codes_away_from_ties(hi, lo, quot, magnitude=np.array([4096.0 * q]))
    assert st["max_step"] == 1 and st["exact_frac"] == 0.0
    with pytest.raises(AssertionError, match="steps apart"):
        assert_codes_away_from_ties(hi + 1, lo, quot, magnitude=np.array([4096.0 * q]))
