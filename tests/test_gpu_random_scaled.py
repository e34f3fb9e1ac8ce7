"""The seeded random shapes of test_gpu_random_shapes and test_gpu_random_wide
with every generated input scaled by 2^-14, 2^-8 or 2^6: f16 subnormal inputs
and outputs, rows whose mean square is far below eps, FP8 scales at their
floor, and large magnitudes.  Same generators, oracle and bars; only the
inputs' scale differs."""
import pytest

from quant_row_workgroup_amd import synth
from tests import test_gpu_random_shapes as shapes
from tests import test_gpu_random_wide as wide

pytestmark = pytest.mark.gpu

SEEDS = range(3000, 3012)
NAMES = [(shapes, n) for n in ("test_random_norms", "test_random_rope", "test_random_fused",
                               "test_random_act_quant", "test_random_qk_norm_rope",
                               "test_random_qk_kv", "test_random_staged_fused")] + \
        [(wide, n) for n in ("test_random_wide_fused", "test_random_wide_rope",
                             "test_random_wide_norms", "test_random_wide_act_quant")]


# at 2^6 the filler of the norms' row padding (std 300) can round to f16
# infinities: the kernels never read that padding, so they must not show
@pytest.mark.filterwarnings("ignore:overflow encountered in cast:RuntimeWarning")
@pytest.mark.parametrize("i", SEEDS)
@pytest.mark.parametrize("mod,name", NAMES, ids=[n for _, n in NAMES])
def test_random_scaled_inputs(monkeypatch, mod, name, i):
    f = [2.0 ** -14, 2.0 ** -8, 2.0 ** 6][i % 3]
    normal = synth.normal

    def scaled(seed, shape, mean, std, dtype, **kw):
        return normal(seed, shape, mean * f, std * f, dtype, **kw)

    monkeypatch.setattr(synth, "normal", scaled)
    getattr(mod, name)(i)
