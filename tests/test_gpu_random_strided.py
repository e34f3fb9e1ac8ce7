"""The seeded random fused shapes of test_gpu_random_shapes and
test_gpu_random_wide with x given as a view into rows padded by 8, 24 or 64
elements of NaN: the strided instances of every fused kernel, and a check
that no padding element reaches a row's statistics.  Same generators, oracle
and bars; only x's row stride differs."""
import pytest
import torch

import quant_row_workgroup_amd as qrw
from tests import test_gpu_fused as fused
from tests import test_gpu_random_shapes as shapes
from tests import test_gpu_random_wide as wide
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu

SEEDS = range(4000, 4012)


def _strided_run(pad):
    def run(x, w, c, s, H, D, R, dt, cs, neox, eps=1e-6):
        T, n = x.shape
        xd = dev(x, dt)
        rows = torch.full((T, n + pad), float("nan"), dtype=xd.dtype, device="cuda")
        rows[:, :n] = xd
        q, sc = qrw.rmsnorm_rope_fp8_fwd(rows[:, :n], None if w is None else dev(w, dt),
                                         dev(c, cs), dev(s, cs), H, D, R, neox=neox, eps=eps)
        return host(q), host(sc)
    return run


@pytest.mark.parametrize("i", SEEDS)
@pytest.mark.parametrize("mod,name", [(shapes, "test_random_fused"),
                                      (wide, "test_random_wide_fused")],
                         ids=["test_random_fused", "test_random_wide_fused"])
def test_random_fused_strided_rows(monkeypatch, mod, name, i):
    monkeypatch.setattr(fused, "_run", _strided_run([8, 24, 64][i % 3]))
    getattr(mod, name)(i)
