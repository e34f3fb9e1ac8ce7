"""The seeded random RoPE shapes of test_gpu_random_shapes and
test_gpu_random_wide with x given as a view into rows padded by 8, 24 or 64
elements of NaN, rotated out of place or in place into that view: the
strided and in-place forms of every RoPE kernel, and a check that no padding
element reaches an output.  Same generators, oracle and bars; only x's row
stride and the output buffer differ."""
import pytest
import torch

import quant_row_workgroup_amd as qrw
from tests import test_gpu_random_shapes as shapes
from tests import test_gpu_random_wide as wide

pytestmark = pytest.mark.gpu

SEEDS = range(5000, 5012)


class _StridedRope:
    """qrw with both RoPE entry points taking x as a padded-row view."""

    def __init__(self, pad, in_place):
        self.pad, self.in_place = pad, in_place

    def __getattr__(self, name):
        return getattr(qrw, name)

    def _wrap(self, fn, x, *args):
        T, n = x.shape
        rows = torch.full((T, n + self.pad), float("nan"), dtype=x.dtype, device=x.device)
        rows[:, :n] = x
        view = rows[:, :n]
        if self.in_place:
            fn(view, *args, out=view)
            return view
        return fn(view, *args)

    def rope_apply_neox(self, x, *args):
        return self._wrap(qrw.rope_apply_neox, x, *args)

    def rope_apply_interleaved(self, x, *args):
        return self._wrap(qrw.rope_apply_interleaved, x, *args)


@pytest.mark.parametrize("i", SEEDS)
@pytest.mark.parametrize("mod,name", [(shapes, "test_random_rope"),
                                      (wide, "test_random_wide_rope")],
                         ids=["test_random_rope", "test_random_wide_rope"])
def test_random_rope_strided_rows(monkeypatch, mod, name, i):
    monkeypatch.setattr(mod, "qrw", _StridedRope([8, 24, 64][i % 3], bool(i % 2)))
    getattr(mod, name)(i)
