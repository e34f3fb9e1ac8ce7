"""The seeded random shapes of test_gpu_random_shapes and test_gpu_random_wide
(QK operators included) at 300 to 2500 rows (40 to 400 for norm and act-quant rows over 16384
channels): many workgroups per launch, several rounds of the grid and a
partial last workgroup on every dispatch path those tests reach.  Same
generators, oracle and bars; only the row count differs."""
import pytest

from tests import test_gpu_random_shapes as shapes
from tests import test_gpu_random_wide as wide

pytestmark = pytest.mark.gpu

SEEDS = range(2000, 2012)


def _many(r, n):
    return int(r.integers(300, 2500)) if n <= 16384 else int(r.integers(40, 400))


@pytest.mark.parametrize("i", SEEDS)
@pytest.mark.parametrize("name", ["test_random_norms", "test_random_rope", "test_random_fused",
                                  "test_random_act_quant", "test_random_staged_fused"])
def test_random_many_rows(monkeypatch, name, i):
    monkeypatch.setattr(shapes, "_tokens", _many)
    getattr(shapes, name)(i)


@pytest.mark.parametrize("i", SEEDS)
@pytest.mark.parametrize("name", ["test_random_wide_fused", "test_random_wide_rope"])
def test_random_wide_many_rows(monkeypatch, name, i):
    monkeypatch.setattr(wide, "_tokens", lambda r: int(r.integers(300, 2500)))
    getattr(wide, name)(i)


@pytest.mark.parametrize("i", SEEDS)
@pytest.mark.parametrize("name", ["test_random_qk_norm_rope", "test_random_qk_kv"])
def test_random_qk_many_rows(monkeypatch, name, i):
    shape = shapes._qk_shape

    def many(r):
        T = int(r.integers(300, 2500))
        return (T,) + shape(r)[1:]

    monkeypatch.setattr(shapes, "_qk_shape", many)
    getattr(shapes, name)(i)
