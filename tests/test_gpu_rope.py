"""GPU parity of rope_apply_interleaved / rope_apply_neox against the fp64
oracle through the C ABI: the benchmark configuration in both pairings,
partial rotation, table dtypes, head layouts that do and do not allow the
one-table-granule-per-lane path, strides, in-place calls and the page's
self-checks (identity rotation, quarter turn)."""
import numpy as np
import pytest

import oracle
import quant_row_workgroup_amd as qrw
from quant_row_workgroup_amd import synth
from tests.gpu_util import assert_close16, dev, host, rope_terms

pytestmark = pytest.mark.gpu


def _fn(neox):
    return qrw.rope_apply_neox if neox else qrw.rope_apply_interleaved


@pytest.mark.parametrize("neox", [True, False])
def test_rope_workload(neox):
    name = "rope_4096x32x128_f16"
    inp = synth.make_inputs(name)
    dt, cs = inp["dtype"], inp["cs_dtype"]
    H, D, R = inp["heads"], inp["head_dim"], inp["rope_dim"]
    got = host(_fn(neox)(dev(inp["x"], dt), dev(inp["cos"], cs), dev(inp["sin"], cs), H, D, R))
    want = oracle.rope(inp["x"], inp["cos"], inp["sin"], H, D, R, dt, cs, neox)
    ts = rope_terms(inp["x"], inp["cos"], inp["sin"], H, D, R, dt, cs, neox)
    st = assert_close16(got, want, dt, term_scale=ts, what=name)
    print(name, "neox" if neox else "interleaved", st)
    assert st["within_2ulp_of_result"] >= 0.9999


SHAPES = [
    # tokens, heads, head_dim, rope_dim
    (5, 32, 128, 128),
    (3, 8, 128, 64),      # partial span
    (7, 3, 48, 32),       # rope_dim/16 = 2
    (4, 5, 96, 96),       # rope_dim/16 = 6 does not divide 64: per-item table loads
    (2, 1, 4096, 128),    # one wide head, rotated tail only
    (6, 64, 128, 128),    # 8192 channels, two passes of items
    (1, 1, 16, 16),
    (9, 2, 1000, 16),     # odd number of pass-through granules per token
    (3, 4, 512, 512),
    # whole heads of head_dim/16 in {1, 2, 4, 8, 16} on rows of 1, 2, 4 or 8
    # blocks of 512 channels
    (3, 4, 128, 128),     # one block
    (2, 16, 64, 64),      # two blocks, head of 8 lanes
    (4, 64, 32, 32),      # four blocks, head of 4 lanes
    (3, 256, 16, 16),     # eight blocks, head of 2 lanes
    (2, 16, 256, 256),    # eight blocks, head of 32 lanes
    # 3, 5, 6, 7, 10, 12, 14 blocks: heads of 128 or 64 (NeoX: whole heads)
    (3, 12, 128, 128), (5, 20, 128, 128), (2, 48, 64, 64), (3, 28, 128, 128),
    (4, 40, 128, 128), (2, 96, 64, 64), (3, 56, 128, 128),
    (4, 40, 128, 64),     # partial span: contiguous when interleaved, items for NeoX
]


@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("dtype,cs", [("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32"),
                                      ("f16", "f16")])
@pytest.mark.parametrize("T,H,D,R", SHAPES)
def test_rope_shapes(neox, dtype, cs, T, H, D, R):
    x = synth.normal(T * 7 + H + D + R, (T, H * D), 0.0, 1.0, dtype)
    c, s = synth.rope_table(T, R, cs, base=10000.0 if T < 8 else 7.0)
    got = host(_fn(neox)(dev(x, dtype), dev(c, cs), dev(s, cs), H, D, R))
    want = oracle.rope(x, c, s, H, D, R, dtype, cs, neox)
    assert_close16(got, want, dtype, term_scale=rope_terms(x, c, s, H, D, R, dtype, cs, neox),
                   what=f"rope {T}x{H}x{D}/{R}")
    # pass-through channels are bit copies
    P = D - R
    if P:
        assert np.array_equal(got.reshape(T, H, D)[..., :P], x.reshape(T, H, D)[..., :P])


@pytest.mark.parametrize("neox", [True, False])
def test_rope_identity_and_quarter_turn_bit_exact(neox):
    T, H, D = 4, 8, 128
    x = synth.normal(3, (T, H * D), 0.0, 1.0, "bf16")
    one = synth.to_storage(np.ones((T, D // 2)), "bf16")
    zero = synth.to_storage(np.zeros((T, D // 2)), "bf16")
    got = host(_fn(neox)(dev(x, "bf16"), dev(one, "bf16"), dev(zero, "bf16"), H, D, D))
    assert np.array_equal(got, x)
    got = host(_fn(neox)(dev(x, "bf16"), dev(zero, "bf16"), dev(one, "bf16"), H, D, D))
    assert np.array_equal(got, oracle.rope(x, zero, one, H, D, D, "bf16", "bf16", neox))


def test_rope_conventions_differ_and_strides_and_in_place():
    T, H, D, R = 33, 4, 64, 32
    dt, cs = "f16", "f32"
    xs, ys = H * D + 24, H * D + 8
    xw = synth.normal(11, (T, xs), 0.0, 1.0, dt)
    c, s = synth.rope_table(T, R, cs)
    xt = dev(xw, dt)
    import torch

    out = torch.zeros((T, ys), dtype=torch.float16, device="cuda")
    qrw.rope_apply_neox(xt[:, :H * D], dev(c, cs), dev(s, cs), H, D, R, out=out[:, :H * D])
    want = oracle.rope(xw, c, s, H, D, R, dt, cs, True)
    got = host(out)
    assert_close16(got[:, :H * D], want, dt,
                   term_scale=rope_terms(xw, c, s, H, D, R, dt, cs, True))
    assert np.all(got[:, H * D:] == 0)
    inter = host(qrw.rope_apply_interleaved(xt[:, :H * D], dev(c, cs), dev(s, cs), H, D, R))
    assert not np.array_equal(inter, got[:, :H * D])
    # in place: the rotated span changes, the pass-through channels stay
    qrw.rope_apply_neox(xt[:, :H * D], dev(c, cs), dev(s, cs), H, D, R, out=xt[:, :H * D])
    gi = host(xt)
    assert np.array_equal(gi[:, :H * D], got[:, :H * D])
    assert np.array_equal(gi[:, H * D:], xw[:, H * D:])


# the contiguous kernel in place and on strided rows: the rotated span equals
# the out-of-place result, pass-through channels and the row padding keep
# their bits (in place the kernel stores only rotated granules)
@pytest.mark.parametrize("neox,H,D,R", [(True, 8, 128, 64), (False, 40, 128, 64),
                                        (True, 24, 128, 128), (False, 16, 256, 32)])
def test_rope_contiguous_in_place_and_strided(neox, H, D, R):
    import torch

    T, dt, cs = 21, "bf16", "f32"
    n = H * D
    xw = synth.normal(H + D + R, (T, n + 24), 0.0, 1.0, dt)
    c, s = synth.rope_table(T, R, cs)
    fn = qrw.rope_apply_neox if neox else qrw.rope_apply_interleaved
    xt = dev(xw, dt)
    out = torch.full((T, n + 8), 3.0, dtype=torch.bfloat16, device="cuda")
    fn(xt[:, :n], dev(c, cs), dev(s, cs), H, D, R, out=out[:, :n])
    got = host(out)
    want = oracle.rope(np.ascontiguousarray(xw[:, :n]), c, s, H, D, R, dt, cs, neox)
    assert_close16(got[:, :n], want, dt,
                   term_scale=rope_terms(np.ascontiguousarray(xw[:, :n]), c, s, H, D, R, dt, cs, neox))
    assert np.all(got[:, n:] == got[0, n]) and got[0, n] != 0  # padding untouched (3.0)
    fn(xt[:, :n], dev(c, cs), dev(s, cs), H, D, R, out=xt[:, :n])
    gi = host(xt)
    assert np.array_equal(gi[:, :n], got[:, :n])
    assert np.array_equal(gi[:, n:], xw[:, n:])
    P = D - R
    if P:
        assert np.array_equal(gi[:, :n].reshape(T, H, D)[..., :P], xw[:, :n].reshape(T, H, D)[..., :P])


def test_rope_empty_and_deterministic():
    T, H, D = 257, 32, 128
    x = synth.normal(12, (T, H * D), 0.0, 1.0, "f16")
    c, s = synth.rope_table(T, D, "f32")
    xt, ct, st = dev(x, "f16"), dev(c, "f32"), dev(s, "f32")
    assert qrw.rope_apply_neox(xt[:0], ct[:0], st[:0], H, D).shape == (0, H * D)
    a = host(qrw.rope_apply_neox(xt, ct, st, H, D))
    b = host(qrw.rope_apply_neox(xt, ct, st, H, D))
    assert np.array_equal(a, b)
