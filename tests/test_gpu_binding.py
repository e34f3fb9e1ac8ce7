"""The Python binding checks every tensor against the one that fixes the shape
(x, qkv or a): device, dtype and exact shape of outputs, weights, tables,
codes, scales, caches and slots.  A mismatch raises ValueError before the
library is called, so nothing is launched: the outputs keep a sentinel.  A
buffer that is too small would otherwise be read or written past its end."""
import pytest
import torch

import quant_row_workgroup_amd as qrw

pytestmark = pytest.mark.gpu

BF, F16, F32, U8 = torch.bfloat16, torch.float16, torch.float32, torch.uint8


def _t(shape, dtype, fill=0):
    return torch.full(shape, fill, dtype=dtype, device="cuda")


def _refused(call, *outs):
    saved = [o.clone() for o in outs]
    with pytest.raises(ValueError):
        call()
    torch.cuda.synchronize()
    for o, s in zip(outs, saved):
        assert torch.equal(o, s)


T, H, D = 4, 2, 128
N = H * D


def test_norm_outputs_and_weights():
    x = _t((T, N), BF, 1.0)
    y_short, y_f16 = _t((T - 1, N), BF, 7.0), _t((T, N), F16, 7.0)
    _refused(lambda: qrw.rmsnorm_fwd(x, None, out=y_short), y_short)
    _refused(lambda: qrw.rmsnorm_fwd(x, None, out=y_f16), y_f16)
    y = _t((T, N), BF, 7.0)
    _refused(lambda: qrw.rmsnorm_fwd(x, _t((N,), F16, 1.0), out=y), y)
    _refused(lambda: qrw.rmsnorm_fwd(x, _t((N - 8,), BF, 1.0), out=y), y)
    _refused(lambda: qrw.rmsnorm_fwd(x, torch.ones(N, dtype=BF), out=y), y)
    _refused(lambda: qrw.layernorm_fwd(x, _t((N,), BF, 1.0), _t((N,), F32), out=y), y)
    _refused(lambda: qrw.layernorm_fwd(x, None, None, out=_t((T, N - 8), BF)), y)


def test_rope_tables_and_outputs():
    x = _t((T, N), F16, 1.0)
    c = _t((T, D // 2), F32, 1.0)
    y = _t((T, N), F16, 7.0)
    _refused(lambda: qrw.rope_apply_neox(x, c[:T - 1], c[:T - 1], H, D, out=y), y)
    _refused(lambda: qrw.rope_apply_neox(x, c, c.to(F16), H, D, out=y), y)
    _refused(lambda: qrw.rope_apply_interleaved(x, _t((T, D // 4), F32), _t((T, D // 4), F32), H,
                                                D, out=y), y)
    _refused(lambda: qrw.rope_apply_interleaved(x, c, c, H, D, out=_t((T, N), BF)), y)


@pytest.mark.parametrize("fn", [qrw.rmsnorm_rope_fp8_fwd, qrw.rmsnorm_rope_fp8_rounded_fwd])
def test_fused_codes_scales_and_tables(fn):
    x = _t((T, N), BF, 1.0)
    w = _t((N,), BF, 1.0)
    c = _t((T, D // 2), BF, 1.0)
    q, sc = _t((T, N), U8, 0x5C), _t((T,), F32, -1.0)
    _refused(lambda: fn(x, w, c, c, H, D, q=_t((T - 1, N), U8), scales=sc), q, sc)
    _refused(lambda: fn(x, w, c, c, H, D, q=_t((T, N), torch.int8), scales=sc), q, sc)
    _refused(lambda: fn(x, w, c, c, H, D, q=q, scales=_t((T - 1,), F32)), q, sc)
    _refused(lambda: fn(x, w, c, c, H, D, q=q, scales=_t((T,), F16)), q, sc)
    _refused(lambda: fn(x, w, c[:, :16], c[:, :16], H, D, q=q, scales=sc), q, sc)
    _refused(lambda: fn(x, w.float(), c, c, H, D, q=q, scales=sc), q, sc)


def test_act_quant_codes_and_scales():
    x = _t((T, N), BF, 1.0)
    q, sc = _t((T, N), U8, 0x5C), _t((T, N // 128), F32, -1.0)
    _refused(lambda: qrw.act_quant_fp8_fwd(x, 128, q=_t((T, N - 8), U8), scales=sc), q, sc)
    _refused(lambda: qrw.act_quant_fp8_fwd(x, 128, q=q, scales=_t((T, 1), F32)), q, sc)
    _refused(lambda: qrw.act_quant_fp8_fwd(x, 128, q=q, scales=_t((T, N // 128), F16)), q, sc)
    _refused(lambda: qrw.act_quant_fp8_fwd(x, 0, q=q, scales=sc), q, sc)


def test_qk_weights_tables_caches_and_slots():
    Hq, Hk = 2, 1
    qkv = _t((T, (Hq + 2 * Hk) * D), BF, 1.0)
    hw = _t((D,), BF, 1.0)
    c = _t((T, D // 2), BF, 1.0)
    keep = qkv.clone()
    _refused(lambda: qrw.qk_norm_rope_fwd(qkv, hw.half(), hw, c, c, Hq, Hk, D), qkv)
    _refused(lambda: qrw.qk_norm_rope_fwd(qkv, hw, hw, c[:2], c[:2], Hq, Hk, D), qkv)
    assert torch.equal(qkv, keep)
    ns = 16
    kc, vc = _t((ns, Hk * D), U8, 0x5C), _t((ns, Hk * D), U8, 0x5C)
    ks, vs = _t((ns, Hk), F32, -1.0), _t((ns, Hk), F32, -1.0)
    sl = torch.arange(T, dtype=torch.int64, device="cuda")

    def kv(**kw):
        a = dict(k_cache=kc, v_cache=vc, k_scales=ks, v_scales=vs, slots=sl)
        a.update(kw)
        return lambda: qrw.qk_norm_rope_fp8_kv_fwd(qkv, hw, hw, c, c, a["k_cache"], a["v_cache"],
                                                   a["k_scales"], a["v_scales"], Hq, Hk, D,
                                                   slots=a["slots"])
    outs = (qkv, kc, vc, ks, vs)
    _refused(kv(k_cache=_t((ns, 2 * Hk * D), U8)[:, :Hk * D // 2]), *outs)   # rows too short
    _refused(kv(v_cache=_t((ns - 1, Hk * D), U8)), *outs)
    _refused(kv(v_cache=_t((ns, Hk * D), torch.int8)), *outs)
    _refused(kv(k_scales=_t((ns - 1, Hk), F32)), *outs)
    _refused(kv(v_scales=_t((ns, Hk), F16)), *outs)
    _refused(kv(slots=sl.int()), *outs)
    _refused(kv(slots=sl[:T - 1]), *outs)
    _refused(kv(slots=sl.cpu()), *outs)


def test_elementwise_operands_and_outputs():
    a = _t((1000,), F16, 1.0)
    y = _t((1000,), F16, 7.0)
    _refused(lambda: qrw.ew_add_fwd(a, _t((999,), F16), out=y), y)
    _refused(lambda: qrw.ew_add_fwd(a, _t((1000,), BF), out=y), y)
    _refused(lambda: qrw.ew_add_fwd(a, a, out=_t((999,), F16)), y)
    _refused(lambda: qrw.ew_scale_add_fwd(a, a, 2.0, out=_t((1000,), F32)), y)
    _refused(lambda: qrw.ew_scale_cast_fwd(a, 2.0, torch.float32, out=_t((1000,), F16)), y)
    _refused(lambda: qrw.ew_scale_cast_fwd(a, 2.0, out=_t((500,), F32)), y)
