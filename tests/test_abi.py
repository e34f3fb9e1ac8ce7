"""The C ABI on the CPU: the library loads, exports every function that
include/qrw.h declares, and rejects bad arguments with the documented status
before touching the device.  Every call below is invalid (or empty) by
construction, so none reaches a HIP call."""
import ctypes
import os
import re

import pytest

import quant_row_workgroup_amd as qrw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qrw.h")
PROBE_HEADER = os.path.join(ROOT, "include", "qrw_probe.h")

OK, NULL, DTYPE, SHAPE, STRIDE, ALIGN, ALIAS, LAUNCH, VALUE = 0, -1, -2, -3, -4, -5, -6, -7, -8
F16, BF16, F32 = 1, 2, 3

# fake, 16-byte aligned, far-apart "device" addresses; never dereferenced
X, Y, W, C, S, Q, SC = (ctypes.c_void_p(a << 32) for a in range(1, 8))
Q_ADDR = 6 << 32


@pytest.fixture(autouse=True)
def _host_only():
    # every case below is meant to fail validation (or be empty) before any HIP
    # call; the fake addresses must never meet a visible device
    import torch

    if torch.cuda.is_available():
        pytest.skip("argument-validation cases use fake device addresses: run without a GPU")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_every_exported_function():
    assert declared_functions() == sorted(qrw.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = qrw.load()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_probe_header_matches_the_probe_library():
    # include/qrw_probe.h: the measurement and self-check kernels' library
    assert declared_functions(PROBE_HEADER) == sorted(qrw.PROBE_EXPORTS)
    P = qrw.load_probe()
    for name in declared_functions(PROBE_HEADER):
        assert hasattr(P, name), name


def test_probe_validation():
    P = qrw.load_probe()
    # wrong row length, negative sizes, bad sweep ranges, bad block counts:
    # refused before anything is enqueued
    assert P.qrw_probe_copy_fused_traffic(X, W, C, S, Q, SC, 4, 2048, 1, None) == SHAPE
    assert P.qrw_probe_copy_fused_traffic(X, W, C, S, Q, SC, 0, 4096, 1, None) == OK
    assert P.qrw_probe_copy_fused_traffic(None, W, C, S, Q, SC, 4, 4096, 1, None) == NULL
    assert P.qrw_probe_copy_fused_traffic(ctypes.c_void_p((1 << 32) + 8), W, C, S, Q, SC, 4,
                                          4096, 1, None) == ALIGN
    # QK probe: qkv, q_weight, k_weight, cos, sin, k/v caches, k/v scales, slots
    qk = (X, W, W, C, S)
    kvb = (Q, Q, SC, SC, Y)
    assert P.qrw_probe_copy_qk_traffic(*qk, None, None, None, None, None, 0, -1, 0, None) == SHAPE
    assert P.qrw_probe_copy_qk_traffic(*qk, *kvb, -1, 4, 1, None) == SHAPE
    assert P.qrw_probe_copy_qk_traffic(*qk, *kvb, 16, 0, 1, None) == OK
    assert P.qrw_probe_copy_qk_traffic(None, W, W, C, S, *kvb, 16, 4, 1, None) == NULL
    assert P.qrw_probe_copy_qk_traffic(*qk, Q, Q, SC, SC, None, 16, 4, 1, None) == NULL
    assert P.qrw_probe_copy_qk_traffic(ctypes.c_void_p((1 << 32) + 8), W, W, C, S, *kvb, 16, 4,
                                       1, None) == ALIGN
    assert P.qrw_probe_copy_qk_traffic(*qk, ctypes.c_void_p(Q_ADDR + 4), Q, SC, SC, Y, 16, 4, 1,
                                       None) == ALIGN
    assert P.qrw_probe_empty(X, -1, None) == SHAPE
    assert P.qrw_probe_empty(None, 4, None) == NULL
    assert P.qrw_probe_fused_timeline(X, W, C, S, Q, SC, 4, -1.0, Y, None) == VALUE
    assert P.qrw_probe_fused_timeline(X, W, C, S, Q, SC, 4, 1e-6, None, None) == NULL
    assert P.qrw_probe_sweep(3, 1, 2, 1, Y, 1, None) == VALUE
    assert P.qrw_probe_sweep(0, 2, 2, 1, Y, 1, None) == SHAPE
    assert P.qrw_probe_sweep(0, 0, 0x7F800001, 1, Y, 1, None) == SHAPE
    assert P.qrw_probe_sweep(0, 0, 512, 1, Y, 1, None) == SHAPE      # needs 2 blocks
    assert P.qrw_probe_sweep(0, 0, 512, 4097, Y, 1, None) == SHAPE
    assert P.qrw_probe_sweep(0, 0, 512, 1, None, 2, None) == NULL
    assert P.qrw_probe_recip_values(X, Y, W, -1, None) == SHAPE
    assert P.qrw_probe_recip_values(X, Y, W, 0, None) == OK


def test_status_strings():
    L = qrw.load()
    for code in (OK, NULL, DTYPE, SHAPE, STRIDE, ALIGN, ALIAS, LAUNCH, VALUE):
        s = L.qrw_status_string(code).decode()
        assert s and s != "unknown status"
    assert L.qrw_status_string(-99).decode() == "unknown status"


def rms(**kw):
    a = dict(x=X, w=W, y=Y, rows=4, n=64, xs=64, ys=64, dtype=BF16, eps=1e-6)
    a.update(kw)
    return qrw.load().rmsnorm_fwd(a["x"], a["w"], a["y"], a["rows"], a["n"], a["xs"], a["ys"],
                                  a["dtype"], a["eps"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL), (dict(y=None), NULL),
    (dict(dtype=F32), DTYPE), (dict(dtype=0), DTYPE), (dict(dtype=7), DTYPE),
    (dict(n=0), SHAPE), (dict(n=(1 << 26) + 1, xs=(1 << 26) + 8, ys=(1 << 26) + 8), SHAPE),
    (dict(rows=-1), SHAPE), (dict(n=8200), STRIDE),
    (dict(rows=1 << 31, n=8200, xs=8200, ys=8200), SHAPE),   # one workgroup per long row
    (dict(xs=56), STRIDE), (dict(ys=60, n=56), STRIDE), (dict(xs=68), STRIDE),
    (dict(x=ctypes.c_void_p((1 << 32) + 8)), ALIGN), (dict(y=ctypes.c_void_p((2 << 32) + 4)), ALIGN),
    (dict(w=ctypes.c_void_p((3 << 32) + 2)), ALIGN),
    (dict(eps=-1e-6), VALUE), (dict(eps=float("nan")), VALUE), (dict(eps=float("inf")), VALUE),
    (dict(y=ctypes.c_void_p((1 << 32) + 64)), ALIAS),          # partial overlap with x
    (dict(y=X, ys=72), ALIAS),                                  # same base, other stride
    (dict(w=ctypes.c_void_p((2 << 32) + 32)), ALIAS),           # weight inside the output
    (dict(rows=0), OK),                                         # empty: nothing launched
    (dict(rows=0, x=None, y=None, w=None), OK),                 # empty tensors may have no storage
    (dict(rows=0, dtype=F32), DTYPE),                           # but still a valid call
    (dict(xs=1 << 54), STRIDE), (dict(ys=1 << 60), STRIDE),     # rows spanning > 2^56 bytes
])
def test_rmsnorm_validation(kw, want):
    assert rms(**kw) == want


def ln(**kw):
    a = dict(x=X, g=W, b=C, y=Y, rows=4, n=64, xs=64, ys=64, dtype=F16, eps=1e-5)
    a.update(kw)
    return qrw.load().layernorm_fwd(a["x"], a["g"], a["b"], a["y"], a["rows"], a["n"], a["xs"],
                                    a["ys"], a["dtype"], a["eps"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL), (dict(dtype=F32), DTYPE), (dict(n=0), SHAPE),
    (dict(n=65537, xs=65544, ys=65544), SHAPE),                 # no two-pass LayerNorm
    (dict(xs=32), STRIDE), (dict(n=13, xs=13, ys=16), STRIDE),
    (dict(b=ctypes.c_void_p((4 << 32) + 8)), ALIGN), (dict(eps=-1.0), VALUE),
    (dict(y=ctypes.c_void_p((1 << 32) + 16)), ALIAS), (dict(rows=0), OK),
    (dict(xs=1 << 58), STRIDE),
])
def test_layernorm_validation(kw, want):
    assert ln(**kw) == want


def rope(neox=True, **kw):
    a = dict(x=X, c=C, s=S, y=Y, T=4, H=2, D=64, R=64, xs=128, ys=128, dtype=F16, cs=F32)
    a.update(kw)
    fn = qrw.load().rope_apply_neox if neox else qrw.load().rope_apply_interleaved
    return fn(a["x"], a["c"], a["s"], a["y"], a["T"], a["H"], a["D"], a["R"], a["xs"], a["ys"],
              a["dtype"], a["cs"], None)


@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("kw,want", [
    (dict(c=None), NULL), (dict(s=None), NULL),
    (dict(cs=BF16), DTYPE), (dict(dtype=F32), DTYPE),
    (dict(R=8), SHAPE), (dict(R=24), SHAPE), (dict(R=80), SHAPE), (dict(D=60, R=16), SHAPE),
    (dict(H=0), SHAPE), (dict(T=-2), SHAPE), (dict(H=200, D=64), SHAPE),
    (dict(xs=120), STRIDE), (dict(ys=130), STRIDE),
    (dict(c=ctypes.c_void_p((4 << 32) + 4)), ALIGN),
    (dict(y=ctypes.c_void_p((1 << 32) + 128)), ALIAS),
    (dict(c=ctypes.c_void_p((2 << 32) + 64)), ALIAS),
    (dict(T=0), OK), (dict(T=0, x=None, y=None, c=None, s=None), OK),
    (dict(xs=1 << 58), STRIDE), (dict(ys=1 << 62), STRIDE),
])
def test_rope_validation(neox, kw, want):
    assert rope(neox, **kw) == want


def fused(**kw):
    a = dict(x=X, w=W, c=C, s=S, q=Q, sc=SC, T=4, H=32, D=128, R=128, xs=4096, qs=4096,
             dtype=BF16, cs=BF16, neox=1, eps=1e-6)
    a.update(kw)
    return qrw.load().rmsnorm_rope_fp8_fwd(a["x"], a["w"], a["c"], a["s"], a["q"], a["sc"],
                                           a["T"], a["H"], a["D"], a["R"], a["xs"], a["qs"],
                                           a["dtype"], a["cs"], a["neox"], a["eps"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL), (dict(q=None), NULL), (dict(sc=None), NULL), (dict(c=None), NULL),
    (dict(dtype=F32), DTYPE), (dict(cs=F16), DTYPE),
    (dict(H=65), SHAPE), (dict(R=136), SHAPE), (dict(R=0), SHAPE),
    (dict(xs=4000), STRIDE), (dict(qs=4100), STRIDE),
    (dict(q=ctypes.c_void_p((5 << 32) + 8)), ALIGN), (dict(sc=ctypes.c_void_p((6 << 32) + 2)), ALIGN),
    (dict(eps=float("-inf")), VALUE), (dict(neox=2), VALUE),
    (dict(sc=ctypes.c_void_p(Q_ADDR + 64)), ALIAS),      # scales inside the codes
    (dict(q=ctypes.c_void_p((1 << 32) + 4096)), ALIAS),  # codes inside x
    (dict(T=0), OK), (dict(T=0, x=None, q=None, sc=None, c=None, s=None), OK),
    (dict(T=0, R=24), SHAPE),
    (dict(xs=1 << 58), STRIDE), (dict(qs=1 << 58), STRIDE),
])
def test_fused_validation(kw, want):
    assert fused(**kw) == want


def aq(**kw):
    a = dict(x=X, q=Q, sc=SC, rows=4, n=4096, group=128, xs=4096, qs=4096, dtype=BF16)
    a.update(kw)
    return qrw.load().act_quant_fp8_fwd(a["x"], a["q"], a["sc"], a["rows"], a["n"], a["group"],
                                        a["xs"], a["qs"], a["dtype"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL), (dict(q=None), NULL), (dict(sc=None), NULL),
    (dict(dtype=F32), DTYPE),
    (dict(group=96), SHAPE), (dict(group=1024), SHAPE), (dict(group=4), SHAPE),
    (dict(n=1000, xs=1000, qs=1000, group=128), SHAPE), (dict(n=8200), SHAPE),
    (dict(n=65544, xs=65544, qs=65544, group=8), SHAPE),          # longer than 65536
    (dict(n=16384, xs=16384, qs=16384, rows=0x7FFFFFFF // 8 + 1), SHAPE),  # long rows: grid
    (dict(xs=4088), STRIDE), (dict(qs=4100), STRIDE),
    (dict(q=ctypes.c_void_p((5 << 32) + 8)), ALIGN), (dict(sc=ctypes.c_void_p((6 << 32) + 2)), ALIGN),
    (dict(sc=ctypes.c_void_p(Q_ADDR + 64)), ALIAS),      # scales inside the codes
    (dict(q=ctypes.c_void_p((1 << 32) + 256)), ALIAS),   # codes inside x
    (dict(rows=0), OK), (dict(rows=0, x=None, q=None, sc=None), OK),
    (dict(xs=1 << 58), STRIDE), (dict(qs=1 << 58), STRIDE),
])
def test_act_quant_validation(kw, want):
    assert aq(**kw) == want


def qk(**kw):
    a = dict(x=X, wq=W, wk=Y, c=C, s=S, T=4, Hq=32, Hkv=8, D=128, R=128, xs=6144,
             dtype=BF16, cs=BF16, neox=1, eps=1e-6)
    a.update(kw)
    return qrw.load().qk_norm_rope_fwd(a["x"], a["wq"], a["wk"], a["c"], a["s"], a["T"],
                                       a["Hq"], a["Hkv"], a["D"], a["R"], a["xs"], a["dtype"],
                                       a["cs"], a["neox"], a["eps"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL), (dict(c=None), NULL), (dict(s=None), NULL),
    (dict(dtype=F32), DTYPE), (dict(cs=F16), DTYPE),
    (dict(D=96, xs=4608), SHAPE), (dict(D=512, xs=24576), SHAPE), (dict(R=8), SHAPE),
    (dict(R=96), SHAPE), (dict(R=256), SHAPE), (dict(Hq=0), SHAPE), (dict(Hkv=-1), SHAPE),
    (dict(xs=6136), STRIDE), (dict(xs=6148), STRIDE),
    (dict(x=ctypes.c_void_p((1 << 32) + 8)), ALIGN), (dict(wk=ctypes.c_void_p((2 << 32) + 4)), ALIGN),
    (dict(eps=float("nan")), VALUE), (dict(neox=-1), VALUE),
    (dict(c=ctypes.c_void_p((1 << 32) + 1024)), ALIAS),   # table inside the q/k columns
    (dict(wq=ctypes.c_void_p((1 << 32) + 12288)), ALIAS),  # weight inside row 1
    (dict(T=0), OK), (dict(T=0, x=None, c=None, s=None), OK),
    (dict(T=0, R=24), SHAPE),
    (dict(xs=1 << 58), STRIDE),
])
def test_qk_norm_rope_validation(kw, want):
    assert qk(**kw) == want


KC, VC, KS, VS, SL = (ctypes.c_void_p(a << 32) for a in range(8, 13))


def qkv_cache(**kw):
    a = dict(x=X, wq=W, wk=Y, c=C, s=S, kc=KC, vc=VC, ks=KS, vs=VS, sl=SL, ns=64, T=4, Hq=32,
             Hkv=8, D=128, R=128, xs=6144, cst=1024, dtype=BF16, cs=BF16, neox=1, eps=1e-6)
    a.update(kw)
    return qrw.load().qk_norm_rope_fp8_kv_fwd(
        a["x"], a["wq"], a["wk"], a["c"], a["s"], a["kc"], a["vc"], a["ks"], a["vs"], a["sl"],
        a["ns"], a["T"], a["Hq"], a["Hkv"], a["D"], a["R"], a["xs"], a["cst"], a["dtype"],
        a["cs"], a["neox"], a["eps"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL), (dict(kc=None), NULL), (dict(vs=None), NULL), (dict(c=None), NULL),
    (dict(dtype=F32), DTYPE), (dict(cs=F16), DTYPE),
    (dict(Hkv=0, xs=4096), SHAPE), (dict(D=96, xs=4608), SHAPE), (dict(R=8), SHAPE),
    (dict(ns=-1), SHAPE), (dict(sl=None, ns=3), SHAPE),
    (dict(xs=6136), STRIDE), (dict(cst=1000), STRIDE), (dict(cst=1028), STRIDE),
    (dict(kc=ctypes.c_void_p((8 << 32) + 8)), ALIGN), (dict(ks=ctypes.c_void_p((10 << 32) + 2)), ALIGN),
    (dict(sl=ctypes.c_void_p((12 << 32) + 4)), ALIGN),
    (dict(eps=-1.0), VALUE), (dict(neox=3), VALUE),
    (dict(vc=ctypes.c_void_p((8 << 32) + 4096)), ALIAS),     # v cache inside the k cache
    (dict(ks=ctypes.c_void_p((1 << 32) + 64)), ALIAS),       # scales inside qkv
    (dict(vs=ctypes.c_void_p((10 << 32) + 16)), ALIAS),      # v scales inside k scales
    (dict(sl=ctypes.c_void_p((9 << 32) + 256)), ALIAS),      # slots inside the v cache
    (dict(c=ctypes.c_void_p((8 << 32) + 1024)), ALIAS),      # table inside the k cache
    (dict(T=0), OK), (dict(T=0, x=None, kc=None, vc=None, ks=None, vs=None, sl=None, ns=0), OK),
    (dict(T=0, R=24), SHAPE),
    (dict(xs=1 << 58), STRIDE), (dict(cst=1 << 58), STRIDE), (dict(ns=1 << 50), STRIDE),
])
def test_qk_kv_cache_validation(kw, want):
    assert qkv_cache(**kw) == want


@pytest.mark.parametrize("call,want", [
    (lambda L: L.ew_add_fwd(X, None, Y, 16, BF16, None), NULL),
    (lambda L: L.ew_add_fwd(None, W, Y, 16, BF16, None), NULL),
    (lambda L: L.ew_add_fwd(X, W, Y, 16, 4, None), DTYPE),
    (lambda L: L.ew_add_fwd(X, W, Y, -1, BF16, None), SHAPE),
    (lambda L: L.ew_add_fwd(X, W, Y, (1 << 40) + 1, BF16, None), SHAPE),
    (lambda L: L.ew_add_fwd(X, W, ctypes.c_void_p((2 << 32) + 8), 16, BF16, None), ALIGN),
    (lambda L: L.ew_add_fwd(X, W, ctypes.c_void_p((1 << 32) + 16), 16, BF16, None), ALIAS),
    (lambda L: L.ew_add_fwd(X, W, Y, 0, BF16, None), OK),
    (lambda L: L.ew_add_fwd(None, None, None, 0, BF16, None), OK),
    (lambda L: L.ew_scale_cast_fwd(X, Y, 16, 0.5, F32, 0, None), DTYPE),
    (lambda L: L.ew_scale_cast_fwd(X, None, 16, 0.5, F32, F16, None), NULL),
    (lambda L: L.ew_scale_cast_fwd(X, X, 16, 0.5, F32, F16, None), ALIAS),  # in place needs one dtype
    (lambda L: L.ew_scale_cast_fwd(X, ctypes.c_void_p((1 << 32) + 32), 64, 0.5, F16, F16, None), ALIAS),
    (lambda L: L.ew_scale_add_fwd(X, None, Y, 16, 0.5, F32, None), NULL),
    (lambda L: L.ew_scale_add_fwd(X, ctypes.c_void_p((3 << 32) + 4), Y, 16, 0.5, F32, None), ALIGN),
    (lambda L: L.ew_scale_add_fwd(X, ctypes.c_void_p((2 << 32) + 16), Y, 64, 0.5, F32, None), ALIAS),
])
def test_elementwise_validation(call, want):
    assert call(qrw.load()) == want


def test_staged_fused_validates_like_the_exact_one():
    L = qrw.load()
    args = [X, W, C, S, Q, SC, 4, 32, 128, 128, 4096, 4096, BF16, BF16, 1, 1e-6, None]
    for i, bad, want in [(0, None, NULL), (12, F32, DTYPE), (8, 100, SHAPE), (10, 4000, STRIDE),
                         (14, 2, VALUE), (4, ctypes.c_void_p((1 << 32) + 4096), ALIAS), (6, 0, OK)]:
        a = list(args)
        a[i] = bad
        assert L.rmsnorm_rope_fp8_rounded_fwd(*a) == want == L.rmsnorm_rope_fp8_fwd(*a), i
