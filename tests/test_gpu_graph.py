"""The operators inside a captured HIP graph: one graph holding a copy (by
the library's own elementwise kernel), the in-place QK-norm + RoPE, RMSNorm,
the fused RMSNorm + RoPE + FP8, the per-group FP8 cast and an elementwise
add is replayed several times, with unrelated eager work and
synchronisations between the replays; every replay must reproduce the eager
results bit for bit.  A second graph holds every other entry point (the KV-cache
write, LayerNorm, both RoPE conventions, the staged fused form, scale-add) and
the ragged, row-block, split-K and tail-rotation paths; there, bytes the
operators do not own (cache rows no token maps to, row padding) must keep
their fill.  (No memset node is recorded: the graphs contain only the
library's kernels.)  A third test makes a process's first call of the
pipelined RMSNorm inside a capture."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import quant_row_workgroup_amd as qrw
from quant_row_workgroup_amd import synth
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu


def _inputs():
    T, Hq, Hk, D = 64, 8, 2, 128
    n = (Hq + 2 * Hk) * D
    qkv0 = dev(synth.normal(1, (T, n), 0.0, 1.0, "bf16"), "bf16")
    qw = dev(synth.normal(2, (D,), 1.0, 0.1, "bf16"), "bf16")
    c, s = (dev(t, "bf16") for t in synth.rope_table(T, D, "bf16"))
    x = dev(synth.normal(3, (T, 4096), 0.0, 3.0, "bf16", outlier_frac=0.01, outlier_mul=10.0),
            "bf16")
    w = dev(synth.normal(4, (4096,), 1.0, 0.1, "bf16"), "bf16")
    c2, s2 = (dev(t, "bf16") for t in synth.rope_table(T, 128, "bf16"))
    return dict(T=T, Hq=Hq, Hk=Hk, D=D, qkv0=qkv0, qw=qw, c=c, s=s, x=x, w=w, c2=c2, s2=s2)


def _run(i, o):
    """All operators once; o holds the output buffers (written in place)."""
    qrw.ew_scale_cast_fwd(i["qkv0"], 1.0, out=o["qkv"])          # exact copy
    qrw.qk_norm_rope_fwd(o["qkv"], i["qw"], i["qw"], i["c"], i["s"], i["Hq"], i["Hk"], i["D"])
    qrw.rmsnorm_fwd(i["x"], i["w"], 1e-6, out=o["y"])
    qrw.rmsnorm_rope_fp8_fwd(i["x"], i["w"], i["c2"], i["s2"], 32, 128, q=o["q"],
                             scales=o["sc"])
    qrw.act_quant_fp8_fwd(i["x"], 128, q=o["q2"], scales=o["sc2"])
    qrw.ew_add_fwd(o["y"], i["x"], out=o["z"])


def _outputs(i):
    T = i["T"]
    return dict(qkv=torch.empty_like(i["qkv0"]), y=torch.empty_like(i["x"]),
                q=torch.empty((T, 4096), dtype=torch.uint8, device="cuda"),
                sc=torch.empty((T,), dtype=torch.float32, device="cuda"),
                q2=torch.empty((T, 4096), dtype=torch.uint8, device="cuda"),
                sc2=torch.empty((T, 32), dtype=torch.float32, device="cuda"),
                z=torch.empty_like(i["x"]))


def test_graph_replays_match_eager():
    i = _inputs()
    ref = _outputs(i)
    _run(i, ref)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in ref.items()}

    o = _outputs(i)
    _run(i, o)  # warm-up outside the capture
    torch.cuda.synchronize()
    for v in o.values():
        v.view(torch.uint8).fill_(0xAB)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        _run(i, o)
    torch.cuda.synchronize()
    other = _outputs(i)
    for rep in range(4):
        for v in o.values():
            v.view(torch.uint8).fill_(0x5C)  # the replay must rewrite every byte it owns
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(o[k].view(torch.uint8), ref[k].view(torch.uint8)), (rep, k)
        # unrelated eager work between replays
        _run(i, other)
        torch.matmul(i["x"][:, :128].float(), i["x"][:, :128].float().t())
        torch.cuda.synchronize()


def _inputs_rest():
    T, Hq, Hk, D = 16, 8, 2, 128
    n = (Hq + 2 * Hk) * D
    g = lambda seed, shape, m=0.0, s=1.0: dev(synth.normal(seed, shape, m, s, "bf16"), "bf16")
    ns = 2 * T + 3
    return dict(
        T=T, Hq=Hq, Hk=Hk, D=D, ns=ns,
        qkv0=g(11, (T, n)), qw=g(12, (D,), 1.0, 0.1), kw=g(13, (D,), 1.0, 0.1),
        c=dev(synth.rope_table(T, D, "bf16")[0], "bf16"),
        s=dev(synth.rope_table(T, D, "bf16")[1], "bf16"),
        slots=torch.from_numpy(synth.cache_slots(14, T, ns)).cuda(),
        x=g(15, (T, 4096), 0.0, 3.0), w=g(16, (4096,), 1.0, 0.1), b=g(17, (4096,), 0.0, 0.1),
        xr=g(18, (T, 4096))[:, :4095],                      # ragged rows, stride 4096
        xl=g(19, (3, 40000)), wl=g(20, (40000,), 1.0, 0.1),  # one workgroup per row
        xs=g(21, (2, 131072)), ws=g(22, (131072,), 1.0, 0.1))  # two-pass split-K


def _outputs_rest(i):
    T, e8 = i["T"], lambda shape: torch.empty(shape, dtype=torch.uint8, device="cuda")
    f32 = lambda shape: torch.empty(shape, dtype=torch.float32, device="cuda")
    like = torch.empty_like
    return dict(qkv=like(i["qkv0"]), kc=e8((i["ns"], i["Hk"] * i["D"])),
                vc=e8((i["ns"], i["Hk"] * i["D"])), ks=f32((i["ns"], i["Hk"])),
                vs=f32((i["ns"], i["Hk"])), ln=like(i["x"]), ri=like(i["x"]), rn=like(i["x"]),
                qs=e8((T, 4096)), ss=f32((T,)), qt=e8((T, 4096)), st=f32((T,)),
                sa=like(i["x"]), yr=torch.empty((T, 4096), dtype=torch.bfloat16, device="cuda"),
                yl=like(i["xl"]), ys=like(i["xs"]), lnl=like(i["xl"]))


def _run_rest(i, o):
    """Every entry point the first graph test does not hold, and the ragged,
    row-block, split-K and tail-rotation paths."""
    qrw.ew_scale_cast_fwd(i["qkv0"], 1.0, out=o["qkv"])          # exact copy
    qrw.qk_norm_rope_fp8_kv_fwd(o["qkv"], i["qw"], i["kw"], i["c"], i["s"], o["kc"], o["vc"],
                                o["ks"], o["vs"], i["Hq"], i["Hk"], i["D"], slots=i["slots"])
    qrw.layernorm_fwd(i["x"], i["w"], i["b"], 1e-5, out=o["ln"])
    qrw.rope_apply_interleaved(i["x"], i["c"], i["s"], 32, 128, out=o["ri"])
    qrw.rope_apply_neox(i["x"], i["c"], i["s"], 32, 128, out=o["rn"])
    qrw.rmsnorm_rope_fp8_rounded_fwd(i["x"], i["w"], i["c"], i["s"], 32, 128, q=o["qs"],
                                     scales=o["ss"])
    qrw.rmsnorm_rope_fp8_fwd(i["x"], i["w"], i["c"], i["s"], 1, 4096, 128, q=o["qt"],
                             scales=o["st"])                      # one head, tail rotation
    qrw.ew_scale_add_fwd(i["x"], i["x"], 0.5, out=o["sa"])
    qrw.rmsnorm_fwd(i["xr"], i["w"][:4095], 1e-6, out=o["yr"][:, :4095])
    qrw.rmsnorm_fwd(i["xl"], i["wl"], 1e-6, out=o["yl"])
    qrw.rmsnorm_fwd(i["xs"], i["ws"], 1e-6, out=o["ys"])
    qrw.layernorm_fwd(i["xl"], i["wl"], None, 1e-5, out=o["lnl"])


def test_graph_replays_match_eager_all_entry_points():
    i = _inputs_rest()

    def fill(o):
        for v in o.values():
            v.view(torch.uint8).fill_(0x5C)

    ref = _outputs_rest(i)
    fill(ref)
    _run_rest(i, ref)
    torch.cuda.synchronize()
    o = _outputs_rest(i)
    _run_rest(i, o)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        _run_rest(i, o)
    torch.cuda.synchronize()
    other = _outputs_rest(i)
    for rep in range(4):
        fill(o)  # bytes the replay does not own must stay as filled
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(o[k].view(torch.uint8), ref[k].view(torch.uint8)), (rep, k)
        _run_rest(i, other)  # unrelated eager work between replays
        torch.cuda.synchronize()


_FIRST_CALL = r"""
import hashlib, sys
import torch
sys.path.insert(0, sys.argv[2])
import quant_row_workgroup_amd as qrw
op = sys.argv[3]
rows, n = {"rms_long": (1500, 32768), "ln_long": (1500, 32768), "rms_4096": (4096, 4096)}[op]
g0 = torch.Generator(device="cuda").manual_seed(5)
x = (torch.randn(rows, n, device="cuda", generator=g0) * 2 + 0.3).to(torch.bfloat16)
w = (torch.randn(n, device="cuda", generator=g0) * 0.1 + 1).to(torch.bfloat16)
b = (torch.randn(n, device="cuda", generator=g0) * 0.1).to(torch.bfloat16)
def run(out):
    if op == "ln_long":
        qrw.layernorm_fwd(x, w, b, 1e-5, out=out)
    else:
        qrw.rmsnorm_fwd(x, w, 1e-6, out=out)
y = torch.empty_like(x)
if sys.argv[1] == "graph":
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        run(y)  # this process's first call of the operator
    ref = torch.empty_like(x)
    for rep in range(3):
        y.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        run(ref)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), rep
else:
    run(y)
    torch.cuda.synchronize()
print(hashlib.sha256(y.view(torch.int16).cpu().numpy().tobytes()).hexdigest())
"""


@pytest.mark.parametrize("op", ["rms_long", "ln_long", "rms_4096"])
def test_first_call_inside_a_capture(op):
    # The first call of an operator on a device may query the device: the
    # pipelined norms ask for their occupancy (LayerNorm's also raises its
    # dynamic LDS limit), the one-wave RMSNorm for the CU count.  When that
    # call is being captured, the replays must still give the eager result of
    # a process that never captured, bit for bit.
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = {}
    for mode in ("graph", "eager"):
        print(f"[first call] {op} {mode}", flush=True)
        r = subprocess.run([sys.executable, "-c", _FIRST_CALL, mode, root, op],
                           capture_output=True, text=True, timeout=240)
        assert r.returncode == 0, (mode, r.stderr[-2000:])
        out[mode] = r.stdout.strip().splitlines()[-1]
    assert out["graph"] == out["eager"], out
