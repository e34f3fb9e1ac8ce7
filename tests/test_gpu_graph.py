"""The operators inside a captured HIP graph: one graph holding a copy (by
the library's own elementwise kernel), the in-place QK-norm + RoPE, RMSNorm,
the fused RMSNorm + RoPE + FP8, the per-group FP8 cast and an elementwise
add is replayed several times, with unrelated eager work and
synchronisations between the replays; every replay must reproduce the eager
results bit for bit.  (No memset node is recorded: the graph contains only
the library's kernels.)"""
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
