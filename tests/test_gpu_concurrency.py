"""The library keeps no mutable global state, so independent calls may run
concurrently: on several streams from one host thread, and from several host
threads at once (ctypes releases the interpreter lock during each call, so
the threads are inside the C ABI together).  Each operator works on its own
buffers on its own stream (default priority); every output must equal, bit
for bit, the output of the same calls made one after another."""
import threading

import pytest
import torch

import quant_row_workgroup_amd as qrw
from quant_row_workgroup_amd import synth
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu

ITERS = 12


def _jobs():
    """(name, run, outputs) triples; run() launches on the current stream.
    Inputs are never written, except the in-place QK job's, which is restored
    from a pristine copy on the same stream first."""
    jobs = []
    T, H, D = 512, 32, 128
    x = dev(synth.normal(1, (T, H * D), 0.0, 3.0, "bf16", outlier_frac=0.01, outlier_mul=10.0),
            "bf16")
    w = dev(synth.normal(2, (H * D,), 1.0, 0.1, "bf16"), "bf16")
    c, s = (dev(a, "bf16") for a in synth.rope_table(T, D, "bf16"))
    q = torch.empty((T, H * D), dtype=torch.uint8, device="cuda")
    sc = torch.empty(T, dtype=torch.float32, device="cuda")

    jobs.append(("fused", lambda: qrw.rmsnorm_rope_fp8_fwd(x, w, c, s, H, D, D, neox=True,
                                                           eps=1e-6, q=q, scales=sc), [q, sc]))

    xn = dev(synth.normal(3, (1024, 4096), 0.0, 1.0, "f16"), "f16")
    wn = dev(synth.normal(4, (4096,), 1.0, 0.1, "f16"), "f16")
    yn = torch.empty_like(xn)
    jobs.append(("rmsnorm", lambda: qrw.rmsnorm_fwd(xn, wn, 1e-6, out=yn), [yn]))

    xl = dev(synth.normal(5, (1024, 4096), 0.5, 2.0, "bf16"), "bf16")
    g = dev(synth.normal(6, (4096,), 1.0, 0.1, "bf16"), "bf16")
    b = dev(synth.normal(7, (4096,), 0.0, 0.1, "bf16"), "bf16")
    yl = torch.empty_like(xl)
    jobs.append(("layernorm", lambda: qrw.layernorm_fwd(xl, g, b, 1e-5, out=yl), [yl]))

    xr = dev(synth.normal(8, (T, H * D), 0.0, 1.0, "f16"), "f16")
    cr, sr = (dev(a, "f32") for a in synth.rope_table(T, D, "f32"))
    yr = torch.empty_like(xr)
    jobs.append(("rope", lambda: qrw.rope_apply_interleaved(xr, cr, sr, H, D, D, out=yr), [yr]))

    xa = dev(synth.normal(9, (T, 4096), 0.0, 1.0, "bf16", outlier_frac=0.01, outlier_mul=20.0),
             "bf16")
    qa = torch.empty((T, 4096), dtype=torch.uint8, device="cuda")
    sa = torch.empty((T, 32), dtype=torch.float32, device="cuda")

    jobs.append(("act_quant", lambda: qrw.act_quant_fp8_fwd(xa, 128, q=qa, scales=sa), [qa, sa]))

    Hq, Hk = 32, 8
    pristine = dev(synth.normal(10, (T, (Hq + 2 * Hk) * D), 0.0, 2.0, "bf16"), "bf16")
    qkv = torch.empty_like(pristine)
    qw = dev(synth.normal(11, (D,), 1.0, 0.2, "bf16"), "bf16")
    kw = dev(synth.normal(12, (D,), 1.0, 0.2, "bf16"), "bf16")

    def qk():
        qkv.copy_(pristine)
        qrw.qk_norm_rope_fwd(qkv, qw, kw, c, s, Hq, Hk, D, D, True, 1e-6)
    jobs.append(("qk_norm_rope", qk, [qkv]))

    xe = dev(synth.normal(13, (1 << 20,), 0.0, 4.0, "bf16"), "bf16")
    be = dev(synth.normal(14, (1 << 20,), 0.0, 4.0, "bf16"), "bf16")
    ye = torch.empty_like(xe)
    jobs.append(("ew_add", lambda: qrw.ew_add_fwd(xe, be, out=ye), [ye]))
    return jobs


def _snapshot(outs):
    return [o.clone() for o in outs]


def _reference(jobs):
    ref = {}
    for name, run, outs in jobs:
        run()
        ref[name] = _snapshot(outs)
    torch.cuda.synchronize()
    # a sentinel in every output, so a call that did not run shows
    for _, _, outs in jobs:
        for o in outs:
            o.fill_(0x5C if o.dtype == torch.uint8 else float("nan"))
    torch.cuda.synchronize()
    return ref


def _check(jobs, ref, got):
    for name, _, _ in jobs:
        assert name in got, name
        for a, b in zip(ref[name], got[name]):
            assert torch.equal(a, b), name


def test_calls_on_several_streams_match_sequential_calls():
    jobs = _jobs()
    ref = _reference(jobs)
    streams = [torch.cuda.Stream() for _ in jobs]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    got = {}
    for it in range(ITERS):
        for (name, run, outs), st in zip(jobs, streams):
            with torch.cuda.stream(st):
                run()
                if it == ITERS - 1:
                    got[name] = _snapshot(outs)
    torch.cuda.synchronize()
    _check(jobs, ref, got)


def test_calls_from_several_host_threads_match_sequential_calls():
    jobs = _jobs()
    ref = _reference(jobs)
    got, errors = {}, []
    start = threading.Barrier(len(jobs))

    def worker(name, run, outs):
        try:
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.default_stream())
            start.wait(timeout=60)
            with torch.cuda.stream(st):
                for _ in range(ITERS):
                    run()
                got[name] = _snapshot(outs)
            st.synchronize()
        except Exception as e:  # reported on the main thread
            errors.append((name, repr(e)))

    threads = [threading.Thread(target=worker, args=j, daemon=True) for j in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    _check(jobs, ref, got)
