#!/usr/bin/env python3
"""Benchmark: achieved HBM bandwidth of the fused RMSNorm -> RoPE -> per-token
FP8 row operator on one MI355X (4096 tokens x 4096 channels = 32 heads x 128,
bf16 in, NeoX rotation over every head with bf16 cos/sin [4096, 64],
E4M3FN codes + binary32 per-token scales out).

One step = one launch of the operator over one 4096 x 4096 batch.  The batch
rotates over --sets independent input/output buffer sets (default 8 x 51.4 MB,
more than the 256 MB last-level cache), so every launch reads inputs that sit
in HBM rather than in cache.  The K steps are captured once into a HIP graph,
whose untimed replays run for about 50 ms first (the GPU settles at its
steady clocks); behind them, still queued, the host enqueues a HIP event, the
K launches and a second event on the same stream, and checks that the first
event had not yet fired when it finished, so the timed region holds exactly
K launches back to back, with neither host time nor a graph boundary in it
(see timed_launches).  The events give the average launch duration, and

    achieved GB/s = counted bytes per launch / average launch duration

where counted bytes are the byte-ledger minimum of one launch (every input
read once, every output written once): 51,404,800 B for this workload.

`traffic` reports HBM bytes per launch measured with rocprofv3 counters
(FETCH_SIZE, WRITE_SIZE, scaled by the same counters on a plain copy of known
size) as recorded in profiles/<workload>_traffic.txt, and only while the
kernel sources are the ones those counters were taken on; otherwise null.

`cpu_baseline` times the CPU checker (plain C, float64) on a bounded sample of
the same workload on this host: on one thread per core (at most 16) over
contiguous blocks of rows (`value`, `cores`), and on one thread
(`single_thread_value`).

`copy_ceiling` (fused workloads with rows of 4096 bf16 channels, and the QK
workloads of 32 query and 8 key/value heads of 128 channels; on by default):
the same launches with the operator's arithmetic replaced by byte selection --
the same grid, loads and stores on the same buffers
(qrw_probe_copy_fused_traffic, qrw_probe_copy_qk_traffic) -- i.e. what a
kernel with this access structure reaches at this size, for the fused
operator also its variant without the row dependency, and the same grid doing
nothing (the fixed cost of a launch).

Options: --workload runs any of the named workloads instead, --rows runs it at
another row (token) count, --plain-copy MIB adds `plain_copy`, a bare copy of
that size through the library's elementwise kernel, --timeline L adds
per-wave timestamps of the fused kernel over L consecutive launches, and
--host-cost adds the C ABI's host time per call measured from plain C, and
--trace-summary CSV prints p10/p50/p90 kernel durations of a rocprofv3
kernel-trace file (or per-kernel counter values of a --pmc file).

Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "achieved HBM GB/s (% of MI355X peak), fused RMSNorm+RoPE+FP8 4096x4096"
DEFAULT_WORKLOAD = "rmsnorm_rope_fp8_4096x4096_bf16"


# Source files that define each operator's kernels and their launch.
KERNEL_SOURCES = {
    "rmsnorm": ("qrw_norm.hip", "qrw_device.h", "qrw_launch.h"),
    "layernorm": ("qrw_norm.hip", "qrw_device.h", "qrw_launch.h"),
    "rope": ("qrw_rope.hip", "qrw_rope_contig.hip", "qrw_contig.h", "qrw_plan.h", "qrw_device.h",
             "qrw_launch.h"),
    "fused": ("qrw_rope.hip", "qrw_fused_contig.h", "qrw_fused_contig_bf16.hip",
              "qrw_fused_contig_f16.hip", "qrw_fused_tail.hip", "qrw_fused_tail.h",
              "qrw_fused_tail_bf16.hip", "qrw_fused_tail_f16.hip", "qrw_contig.h", "qrw_plan.h",
              "qrw_device.h", "qrw_launch.h"),
    "act_quant": ("qrw_quant.hip", "qrw_device.h", "qrw_launch.h"),
    "qk_norm_rope": ("qrw_qknorm.hip", "qrw_qknorm.h", "qrw_qknorm_gc_a.hip",
                     "qrw_qknorm_gc_b.hip", "qrw_qknorm_gc_c.hip", "qrw_device.h", "qrw_launch.h"),
    "qk_kv": ("qrw_qknorm.hip", "qrw_qknorm.h", "qrw_qknorm_gc_a.hip", "qrw_qknorm_gc_b.hip",
              "qrw_qknorm_gc_c.hip", "qrw_device.h", "qrw_launch.h"),
    "ew": ("qrw_ew.hip", "qrw_device.h", "qrw_launch.h"),
}


def kernel_source_hash(op: str = "fused") -> str:
    """sha256 (first 16 hex digits) of the sources of one operator's kernels."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[op]:
        h.update(name.encode())
        with open(os.path.join(ROOT, "quant_row_workgroup_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, src_hash: str):
    """HBM bytes per launch from the committed counter summary of this workload, if
    it was taken on the current kernel sources (``key: value`` lines at its end)."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("workload") != workload or rec.get("kernel_src_hash") != src_hash:
        return None
    try:
        return int(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


# ---------------------------------------------------------------- GPU side
class Workload:
    """Device buffers for `sets` independent batches and one raw C-ABI call per step."""

    def __init__(self, name: str, sets: int):
        import numpy as np
        import torch

        import quant_row_workgroup_amd as qrw
        from quant_row_workgroup_amd import ledger, synth

        self.name = name
        self.cfg = dict(synth.WORKLOADS[name])
        self.inp = synth.make_inputs(name)
        self.counted = ledger.counted_bytes(self.cfg)
        self.lib = qrw.load()
        dev = torch.device("cuda:0")
        tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}

        def up(bits, dt):
            if bits.dtype == np.int64:
                return torch.from_numpy(np.ascontiguousarray(bits)).to(dev)
            if dt == "f32":
                return torch.from_numpy(np.ascontiguousarray(bits)).to(dev)
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt[dt]).to(dev)

        op = self.cfg["op"]
        dt = self.cfg["dtype"]
        code = {"f16": 1, "bf16": 2, "f32": 3}
        base = {k: up(v, self.cfg.get("cs_dtype", dt) if k in ("cos", "sin") else dt)
                for k, v in self.inp.items()
                if k in ("x", "b", "w", "gamma", "beta", "cos", "sin", "q_weight", "k_weight",
                         "slots")}
        if op in ("rmsnorm", "layernorm") and self.cfg["n"] % 8:
            # rows stored padded to a multiple of 8 elements (16-byte aligned rows)
            n = self.cfg["n"]
            wide = torch.zeros((self.cfg["rows"], (n + 7) // 8 * 8), dtype=base["x"].dtype,
                               device=dev)
            wide[:, :n] = base["x"]
            base["x"] = wide
        self.sets = []
        for _ in range(sets):
            s = {k: v.clone() for k, v in base.items()}
            if op == "act_quant":
                R, n = self.cfg["rows"], self.cfg["n"]
                g = self.cfg.get("group") or n
                s["q"] = torch.empty((R, n), dtype=torch.uint8, device=dev)
                s["scales"] = torch.empty((R, n // g), dtype=torch.float32, device=dev)
            elif op == "fused":
                T = self.cfg["tokens"]
                n = self.cfg["heads"] * self.cfg["head_dim"]
                s["q"] = torch.empty((T, n), dtype=torch.uint8, device=dev)
                s["scales"] = torch.empty((T,), dtype=torch.float32, device=dev)
            elif op == "ew":
                yd = self.cfg.get("y_dtype", dt)
                s["y"] = torch.empty(s["x"].shape, dtype=tdt[yd], device=dev)
            elif op == "qk_kv":
                ns, kvn = self.cfg["num_slots"], self.cfg["kv_heads"] * self.cfg["head_dim"]
                for k in ("k_cache", "v_cache"):
                    s[k] = torch.zeros((ns, kvn), dtype=torch.uint8, device=dev)
                for k in ("k_scales", "v_scales"):
                    s[k] = torch.zeros((ns, self.cfg["kv_heads"]), dtype=torch.float32,
                                       device=dev)
            elif op != "qk_norm_rope":  # qk_norm_rope works in place on x
                s["y"] = torch.empty_like(s["x"])
            self.sets.append(s)
        self.op = op
        self.code = code
        self.pristine = base["x"]
        torch.cuda.synchronize()

    def reset(self) -> None:
        """Restore the inputs an in-place operator overwrote."""
        if self.op in ("qk_norm_rope", "qk_kv"):
            for s in self.sets:
                s["x"].copy_(self.pristine)

    def launch(self, i: int, stream_ptr: int) -> None:
        s = self.sets[i % len(self.sets)]
        c = self.cfg
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        st = ctypes.c_void_p(stream_ptr)
        if self.op == "fused":
            T, H, D, R = c["tokens"], c["heads"], c["head_dim"], c["rope_dim"]
            fn = (self.lib.rmsnorm_rope_fp8_rounded_fwd if c.get("staged")
                  else self.lib.rmsnorm_rope_fp8_fwd)
            rc = fn(p(s["x"]), p(s["w"]), p(s["cos"]), p(s["sin"]), p(s["q"]), p(s["scales"]),
                    T, H, D, R, H * D, H * D, self.code[c["dtype"]], self.code[c["cs_dtype"]],
                    int(c["neox"]), c["eps"], st)
        elif self.op == "qk_norm_rope":
            T, D = c["tokens"], c["head_dim"]
            n = (c["q_heads"] + 2 * c["kv_heads"]) * D
            rc = self.lib.qk_norm_rope_fwd(p(s["x"]), p(s["q_weight"]), p(s["k_weight"]),
                                           p(s["cos"]), p(s["sin"]), T, c["q_heads"],
                                           c["kv_heads"], D, c["rope_dim"], n,
                                           self.code[c["dtype"]], self.code[c["cs_dtype"]],
                                           int(c["neox"]), c["eps"], st)
        elif self.op == "ew":
            n = c["n"]
            if c["kind"] == "add":
                rc = self.lib.ew_add_fwd(p(s["x"]), p(s["b"]), p(s["y"]), n,
                                         self.code[c["dtype"]], st)
            elif c["kind"] == "scale_add":
                rc = self.lib.ew_scale_add_fwd(p(s["x"]), p(s["b"]), p(s["y"]), n, c["alpha"],
                                               self.code[c["dtype"]], st)
            else:
                rc = self.lib.ew_scale_cast_fwd(p(s["x"]), p(s["y"]), n, c["alpha"],
                                                self.code[c["dtype"]],
                                                self.code[c.get("y_dtype", c["dtype"])], st)
        elif self.op == "qk_kv":
            T, D = c["tokens"], c["head_dim"]
            n = (c["q_heads"] + 2 * c["kv_heads"]) * D
            rc = self.lib.qk_norm_rope_fp8_kv_fwd(
                p(s["x"]), p(s["q_weight"]), p(s["k_weight"]), p(s["cos"]), p(s["sin"]),
                p(s["k_cache"]), p(s["v_cache"]), p(s["k_scales"]), p(s["v_scales"]),
                p(s["slots"]), c["num_slots"], T, c["q_heads"], c["kv_heads"], D, c["rope_dim"],
                n, c["kv_heads"] * D, self.code[c["dtype"]], self.code[c["cs_dtype"]],
                int(c["neox"]), c["eps"], st)
        elif self.op == "act_quant":
            g = c.get("group") or c["n"]
            rc = self.lib.act_quant_fp8_fwd(p(s["x"]), p(s["q"]), p(s["scales"]), c["rows"],
                                            c["n"], g, c["n"], c["n"], self.code[c["dtype"]], st)
        elif self.op == "rmsnorm":
            rc = self.lib.rmsnorm_fwd(p(s["x"]), p(s["w"]), p(s["y"]), c["rows"], c["n"],
                                      s["x"].stride(0), s["y"].stride(0), self.code[c["dtype"]],
                                      c["eps"], st)
        elif self.op == "layernorm":
            rc = self.lib.layernorm_fwd(p(s["x"]), p(s["gamma"]), p(s["beta"]), p(s["y"]),
                                        c["rows"], c["n"], s["x"].stride(0), s["y"].stride(0),
                                        self.code[c["dtype"]], c["eps"], st)
        else:
            T, H, D, R = c["tokens"], c["heads"], c["head_dim"], c["rope_dim"]
            fn = self.lib.rope_apply_neox if c.get("neox", True) else self.lib.rope_apply_interleaved
            rc = fn(p(s["x"]), p(s["cos"]), p(s["sin"]), p(s["y"]), T, H, D, R, H * D, H * D,
                    self.code[c["dtype"]], self.code[c["cs_dtype"]], st)
        if rc != 0:
            raise RuntimeError(f"{self.name}: launch returned status {rc}")

    def outputs(self, i: int):
        s = self.sets[i % len(self.sets)]
        keys = {"qk_norm_rope": ("x",),
                "qk_kv": ("x", "k_cache", "v_cache", "k_scales", "v_scales")}.get(
                    self.op, ("q", "scales", "y"))
        return [s[k].clone() for k in keys if k in s]


def time_gpu(wl: Workload, steps: int, warmup: int, mode: str):
    """Milliseconds per step of the workload (see timed_launches); first checks
    that a graph replay of the steps gives the same outputs as the same launches
    made eagerly, bit for bit (from the same starting inputs, since an in-place
    operator consumes them), since the backlog is made of graph replays."""
    import torch

    cur = torch.cuda.current_stream()
    for i in range(warmup):
        wl.launch(i, cur.cuda_stream)
    torch.cuda.synchronize()
    g = capture(wl.launch, steps)
    wl.reset()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    ref = wl.outputs(steps - 1)
    wl.reset()
    for i in range(steps):
        wl.launch(i, cur.cuda_stream)
    torch.cuda.synchronize()
    for a, b in zip(ref, wl.outputs(steps - 1)):
        if not torch.equal(a, b):
            raise RuntimeError("graph replay differs from eager launches")
    return timed_launches(wl.launch, steps, 0, mode, graph=g)


# ---------------------------------------------------------------- CPU side
def compute_dtype(cfg: dict) -> str:
    """The arithmetic type of the kernel: binary32, except the elementwise family's
    16-bit outputs, which are formed in binary64 (a plain sum of two 16-bit
    values, alpha == 1, stays binary32)."""
    if cfg["op"] == "ew" and cfg.get("y_dtype", cfg["dtype"]) != "f32":
        plain_sum = cfg.get("kind") == "add" or (cfg.get("kind") == "scale_add"
                                                 and cfg.get("alpha") == 1.0)
        return "f32" if plain_sum and cfg["dtype"] != "f32" else "f64"
    return "f32"


SETTLE_MS = 50.0


def settle(g, ms: float = None) -> None:
    """Replay graph ``g`` untimed for about ``ms`` (default SETTLE_MS) of GPU
    time and return while those replays are still queued: the GPU reaches its
    steady clocks before a timed region (a short run otherwise times part of
    the ramp), and the host can enqueue the timed work behind them."""
    import torch

    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    b.synchronize()
    per = max(a.elapsed_time(b), 1e-3)
    for _ in range(max(1, min(4000, int((ms or SETTLE_MS) / per) + 1))):
        g.replay()


def capture(launch, steps: int):
    """A HIP graph of ``launch(i, stream_ptr)`` for i = 0 .. steps-1."""
    import torch

    cur = torch.cuda.current_stream()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(cur)
    with torch.cuda.graph(g, stream=cap):
        sp = torch.cuda.current_stream().cuda_stream
        for i in range(steps):
            launch(i, sp)
    torch.cuda.synchronize()
    return g


# How the last timed region was measured (reported in the JSON line).
TIMING = {}


def timed_launches(launch, steps: int, warmup: int = 3, mode: str = "stream", graph=None):
    """Milliseconds per launch of ``launch(i, stream_ptr)``, i = 0 .. steps-1,
    between two HIP events on the launch stream.

    mode "stream" (the default): the graph of the same launches is replayed
    untimed for about SETTLE_MS of GPU time, then the start event and the
    `steps` launches are enqueued directly on the stream behind that backlog,
    then the end event.  If the start event is still pending once the host has
    enqueued everything, every timed launch was queued before the first one
    ran, so the region holds the launches back to back with no host time in
    it.  Otherwise (a kernel shorter than the host's launch cost outran a
    too-short backlog) the backlog is doubled, twice at most, and then the
    graph mode is used.

    mode "graph": the same backlog, then the launches as one graph replay.  A
    replay carries a fixed cost of its own on the GPU (about 4 us on MI355X),
    part of the region.

    mode "eager": the launches enqueued from an idle GPU (the host's launch
    cost is part of the region whenever it exceeds the kernel's)."""
    import torch

    cur = torch.cuda.current_stream()
    for i in range(warmup):
        launch(i, cur.cuda_stream)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if mode == "eager":
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            launch(i, cur.cuda_stream)
        end.record()
        end.synchronize()
        TIMING.update(mode="eager", ahead=None)
        return start.elapsed_time(end) / steps
    g = graph if graph is not None else capture(launch, steps)
    if mode == "stream":
        for attempt in range(3):
            settle(g, SETTLE_MS * 2 ** attempt)
            start.record()
            for i in range(steps):
                launch(i, cur.cuda_stream)
            end.record()
            ahead = not start.query()
            end.synchronize()
            torch.cuda.synchronize()
            if ahead:
                TIMING.update(mode="stream", ahead=True, backlog_ms=SETTLE_MS * 2 ** attempt)
                return start.elapsed_time(end) / steps
    settle(g)
    start.record()
    g.replay()
    end.record()
    end.synchronize()
    torch.cuda.synchronize()
    TIMING.update(mode="graph", ahead=None if mode == "graph" else False)
    return start.elapsed_time(end) / steps


def plain_copy(mib: int, sets: int, steps: int = 50):
    """A plain device copy of ``mib`` MiB (f32, y = x * 1) through the library's
    elementwise kernel, over ``sets`` rotating buffer pairs and timed like the
    workload: what a bare 16-byte-per-lane copy of that size reaches here."""
    import torch

    import quant_row_workgroup_amd as qrw

    lib = qrw.load()
    n = (mib << 20) // 4
    xs = [torch.empty(n, dtype=torch.float32, device="cuda").uniform_() for _ in range(sets)]
    ys = [torch.empty_like(x) for x in xs]

    def go(i, sp):
        rc = lib.ew_scale_cast_fwd(ctypes.c_void_p(xs[i % sets].data_ptr()),
                                   ctypes.c_void_p(ys[i % sets].data_ptr()), n, 1.0, 3, 3,
                                   ctypes.c_void_p(sp))
        if rc != 0:
            raise RuntimeError(f"ew_scale_cast_fwd failed: {rc}")

    ms = timed_launches(go, steps)
    torch.cuda.synchronize()
    if not torch.equal(ys[(steps - 1) % sets], xs[(steps - 1) % sets]):
        raise RuntimeError("copy through the elementwise kernel is not exact")
    us = ms * 1e3
    moved = 2 * n * 4
    print(f"[bench] plain copy: {mib} MiB in {us:.2f} us, {moved / us / 1e3:.1f} GB/s",
          file=sys.stderr, flush=True)
    return {"mib": mib, "us_per_copy": round(us, 3), "GB/s": round(moved / us / 1e3, 1),
            "frac": round(moved / us / 1e3 / PEAK_HBM_GBS, 4),
            "kernel": "ew_scale_cast_fwd f32 -> f32, alpha 1 (16 B per lane)"}


def fused_probe_shape(cfg: dict) -> bool:
    """The probes reproduce the fused operator's benchmark layout only: rows of
    4096 bf16 channels in 32 heads of 128 rotating whole (NeoX), bf16 tables."""
    return (cfg["op"] == "fused" and cfg["heads"] * cfg["head_dim"] == 4096
            and cfg["head_dim"] == 128 and cfg["rope_dim"] == 128 and cfg["dtype"] == "bf16"
            and cfg["cs_dtype"] == "bf16" and cfg["neox"] and not cfg.get("staged"))


def qk_probe_shape(cfg: dict) -> bool:
    """The QK probe reproduces the QK operators' benchmark layout only: 32 query
    heads and 8 key/value heads of 128 16-bit channels, NeoX over the whole head."""
    return (cfg["op"] in ("qk_norm_rope", "qk_kv") and cfg["q_heads"] == 32
            and cfg["kv_heads"] == 8 and cfg["head_dim"] == 128 and cfg["rope_dim"] == 128
            and cfg["dtype"] in ("bf16", "f16") and cfg["cs_dtype"] in ("bf16", "f16")
            and cfg["neox"])


def probe_shape(cfg: dict) -> bool:
    return fused_probe_shape(cfg) or qk_probe_shape(cfg)


def same_traffic_ceiling(wl, steps: int):
    """The operator's memory traffic and grid with no arithmetic
    (qrw_probe_copy_fused_traffic or qrw_probe_copy_qk_traffic,
    include/qrw_probe.h) on the workload's own buffers, and the same grid doing
    nothing (qrw_probe_empty): what a kernel with this access structure reaches
    at this size, and a launch's fixed cost."""
    import torch

    import quant_row_workgroup_amd as qrw

    P = qrw.load_probe()
    T = wl.cfg["tokens"]
    blocks = (T + 3) // 4
    empty = torch.zeros(4 * blocks, dtype=torch.int32, device="cuda")
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())

    def nothing(i, sp):
        rc = P.qrw_probe_empty(ptr(empty), blocks, ctypes.c_void_p(sp))
        if rc != 0:
            raise RuntimeError(f"qrw_probe_empty: status {rc}")

    def empty_grid():
        ms = timed_launches(nothing, steps)
        mode = TIMING["mode"]
        torch.cuda.synchronize()
        if not torch.equal(empty.view(-1, 4)[:, 0].cpu(), torch.arange(blocks, dtype=torch.int32)):
            raise RuntimeError("empty-grid probe wrote the wrong words")
        return ms, mode

    if wl.cfg["op"] in ("qk_norm_rope", "qk_kv"):
        kv = wl.cfg["op"] == "qk_kv"

        def qk_copy(i, sp):
            s = wl.sets[i % len(wl.sets)]
            if kv:
                rc = P.qrw_probe_copy_qk_traffic(
                    ptr(s["x"]), ptr(s["q_weight"]), ptr(s["k_weight"]), ptr(s["cos"]),
                    ptr(s["sin"]), ptr(s["k_cache"]), ptr(s["v_cache"]), ptr(s["k_scales"]),
                    ptr(s["v_scales"]), ptr(s["slots"]), wl.cfg["num_slots"], T, 1,
                    ctypes.c_void_p(sp))
            else:
                rc = P.qrw_probe_copy_qk_traffic(
                    ptr(s["x"]), ptr(s["q_weight"]), ptr(s["k_weight"]), ptr(s["cos"]),
                    ptr(s["sin"]), None, None, None, None, None, 0, T, 0, ctypes.c_void_p(sp))
            if rc != 0:
                raise RuntimeError(f"qrw_probe_copy_qk_traffic: status {rc}")

        ms = timed_launches(qk_copy, steps)
        timing = TIMING["mode"]
        gbs = wl.counted / (ms * 1e-3) / 1e9
        ems, empty_timing = empty_grid()
        wl.reset()
        print(f"[bench] same-traffic copy: {ms * 1e3:.3f} us; empty grid of {blocks} workgroups "
              f"{ems * 1e3:.3f} us", file=sys.stderr, flush=True)
        what = ("q heads written back in place, k and v heads as 8 bytes per lane to the "
                "cache rows of their slots, one 4-byte scale per slot and head" if kv else
                "q and k heads written back in place")
        return {
            "kernel": (f"qrw_probe_copy_qk_traffic: the operator's grid (one wave per token), "
                       f"loads and stores ({what}) with byte selection in place of arithmetic"),
            "us_per_launch": round(ms * 1e3, 3),
            "GB/s": round(gbs, 1),
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "timing": timing,
            "empty_grid_us_per_launch": round(ems * 1e3, 3),
            "empty_grid_timing": empty_timing,
        }

    def copy(dep):
        def go(i, sp):
            s = wl.sets[i % len(wl.sets)]
            rc = P.qrw_probe_copy_fused_traffic(ptr(s["x"]), ptr(s["w"]), ptr(s["cos"]),
                                                ptr(s["sin"]), ptr(s["q"]), ptr(s["scales"]), T,
                                                4096, dep, ctypes.c_void_p(sp))
            if rc != 0:
                raise RuntimeError(f"qrw_probe_copy_fused_traffic: status {rc}")
        return go

    out = {}
    for key, fn in (("row_dependency", copy(1)), ("no_dependency", copy(0))):
        ms = timed_launches(fn, steps)
        gbs = wl.counted / (ms * 1e-3) / 1e9
        out[key] = {"us_per_launch": round(ms * 1e3, 3), "GB/s": round(gbs, 1),
                    "frac": round(gbs / PEAK_HBM_GBS, 4), "timing": TIMING["mode"]}
    ms, empty_timing = empty_grid()
    wl.reset()
    print(f"[bench] same-traffic copy: {out['row_dependency']['us_per_launch']:.3f} us "
          f"(no row dependency {out['no_dependency']['us_per_launch']:.3f} us); empty grid "
          f"of {blocks} workgroups {ms * 1e3:.3f} us", file=sys.stderr, flush=True)
    return {
        "kernel": ("qrw_probe_copy_fused_traffic: the fused operator's grid, loads and stores "
                   "(51.4 MB at 4096 tokens) with byte selection in place of arithmetic; no "
                   "store before the wave's whole row has arrived"),
        "us_per_launch": out["row_dependency"]["us_per_launch"],
        "GB/s": out["row_dependency"]["GB/s"],
        "frac": out["row_dependency"]["frac"],
        "timing": out["row_dependency"]["timing"],
        "no_row_dependency": out["no_dependency"],
        "empty_grid_us_per_launch": round(ms * 1e3, 3),
        "empty_grid_timing": empty_timing,
    }


def timeline(wl, launches: int):
    """Per-wave timestamps of the fused kernel (qrw_probe_fused_timeline: the
    library's contiguous kernel with the constant 100 MHz clock read at entry,
    once the row's sum of squares is known, after the last store is issued and
    once the stores are done) over ``launches`` consecutive launches on
    rotating buffer sets, timed like the workload.  Times are microseconds from each
    launch's first wave; ``gap_to_next`` runs from a launch's last completed
    store to the next launch's first wave."""
    import numpy as np
    import torch

    import quant_row_workgroup_amd as qrw

    P = qrw.load_probe()
    T = wl.cfg["tokens"]
    stamps = torch.zeros((launches, T, 4), dtype=torch.int64, device="cuda")
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())

    def go(i, sp):
        s = wl.sets[i % len(wl.sets)]
        rc = P.qrw_probe_fused_timeline(ptr(s["x"]), ptr(s["w"]), ptr(s["cos"]), ptr(s["sin"]),
                                        ptr(s["q"]), ptr(s["scales"]), T, wl.cfg["eps"],
                                        ptr(stamps[i % launches]), ctypes.c_void_p(sp))
        if rc != 0:
            raise RuntimeError(f"qrw_probe_fused_timeline: status {rc}")

    ms = timed_launches(go, launches)
    st = stamps.cpu().numpy().astype(np.float64) * 0.01  # 100 MHz ticks -> us
    names = ("entry", "row_arrived", "stores_issued", "stores_done")
    per = {k: [] for k in names}
    gaps, spans = [], []
    for k in range(launches):
        t0 = st[k, :, 0].min()
        for j, nm in enumerate(names):
            per[nm].append(st[k, :, j] - t0)
        spans.append(st[k, :, 3].max() - t0)
        if k + 1 < launches:
            gaps.append(st[k + 1, :, 0].min() - st[k, :, 3].max())
    q = lambda a, p: round(float(np.percentile(np.concatenate(a), p)), 3)
    out = {"launches": launches, "us_per_launch": round(ms * 1e3, 3), "timing": TIMING["mode"],
           "first_wave_to_last_store_done_us": round(float(np.median(spans)), 3),
           "gap_to_next_us": round(float(np.median(gaps)), 3) if gaps else None}
    for nm in names:
        out[nm] = {f"p{p}": q(per[nm], p) for p in (0, 10, 50, 90, 99, 100)}
    arith = [per["stores_issued"][k] - per["row_arrived"][k] for k in range(launches)]
    out["arrived_to_issued"] = {f"p{p}": q(arith, p) for p in (0, 50, 99, 100)}
    print(f"[bench] timeline: {json.dumps(out)}", file=sys.stderr, flush=True)
    return out


def host_cost(wl) -> dict:
    """Host time per call of the fused operator's launch path.  From plain C
    (csrc/probe/host_cost.c, a child process with its own buffers): argument
    validation alone (invalid and empty calls, nanoseconds), and valid
    asynchronous calls at the benchmark shape beside bare launches of the same
    grid (microseconds).  From Python, on the workload's buffers: the raw
    ctypes call bench.py times in eager mode, and the torch binding with
    preallocated outputs (microseconds)."""
    import time as _time

    import torch

    import quant_row_workgroup_amd as qrw
    from quant_row_workgroup_amd import build

    out = {}
    for mode, n in (("validate", "1000000"), ("launch", "200")):
        r = subprocess.run([build.HOST_COST, mode, n], capture_output=True, text=True,
                           timeout=300)
        if r.returncode != 0:
            raise RuntimeError(f"host_cost {mode}: {r.stderr.strip()}")
        out.update({f"c_{k}": float(v)
                    for k, v in (ln.split() for ln in r.stdout.strip().splitlines())})
    n = 200
    cur = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    t0 = _time.perf_counter()
    for i in range(n):
        wl.launch(i, cur)
    t1 = _time.perf_counter()
    torch.cuda.synchronize()
    s = wl.sets[0]
    c = wl.cfg
    args = (s["x"], s["w"], s["cos"], s["sin"], c["heads"], c["head_dim"], c["rope_dim"],
            c["neox"], c["eps"], s["q"], s["scales"])
    qrw.rmsnorm_rope_fp8_fwd(*args)
    torch.cuda.synchronize()
    t2 = _time.perf_counter()
    for _ in range(n):
        qrw.rmsnorm_rope_fp8_fwd(*args)
    t3 = _time.perf_counter()
    torch.cuda.synchronize()
    wl.reset()
    out["python_ctypes_launch_us_per_call"] = round((t1 - t0) / n * 1e6, 3)
    out["python_binding_us_per_call"] = round((t3 - t2) / n * 1e6, 3)
    print(f"[bench] host cost: {json.dumps(out)}", file=sys.stderr, flush=True)
    return out


def trace_summary(path: str, last: int = 0) -> str:
    """Summary of a rocprofv3 CSV, in microseconds.  A --kernel-trace file:
    per kernel the dispatch count and mean, p10, p50, p90, min and max
    duration, its launch shape, and, with ``last``, the same statistics over
    its last ``last`` dispatches (bench.py's timed launches come last).  A
    --pmc counter file: per kernel and counter the dispatch count and the
    median, min and max value."""
    import csv

    import numpy as np

    with open(path, newline="") as fh:
        rows = list(csv.DictReader(fh))
    if not rows:
        return "empty"
    stat = lambda a: (f"{len(a):>7} {a.mean():9.3f} {np.percentile(a, 10):9.3f} "
                      f"{np.percentile(a, 50):9.3f} {np.percentile(a, 90):9.3f} "
                      f"{a.min():9.3f} {a.max():9.3f}")
    head = (f"{'count':>7} {'mean_us':>9} {'p10_us':>9} {'p50_us':>9} {'p90_us':>9} "
            f"{'min_us':>9} {'max_us':>9}  kernel")
    if "Counter_Name" in rows[0]:
        vals = {}
        for r in rows:
            vals.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(
                float(r["Counter_Value"]))
        lines = [f"{'count':>7} {'median':>14} {'min':>14} {'max':>14}  counter  kernel"]
        for (name, ctr), v in sorted(vals.items(), key=lambda kv: -len(kv[1])):
            a = np.array(v)
            lines.append(f"{len(a):>7} {np.median(a):14.1f} {a.min():14.1f} {a.max():14.1f}  "
                         f"{ctr}  {name[:160]}")
        return "\n".join(lines)
    durs, shape = {}, {}
    for r in sorted(rows, key=lambda r: int(r["Start_Timestamp"])):
        name = r["Kernel_Name"]
        durs.setdefault(name, []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
        if name not in shape:
            grid = r.get("Grid_Size") or r.get("Grid_Size_X", "?")
            wg = r.get("Workgroup_Size") or r.get("Workgroup_Size_X", "?")
            vg = r.get("Arch_VGPR_Count") or r.get("VGPR_Count", "?")
            shape[name] = f"grid {grid} threads, workgroups of {wg}, {vg} arch VGPRs"
    lines = [head]
    order = sorted(durs.items(), key=lambda kv: -sum(kv[1]))
    for name, v in order:
        lines.append(f"{stat(np.array(v))}  {name[:160]}")
    lines.append("")
    for name, v in order:
        lines.append(f"launch: {shape[name]}  {name[:160]}")
    if last:
        lines += ["", f"last {last} dispatches of each kernel with at least that many:", head]
        for name, v in order:
            if len(v) >= last:
                lines.append(f"{stat(np.array(v[-last:]))}  {name[:160]}")
    return "\n".join(lines)


def resized_workload(name: str, rows: int) -> str:
    """Register ``name`` with another row count as ``name@rows`` and return that
    name (a paged-cache workload keeps at least four cache slots per token)."""
    from quant_row_workgroup_amd import synth

    cfg = dict(synth.WORKLOADS[name])
    key = {"rope": "tokens", "fused": "tokens", "qk_norm_rope": "tokens", "qk_kv": "tokens",
           "ew": "n"}.get(cfg["op"], "rows")
    cfg[key] = rows
    if cfg["op"] == "qk_kv":
        cfg["num_slots"] = max(cfg["num_slots"], 4 * rows)
    new = f"{name}@{rows}"
    synth.WORKLOADS[new] = cfg
    return new


def op_of(name: str) -> str:
    from quant_row_workgroup_amd import synth

    return synth.WORKLOADS[name]["op"]


def full_rows(name: str) -> int:
    from quant_row_workgroup_amd import synth

    c = synth.WORKLOADS[name]
    return c.get("tokens", c.get("rows", c.get("n")))


def cpu_baseline(name: str, seconds: float):
    """The float64 C oracle on a bounded sample of the workload, on the host's
    cores: first one thread, then one thread per core (at most 16) over
    contiguous row blocks, each half of ``seconds``.  ctypes releases the
    interpreter lock during each oracle call, so the threads run in parallel."""
    import concurrent.futures

    import oracle
    from quant_row_workgroup_amd import ledger, synth

    rows = 1 << 20 if op_of(name) == "ew" else 256
    inp = synth.make_inputs(name, rows=rows)
    cfg = dict(synth.WORKLOADS[name])
    op = cfg["op"]
    key = {"rope": "tokens", "fused": "tokens", "qk_norm_rope": "tokens", "qk_kv": "tokens",
           "ew": "n"}.get(op, "rows")
    cfg[key] = rows
    bytes_per_call = ledger.counted_bytes(cfg)

    def call(lo, hi):
        x = inp["x"][lo:hi]
        if op in ("fused", "rope", "qk_norm_rope", "qk_kv"):
            cos, sin = inp["cos"][lo:hi], inp["sin"][lo:hi]
        if op == "fused":
            fn = oracle.rmsnorm_rope_fp8_rounded if cfg.get("staged") else oracle.rmsnorm_rope_fp8
            fn(x, inp["w"], cos, sin, cfg["heads"], cfg["head_dim"], cfg["rope_dim"],
               cfg["dtype"], cfg["cs_dtype"], cfg["neox"], cfg["eps"])
        elif op == "act_quant":
            oracle.act_quant_fp8(x, cfg["dtype"], cfg.get("group"))
        elif op == "ew":
            alpha = 1.0 if cfg["kind"] == "add" else cfg["alpha"]
            b = inp.get("b")
            oracle.ew_scale_add(x, None if b is None else b[lo:hi], alpha, cfg["dtype"],
                                cfg.get("y_dtype", cfg["dtype"]))
        elif op == "qk_kv":
            oracle.qk_norm_rope_fp8_kv(x, inp["q_weight"], inp["k_weight"], cos, sin,
                                       cfg["q_heads"], cfg["kv_heads"], cfg["head_dim"],
                                       cfg["rope_dim"], cfg["dtype"], cfg["cs_dtype"],
                                       cfg["neox"], cfg["eps"], slots=inp["slots"][lo:hi],
                                       num_slots=cfg["num_slots"])
        elif op == "qk_norm_rope":
            oracle.qk_norm_rope(x, inp["q_weight"], inp["k_weight"], cos, sin, cfg["q_heads"],
                                cfg["kv_heads"], cfg["head_dim"], cfg["rope_dim"],
                                cfg["dtype"], cfg["cs_dtype"], cfg["neox"], cfg["eps"])
        elif op == "rmsnorm":
            oracle.rmsnorm(x, inp["w"], cfg["dtype"], cfg["eps"])
        elif op == "layernorm":
            oracle.layernorm(x, inp["gamma"], inp["beta"], cfg["dtype"], cfg["eps"])
        else:
            oracle.rope(x, cos, sin, cfg["heads"], cfg["head_dim"], cfg["rope_dim"],
                        cfg["dtype"], cfg["cs_dtype"], cfg.get("neox", True))

    def timed(step, budget):
        step()  # warm-up
        reps = 0
        t0 = time.perf_counter()
        while True:
            step()
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return reps, el

    reps1, el1 = timed(lambda: call(0, rows), seconds / 2)
    threads = max(1, min(16, os.cpu_count() or 1, rows))
    cuts = [rows * i // threads for i in range(threads + 1)]
    with concurrent.futures.ThreadPoolExecutor(threads) as pool:
        def all_blocks():
            for f in [pool.submit(call, cuts[i], cuts[i + 1]) for i in range(threads)]:
                f.result()
        repsn, eln = timed(all_blocks, seconds / 2)
    gbs1 = bytes_per_call * reps1 / el1 / 1e9
    gbsn = bytes_per_call * repsn / eln / 1e9
    unit = "elements" if op == "ew" else "rows"
    return {
        "value": round(gbsn, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "single_thread_value": round(gbs1, 4),
        "sample": (f"{rows} of {full_rows(name)} {unit} of the same workload; float64 C "
                   f"checker on {cpu_model()} ({os.cpu_count()} logical CPUs present): "
                   f"{threads} threads over contiguous blocks of {unit}, {repsn} passes in "
                   f"{eln:.1f} s; one thread, {reps1} passes in {el1:.1f} s"),
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--sets", type=int, default=8)
    ap.add_argument("--mode", choices=["stream", "graph", "eager"], default="stream",
                    help="how the timed launches are enqueued (see timed_launches)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--rows", type=int, default=0,
                    help="run the workload with this many rows (tokens, or elements for the "
                         "elementwise family) instead of its own count; every other size stays")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--plain-copy", type=int, default=0, metavar="MIB",
                    help="also time a plain copy of MIB MiB through the library's 16-byte-per-lane "
                         "elementwise kernel (f32, alpha 1), timed like the workload, and "
                         "report it as plain_copy (context: what a bare copy of that size reaches)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the same-traffic copy and empty-grid probes (fused 4096-wide "
                         "and QK workloads run them by default and report copy_ceiling)")
    ap.add_argument("--timeline", type=int, default=0, metavar="LAUNCHES",
                    help="fused 4096-wide workloads: per-wave timestamps over LAUNCHES "
                         "consecutive launches, reported as timeline")
    ap.add_argument("--host-cost", action="store_true",
                    help="also time the C ABI's host path from plain C (validation alone; valid "
                         "calls of the fused operator and bare launches), reported as host_cost")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="print per-kernel duration statistics of a rocprofv3 kernel-trace CSV, "
                         "or per-kernel counter statistics of a --pmc counter CSV, and exit (no "
                         "GPU work)")
    ap.add_argument("--trace-last", type=int, default=0, metavar="K",
                    help="with --trace-summary: also the statistics of each kernel's last K "
                         "dispatches (the timed launches)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="after timing, run 5 plain device copies of MIB MiB (a known-size "
                         "reference for rocprofv3 FETCH_SIZE / WRITE_SIZE scaling)")
    args = ap.parse_args()

    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.trace_last))
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the row operators shard by tokens with no "
              "exchange between GPUs, so one GPU's throughput is the figure. Use --gpus 1.",
              file=sys.stderr)
        return 2

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no ROCm device visible", file=sys.stderr)
        return 1

    from quant_row_workgroup_amd import synth

    if args.rows:
        args.workload = resized_workload(args.workload, args.rows)
    wl = Workload(args.workload, args.sets)
    print(f"[bench] {args.workload}: {args.sets} sets, warmup {args.warmup}, steps {args.steps}, "
          f"mode {args.mode}", file=sys.stderr, flush=True)
    ms = time_gpu(wl, args.steps, args.warmup, args.mode)
    timing = dict(TIMING)
    gbs = wl.counted / (ms * 1e-3) / 1e9
    print(f"[bench] {ms * 1e3:.3f} us/launch, {gbs:.1f} GB/s", file=sys.stderr, flush=True)

    ceiling = None
    if probe_shape(wl.cfg) and not args.no_ceiling:
        ceiling = same_traffic_ceiling(wl, args.steps)
        ceiling["kernel_over_ceiling"] = round(ms * 1e3 / ceiling["us_per_launch"], 4)
    tl = timeline(wl, args.timeline) if args.timeline and fused_probe_shape(wl.cfg) else None
    plain = plain_copy(args.plain_copy, args.sets) if args.plain_copy else None
    hcost = host_cost(wl) if args.host_cost and wl.cfg["op"] == "fused" else None

    if args.calibrate_copy:
        nb = args.calibrate_copy << 20
        a = torch.empty(nb, dtype=torch.uint8, device="cuda").random_(0, 255)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(f"[bench] calibration: 5 copies of {nb} B", file=sys.stderr, flush=True)

    src_hash = kernel_source_hash(wl.cfg["op"])
    traffic = stored_traffic(args.workload, src_hash)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.workload, args.cpu_seconds)

    c = wl.cfg
    if c["op"] == "fused":
        cfg = {"workload": (f"fused RMSNorm+RoPE(NeoX)+per-token E4M3 quant, {c['tokens']} tokens x "
                            f"{c['heads'] * c['head_dim']} ({c['heads']} heads x {c['head_dim']}) "
                            f"{c['dtype']} in, {c['cs_dtype']} cos/sin [{c['tokens']},"
                            f"{c['rope_dim'] // 2}], e4m3 codes + f32 scales out"),
               "tokens": c["tokens"], "hidden": c["heads"] * c["head_dim"], "heads": c["heads"],
               "head_dim": c["head_dim"], "rope_dim": c["rope_dim"]}
    else:
        cfg = {"workload": args.workload}
    cfg.update({"input_sets": args.sets, "counted_bytes_per_step": wl.counted,
                "timing": (f"{timing['mode']}: HIP events on the launch stream"
                           + (", launches queued behind a backlog before the first ran"
                              if timing.get("ahead") else ""))})

    line = {
        "metric": METRIC if args.workload == DEFAULT_WORKLOAD else f"achieved HBM GB/s, {args.workload}",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": compute_dtype(wl.cfg),
        "data": "synthetic",
        "config": cfg,
        "pct_of_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
        "kernel_src_hash": src_hash,
    }
    if ceiling is not None:
        line["copy_ceiling"] = ceiling
    if tl is not None:
        line["timeline"] = tl
    if plain is not None:
        line["plain_copy"] = plain
    if hcost is not None:
        line["host_cost"] = hcost
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
