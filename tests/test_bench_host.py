"""Host logic of bench.py on the CPU: the row-count override, the reported
arithmetic type, the layouts the same-traffic probes reproduce, the refusal of
more than one GPU, the oracle baseline, and the summaries of rocprofv3
kernel-trace and counter files."""
import subprocess
import sys

import pytest

import bench
from quant_row_workgroup_amd import ledger, synth


@pytest.fixture(autouse=True)
def _restore_workloads():
    saved = dict(synth.WORKLOADS)
    yield
    synth.WORKLOADS.clear()
    synth.WORKLOADS.update(saved)


ROW_KEY = {"rope": "tokens", "fused": "tokens", "qk_norm_rope": "tokens", "qk_kv": "tokens",
           "ew": "n"}


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_resized_workload_changes_only_the_row_count(name):
    base = dict(synth.WORKLOADS[name])
    key = ROW_KEY.get(base["op"], "rows")
    a, b = bench.resized_workload(name, 64), bench.resized_workload(name, 128)
    ca, cb = synth.WORKLOADS[a], synth.WORKLOADS[b]
    assert a == f"{name}@64" and ca[key] == 64 and cb[key] == 128
    for k in base:
        if k not in (key, "num_slots"):
            assert ca[k] == base[k], k
    if base["op"] == "qk_kv":
        assert ca["num_slots"] >= 4 * 64 and cb["num_slots"] >= 4 * 128
    # bytes grow by the same amount for each further 64 rows (the per-row cost);
    # weights, tables of other rows and the like stay
    c192 = synth.WORKLOADS[bench.resized_workload(name, 192)]
    d1 = ledger.counted_bytes(cb) - ledger.counted_bytes(ca)
    d2 = ledger.counted_bytes(c192) - ledger.counted_bytes(cb)
    assert d1 == d2 > 0
    inp = synth.make_inputs(a, rows=8)
    assert inp["x"].shape[0] == 8
    assert bench.full_rows(a) == 64


def test_compute_dtype():
    assert bench.compute_dtype(synth.WORKLOADS["rmsnorm_rope_fp8_4096x4096_bf16"]) == "f32"
    assert bench.compute_dtype(synth.WORKLOADS["add_16M_bf16"]) == "f32"
    assert bench.compute_dtype(synth.WORKLOADS["scale_cast_16M_f32_to_f16"]) == "f64"
    assert bench.compute_dtype(synth.WORKLOADS["scale_add_1M_f32"]) == "f32"
    assert bench.compute_dtype(dict(op="ew", kind="scale_add", alpha=0.5, dtype="bf16")) == "f64"
    assert bench.compute_dtype(dict(op="ew", kind="scale_add", alpha=1.0, dtype="f16")) == "f32"


def test_same_traffic_probes_cover_only_their_own_layouts():
    covered = {n for n, c in synth.WORKLOADS.items() if bench.probe_shape(c)}
    assert covered == {"rmsnorm_rope_fp8_4096x4096_bf16", "qk_norm_rope_4096_q32_kv8_d128_bf16",
                       "qk_norm_rope_fp8_kv_4096_q32_kv8_d128_bf16"}
    base = dict(synth.WORKLOADS["rmsnorm_rope_fp8_4096x4096_bf16"])
    for k, v in (("neox", False), ("rope_dim", 64), ("dtype", "f16"), ("cs_dtype", "f32"),
                 ("staged", True)):
        assert not bench.probe_shape(dict(base, **{k: v})), k
    qk = dict(synth.WORKLOADS["qk_norm_rope_4096_q32_kv8_d128_bf16"])
    for k, v in (("q_heads", 16), ("kv_heads", 4), ("head_dim", 64), ("neox", False),
                 ("cs_dtype", "f32")):
        assert not bench.probe_shape(dict(qk, **{k: v})), k
    assert bench.probe_shape(dict(qk, tokens=17))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


@pytest.mark.parametrize("name", ["rmsnorm_rope_fp8_4096x4096_bf16", "scale_add_1M_f32",
                                  "qk_norm_rope_fp8_kv_4096_q32_kv8_d128_bf16"])
def test_cpu_baseline_reports_both_thread_counts(name):
    r = bench.cpu_baseline(name, 0.2)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s"
    assert 1 <= r["cores"] <= 16 and r["value"] > 0 and r["single_thread_value"] > 0
    assert f"{r['cores']} threads" in r["sample"]


def _write_csv(path, rows):
    import csv

    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_trace_summary_of_a_kernel_trace(tmp_path):
    # rocprofv3 --kernel-trace rows: durations from the timestamps (ns), per
    # kernel in launch order, and the statistics of each kernel's last K
    # dispatches (bench.py's timed launches come last)
    rows, t = [], 0
    for i in range(30):
        for name, d in (("kA", 1000 * (i + 1)), ("kB", 500)):
            rows.append({"Kind": "KERNEL_DISPATCH", "Kernel_Name": name, "Start_Timestamp": t,
                         "End_Timestamp": t + d, "Grid_Size": 4096, "Workgroup_Size": 256,
                         "Arch_VGPR_Count": 40})
            t += d + 10
    p = tmp_path / "k_kernel_trace.csv"
    _write_csv(p, rows)
    out = bench.trace_summary(str(p), last=10).splitlines()
    a = next(l for l in out if l.endswith("kA"))
    assert a.split()[:2] == ["30", "15.500"]  # mean of 1..30 us
    assert any(l.startswith("launch: grid 4096 threads, workgroups of 256, 40 arch VGPRs  kA")
               for l in out)
    i = next(k for k, l in enumerate(out) if l.startswith("last 10 dispatches"))
    a10 = next(l for l in out[i:] if l.endswith("kA"))
    assert a10.split()[:2] == ["10", "25.500"]  # mean of 21..30 us
    assert float(a10.split()[5]) == 21.0 and float(a10.split()[6]) == 30.0


def test_trace_summary_of_a_counter_file(tmp_path):
    rows = [{"Dispatch_Id": i, "Kernel_Name": "kA", "Counter_Name": "FETCH_SIZE",
             "Counter_Value": 100.0 + (i % 3)} for i in range(9)]
    rows += [{"Dispatch_Id": 9, "Kernel_Name": "copy", "Counter_Name": "FETCH_SIZE",
              "Counter_Value": 131072.0}]
    p = tmp_path / "k_counter_collection.csv"
    _write_csv(p, rows)
    out = bench.trace_summary(str(p)).splitlines()
    a = next(l for l in out if l.endswith("kA"))
    assert a.split()[:4] == ["9", "101.0", "100.0", "102.0"] and "FETCH_SIZE" in a
