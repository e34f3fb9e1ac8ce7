"""Host-side checks of the kernels' index math, run on the CPU before any
launch: the token-row plan (qrw_plan.h) compiled with g++ and exercised over
every accepted shape class (tests/plan_check.cpp)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_row_plan_bounds_and_coverage(tmp_path):
    exe = tmp_path / "plan_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-I",
                    os.path.join(ROOT, "quant_row_workgroup_amd", "csrc"),
                    os.path.join(ROOT, "tests", "plan_check.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout
