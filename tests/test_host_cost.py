"""The C ABI's argument validation timed from plain C (csrc/probe/host_cost.c,
built by build()): calls that fail validation and empty calls never touch a
device, so this runs on the CPU.  The page "The TileLang kernel DSL in
DeepSeek-V4" (host code generation) puts its generated launchers' checks
under one microsecond; the figures are printed, not asserted (timing depends
on the host), and the program itself checks every returned status."""
import os
import subprocess

import pytest

import quant_row_workgroup_amd as qrw
from quant_row_workgroup_amd import build


@pytest.fixture(scope="module")
def harness():
    if not os.path.exists(build.HOST_COST):
        build.build_host_cost()
    return build.HOST_COST


def test_validation_cost_from_c(harness):
    qrw.load()  # the library the harness links is built
    r = subprocess.run([harness, "validate", "200000"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    figures = dict(line.split() for line in r.stdout.strip().splitlines())
    print(figures)
    assert int(figures["calls"]) == 200000
    for k in ("fused_invalid_ns_per_call", "fused_empty_ns_per_call",
              "rmsnorm_invalid_ns_per_call", "rmsnorm_empty_ns_per_call"):
        assert float(figures[k]) > 0
