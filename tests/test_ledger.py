"""The byte/FLOP ledger reproduces every number the pages print for it
(tests/golden/ledger_table.txt, from "TileLang tutorial, ch. 13", s1.2)."""
import os

from quant_row_workgroup_amd import ledger, synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ledger_table.txt")


def _golden():
    rows = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, *vals = line.split()
        rows[name] = vals
    return rows


def test_printed_ledger_values():
    g = _golden()
    sc = ledger.page_scenarios()
    for name, (unf, fus, _) in sc.items():
        pu, pf, pr = g[name]
        assert f"{unf / 1e6:.2f}" == pu, name
        assert f"{fus / 1e6:.2f}" == pf, name
        assert f"{unf / fus:.2f}" == pr, name


def test_exact_reconstructions():
    E = 4096 * 4096
    sc = ledger.page_scenarios()
    assert sc["scale_add"][:2] == (20 * (1 << 20), 12 * (1 << 20))
    assert sc["rmsnorm"][:2] == (14 * E + 26 * 4096, 4 * E + 2 * 4096)
    assert sc["rmsnorm"][:2] == (234_987_520, 67_117_056)
    assert sc["layernorm"][1] == 67_125_248
    assert sc["rope"][:2] == (22 * E, 6 * E) == (369_098_752, 100_663_296)
    assert sc["rmsnorm_rope_fp8"][:2] == (185_622_528, 51_404_800)


def test_arithmetic_intensity_range():
    g = _golden()["ai_range"]
    ais = []
    for unf, fus, flops in ledger.page_scenarios().values():
        ais += [flops / unf, flops / fus]
    assert f"{min(ais):.3f}" == g[0]
    assert f"{max(ais):.3f}" == g[1]


def test_counted_bytes_of_the_workloads():
    want = {
        "rmsnorm_256x1024_f16": 1_050_624,
        "rmsnorm_4096x4096_f16": 67_117_056,
        "layernorm_4096x4096_bf16": 67_125_248,
        "rope_4096x32x128_f16": 69_206_016,
        "rmsnorm_rope_fp8_4096x4096_bf16": 51_404_800,
    }
    for name, b in want.items():
        assert ledger.counted_bytes(synth.WORKLOADS[name]) == b, name


def test_qk_norm_rope_bytes_count_only_q_and_k():
    # 4096 tokens, 32 query + 8 key heads of 128 bf16 channels read and written,
    # two 128-wide weights, bf16 cos/sin of 64 entries per token; value heads free
    cfg = synth.WORKLOADS["qk_norm_rope_4096_q32_kv8_d128_bf16"]
    qk = 4096 * 40 * 128 * 2
    assert ledger.counted_bytes(cfg) == 2 * qk + 2 * 128 * 2 + 2 * 4096 * 64 * 2 == 84_935_168
    unfused, fused, _ = ledger.qk_norm_rope(4096, 32, 8, 128, 128)
    assert unfused - fused == 2 * qk  # the intermediate is written once and read once
