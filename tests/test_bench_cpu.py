"""Host-side logic of bench.py: the one-GPU guard, the source-hash gating of the stored
counter figures, the update roofline arithmetic and the CPU oracle baseline's record."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout


def test_stored_traffic_is_used_only_for_its_source_and_workload():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    if t["source_sha256"] == bench.source_hash(bench.PERTURB_SOURCES):
        assert bench.stored_traffic(t["workload"], 0.0) == float(t["bytes_per_pass"])
    else:
        assert bench.stored_traffic(t["workload"], 0.0) is None
    assert bench.stored_traffic("some/other-workload", 0.0) is None


def test_stored_philox_peak_matches_its_sources():
    with open(bench.PHILOX_FILE) as f:
        t = json.load(f)
    got = bench.stored_philox_peak()
    if t["source_sha256"] == bench.source_hash(bench.PHILOX_SOURCES):
        assert got == float(t["calls_per_s"])
    else:
        assert got is None


def test_update_roofline_arithmetic():
    M, n, ms = 1 << 30, 160, 10.0
    r = bench.update_roofline(M, n, 4.0 * M, ms, "bf16", True)
    assert r["kernel"] == "k_update" and r["bound"] == "alu"
    assert abs(r["achieved_GBps"] - 4.0 * M / 1e-2 / 1e9) < 1e-6
    assert abs(r["probe_params_per_s"] - n * M / 1e-2) < 1.0
    assert abs(r["philox_calls_per_s"] - M * n / 128 / 1e-2) < 1.0
    if r["philox_peak_calls_per_s"]:
        assert abs(r["philox_frac"] - r["philox_calls_per_s"] / r["philox_peak_calls_per_s"]) < 1e-12
    # 256 CUs x 4 SIMDs x 2.4 GHz / 4 cycles per wave64 instruction
    assert r["peak"] == 6.144e11
    per = r["valu_insts_per_param_group"]
    if per is not None:
        assert abs(r["achieved"] - per * M * 20 / 64 / 1e-2) < 1e-3 * r["achieved"]
        assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-12
    # counts of another kernel form are not used
    other = bench.update_roofline(M, 32, 8.0 * M, ms, "fp32", True)
    assert other["achieved"] is None and other["frac"] is None
    assert bench.update_roofline(M, n, 4.0 * M, None, "bf16", True) is None


def test_stored_update_valu_matches_its_sources():
    with open(bench.UPDATE_VALU_FILE) as f:
        t = json.load(f)
    got = bench.stored_update_valu(t["dtype"], t["n_pert"], t["restore"])
    if t["source_sha256"] == bench.source_hash(bench.UPDATE_SOURCES):
        assert got == float(t["valu_insts_per_param_group"])
    else:
        assert got is None


def test_cpu_baseline_record_on_a_tiny_slice():
    from workloads import CONFIGS
    r = bench.cpu_baseline(CONFIGS["opt30b"], 1024, 2, "S2f")
    assert r["kind"] == "oracle" and r["unit"] == "probe*params/s" and r["cores"] == 2
    assert r["value"] > 0 and r["single_core_value"] > 0
    assert "2 windows x 1024 bf16 params" in r["sample"]
    assert r["host_cpus"] >= 1 and r["cpu_model"]
