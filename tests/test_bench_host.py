"""Host-side logic of bench.py (no GPU): the one-GPU contract, the roofline and work
formulas, the code hash that tags counter traffic, and counter ingestion."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth.configs import CONFIGS  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "single GPU" in p.stderr and "--gpus 2" in p.stderr
    assert p.stdout == ""


def test_quantized_secondary_workloads_are_refused_before_any_gpu_work():
    # secondary workloads reuse the primary's bf16 weights: a quantized name would run the bf16
    # layer under the quantized label, so it is refused up front
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--secondary", "skew_t6000,prefill_t8192_fp8"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "prefill_t8192_fp8" in p.stderr and "bf16 workloads only" in p.stderr
    assert p.stdout == ""


def test_roofline_picks_the_binding_resource():
    # 2.5 PFLOP and 8 GB in one second: the flops take 1 s at peak, the bytes 1 ms -> mfma
    r = bench.roofline(2.5e15, 8e9, 2.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(1250.0) and r["frac"] == pytest.approx(0.5)
    # 1 GFLOP and 8 GB: the bytes bind
    r = bench.roofline(1e9, 8e9, 2e-3, traffic={"bytes": 1})
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(4000.0) and r["frac"] == pytest.approx(0.5)
    assert r["traffic"] == {"bytes": 1}


def test_bytes_per_stored_weight():
    assert bench.weight_bytes_per_element(CONFIGS["decode_t64"]) == 2.0
    assert bench.weight_bytes_per_element(CONFIGS["decode_t64_fp8"]) == 1.0 + 1.0 / 32
    assert bench.weight_bytes_per_element(CONFIGS["decode_t64_mxfp4"]) == 0.5 + 1.0 / 32


def test_gemm_work_formulas():
    cfg = CONFIGS["decode_t64"]
    H, I, T, k = 5120, 2560, 64, 8
    f, b = bench.gate_up_work(cfg, 209)
    assert f == 4.0 * H * I * T * k
    assert b == 209 * 2.0 * I * H * 2 + T * H * 2 + T * k * I * 2
    f, b = bench.down_work(cfg, 209)
    assert f == 2.0 * H * I * T * k
    assert b == 209 * H * I * 2 + T * k * (I + H) * 2
    f8, b8 = bench.gate_up_work(CONFIGS["decode_t64_fp8"], 209)
    assert f8 == f * 2 and b8 == 209 * 2.0 * I * H * (1 + 1 / 32) + T * H * 2 + T * k * I * 2


def test_code_hash_ignores_comments_and_blank_space_only():
    src = "int f(int a) {\n    return a + 1;  // one more\n}\n/* block\n comment */\n"
    h = bench.kernel_source_hash(src)
    assert bench.kernel_source_hash("// header\n" + src.replace("    ", "  ") + "\n\n") == h
    assert bench.kernel_source_hash(src.replace("a + 1", "a + 2")) != h
    # the recorded hash covers every expert-GEMM source
    assert bench.kernel_source_hash() == bench.kernel_source_hash(
        "\n".join(open(p).read() for p in bench.GEMM_SOURCES))


def _pmc_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, v in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_counter_ingestion_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "traffic.json"))
    gu = "void beam::moe_gemm_line_kernel<true, 0, 8, 2, 2>(...)"
    dn = "void beam::moe_gemm_line_kernel<false, 0, 8, 2, 2>(...)"
    _pmc_csv(tmp_path / "f.csv", "FETCH_SIZE", [(gu, 100.0), (gu, 300.0), (dn, 50.0), ("other", 7.0)])
    _pmc_csv(tmp_path / "w.csv", "WRITE_SIZE", [(gu, 10.0), (dn, 20.0)])
    # a 1 MiB copy that reads half its bytes by FETCH_SIZE and all of them by WRITE_SIZE
    _pmc_csv(tmp_path / "cf.csv", "FETCH_SIZE", [("copy", 512.0), ("small", 1.0)])
    _pmc_csv(tmp_path / "cw.csv", "WRITE_SIZE", [("copy", 1024.0)])
    bench.ingest_counters("prefill_t8192", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                          str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), 1)
    d = json.load(open(tmp_path / "traffic.json"))["prefill_t8192"]
    assert d["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert d["calibration"]["write_factor"] == pytest.approx(1.0)
    assert d["gate_up"]["fetch_bytes"] == pytest.approx(200.0 * 1024 * 2.0)   # mean of 100 and 300 KiB
    assert d["gate_up"]["write_bytes"] == pytest.approx(10.0 * 1024)
    assert d["down"]["fetch_bytes"] == pytest.approx(50.0 * 1024 * 2.0)
    # the record is used while the GEMM code is unchanged, and only then
    t = bench.load_traffic("prefill_t8192", "gate_up")
    assert t["bytes"] == pytest.approx(200.0 * 1024 * 2.0 + 10.0 * 1024)
    rec = json.load(open(tmp_path / "traffic.json"))
    rec["prefill_t8192"]["experts_hip_code_sha256_16"] = "0" * 16
    json.dump(rec, open(tmp_path / "traffic.json", "w"))
    assert bench.load_traffic("prefill_t8192", "gate_up") is None
    assert bench.load_traffic("decode_t64", "gate_up") is None


def test_expert_histogram():
    h = bench.expert_histogram([0, 3, 5, 0, 9, 1, 2, 2, 7, 4])
    assert h == {"touched": 8, "min": 0, "median": 2.5, "max": 9, "empty": 2, "top8": [9, 7, 5, 4, 3, 2, 2, 1]}


def test_layer_work_counts_touched_experts_router_and_activations():
    cfg = CONFIGS["prefill_t8192"]
    f, b = bench.layer_work(cfg, 256)
    assert f == 6.0 * 5120 * 2560 * 8192 * 8
    assert b == 256 * 3.0 * 5120 * 2560 * 2 + 256 * 5120 * 4 + 2 * 8192 * 5120 * 2
    tiny = CONFIGS["tiny_f32"]
    f, b = bench.layer_work(tiny, 16)
    assert b == 16 * 3.0 * 64 * 32 * 4 + 16 * 64 * 4 + 2 * 32 * 64 * 4     # fp32 weights and activations


def test_trace_summary_leaves_out_the_warm_up_dispatches(tmp_path):
    path = tmp_path / "trace.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for i, us in enumerate([50, 40, 10, 10, 12]):      # two warm-ups, then three timed
            w.writerow({"Kernel_Name": "void beam::k<true>(int)", "Start_Timestamp": 1000 * i,
                        "End_Timestamp": 1000 * i + us * 1000})
        w.writerow({"Kernel_Name": "other(int)", "Start_Timestamp": 0, "End_Timestamp": 5000})
    table = bench.trace_summary(str(path), 2)
    line = [l for l in table.splitlines() if "beam::k<true>" in l][0]
    cells = [c.strip() for c in line.split("|")]
    assert cells[2] == "3" and cells[3] == "10.7" and cells[4] == "10.0" and cells[5] == "10.0" and cells[6] == "12.0"
    assert "other" in table      # a kernel with fewer dispatches than the skip keeps them all
