"""Host-side logic of bench.py (no GPU): the multi-GPU refusal, the per-kernel
algorithmic work model, the choice of bound, and the counter table that
supplies roofline.traffic."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_work_model_counts():
    w = WORKLOADS[2]  # B=1, N=128, D=128, h=4, fp32
    m = bench.work_model(w)
    P, D, h, s = 128 * 128, 128, 4, 4
    assert m["positions"] == P
    assert m["k1_ln_proj"]["flops"] == 2 * P * D * (4 * D + h)
    assert m["k1_ln_proj"]["bytes"] == P * D * s + P + 4 * P * D * s + 4 * h * 128 * 128
    assert m["k2_attention"]["flops"] == 4 * 128 ** 3 * D
    assert m["k2_attention"]["bytes"] == 4 * P * D * s + 4 * h * 128 * 128 + P * D * s
    assert m["k3_out_proj"]["flops"] == 2 * P * D * D
    assert m["k3_out_proj"]["bytes"] == 2 * P * D * s
    m5 = bench.work_model(WORKLOADS[5])
    assert m5["k1_ln_proj"]["bytes"] == 4 * 512 * 512 * (128 * 2 + 1 + 4 * 128 * 2 + 4 * 8)


def test_bound_selection():
    # bf16 kernel 1 and kernel 3 sit below the HBM ridge; fp32 kernel 1 above the fp32 one
    m5 = bench.work_model(WORKLOADS[5])
    assert bench.roofline_of("k1_ln_proj", WORKLOADS[5], m5, 1.0)["bound"] == "hbm"
    assert bench.roofline_of("k3_out_proj", WORKLOADS[5], m5, 1.0)["bound"] == "hbm"
    assert bench.roofline_of("k2_attention", WORKLOADS[5], m5, 1.0)["bound"] == "mfma"
    m2 = bench.work_model(WORKLOADS[2])
    r = bench.roofline_of("k1_ln_proj", WORKLOADS[2], m2, 0.05)
    assert r["bound"] == "mfma" and r["peak"] == 157.3
    assert r["achieved"] == pytest.approx(m2["k1_ln_proj"]["flops"] / 0.05e-3 / 1e12)
    assert r["frac"] == pytest.approx(r["achieved"] / 157.3)


def test_attention_roofline_on_valid_pairs():
    import numpy as np
    w = WORKLOADS[5]
    m = bench.work_model(w)
    mask = np.zeros((4, 512, 512), np.uint8)
    mask[:, :100, :200] = 1
    r = bench.roofline_of("k2_attention", w, m, 1.0, mask)
    assert r["achieved"] == pytest.approx(4 * 512 * 128 * (4 * 100 * 200) / 1e-3 / 1e12)
    assert r["frac"] == pytest.approx(r["achieved"] / 2500.0)
    assert r["achieved_dense"] == pytest.approx(m["k2_attention"]["flops"] / 1e-3 / 1e12)
    assert "achieved_dense" not in bench.roofline_of("k1_ln_proj", w, m, 1.0, mask)


def test_split_products_ceiling():
    # float32 kernels 1 and 3 run six bf16 products per float32 product
    m2 = bench.work_model(WORKLOADS[2])
    r = bench.roofline_of("k3_out_proj", WORKLOADS[2], m2, 0.01)
    assert r["split_products"]["ceiling"] == pytest.approx(2500.0 / 6)
    assert r["split_products"]["frac_of_ceiling"] == pytest.approx(r["achieved"] / (2500.0 / 6))
    assert "split_products" not in bench.roofline_of("k2_attention", WORKLOADS[2], m2, 0.01)
    assert "split_products" not in bench.roofline_of("k2_attention", WORKLOADS[5], bench.work_model(WORKLOADS[5]), 1.0)


def test_float32_kernel1_source():
    assert bench.kernel_source("k1_ln_proj", "f32").endswith("k1_split.hip")
    assert bench.kernel_source("k1_ln_proj", "bf16").endswith("k1_ln_proj.hip")
    assert bench.source_hash("k1_ln_proj", "f32") != bench.source_hash("k1_ln_proj", "bf16")


def test_traffic_table_is_used_only_for_the_current_source(tmp_path, monkeypatch):
    k = "k1_ln_proj"
    good = bench.source_hash(k)
    table = tmp_path / "hbm_traffic.md"
    table.write_text(
        "| workload | kernel | source sha256[:16] | FETCH_SIZE KiB | WRITE_SIZE KiB | fetch scale | write scale |\n"
        "|---|---|---|---|---|---|---|\n"
        f"| wl_a | {k} | {good} | 100.0 | 50.0 | 2.000 | 1.000 |\n"
        f"| wl_b | {k} | 0000000000000000 | 100.0 | 50.0 | 2.000 | 1.000 |\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(table))
    assert bench.stored_traffic("wl_a", k) == pytest.approx((100.0 * 2 + 50.0) * 1024)
    assert bench.stored_traffic("wl_b", k) is None  # counters taken on another kernel source
    assert bench.stored_traffic("wl_c", k) is None  # no row


def test_committed_traffic_table_parses():
    # every row of the committed table has the seven cells bench.py reads
    rows = 0
    with open(bench.TRAFFIC_FILE) as f:
        for line in f:
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) == 7 and cells[1] in bench.KERNEL_SOURCES:
                float(cells[3]), float(cells[4]), float(cells[5]), float(cells[6])
                rows += 1
    assert rows >= 6


def test_attention_floor():
    import numpy as np
    w = WORKLOADS[5]
    m = bench.work_model(w)
    exps = 4 * 8 * 512 ** 3
    t_floor = exps / (bench.CALIB["v_exp_f32_Gops"] * 1e9) + m["k2_attention"]["flops"] / (
        bench.CALIB["mfma_bf16_random_TFLOPs"] * 1e12)
    mask = np.zeros((4, 512, 512), np.uint8)
    mask[:, :100, :200] = 1
    r = bench.attention_floor(w, m, 1.0, mask)
    assert r["exps"] == exps
    assert r["floor_ms"] == pytest.approx(t_floor * 1e3)
    assert r["frac_of_floor"] == pytest.approx(t_floor * 1e3 / 1.0)
    assert r["valid_tflops"] == pytest.approx(4 * 512 * 128 * (4 * 100 * 200) / 1e-3 / 1e12)


def test_source_hash_ignores_comments():
    code = "int f(int x) {\n  return x + 1;  // one more\n}\n/* block\ncomment */\n"
    same = "int f(int x) { return x + 1; }  // other words\n"
    other = "int f(int x) { return x + 2; }\n"
    assert bench._code_only(code) == bench._code_only(same)
    assert bench._code_only(code) != bench._code_only(other)
