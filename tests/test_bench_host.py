"""Host-side logic of bench.py: the one-GPU contract, the algorithmic byte and
flop counts behind the roofline fractions, and the counter summaries."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from transformer_llama_decode_amd.configs import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_w13_launch_bytes_of_the_7b_shape():
    cfg = WORKLOADS["C5"].model
    d, f = 4096, 11008
    # W1 and W3 (fp32), the input row and its gain read, the gate row written
    assert bench.w13_launch_bytes(cfg) == 4 * 2 * f * d + 4 * (2 * d + f) == 360786944
    assert bench.w13_launch_bytes(WORKLOADS["C5bf16"].model) == 2 * 2 * f * d + 4 * (2 * d + f)


def test_step_bytes_count_every_matrix_once_and_the_visible_history():
    cfg = WORKLOADS["C5"].model
    d, f, V, L = 4096, 11008, 32000, 32
    weights = 4 * (L * (4 * d * d + 3 * d * f) + V * d)
    assert weights == 4 * 6738415616 - 4 * (2 * L + 1) * d - 4 * V * d   # untied: embedding not read
    p = 700
    per_seq = 4 * (d + 2 * L * (p + 1) * d + 2 * L * d + V)
    assert bench.step_bytes(cfg, p) == weights + 4 * (2 * L + 1) * d + per_seq
    # past max_seq only the window's max_seq positions are read
    win = WORKLOADS["C5w"].model
    assert bench.step_bytes(win, 1500) == bench.step_bytes(win, win.max_seq - 1)


def test_gemm_flops_of_the_batched_15m_step():
    cfg = WORKLOADS["C3"].model
    d, f, V, L, B = 288, 768, 32000, 6, 256
    assert bench.gemm_flops_per_step(cfg, B) == 2 * B * (L * (4 * d * d + 3 * d * f) + V * d) == 7776239616


def _write_pmc_csv(path, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(cols, r)))


def test_mfma_summary_from_counters(tmp_path):
    # two launches of one GEMM: 1000 kernel cycles on each of 8 XCDs, the matrix
    # cores of 1024 SIMDs busy for 256000 cycles in all -> 25%; 2e6 MOPS = 1.024e9 flops
    name = "void ld::(anonymous namespace)::k_gemm_sk<0, false, false, 32>(ld::GemmArgs, int, int)"
    rows = []
    for disp in (1, 2):
        rows += [(disp, name, "GRBM_GUI_ACTIVE", 8000.0, 0, 1),
                 (disp, name, "SQ_VALU_MFMA_BUSY_CYCLES", 256000.0, 0, 1),
                 (disp, name, "SQ_BUSY_CYCLES", 1.0, 0, 1),
                 (disp, name, "SQ_INSTS_VALU_MFMA_MOPS_F32", 1e6, 0, 1)]
    rows.append((3, "void ld::(anonymous namespace)::k_fill(float*, float, unsigned long)", "GRBM_GUI_ACTIVE",
                 5.0, 0, 1))
    _write_pmc_csv(tmp_path / "m_counter_collection.csv", rows)
    out = tmp_path / "mfma.txt"
    bench.summarize_mfma(str(tmp_path), "C3", str(out))
    text = out.read_text()
    line = [ln for ln in text.splitlines() if ln.startswith("k_gemm_sk<0")][0].split()
    assert line[-1] == "25.0%"
    assert float(line[-3]) == pytest.approx(512e6)      # flops per call
    assert "k_fill" not in text                          # no matrix-core work, no line
    assert "all matrix-core kernels: MFMA busy 25.0%" in text


def test_trace_summary_table(tmp_path):
    cols = ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"]
    with open(tmp_path / "x_kernel_stats.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=cols)
        w.writeheader()
        w.writerow(dict(zip(cols, ["void ld::(anonymous namespace)::k_small(int)", 4, 8000, 2000, 1, 1500, 2500, 1])))
        w.writerow(dict(zip(cols, ["void ld::(anonymous namespace)::k_big(ld::GemvArgs)", 2, 100000, 50000, 99, 49000,
                                   51000, 1])))
    out = tmp_path / "t.txt"
    bench.summarize_trace(str(tmp_path), "a title", "rocprofv3 ...", str(out))
    text = out.read_text().splitlines()
    assert text[0].startswith("rocprofv3 kernel statistics: a title")
    body = [ln for ln in text if ln.startswith("k_")]
    assert body[0].split()[0] == "k_big(GemvArgs)" and body[1].split()[0] == "k_small(int)"   # by total time
    assert body[0].split()[1:4] == ["2", "0.100", "50.00"]


def test_w13_traffic_is_taken_from_the_streamed_7b_kernel(tmp_path):
    # two W1/W3 instantiations (the 7B one streams 360 MB, a small model's 6 MB):
    # the summary must report the 7B one
    big = "void ld::(anonymous namespace)::k_gemv<2, 1, 4, true, false, 0, true>(ld::GemvArgs)"
    small = "void ld::(anonymous namespace)::k_gemv<2, 1, 4, false, false, 0, false>(ld::GemvArgs)"
    copy = "__amd_rocclr_copyBuffer"
    dirs = {k: tmp_path / k for k in ("f", "w", "cf", "cw")}
    for d in dirs.values():
        d.mkdir()
    kib = 1024.0
    _write_pmc_csv(dirs["f"] / "f_counter_collection.csv",
                   [(1, big, "FETCH_SIZE", 360786944 / 2 / kib, 0, 1), (2, small, "FETCH_SIZE", 6e6 / 2 / kib, 0, 1)])
    _write_pmc_csv(dirs["w"] / "w_counter_collection.csv",
                   [(1, big, "WRITE_SIZE", 0.0, 0, 1), (2, small, "WRITE_SIZE", 0.0, 0, 1)])
    _write_pmc_csv(dirs["cf"] / "f_counter_collection.csv", [(1, copy, "FETCH_SIZE", (4 << 29) / 2 / kib, 0, 1)])
    _write_pmc_csv(dirs["cw"] / "w_counter_collection.csv", [(1, copy, "WRITE_SIZE", (4 << 29) / kib, 0, 1)])
    out_json, out_txt = tmp_path / "t.json", tmp_path / "t.txt"
    bench.summarize_counters(str(dirs["f"]), str(dirs["w"]), str(dirs["cf"]), str(dirs["cw"]), str(out_json),
                             str(out_txt))
    import json
    rec = json.loads(out_json.read_text())
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["bytes_per_launch"] == 360786944
