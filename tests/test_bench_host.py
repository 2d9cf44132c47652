"""bench.py's host-side logic, on the CPU: the one-GPU guard, the counter
summary (FETCH_SIZE / WRITE_SIZE scaled by the runtime copy kernel of known
size), and the rule that a stored traffic figure is used only while the
kernel source is the one that was profiled."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402

FANOUT = ("void ms::dispatch_fanout_kernel<1, true, 4, 2>(unsigned int __vector(4) const*, "
          "unsigned int __vector(4)*, int const*, int, long, int const*, ms::RowSplit, int const*)")
COPY = "__amd_rocclr_copyBuffer"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, counter, value) in enumerate(rows):
            w.writerow([i + 1, name, counter, value])


def test_counter_summary_scales_by_the_copy_kernel(tmp_path):
    cfg = synth.CONFIGS[0]
    copy_bytes = min(cfg.T * cfg.k * cfg.H * 2, 2 << 30)
    # the copy reads copy_bytes / 2 KiB on FETCH_SIZE (scale 2) and copy_bytes KiB on WRITE_SIZE (scale 1)
    fetch_kib, write_kib = 100.0, 30.0
    _counter_csv(tmp_path / "fetch.csv", [(COPY, "FETCH_SIZE", copy_bytes / 2 / 1024),
                                          (FANOUT, "FETCH_SIZE", fetch_kib), (FANOUT, "FETCH_SIZE", fetch_kib)])
    _counter_csv(tmp_path / "write.csv", [(COPY, "WRITE_SIZE", copy_bytes / 1024),
                                          (FANOUT, "WRITE_SIZE", write_kib), (FANOUT, "WRITE_SIZE", write_kib)])
    with open(tmp_path / "stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow([FANOUT, 2, 2000, 1000.0, 100, 900, 1100, 0])
    out = tmp_path / "out"
    out.mkdir()
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--pmc-summary", "--config", "0",
                        "--src-sha", "0123456789abcdef", "--fetch-csv", str(tmp_path / "fetch.csv"),
                        "--write-csv", str(tmp_path / "write.csv"), "--trace-stats", str(tmp_path / "stats.csv"),
                        "--out-dir", str(out)], capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "--commands" in r.stderr, "a summary without its commands is refused"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--pmc-summary", "--config", "0",
                        "--src-sha", "0123456789abcdef", "--fetch-csv", str(tmp_path / "fetch.csv"),
                        "--write-csv", str(tmp_path / "write.csv"), "--trace-stats", str(tmp_path / "stats.csv"),
                        "--out-dir", str(out), "--commands", "rocprofv3 --pmc FETCH_SIZE ..."],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert "    rocprofv3 --pmc FETCH_SIZE ..." in (out / f"kernels_{cfg.name}.md").read_text()
    rec = json.load(open(out / f"traffic_dispatch_fanout_kernel_{cfg.name}.json"))
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["hbm_bytes_per_launch"] == round(fetch_kib * 1024 * 2 + write_kib * 1024)
    idx, _ = synth.make_routing(cfg, 0)
    N = bench.n_rank_rows(idx, cfg.E, cfg.R)
    assert rec["alg_bytes_per_launch"] == bench.algorithmic_bytes(cfg.T, cfg.H, cfg.k, N)["fanout"]
    assert rec["kernel_src_sha256_16"] == "0123456789abcdef"
    assert (out / f"kernels_{cfg.name}.md").exists()


def test_path_counter_summary_sums_the_kernels_of_each_call(tmp_path, monkeypatch):
    """--path backward: the three kernels of the combine backward count as
    one call; counters equal to the algorithmic bytes give a ratio of 1."""
    cfg = synth.CONFIGS[0]
    copy_bytes = bench.copy_bytes_of(cfg.T, cfg.H, cfg.k)
    idx, _ = synth.make_routing(cfg, 0)
    N = bench.n_rank_rows(idx, cfg.E, cfg.R)
    B = bench.path_bytes("backward", cfg.T, cfg.H, cfg.k, N)
    sig = "(unsigned int __vector(4) const*, int)"
    # the combine backward's bytes split over its three kernels, all reads (FETCH_SIZE scale 2)
    parts = {"void ms::combine_bwd_grad_kernel<1, true>": B["combine_bwd"] * 0.5,
             "void ms::combine_bwd_dot_kernel<2, true>": B["combine_bwd"] * 0.25,
             "ms::gate_grad_kernel": B["combine_bwd"] * 0.25,
             "void ms::sum_expert_rows_kernel<2, true, 0, 4, 8, 1, 0>": B["sum_expert_rows"],
             "void ms::sum_rank_rows_kernel<1, true, 0, 4, 8, 1, 0>": B["sum_rank_rows"]}
    fetch = [(COPY, "FETCH_SIZE", copy_bytes / 2 / 1024)]
    write = [(COPY, "WRITE_SIZE", copy_bytes / 1024)]
    for name, b in parts.items():
        for _ in range(3):  # three launches of each, same counts
            fetch.append((name + sig, "FETCH_SIZE", b / 2 / 1024))
            write.append((name + sig, "WRITE_SIZE", 0.0))
    _counter_csv(tmp_path / "fetch.csv", fetch)
    _counter_csv(tmp_path / "write.csv", write)
    with open(tmp_path / "stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        for name in parts:
            w.writerow([name + sig, 3, 3000, 1000.0, 20, 900, 1100, 0])
    out = tmp_path / "profiles"
    out.mkdir()
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--pmc-summary", "--path", "backward",
                        "--config", "0", "--src-sha", bench.source_digest(),
                        "--fetch-csv", str(tmp_path / "fetch.csv"),
                        "--write-csv", str(tmp_path / "write.csv"), "--trace-stats", str(tmp_path / "stats.csv"),
                        "--out-dir", str(out), "--commands", "rocprofv3 ..."],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    text = open(out / f"kernels_backward_{cfg.name}.md").read()
    calls = {ln.split("|")[1].strip(): ln.split("|") for ln in text.splitlines()
             if ln.startswith("| combine_bwd") or ln.startswith("| sum_")}
    assert set(calls) == {"combine_bwd", "sum_expert_rows", "sum_rank_rows"}
    assert calls["combine_bwd"][2].strip() == "combine_bwd_dot_kernel, combine_bwd_grad_kernel, gate_grad_kernel"
    assert float(calls["combine_bwd"][3]) == pytest.approx(3.0)  # three kernels of 1 us each
    for c in calls.values():
        assert c[7].strip() == "1.000"
    # one traffic record per call, read back by the bench of that path
    rec = json.load(open(out / f"traffic_backward_combine_bwd_{cfg.name}.json"))
    assert rec["hbm_bytes_per_call"] == round(B["combine_bwd"])
    assert rec["kernels"] == ["combine_bwd_dot_kernel", "combine_bwd_grad_kernel", "gate_grad_kernel"]
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_path_traffic(cfg.name, "backward", ("combine_bwd",)) == round(B["combine_bwd"])
    both = bench.load_path_traffic(cfg.name, "backward", ("sum_expert_rows", "sum_rank_rows"))
    assert both == round(B["sum_expert_rows"]) + round(B["sum_rank_rows"])
    assert bench.load_path_traffic(cfg.name, "rank-partial", ("sum_rank_rows",)) is None  # not profiled


def test_stored_traffic_is_used_only_for_the_profiled_source(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    path = tmp_path / "profiles" / "traffic_dispatch_fanout_kernel_w.json"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    json.dump({"data_kernel_src_sha256_16": bench.data_source_digest(), "hbm_bytes_per_launch": 1234},
              open(path, "w"))
    assert bench.load_traffic("w", "fanout") == 1234
    json.dump({"data_kernel_src_sha256_16": "not-this-source", "hbm_bytes_per_launch": 1234}, open(path, "w"))
    assert bench.load_traffic("w", "fanout") is None
    # a record stamped with the hash of every source, plan included, is not enough
    json.dump({"kernel_src_sha256_16": bench.source_digest(), "hbm_bytes_per_launch": 1234}, open(path, "w"))
    assert bench.load_traffic("w", "fanout") is None
    assert bench.load_traffic("absent", "fanout") is None


def test_row_kernel_hash_leaves_out_only_the_plan():
    """The traffic records cover row kernels only; their hash covers every
    device source except the plan's, so a plan change keeps them valid and a
    row-kernel change drops them."""
    assert "plan.hip" in bench.KERNEL_SRCS and "plan.hip" not in bench.DATA_KERNEL_SRCS
    assert set(bench.KERNEL_SRCS) - set(bench.DATA_KERNEL_SRCS) == {"plan.hip"}
    assert bench.data_source_digest() == bench.source_digest(bench.DATA_KERNEL_SRCS)
    assert bench.data_source_digest() != bench.source_digest()


def test_algorithmic_bytes_count_each_step_once():
    # T = 1, H = 8 (16-byte rows), k = 2 experts on N = 2 ranks: every term by hand
    b = bench.algorithmic_bytes(1, 8, 2, 2)
    row = 16
    assert b["send"] == row * (1 + 2) + 4 * 2           # read x once, write 2 rank rows, 2 indices
    assert b["fanout"] == row * (2 + 2) + 4 * 2         # read 2 rank rows, write 2 expert rows
    assert b["combine"] == row * (2 + 1) + 8 * 2        # read 2 expert rows, write 1, rows + gates
    assert b["total"] == b["send"] + b["fanout"] + b["combine"]


def test_occupancy_and_latency_summary_derives_each_figure(tmp_path):
    """--counter-summary: each derived column follows its stated formula
    from the per-dispatch means (G = GRBM_GUI_ACTIVE / XCDs), a dispatch
    counts once however many counter rows it has, the "_sum" suffix of a
    counter name is dropped, and the title carries the kernel source hash."""
    G, cus, wpc, xcc = 1000.0, 256, 32, 8
    counters = {
        "GRBM_GUI_ACTIVE": G * xcc,
        "SQ_WAVE_CYCLES": 0.5 * G * cus * wpc / 4,      # occupancy 0.50
        "SQ_WAIT_INST_ANY": 0.25 * 0.5 * G * cus * wpc / 4,  # issue wait 0.25
        "TCP_TCC_READ_REQ_sum": 1000.0,
        "TCP_TCC_READ_REQ_LATENCY_sum": 1000.0 * 1500,  # 1500 cycles; 5.9 reads in flight per CU
        "TCP_PENDING_STALL_CYCLES_sum": 0.75 * G * cus,  # 0.75
        "TA_TA_BUSY_sum": 0.5 * G * cus,                 # 0.50
        "TCC_EA0_RDREQ_sum": 2000.0,
        "TCC_EA0_RDREQ_LEVEL_sum": 2000.0 * 2000,        # 2000 cycles; 4000 reads in flight
        "TCC_EA0_WRREQ_LEVEL_sum": 3000.0 * G,           # 3000 writes in flight
    }
    name = "void ms::combine_rows_kernel<1, true, 1, 4, 8, 1, 0>(unsigned int __vector(4) const*)"
    d = tmp_path / "pass"
    d.mkdir()
    with open(d / "pmc_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"])
        for i, (c, v) in enumerate(counters.items()):  # two dispatches, one row per counter each
            w.writerow([1, name, c, v, 1000, 1000 + 183000])
            w.writerow([2, name, c, v, 1000, 1000 + 185000])
        w.writerow([3, "void ms::plan_count_kernel<8>(int const*)", "GRBM_GUI_ACTIVE", 1.0, 0, 1000])
    with open(d / "pmc_agent_info.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Node_Id", "Name", "Num_Xcc", "Cu_Count", "Max_Waves_Per_Cu"])
        w.writerow([0, "AMD EPYC", 0, 0, 0])
        w.writerow([1, "gfx950", xcc, cus, wpc])
    out = tmp_path / "out"
    out.mkdir()
    base = [sys.executable, os.path.join(ROOT, "bench.py"), "--counter-summary", "--counter-csv",
            str(d / "pmc_counter_collection.csv"), "--kernel-filter", "combine_rows", "--out-dir", str(out),
            "--out-name", "c.md", "--src-sha", "0123456789abcdef"]
    r = subprocess.run(base, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "--commands" in r.stderr, "a summary without its commands is refused"
    r = subprocess.run(base + ["--title", "combine", "--commands", "rocprofv3 --pmc ..."], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    text = (out / "c.md").read_text()
    assert text.splitlines()[0] == "# Counters — combine (kernel source sha256[:16] 0123456789abcdef)"
    assert "    rocprofv3 --pmc ..." in text
    rows = [ln for ln in text.splitlines() if ln.startswith("| `")]
    assert len(rows) == 1 and "plan_count" not in text  # the filter keeps the combine only
    cells = [c.strip() for c in rows[0].strip("|").split("|")]
    assert cells[0] == "`ms::combine_rows_kernel<1, true, 1, 4, 8, 1, 0>`"
    assert cells[1:] == ["2", "184.0", "0.50", "0.25", "1500", "5.9", "0.75", "0.50", "2000", "4000", "3000"]


def test_path_summary_keeps_the_figures_the_forward_line_reports():
    rec = {"ms_per_step": 0.8, "value": 5800.0, "frac_of_peak": 0.725, "tokens_per_s": 1.0e7,
           "kernel_us": {"combine_bwd": 365.0}, "algorithmic_bytes": {"total": 4.6e9, "combine_bwd": 2e9},
           "roofline": {"kernel": "combine_bwd", "frac": 0.68, "traffic": 2.1e9, "peak": 8000.0},
           "parity": {"grad_x_bitexact": True}, "config": {"T": 8192}}
    s = bench.path_summary(rec)
    assert s == {"ms_per_step": 0.8, "GBps": 5800.0, "frac_of_peak": 0.725, "tokens_per_s": 1.0e7,
                 "kernel_us": {"combine_bwd": 365.0}, "algorithmic_bytes": 4.6e9,
                 "roofline": {"kernel": "combine_bwd", "frac": 0.68, "traffic": 2.1e9},
                 "parity": {"grad_x_bitexact": True}}
