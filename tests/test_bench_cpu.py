"""bench.py's host-side contract, without a GPU: it refuses more than one GPU,
its source hashes ignore comments (they decide whether recorded counter
readings still apply), and its rocprofv3 summarizers turn counter and trace
CSV folders into the figures the bench line reports."""
import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def test_code_hash_ignores_comments_not_code():
    c = "int f(int x) {\n  // twice\n  return 2 * x; /* doubled */\n}\n"
    c_comment = "int f(int x) {\n  // two times x\n  return 2 * x;   /* x + x */\n}\n"
    c_code = "int f(int x) {\n  // twice\n  return 3 * x; /* doubled */\n}\n"
    assert bench._code_only(c, "a.hip") == bench._code_only(c_comment, "a.hip")
    assert bench._code_only(c, "a.hip") != bench._code_only(c_code, "a.hip")
    p = "def f(x):\n    # twice\n    return 2 * x\n"
    assert bench._code_only(p, "a.py") == bench._code_only(p.replace("twice", "doubled"), "a.py")
    assert bench._code_only(p, "a.py") != bench._code_only(p.replace("2 *", "3 *"), "a.py")


def test_kernel_sources_follow_the_kernel_file():
    assert bench.kernel_sources("k_combine<false, 1, 2>")[-1].endswith("moon_combine.hip")
    assert bench.kernel_sources("k_dispatch_expand<4, 1, true>")[-1].endswith("moon_dispatch.hip")
    assert bench.kernel_sources("k_plan_place")[-1].endswith("moon_plan.hip")
    for k in ("k_combine", "k_plan_count"):
        assert set(bench.PMC_COMMON) <= set(bench.kernel_sources(k))


def _write_csv(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _counters(path, launches):
    """launches: [(full kernel name, KiB)]"""
    _write_csv(path, ["Kernel_Name", "Counter_Name", "Counter_Value"],
               [{"Kernel_Name": n, "Counter_Name": "X", "Counter_Value": v} for n, v in launches])


K_COMBINE = "void moon::(anonymous namespace)::k_combine<false, 1, 2>(moon::Dims, ...)"
K_EXPAND = "void moon::(anonymous namespace)::k_dispatch_expand<4, 1, true>(moon::Dims, ...)"
COPY = "void at::native::vectorized_elementwise_kernel<4>(int, ...)"


def test_pmc_summary_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    os.makedirs(bench.PROFILES)
    d = tmp_path / "raw"
    # step runs: two combine launches, three expand launches of another
    # instantiation (the most-launched instantiation is the one reported)
    _counters(str(d / "f" / "run_counter_collection.csv"),
              [(K_COMBINE, 1000.0), (K_COMBINE, 1200.0)] + [(K_EXPAND, 300.0)] * 3 +
              [(COPY, 5.0)])
    _counters(str(d / "w" / "run_counter_collection.csv"),
              [(K_COMBINE, 500.0), (K_COMBINE, 500.0)] + [(K_EXPAND, 100.0)] * 3 +
              [(COPY, 5.0)])
    # calibration: a 1 GiB copy read as 0.5 GiB by the fetch counter, 1 GiB written
    gib_kib = (1 << 30) / 1024.0
    _counters(str(d / "cf" / "run_counter_collection.csv"), [(COPY, gib_kib / 2)] * 5)
    _counters(str(d / "cw" / "run_counter_collection.csv"), [(COPY, gib_kib)] * 5)
    bench.summarize_pmc("wl-test", [str(d / x) for x in ("f", "w", "cf", "cw")], ["cmd"])
    rec = json.load(open(os.path.join(bench.PROFILES, "pmc_wl-test.json")))
    assert rec["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert rec["calibration"]["write_factor"] == pytest.approx(1.0)
    k = rec["kernels"]["k_combine<false, 1, 2>"]
    assert k["launches"] == 2
    assert k["hbm_bytes_per_launch"] == int(1100.0 * 1024 * 2.0 + 500.0 * 1024 * 1.0)
    assert "vectorized_elementwise_kernel<4>" not in json.dumps(rec["kernels"])
    # read back through the bench's lookup: the hashes match the current sources
    assert bench.measured_traffic("k_combine", "wl-test") == k["hbm_bytes_per_launch"]
    assert bench.measured_traffic("k_dispatch_expand", "wl-test") == \
        int(300.0 * 1024 * 2.0 + 100.0 * 1024 * 1.0)
    assert bench.measured_traffic("k_plan_place", "wl-test") is None
    # a recorded hash that no longer matches its source voids the reading
    rec["source_hashes"][bench.PMC_COMMON[0]] = "0" * 16
    json.dump(rec, open(os.path.join(bench.PROFILES, "pmc_wl-test.json"), "w"))
    assert bench.measured_traffic("k_combine", "wl-test") is None


def test_trace_summary_groups_by_kernel_and_grid(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    os.makedirs(bench.PROFILES)
    rows = []
    t = 0
    for name, grid, ns, n in [(K_COMBINE, 4096, 80000, 3), (K_COMBINE, 1024, 20000, 2),
                              (K_EXPAND, 2048, 30000, 4), (COPY, 64, 10, 1)]:
        for _ in range(n):
            rows.append({"Kernel_Name": name, "Grid_Size_X": grid, "Grid_Size_Y": 1,
                         "Grid_Size_Z": 1, "Start_Timestamp": t, "End_Timestamp": t + ns})
            t += ns + 1000
    _write_csv(str(tmp_path / "tr" / "run_kernel_trace.csv"),
               ["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Start_Timestamp",
                "End_Timestamp"], rows)
    log = tmp_path / "b.log"
    log.write_text("[bench] noise\n" + json.dumps(
        {"ms_per_step": 0.2, "call_us": {"combine": 80.0}, "roofline": {"frac": 0.7}}) + "\n")
    bench.summarize_trace("wl-test", str(tmp_path / "tr"), "the command", str(log))
    md = open(os.path.join(bench.PROFILES, "kernels_wl-test.md")).read().splitlines()
    table = [ln for ln in md if ln.startswith("| k_")]
    assert table[0].startswith("| k_combine<false, 1, 2> | 4096 | 3 | 240.0 | 80.00 |")
    assert table[1].startswith("| k_dispatch_expand<4, 1, true> | 2048 | 4 | 120.0 | 30.00 |")
    assert table[2].startswith("| k_combine<false, 1, 2> | 1024 | 2 | 40.0 | 20.00 |")
    assert any("more lines, each under 0.1 %" in ln for ln in md)  # the 10 ns copy
    assert any(ln.startswith("Bench line of the same run: step 0.2 ms") for ln in md)
    assert "    the command" in md


def test_algorithmic_bytes_by_hand():
    """R=2, S=3, K=3, H=8 (a row is 16 bytes), 1 duplicate group with 2
    duplicate rows, 5 padding rows: every term counted out by hand."""
    nb = bench.bytes_from_counts(2, 3, 3, 8, n_grp=1, n_dup=2, n_pad=5)
    routes, row, tokens = 18, 16, 6
    d_min = (tokens * row        # each token row read once
             + routes * row      # every route's row written
             + 5 * row           # padding rows zeroed
             + routes * 12       # dst read, weight read, weight written
             + 5 * 4             # padding weights zeroed
             + 1 * 12 + 2 * 4)   # the duplicate record and its two row offsets
    assert nb["dispatch"] == d_min  # one pass: duplicates stored from the token's row
    assert nb["dispatch_epilogue"] == d_min + 1 * row  # the epilogue reads the primary once
    assert nb["combine"] == routes * row + tokens * row + routes * 12
    assert bench.plan_counts(np.array([[1, 1], [0, 0]]),
                             np.array([[[3, 5], [7, 7]], [[0, 3], [9, 9]]])) == (1, 1, 5)


def test_cpu_baseline_record():
    """The oracle timed on the host: its plan of the full routing, then one
    pass over the token sample is enough to fill the record the bench line
    carries."""
    import synth
    topk, w = synth.routing("r8-e64-k6", 2000)
    rec = bench.cpu_baseline("r8-e64-k6", topk, w, 2000, budget_s=0.0, sample_tokens=64)
    assert rec["kind"] == "oracle" and rec["cores"] == 1 and rec["unit"] == "GB/s"
    assert rec["value"] > 0 and rec["tokens_per_s"] > 0 and rec["plan_full_ms"] > 0
    assert "the first 64 of the 2048 tokens" in rec["sample"] and ") x 1: plan " in rec["sample"]


def test_stall_summary_divides_by_busy_cycles(tmp_path, monkeypatch):
    """The memory-queue table: per kernel (template arguments dropped, means
    over launches), request counts, queue levels and credit stalls over the
    GPU's busy cycles of the same pass."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    os.makedirs(bench.PROFILES)
    K_SCATTER = "void moon::(anonymous namespace)::k_dispatch_scatter<2, true>(moon::Dims, ...)"
    K_FILL = "(anonymous namespace)::k_fill(unsigned int __vector(4)*, long)"

    def pass_csv(path, values):
        rows = []
        for did, (name, cs) in enumerate(values):
            for c, v in cs.items():
                rows.append({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": c,
                             "Counter_Value": v})
        _write_csv(path, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], rows)

    a = {"TCC_EA0_WRREQ_sum": 400.0, "TCC_EA0_WRREQ_64B_sum": 400.0, "TCC_EA0_RDREQ_sum": 50.0,
         "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum": 10.0, "GRBM_GUI_ACTIVE": 100.0}
    b = {"TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum": 30.0, "TCC_TAG_STALL_sum": 20.0,
         "TCC_EA0_WRREQ_LEVEL_sum": 150000.0, "TCC_EA0_RDREQ_LEVEL_sum": 90000.0,
         "GRBM_GUI_ACTIVE": 100.0}
    a2 = dict(a, TCC_EA0_WRREQ_sum=600.0)  # second launch: mean 500 write requests
    pass_csv(str(tmp_path / "A" / "run_counter_collection.csv"),
             [(K_SCATTER, a), (K_SCATTER, a2), (K_FILL, a)])
    pass_csv(str(tmp_path / "B" / "run_counter_collection.csv"),
             [(K_SCATTER, b), (K_SCATTER, b), (K_FILL, b)])
    bench.summarize_stalls("wl-test", [str(tmp_path / "A"), str(tmp_path / "B")], ["cmd a"])
    md = open(os.path.join(bench.PROFILES, "stalls_wl-test.md")).read().splitlines()
    rows = {ln.split("|")[1].strip(): ln for ln in md if ln.startswith("| k_")}
    assert set(rows) == {"k_dispatch_scatter", "k_fill"}
    cells = [c.strip() for c in rows["k_dispatch_scatter"].split("|")[2:-1]]
    assert cells == ["100", "5.000", "0.500", "1500", "900", "0.300", "0.100", "0.200"]
    assert "    cmd a" in md
