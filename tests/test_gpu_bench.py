"""bench.py's JSON line on the GPU (in this process, step only): the keys,
types and relations the benchmark contract fixes."""
import json
import sys

import pytest

import bench

pytestmark = pytest.mark.gpu


def test_step_only_line(monkeypatch, capsys):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[case] bench.py --step-only --steps 3 --warmup 1", file=sys.stderr, flush=True)
    monkeypatch.setattr(sys, "argv", ["bench.py", "--step-only", "--steps", "3", "--warmup", "1"])
    bench.main()
    out = capsys.readouterr().out
    lines = [ln for ln in out.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, out
    d = json.loads(lines[0])
    assert d["metric"] == bench.METRIC and d["unit"] == "GB/s"
    assert (d["n_gpus"], d["steps"], d["warmup"]) == (1, 3, 1)
    assert d["higher_is_better"] is True and d["scaling"] == "weak"
    assert d["vs_baseline"] is None and d["dtype"] == "bf16" and "synthetic" in d["data"]
    assert d["config"]["workload"] == "r16-e384-k8-s8192-h7168-dedup"
    assert d["ms_per_step"] > 0 and d["value"] > 0
    # value = the step's dispatch+combine bytes over the step time
    b = d["bytes_per_step"]
    assert d["value"] == pytest.approx((b["dispatch"] + b["combine"]) / (d["ms_per_step"] * 1e-3)
                                       / 1e9, rel=2e-3)
    # the roofline is the longer-running of the step's two bulk kernels
    assert set(d["kernels"]) == {"k_dispatch_scatter", "k_combine_staged"}
    r = d["roofline"]
    assert r == max(d["kernels"].values(), key=lambda k: k["avg_launch_us"])
    for r in d["kernels"].values():
        assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.PEAK_HBM_GBPS
        assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-4)
        assert r["achieved"] == pytest.approx(r["algorithmic_bytes_per_launch"] /
                                              (r["avg_launch_us"] * 1e-6) / 1e9, rel=2e-3)
        assert r["traffic"] is None or r["traffic"] > 0
    assert d["kernels"]["k_dispatch_scatter"]["algorithmic_bytes_per_launch"] == \
        pytest.approx(b["dispatch"], rel=1e-6)
    assert set(d["call_us"]) == {"plan", "dispatch", "combine"}
    assert "cpu_baseline" in d and d["cpu_baseline"] is None  # not taken in a step-only run
