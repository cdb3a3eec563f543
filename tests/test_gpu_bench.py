"""GPU check of bench.py's one-line JSON contract, which the round's benchmark run parses:
the fused path on the Llama-2-shaped workload with a small oracle sample, the single pass
on the same workload and the RMSNorm path, two timed steps each."""
import json
import sys

import pytest
import torch

import bench

pytestmark = pytest.mark.gpu

REQUIRED = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
            "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("argv", [("--workload", "llama2", "--cpu-rows", "2"),
                                  ("--path", "single", "--workload", "llama2", "--no-cpu-baseline"),
                                  ("--path", "norm", "--no-cpu-baseline")],
                         ids=["fused_llama2", "single_llama2", "norm"])
def test_bench_line(monkeypatch, capsys, argv):
    print("bench", " ".join(argv), flush=True)
    monkeypatch.setattr(sys, "argv", ["bench.py", "--steps", "2", "--warmup", "1", *argv])
    assert bench.main() == 0
    d = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    for k in REQUIRED:
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["data"].startswith("synthetic") and "workload" in d["config"] and d["vs_baseline"] is None
    r = d["roofline"]
    assert r["bound"] in ("mfma", "hbm") and r["achieved"] > 0 and 0 < r["frac"] < 1
    if "llama2" in argv:
        assert r["traffic"] is None  # the committed counter records describe other workloads
    if "--path" not in argv or "single" in argv:
        # per-kernel timing: the roofline names the GEMM kind with the largest time per step
        ks = d["kernels"]
        assert r["kernel"] == max(ks, key=lambda k: ks[k]["ms_per_step"])
        for k in ks.values():
            assert k["launches_per_step"] >= 1 and k["mean_us"] > 0 and 0 < k["frac"] < 1
        assert sum(k["ms_per_step"] for k in ks.values()) < d["kernel_timing_step_ms"]
        print("kernels", json.dumps(ks), "timed-launch step", d["kernel_timing_step_ms"], "plain step",
              d["ms_per_step"], flush=True)
    cb = d["cpu_baseline"]
    if "--no-cpu-baseline" in argv:
        assert cb is None
    else:
        assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
