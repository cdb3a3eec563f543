"""Host-side checks of bench.py's arithmetic (no GPU): the algorithmic byte counts behind
the HBM rooflines, the counter-record summariser and its calibration scaling, and that a
traffic record taken on another kernel source is ignored."""
import csv
import json
import os

import pytest

import bench
from linear_cross_entropy_lm_amd import inputs as I


def test_ce_row_bytes():
    # forward: the row (V es) + label (8) + lse (4) + loss term (8) + flag (4)
    # backward: the row read and written (2 V es) + label (8) + lse (4)
    assert bench.ce_row_bytes(128256, 2) == (128256 * 2 + 24, 4 * 128256 + 12)
    assert bench.ce_row_bytes(7, 4) == (7 * 4 + 24, 2 * 7 * 4 + 12)


def test_norm_bytes():
    N, D, es, grid = 16384, 4096, 2, 512
    fwd, bwd = bench.norm_bytes(N, D, es, grid)
    assert fwd == 2 * N * D * es + 4 * N + D * es
    groups = 16  # 512 partial rows summed 32 at a time
    assert bwd == 3 * N * D * es + 4 * N + D * es + 2 * grid * D * 4 + 2 * groups * D * 4 + D * 4
    assert bench.norm_bytes(3, 8, 4, 3)[1] == 3 * 3 * 8 * 4 + 12 + 32 + 2 * 3 * 8 * 4 + 2 * 1 * 8 * 4 + 32


def _write_counters(path, kernel, counter, values, tag="x"):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, f"{tag}_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, v in enumerate(values):
            # two rows per dispatch (per-XCD style pieces) that the reader must add up
            w.writerow([i, f"void {kernel}(int)", counter, v / 2])
            w.writerow([i, f"void {kernel}(int)", counter, v / 2])
        w.writerow([99, "other_kernel", counter, 1e9])


@pytest.mark.parametrize("path,kinds", [("fused", ["fwd_tiles16", "bwd_dz16", "bwd_dhdw"]),
                                        ("single", ["fwd_tiles16_keep", "bwd_dhdw"]), ("ce", ["ce_rows_bwd"]),
                                        ("norm", ["rms_bwd"])])
def test_summarize_counters_scales_by_the_copy(tmp_path, monkeypatch, path, kinds):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    root = tmp_path / "cnt"
    copy = 1 << 30
    names = {"fwd_tiles16": "(anonymous namespace)::fwd_tiles16<unsigned short, false>",
             "fwd_tiles16_keep": "(anonymous namespace)::fwd_tiles16<unsigned short, true>",
             "bwd_dz16": "(anonymous namespace)::bwd_dz16<unsigned short>",
             "bwd_dhdw": "(anonymous namespace)::bwd_dhdw<unsigned short, true, false, true>",
             "ce_rows_bwd": "(anonymous namespace)::ce_rows_bwd<1>", "rms_bwd": "(anonymous namespace)::rms_bwd<1, 2>"}
    for i, kind in enumerate(kinds):
        _write_counters(root / "F", names[kind], "FETCH_SIZE", [1000.0 * (i + 1), 3000.0 * (i + 1)], f"k{i}")
        _write_counters(root / "W", names[kind], "WRITE_SIZE", [500.0, 500.0], f"k{i}")
    # a 1 GiB copy whose counters read half the fetched bytes and all the written bytes
    _write_counters(root / "FC", "__amd_rocclr_copyBuffer", "FETCH_SIZE", [copy / 2048.0])
    _write_counters(root / "WC", "__amd_rocclr_copyBuffer", "WRITE_SIZE", [copy / 1024.0])
    recs = bench.summarize_counters(str(root), copy, path, kinds, "w")
    for i, (kind, rec) in enumerate(zip(kinds, recs)):
        assert rec["fetch_kib_per_launch"] == 2000.0 * (i + 1) and rec["write_kib_per_launch"] == 500.0
        assert rec["fetch_factor"] == pytest.approx(2.0) and rec["write_factor"] == pytest.approx(1.0)
        assert rec["hbm_bytes_per_launch"] == pytest.approx(2000.0 * (i + 1) * 1024 * 2 + 500.0 * 1024)
        saved = json.loads(open(bench.traffic_path(kind, "w", path)).read())
        assert saved["source_digest"] == bench.source_digest(path)
        assert bench.load_traffic(kind, "w", path) == pytest.approx(rec["hbm_bytes_per_launch"])


def test_kernel_patterns_tell_the_forward_variants_apart():
    import re
    plain = "void (anonymous namespace)::fwd_tiles16<(anonymous namespace)::h16, false>(int)"
    keep = "void (anonymous namespace)::fwd_tiles16<unsigned short, true>(int)"
    assert re.search(bench.KINDS["fwd_tiles16"][0], plain) and not re.search(bench.KINDS["fwd_tiles16"][0], keep)
    assert re.search(bench.KINDS["fwd_tiles16_keep"][0], keep)
    assert not re.search(bench.KINDS["fwd_tiles16_keep"][0], plain)


def test_traffic_record_of_another_source_is_ignored(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    with open(bench.traffic_path("bwd_dhdw", "llama3"), "w") as f:
        f.write(json.dumps({"source_digest": "0" * 16, "workload": "llama3", "hbm_bytes_per_launch": 1.0}))
    assert bench.load_traffic("bwd_dhdw", "llama3") is None


def test_single_pass_record_does_not_shadow_the_default_one(tmp_path, monkeypatch):
    """The dH + dW launch runs in both schedules at other chunk shapes: each schedule's
    record has its own file and is only read back under that schedule."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.traffic_path("bwd_dhdw", "llama3", "single") != bench.traffic_path("bwd_dhdw", "llama3", "fused")
    for path, value in (("fused", 1.0), ("single", 20.0)):
        with open(bench.traffic_path("bwd_dhdw", "llama3", path), "w") as f:
            f.write(json.dumps({"source_digest": bench.source_digest(path), "workload": "llama3", "path": path,
                                "hbm_bytes_per_launch": value}))
    assert bench.load_traffic("bwd_dhdw", "llama3", "fused") == 1.0
    assert bench.load_traffic("bwd_dhdw", "llama3", "single") == 20.0
    # a record written under one schedule and copied to the other's name is refused
    os.replace(bench.traffic_path("bwd_dhdw", "llama3", "fused"), bench.traffic_path("bwd_dhdw", "llama3", "single"))
    assert bench.load_traffic("bwd_dhdw", "llama3", "single") is None


def test_chunk_spans_partition_whole_tiles():
    for total, chunk in [(16384, 4096), (128256, 8192), (4097, 4096), (300, 4096), (152064, 8192)]:
        spans = bench.chunk_spans(total, chunk)
        assert spans[0][0] == 0 and sum(r for _, r in spans) == total
        for (a, r), (b, _) in zip(spans, spans[1:]):
            assert a + r == b and a % 256 == 0 and r % 256 == 0 and r <= chunk
        assert spans[-1][1] <= chunk
    assert bench.chunk_spans(128256, 8192)[0] == (0, 7936)  # 501 tiles over 16 chunks: 31 or 32 tiles


@pytest.mark.parametrize("path,tc,vc", [("fused", 4096, 8192), ("single", 4096, 0), ("single", 8192, 0)])
def test_gemm_launch_flops_cover_the_work_once(path, tc, vc):
    """The GEMM launches of a step add up to the forward (2 N V D; the single pass's keep
    forward) and the backward's contractions (two of 2 N V D for dH and dW, and the dz
    recompute's 2 N V D on the recomputing path)."""
    N, D, V = 16384, 4096, 128256
    launches = bench.gemm_launch_flops(path, N, D, V, tc, vc)
    assert sum(f for _, f in launches) == pytest.approx((4.0 if path == "fused" else 3.0) * 2.0 * N * V * D)
    for kind in bench.GEMM_KINDS[path]["f16"]:
        ids = set(bench.KINDS[kind][1])
        contractions = 2 if kind == "bwd_dhdw" else 1
        assert sum(f for k, f in launches if k in ids) == pytest.approx(contractions * 2.0 * N * V * D)
    if path == "fused":
        assert [k for k, _ in launches] == [0] + [5, 6] * 64
    else:
        assert [k for k, _ in launches] == [1, 6] * (N // tc)


def test_more_than_one_gpu_is_refused(capsys, monkeypatch):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    assert bench.main() == 2
    assert "one GPU" in capsys.readouterr().err


def test_code_digest_ignores_comments_only():
    src = "int f(int x) {  // doubles x\n  return 2 * x; /* twice */ }\n"
    same = "// header\nint f(int x) {\n  return 2 * x;\n}\n"
    other = "int f(int x) { return 3 * x; }\n"
    assert bench.code_digest(src) == bench.code_digest(same)
    assert bench.code_digest(src) != bench.code_digest(other)


def test_summarize_occupancy(tmp_path):
    """Two dispatches of one kernel lasting 1 ms each at 2.0 GHz: GRBM_GUI_ACTIVE is summed
    over the 8 XCDs (8 x 2e6 cycles); MFMA busy half of every SIMD's cycles; LDS active a
    quarter of every CU's; a kernel shorter than 100 us is left out."""
    cyc = 2e6
    vals = {"GRBM_GUI_ACTIVE": 8 * cyc, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * cyc * 1024,
            "SQ_LDS_IDX_ACTIVE": 0.25 * cyc * 256, "SQ_LDS_BANK_CONFLICT": 0.01 * cyc * 256,
            "SQ_LDS_ADDR_CONFLICT": 0.0, "SQ_BUSY_CU_CYCLES": cyc * 256 / 4,
            "SQ_WAIT_INST_LDS": 0.1 * cyc * 1024 / 4, "SQ_LDS_DATA_FIFO_FULL": 0.0}
    assert set(vals) == set(bench.OCCUPANCY_COUNTERS)
    with open(tmp_path / "p_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name", "Counter_Value",
                    "Start_Timestamp", "End_Timestamp"])
        for d, (name, dur) in enumerate([("void (anonymous namespace)::gemm<bf16>(int)", 1_000_000)] * 2
                                        + [("void small(int)", 50_000)]):
            for c, v in vals.items():
                w.writerow([d, name, 131072, 512, c, v, 1000, 1000 + dur])
    recs = bench.summarize_occupancy(str(tmp_path))
    assert len(recs) == 1
    r = recs[0]
    assert (r["kernel"], r["grid"], r["workgroup"], r["dispatches"]) == ("gemm<bf16>", 256, 512, 2)
    assert r["mean_us"] == pytest.approx(1000.0) and r["clock_ghz"] == pytest.approx(2.0)
    assert r["mfma_busy"] == pytest.approx(0.5) and r["mfma_busy_ghz"] == pytest.approx(1.0)
    assert r["lds_active"] == pytest.approx(0.25) and r["lds_bank_conflict"] == pytest.approx(0.01)
    assert r["lds_issue_wait"] == pytest.approx(0.1)


def test_summarize_memstall(tmp_path):
    """Two dispatches of 1 ms at 2.0 GHz: 80% L2 hits, 400 cycles (200 ns) per L1 read
    request to the L2, pending stalls on a quarter of every CU's cycles; a dispatch missing
    a counter is left out."""
    cyc = 2e6
    vals = {"GRBM_GUI_ACTIVE": 8 * cyc, "SQ_VALU_MFMA_BUSY_CYCLES": 0.6 * cyc * 1024, "TCC_HIT_sum": 800.0,
            "TCC_MISS_sum": 200.0, "TCP_TCC_READ_REQ_LATENCY_sum": 400.0 * 5000, "TCP_TCC_READ_REQ_sum": 5000.0,
            "TCP_PENDING_STALL_CYCLES_sum": 0.25 * cyc * 256}
    assert set(vals) == set(bench.MEMSTALL_COUNTERS)
    with open(tmp_path / "s_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                    "End_Timestamp"])
        for d in range(2):
            for c, v in vals.items():
                w.writerow([d, "void (anonymous namespace)::gemm<bf16>(int)", c, v, 1000, 1_001_000])
        w.writerow([2, "void (anonymous namespace)::gemm<bf16>(int)", "GRBM_GUI_ACTIVE", 1.0, 1000, 1_001_000])
    recs = bench.summarize_memstall(str(tmp_path))
    assert len(recs) == 1
    r = recs[0]
    assert (r["kernel"], r["dispatches"]) == ("gemm<bf16>", 2)
    assert r["clock_ghz"] == pytest.approx(2.0) and r["mfma_busy"] == pytest.approx(0.6)
    assert r["l2_hit"] == pytest.approx(0.8)
    assert r["l1_l2_read_latency_cycles"] == pytest.approx(400.0) and r["l1_l2_read_latency_ns"] == pytest.approx(200.0)
    assert r["l1_pending_stall"] == pytest.approx(0.25)


def test_summarize_mops(tmp_path):
    """Two calls of the recomputing schedule at the tiny workload: per call a forward of
    2 N V D, a dz recompute of 2 N V D and two dH + dW launches of 2 N V D each (flops over
    512 in the counter, on two counters' rows), and one fwd_finalize: executed equals the
    credited 8 N V D per call."""
    cfg = I.CONFIGS["tiny_f32"]
    unit = 2 * cfg.N * cfg.V * cfg.D
    rows = []
    for call in range(2):
        rows += [("void (anonymous namespace)::fwd_tiles<float, false>(int)", unit),
                 ("void (anonymous namespace)::bwd_dz<float>(int)", unit),
                 ("void (anonymous namespace)::bwd_dhdw<float, false, false, false>(int)", unit),
                 ("void (anonymous namespace)::bwd_dhdw<float, true, false, false>(int)", unit),
                 ("void (anonymous namespace)::fwd_finalize(int)", 0)]
    with open(tmp_path / "m_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d, (name, flop) in enumerate(rows):
            w.writerow([d, name, "SQ_INSTS_VALU_MFMA_MOPS_F32", flop / 512 * 0.75])
            w.writerow([d, name, "SQ_INSTS_VALU_MFMA_MOPS_F32", flop / 512 * 0.25])
            w.writerow([d, name, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 0])
            w.writerow([d, name, "GRBM_GUI_ACTIVE", 123456])
    recs = bench.summarize_mops(str(tmp_path), "tiny_f32")
    per = {r["kernel"]: r for r in recs[:-1]}
    assert set(per) == {"fwd_tiles<float, false>", "bwd_dz<float>", "bwd_dhdw<float, false, false, false>",
                        "bwd_dhdw<float, true, false, false>"}
    assert all(r["dispatches"] == 2 and r["tflop_per_dispatch"] == pytest.approx(unit / 1e12) for r in per.values())
    tot = recs[-1]
    assert tot["calls"] == 2 and tot["executed_over_credited"] == pytest.approx(1.0)
    assert tot["credited_tflop_per_call"] == pytest.approx(4 * unit / 1e12)
    assert bench.summarize_mops(str(tmp_path), "tiny_f32", "single")[-1]["executed_over_credited"] == pytest.approx(4 / 3)


def test_parse_sclk():
    assert bench._parse_sclk_mhz("0: 500Mhz\n1: 1650Mhz *\n2: 2400Mhz\n") == 1650.0
    assert bench._parse_sclk_mhz("S: 1423MHz *\n") == 1423.0
    assert bench._parse_sclk_mhz("0: 500Mhz\n1: 2400Mhz\n") is None


def test_sclk_sampler_reads_the_current_level(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 1700Mhz *\n2: 2400Mhz\n")
    with bench.SclkSampler(str(f), period=0.001) as s:
        import time
        t0 = time.time()
        while len(s.samples) < 3 and time.time() - t0 < 5:
            time.sleep(0.005)
    r = s.summary()
    assert r["median"] == 1700.0 and r["min"] == 1700.0 and r["samples"] >= 3
    with bench.SclkSampler(None) as s:
        pass
    assert s.summary() is None


def test_traffic_record_of_another_workload_is_ignored(tmp_path, monkeypatch):
    """A record taken on the Llama-3 workload does not describe a run on another one."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    with open(bench.traffic_path("bwd_dhdw", "llama3"), "w") as f:
        f.write(json.dumps({"source_digest": bench.source_digest("fused"), "workload": "llama3",
                            "hbm_bytes_per_launch": 5.0}))
    assert bench.load_traffic("bwd_dhdw", "llama3") == 5.0
    assert bench.load_traffic("bwd_dhdw", "llama2") is None


def test_metric_names_the_sizes_that_ran():
    """The headline workload keeps the headline metric text; any other reports its own sizes."""
    from linear_cross_entropy_lm_amd import inputs as I
    assert bench.workload_metric(bench.METRIC, I.CONFIGS["llama3"]) == bench.METRIC
    m = bench.workload_metric(bench.METRIC, I.CONFIGS["llama2"])
    assert "N=4096,D=4096,V=32000" in m and "16384" not in m
    assert "fp16 MFMA peak" in bench.workload_metric(bench.METRIC_SINGLE, I.CONFIGS["llama3_f16"])
    assert bench.workload_metric(bench.METRIC_CE, I.LOGIT_CONFIGS["ce_llama3"]) == bench.METRIC_CE
    assert bench.workload_metric(bench.METRIC_NORM, I.NORM_CONFIGS["norm_llama3"]) == bench.METRIC_NORM
