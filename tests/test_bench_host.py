"""Host logic of bench.py (no GPU): the algorithmic work and roofline of a launch, the source
digest that ties a traffic file to the kernels it measured, and the parsers of rocprofv3's
csv output (kernel table, routed-launch selection, counter scaling)."""
import csv
import json
import os

import pytest

import bench


def test_kernel_work_gate_up_and_down():
    # Zipf prefill: 4096 tokens x top-6, hidden 4096, inter 1408, 64 touched MXFP4 experts
    b, f, _, _ = bench.kernel_work("gate_up", 64, 4096, 6, 4096, 1408, 1, False)
    assert f == 2 * 24576 * 4096 * 2 * 1408 == 566_935_683_072
    weights = 64 * 2 * 1408 * 4096 * (0.5 + 1 / 32)  # E2M1 codes + one E8M0 byte per 32
    assert b == pytest.approx(weights + 4096 * 4096 * 2 + 24576 * 1408 * 2)
    b, f, _, _ = bench.kernel_work("down", 64, 4096, 6, 4096, 1408, 1, False)
    assert f == 2 * 24576 * 4096 * 1408
    # fp16 routed prefill outputs, fp32 decode outputs
    y16 = b - 64 * 1408 * 4096 * (0.5 + 1 / 32) - 24576 * 1408 * 2
    assert y16 == pytest.approx(24576 * 4096 * 2)
    b32, _, _, _ = bench.kernel_work("down", 64, 4096, 6, 4096, 1408, 1, True)
    assert b32 - b == pytest.approx(24576 * 4096 * 2)
    # NVFP4: one E4M3 byte per 16 codes
    b, _, _, _ = bench.kernel_work("gate_up", 1, 1, 1, 32, 32, 0, True)
    assert b == pytest.approx(2 * 32 * 32 * (0.5 + 1 / 16) + 32 * 2 + 32 * 2)


def test_roofline_bound_and_fraction():
    ridge = bench.BF16_MFMA_PEAK_TFLOPS * 1e12 / (bench.HBM_PEAK_GBS * 1e9)
    # below the ridge: bytes over time against the HBM peak
    r = bench.roofline(1e9, 0.5 * ridge * 1e9, 0.25)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(4000.0)
    assert r["frac"] == pytest.approx(4000.0 / bench.HBM_PEAK_GBS, abs=1e-4)
    # above it: flops over time against the bf16 MFMA peak
    r = bench.roofline(1e9, 2 * ridge * 1e9, 1.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(2 * ridge * 1e9 / 1e-3 / 1e12, rel=1e-3)
    assert r["per_launch"] == 2 * ridge * 1e9


def test_code_only_ignores_comments_and_layout():
    a = 'int x = 1; // one\n/* block\n comment */ float y = "//not a comment";\n'
    b = 'int x = 1;\n\n   float y = "//not a comment";  // other words\n'
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(a.replace("x = 1", "x = 2"))
    assert bench._code_only("char c = '/'; // c") == bench._code_only("char c = '/';")


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_summarize_trace_routed_launches(tmp_path):
    d = str(tmp_path / "trace")
    _write_csv(os.path.join(d, "run_kernel_stats.csv"),
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"],
               [["moe::k_dispatch_scatter", 2, 20000, 10000, 9000, 11000],
                ["void moe::k_pre_gemm<1, 64>(moe::ExpertGemmArgs)", 6, 600000, 100000, 50000, 150000],
                ["at::elementwise_kernel", 3, 90000, 30000, 30000, 30000]])
    # per call: dispatch, a shared-expert launch on stream 2, routed gate+up and down on
    # stream 1, then the blend
    rows, t = [], 0
    for _ in range(2):
        for name, sid, dur in (("moe::k_dispatch_scatter", 1, 10), ("void moe::k_pre_gemm<0>", 2, 40),
                               ("void moe::k_pre_gemm<1>", 1, 150), ("void moe::k_pre_gemm<1>", 1, 50),
                               ("moe::k_combine", 1, 5)):
            rows.append([name, sid, t * 1000, (t + dur) * 1000])
            t += dur + 1
    _write_csv(os.path.join(d, "run_kernel_trace.csv"),
               ["Kernel_Name", "Stream_Id", "Start_Timestamp", "End_Timestamp"], rows)
    md = bench.summarize_trace(d, "cmd")
    assert "elementwise" not in md  # the input generator's kernels are left out
    assert "| gate_up | 2 | 150.00 | 150.00 | 150.00 |" in md
    assert "| down | 2 | 50.00 | 50.00 | 50.00 |" in md


def _counter_rows(seq):
    return [[i, name, "FETCH_SIZE", v] for i, (name, v) in enumerate(seq)]


def test_routed_counter_prefill_decode_and_one_token(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    d = str(tmp_path / "pre")
    _write_csv(os.path.join(d, "run_counter_collection.csv"), hdr, _counter_rows(
        [("moe::k_pre_gemm<shared>", 7.0), ("moe::k_dispatch_count", 1.0), ("moe::k_dispatch_scatter", 1.0),
         ("moe::k_pre_gemm<gu>", 100.0), ("moe::k_pre_gemm<dn>", 40.0), ("moe::k_combine", 3.0),
         ("moe::k_dispatch_count", 1.0), ("moe::k_dispatch_scatter", 1.0),
         ("moe::k_pre_gemm<gu>", 110.0), ("moe::k_pre_gemm<dn>", 50.0)]))
    got = bench._routed_counter(d, "prefill")
    assert got["gate_up"] == (105.0, 2) and got["down"] == (45.0, 2)
    d = str(tmp_path / "t1")
    _write_csv(os.path.join(d, "run_counter_collection.csv"), hdr, _counter_rows(
        [("moe::k_router_mfma", 2.0), ("moe::k_dec_one_topk<0>", 20.0), ("moe::k_dec_one_blend<0>", 9.0)]))
    got = bench._routed_counter(d, "decode")
    assert got["gate_up"] == (20.0, 1) and got["down"] == (9.0, 1)


def test_summarize_traffic_scales_by_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path / "profiles"))
    d = tmp_path / "tr"
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    # a 1 GiB copy reads as 524288 KiB of FETCH_SIZE (factor 2) and 1048576 KiB of WRITE_SIZE
    _write_csv(str(d / "copy_fetch" / "a_counter_collection.csv"), hdr,
               [[1, "copyBuffer", "FETCH_SIZE", 524288.0], [2, "copyBuffer", "FETCH_SIZE", 12.0]])
    _write_csv(str(d / "copy_write" / "a_counter_collection.csv"), hdr,
               [[1, "copyBuffer", "WRITE_SIZE", 1048576.0]])
    for sub, gu, dn in (("fetch", 1000.0, 300.0), ("write", 10.0, 20.0)):
        _write_csv(str(d / sub / "a_counter_collection.csv"), hdr, _counter_rows(
            [("moe::k_dispatch_scatter", 1.0), ("moe::k_pre_gemm<gu>", gu), ("moe::k_pre_gemm<dn>", dn)]))
    out = bench.summarize_traffic(str(d), "w", "prefill", ["c1"])
    doc = json.load(open(out))
    assert doc["source_digest"] == bench.source_digest()
    gu = doc["kernels"]["prefill_gate_up"]
    assert gu["fetch_bytes"] == 1000 * 1024 * 2 and gu["write_bytes"] == 10 * 1024
    assert gu["bytes_per_launch"] == gu["fetch_bytes"] + gu["write_bytes"]
    assert bench.load_traffic("w", "prefill_down") == 300 * 1024 * 2 + 20 * 1024
