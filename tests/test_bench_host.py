"""Host-side checks of the benchmark's bookkeeping (no GPU): the algorithmic
byte counts behind the roofline figures and the single-GPU guard."""
import subprocess
import sys
import os

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_weight_bytes_per_storage():
    # bf16: 2 bytes a weight; FP8 E4M3: 1 byte plus a 4-byte scale per row;
    # MXFP4: half a byte plus one E8M0 byte per 32 weights
    assert bench.weight_bytes(12800, 4096, 2, "bf16") == 12800 * 4096 * 2
    assert bench.weight_bytes(12800, 4096, 2, "fp8") == 12800 * 4096 + 12800 * 4
    assert bench.weight_bytes(12800, 4096, 2, "mxfp4") == 12800 * 4096 // 2 + 12800 * 128


def test_work_counts_only_experts_that_received_tokens():
    wl = W.BY_NAME["phimoe_decode"]
    counts = [0] * wl.E
    counts[3], counts[9] = 40, 24
    for fmt in ("bf16", "fp8", "mxfp4"):
        w = bench.work(wl, counts, weights=fmt)
        assert w["hit"] == 2
        gu = 2 * bench.weight_bytes(2 * wl.I, wl.H, 2, fmt)
        assert w["bytes_gate_up"] == gu + wl.T * wl.H * 2 + wl.T * wl.k * wl.I * 2
        assert w["flop_gate_up"] == 2.0 * wl.T * wl.k * 2 * wl.I * wl.H


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_cpu_baseline_repeats_whole_passes():
    wl = W.BY_NAME["tiny_f32"]
    res = {"inp": W.make_inputs(wl)}
    b = bench.cpu_baseline(res, 64, min_seconds=0.3)
    assert b["kind"] == "oracle" and b["unit"] == "tokens/s" and b["value"] > 0 and b["cores"] >= 1
    assert "passes" in b["sample"] and b["sample"].startswith(f"all {wl.T} tokens of tiny_f32")


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    src = tmp_path / "sparse_mixture_experts_logits_amd" / "csrc"
    src.mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (src / "k.hip").write_text("int f() { return 1; }  // one\n/* block */\n")
    a = bench.source_hash(["k.hip"])
    (src / "k.hip").write_text("// another comment\nint f()  {\n  return 1;\n}\n")
    assert bench.source_hash(["k.hip"]) == a
    (src / "k.hip").write_text("int f() { return 2; }\n")
    assert bench.source_hash(["k.hip"]) != a


def _pmc(dirpath, rows):
    import csv
    dirpath.mkdir(parents=True)
    with open(dirpath / "pmc_counter_collection.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, counter, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_write_traffic_scales_counters_by_the_copy_calibration(tmp_path, monkeypatch):
    # the kernel's FETCH_SIZE / WRITE_SIZE (KiB per dispatch) scaled by what the
    # same counters read for a copy of known size; other kernels are ignored
    (tmp_path / "profiles").mkdir()
    src = tmp_path / "sparse_mixture_experts_logits_amd" / "csrc"
    src.mkdir(parents=True)
    for n in ("gemm_skinny.hip", "gemm_tiled.hip", "moe_internal.h"):
        (src / n).write_text("int x;\n")
    # a change to the other schedule's kernel leaves the figure valid (checked below)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    k = "void skinny_gemm_kernel<true, 0, true>(p)"
    _pmc(tmp_path / "f", [(k, "FETCH_SIZE", 1000.0), (k, "FETCH_SIZE", 1200.0), ("other", "FETCH_SIZE", 9e9)])
    _pmc(tmp_path / "w", [(k, "WRITE_SIZE", 10.0), (k, "WRITE_SIZE", 30.0)])
    copy = 1 << 20
    _pmc(tmp_path / "cf", [("copy", "FETCH_SIZE", copy / 1024 / 2), ("small", "FETCH_SIZE", 1.0)])
    _pmc(tmp_path / "cw", [("copy", "WRITE_SIZE", copy / 1024)])
    bench.write_traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"), str(tmp_path / "cw"),
                        "gate_up", "unit", r"skinny_gemm_kernel<true, 0, true>", copy, "cmd")
    import json
    d = json.load(open(tmp_path / "profiles" / "gate_up_unit_traffic.json"))
    assert d["launches"] == [2, 2]
    assert d["copy_calibration"]["fetch_factor"] == 2.0 and d["copy_calibration"]["write_factor"] == 1.0
    assert d["hbm_bytes_per_launch"] == 1100.0 * 1024 * 2 + 20.0 * 1024
    assert bench.measured_traffic("gate_up", "unit") == d["hbm_bytes_per_launch"]
    (src / "gemm_tiled.hip").write_text("int z;\n")  # another schedule's kernel: still valid
    assert bench.measured_traffic("gate_up", "unit") == d["hbm_bytes_per_launch"]
    (src / "gemm_skinny.hip").write_text("int y;\n")  # the code changed: the figure no longer applies
    assert bench.measured_traffic("gate_up", "unit") is None


def test_roofline_of_decode_and_prefill():
    dec = W.BY_NAME["phimoe_decode"]
    res = dict(wl=dec, counts=[4] * dec.E, weights="bf16", dominant="gate_up",
               stages={"gate_up": 0.25, "down": 0.13})
    r, w = bench.roofline_of(res)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["kernel"] == "gate_up" and r["peak"] == 8000.0
    expect = w["bytes_gate_up"] / 0.25e-3 / 1e9
    assert abs(r["achieved"] - round(expect, 1)) < 1e-6 and abs(r["frac"] - expect / 8000.0) < 1e-4
    assert w["bytes_gate_up"] > 16 * 2 * dec.I * dec.H * 2  # every expert's weights once, plus activations
    pre = W.BY_NAME["phimoe_prefill"]
    res = dict(wl=pre, counts=[512] * pre.E, weights="bf16", dominant="gate_up",
               stages={"gate_up": 0.9, "down": 0.47})
    r, w = bench.roofline_of(res)
    assert r["bound"] == "mfma" and r["kernel"] == "gate_up" and r["peak"] == 2500.0
    assert abs(r["achieved"] - round(2.0 * pre.T * pre.k * 2 * pre.I * pre.H / 0.9e-3 / 1e12, 1)) < 1e-6
    # a dominant stage that is not an expert GEMM falls back to the slower of the two
    res.update(dominant="router", stages={"router": 2.0, "gate_up": 0.4, "down": 0.47})
    r, _ = bench.roofline_of(res)
    assert r["kernel"] == "down"
    assert abs(r["achieved"] - round(2.0 * pre.T * pre.k * pre.H * pre.I / 0.47e-3 / 1e12, 1)) < 1e-6


def test_bound_is_the_longer_of_mfma_and_hbm_time():
    # the Instella-style gate_up moves more bytes than its FLOPs take at peak
    # (intensity below the ridge): HBM bound, although many rows share each expert
    fine = W.BY_NAME["instella_fine"]
    res = dict(wl=fine, counts=[192] * fine.E, weights="bf16", dominant="gate_up", schedule="tiled",
               stages={"gate_up": 0.18, "down": 0.1})
    r, w = bench.roofline_of(res)
    assert w["flop_gate_up"] / 2.5e15 < w["bytes_gate_up"] / 8e12
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert abs(r["achieved"] - round(w["bytes_gate_up"] / 0.18e-3 / 1e9, 1)) < 1e-6
    lay = bench.layer_summary(dict(res, wall_s=0.5e-3 * 10, steps=10), w)
    assert lay["bound"] == "hbm" and abs(lay["roofline_frac"] - w["bytes_layer"] / 8e12 / 0.5e-3) < 1e-4
    assert bench.bound_of(1e12, 1e6, fine)[0] == "mfma" and bench.bound_of(1e6, 1e9, fine)[0] == "hbm"


def test_tiled_executed_flops_counts_padded_tiles():
    pre = W.BY_NAME["phimoe_prefill"]
    # 512 rows: two full 256-row tiles; I = 6400 is 50 whole column blocks: no padding
    ex = bench.tiled_executed_flops(pre, [512] * pre.E)
    assert ex["gate_up"] == 2.0 * pre.T * pre.k * 2 * pre.I * pre.H
    assert ex["down"] == 2.0 * pre.T * pre.k * pre.H * pre.I
    # 557 rows: tiles of 288 (256 + 32 extra) and 269 (256 + 13 extra) both run 288 rows;
    # 20 rows: one 32-row block; 0 rows: nothing
    counts = [557, 20, 0] + [0] * (pre.E - 3)
    ex = bench.tiled_executed_flops(pre, counts)
    assert ex["down"] == 2.0 * (576 + 32) * pre.H * pre.I
    import dataclasses
    one = dataclasses.replace(pre, T=577, k=1)  # T*k = the 577 rows above
    res = dict(wl=one, counts=counts, weights="bf16", dominant="down", schedule="tiled",
               stages={"gate_up": 0.1, "down": 0.2})
    r, w = bench.roofline_of(res)
    assert abs(r["padded_flop_frac"] - (1 - 577 / 608)) < 1e-4


def test_write_stats_and_counters_summaries(tmp_path, monkeypatch):
    import csv
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d = tmp_path / "trace" / "host" / "123"
    d.mkdir(parents=True)
    with open(d / "t_kernel_stats.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage",
                                           "MinNs", "MaxNs", "StdDev"])
        w.writeheader()
        w.writerow(dict(Name="small_kernel(int)", Calls=4, TotalDurationNs=4000, AverageNs=1000, Percentage=10,
                        MinNs=900, MaxNs=1100, StdDev=1))
        w.writerow(dict(Name="void big<1, true>(P)", Calls=4, TotalDurationNs=36000, AverageNs=9000,
                        Percentage=90, MinNs=8000, MaxNs=9500, StdDev=1))
    bench.write_stats(str(tmp_path / "trace"), "unit", "unit_stats", "cmd --x")
    text = (tmp_path / "profiles" / "unit_stats.md").read_text()
    assert "cmd --x" in text and text.index("`void big<1, true>`") < text.index("`small_kernel`")
    assert "| 4 | 9.0 | 8.0 | 9.5 | 90.0% |" in text
    _pmc(tmp_path / "pmc", [("void big<1, true>(P)", "SQ_BUSY_CYCLES", 10.0),
                            ("void big<1, true>(P)", "SQ_BUSY_CYCLES", 30.0),
                            ("tiny(int)", "SQ_BUSY_CYCLES", 0.01)])
    bench.write_counters(str(tmp_path / "pmc"), "unit", "unit_pmc", "cmd")
    text = (tmp_path / "profiles" / "unit_pmc.md").read_text()
    assert "| SQ_BUSY_CYCLES | 20 (2) |" in text and "tiny" not in text
