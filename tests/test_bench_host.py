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
