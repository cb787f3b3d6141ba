"""The benchmark's output contract on a GPU: one JSON line with the metric,
the whole-step throughput, the roofline of the dominant kernel, the CPU
oracle baseline and a nested line for every other workload (a short run:
few steps)."""
import json

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def test_bench_prints_one_json_line_with_roofline_and_cpu_baseline(capsys):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("case bench.py short run", flush=True)
    import bench  # in this process: no second program is started
    try:
        rc = bench.main(["--steps", "5", "--warmup", "1", "--cpu-tokens", "2", "--cpu-seconds", "0.2"])
    finally:  # the full-size weights it keeps on the device
        bench._INPUT_CACHE.clear()
        bench._DEV_CACHE.clear()
        torch.cuda.empty_cache()
    out = capsys.readouterr().out
    assert rc == 0
    lines = [ln for ln in out.splitlines() if ln.strip().startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["unit"] == "tokens/s" and d["value"] > 0
    assert d["config"]["workload"] == "phimoe_decode" and d["dtype"] == "bf16"
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert 0 < roof["frac"] < 1.2 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and "tokens" in cpu["sample"]
    for sec, bound in (("decode_fp8", "hbm"), ("decode_mxfp4", "hbm"), ("phimoe_prefill", "mfma"),
                       ("phimoe_skewed", "mfma"), ("instella_fine", "hbm")):
        sub = d[sec]
        assert sub["roofline"]["bound"] == bound and sub["layer"]["tokens_per_s"] > 0, sec
        assert sub["steps"] == 5 and sub["warmup"] == 1, sec
    assert d["tiny_f32"]["dtype"] == "f32" and d["tiny_f32"]["layer"]["tokens_per_s"] > 0
    assert 0 <= d["phimoe_skewed"]["roofline"]["padded_flop_frac"] < 0.2
    # the other routing rules: their own lines, naming the rule
    for sec, rule in (("instella_fine_noaux_groups", "sigmoid"), ("phimoe_prefill_sparsemixer", "sparsemixer")):
        assert d[sec]["router"]["score_func"] == rule and d[sec]["layer"]["tokens_per_s"] > 0, sec
    assert d["phimoe_prefill_router_stats"]["router"]["router_stats"] is True
