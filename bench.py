"""Benchmark of the MI355X sparse-MoE layer (one GPU).

One step is one moe_forward call -- router, top-k, permutation, gate_up GEMM
with fused SiLU*up, down GEMM with the weighted scatter, shared expert,
combine -- over one batch of seeded synthetic tokens already resident in HBM.
Prints ONE JSON line on stdout.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload (the headline ``value``): the PhiMoE decode step (T=32,
H=4096, I=6400, E=16, top-2), bound by the bandwidth of streaming the
selected experts' weights. Every other workload is measured in the same run
with the same steps and warm-up and nested in the line under its own name:
``phimoe_prefill`` (T=4096), ``instella_fine`` (T=2048, 64 experts, top-6,
scale 2.5, two shared experts), ``phimoe_skewed`` (T=16384, router bias: half
of all assignments to one expert), ``phimoe_skewed_small`` (the same bias on a
256-token batch: the mixed schedule) and ``tiny_f32`` (fp32), plus the decode
step with FP8 (E4M3, per-row scaled) and MXFP4 (E2M1, E8M0 scale per 32)
expert weights under ``decode_fp8`` and ``decode_mxfp4``, and the prefill,
skewed and Instella-style workloads with their bf16 routed weights packed in
tile blocks under ``<workload>_tile_blocks`` (other weight storage, so never
the headline value), and with other routing rules under
``<workload>_<router>``: the Instella-style layer with sigmoid scores, a
selection-only bias and group-limited top-k (``noaux_groups``), the prefill
with PhiMoE's sparsemixer selection (``sparsemixer``) and with the router
statistics and load-balancing loss computed (``router_stats``), and one GPU's
share of the prefill chunk split over 8 GPUs: ``phimoe_prefill_tp8`` (tensor
parallel, I/8 = 800 columns of every expert, all tokens) and
``phimoe_prefill_ep8`` (expert parallel: the GEMMs of 2 experts with 512 rows
each). Each carries a ``roofline`` of its
dominant kernel, bound by max(FLOP / MFMA peak, bytes / HBM bandwidth). A
short untimed pilot with events at every stage boundary finds the dominant
kernel; every timed call then records HIP events around that kernel on the
library's stream, so the roofline figures come from the timed region itself.

Other modes: --copy-calibration (a 1 GiB device copy, for scaling rocprofv3
FETCH_SIZE / WRITE_SIZE), --write-traffic, --write-stats and --write-counters
(summarise rocprofv3 runs into profiles/).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0         # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector
METRIC = "MoE layer tokens/sec + % of bf16 MFMA peak (prefill) / % HBM BW (decode)"
# the sources a counter figure depends on, by the kernel family it was taken on
SCHEDULE_SOURCES = {"skinny": ("gemm_skinny.hip", "moe_internal.h"), "tiled": ("gemm_tiled.hip", "moe_internal.h"),
                    "f32": ("gemm_f32.hip", "moe_internal.h")}


def schedule_of_kernel(regex):
    """Kernel family of a kernel-name pattern (skinny_gemm / tiled_gemm / f32_*)."""
    if "skinny" in regex:
        return "skinny"
    if "tiled" in regex:
        return "tiled"
    return "f32"


def decode_tokens_per_s_bound(bandwidth_Bps: float, bytes_per_token: float) -> float:
    """Bandwidth-bound decode rate: every token streams its active weights once."""
    return bandwidth_Bps / bytes_per_token


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ algorithmic work

WEIGHT_FORMATS = {"bf16": "bf16 as given", "fp8": "OCP FP8 E4M3, one fp32 scale per row",
                  "mxfp4": "OCP MXFP4: FP4 E2M1, one E8M0 scale per 32 weights of a row",
                  "tile_blocks": "bf16 in tile blocks (packed once; read by the tiled kernels)"}


def weight_bytes(rows, cols, es, weights):
    """Bytes of a [rows, cols] expert weight matrix in the given storage."""
    if weights == "fp8":
        return rows * cols + rows * 4
    if weights == "mxfp4":
        return rows * cols // 2 + rows * cols // 32
    return rows * cols * es  # bf16, in either layout


def work(wl, counts, weights="bf16"):
    """Algorithmic FLOPs and bytes of the layer and of its two expert GEMMs.

    Bytes count what the method itself must move once: weights of experts that
    received tokens, hidden, router weights and the output for the layer; for
    a GEMM kernel, its weights once plus its input and output activations once
    (gate_up: hidden in, h out; down: h in, fp32 weighted slots out). With
    FP8 expert weights a weight is one byte plus its row's 4-byte scale; with
    MXFP4 half a byte plus one scale byte per 32 weights."""
    es = 2 if wl.dtype == "bf16" else 4
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    TK = T * k
    hit = int(sum(1 for c in counts if c > 0))
    Is = wl.n_shared * wl.shared_I
    f_gu = 2.0 * TK * 2 * I * H
    f_dn = 2.0 * TK * H * I
    f_router = 2.0 * T * H * E
    f_shared = 2.0 * T * 3 * Is * H
    w_gu = hit * weight_bytes(2 * I, H, es, weights)
    w_dn = hit * weight_bytes(H, I, es, weights)
    b_gu = w_gu + T * H * es + TK * I * es
    b_dn = w_dn + TK * I * es + TK * H * 4
    b_layer = w_gu + w_dn + 2 * T * H * es + E * H * es + 3 * Is * H * es
    return dict(hit=hit, flop_layer=f_gu + f_dn + f_router + f_shared, bytes_layer=b_layer,
                flop_gate_up=f_gu, bytes_gate_up=b_gu, flop_down=f_dn, bytes_down=b_dn)


def source_hash(names):
    """Hash of the kernels' code (comments and spacing removed), so that stored
    counter figures are dropped when the code changes, not when a comment does."""
    import re
    h = hashlib.sha256()
    for n in sorted(set(names)):
        with open(os.path.join(ROOT, "sparse_mixture_experts_logits_amd", "csrc", n)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def _counter_rows(path):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    return rows


def write_traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, kernel, workload, regex, copy_bytes,
                  command):
    """Summarise rocprofv3 FETCH_SIZE / WRITE_SIZE runs of one kernel into
    profiles/<kernel>_<workload>_traffic.json, scaled by the same counters on a
    plain copy of copy_bytes (read copy_bytes, write copy_bytes)."""
    import re
    rx = re.compile(regex)

    def avg(rows, counter, name_rx=None):
        v = [float(r["Counter_Value"]) for r in rows
             if r["Counter_Name"] == counter and (name_rx is None or name_rx.search(r["Kernel_Name"]))]
        return sum(v) / len(v) if v else None, len(v)

    def copy_avg(rows, counter):
        # the largest dispatches of the calibration run are the copies
        v = sorted(float(r["Counter_Value"]) for r in rows if r["Counter_Name"] == counter)
        top = [x for x in v if x >= 0.5 * v[-1]] if v else []
        return sum(top) / len(top) if top else None

    f_k, nf = avg(_counter_rows(fetch_dir), "FETCH_SIZE", rx)
    w_k, nw = avg(_counter_rows(write_dir), "WRITE_SIZE", rx)
    if not nf or not nw:
        raise SystemExit(f"no dispatch of a kernel matching {regex!r} in {fetch_dir} / {write_dir}")
    f_c = copy_avg(_counter_rows(copy_fetch_dir), "FETCH_SIZE")
    w_c = copy_avg(_counter_rows(copy_write_dir), "WRITE_SIZE")
    if f_c is None or w_c is None:
        raise SystemExit(f"no copy dispatch in {copy_fetch_dir} / {copy_write_dir}")
    ff = copy_bytes / (f_c * 1024.0)
    fw = copy_bytes / (w_c * 1024.0)
    d = {
        "kernel": kernel, "workload": workload, "kernel_regex": regex,
        "fetch_size_kib_per_launch": f_k, "write_size_kib_per_launch": w_k, "launches": [nf, nw],
        "copy_calibration": {"bytes": copy_bytes, "fetch_kib": f_c, "write_kib": w_c,
                             "fetch_factor": ff, "write_factor": fw},
        "hbm_bytes_per_launch": f_k * 1024.0 * ff + w_k * 1024.0 * fw,
        "schedule": schedule_of_kernel(regex),
        "source_hash": source_hash(SCHEDULE_SOURCES[schedule_of_kernel(regex)]),
        "command": command,
    }
    out = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    with open(out, "w") as fh:
        json.dump(d, fh, indent=1)
    print(json.dumps(d))


def _csv_rows(path, suffix):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(path, "**", "*" + suffix), recursive=True):
        rows += list(csv.DictReader(open(f)))
    return rows


def _short_kernel_name(name):
    """A kernel's name without its namespace and parameter list (template
    arguments kept); mangled names are demangled first."""
    if name.startswith("_Z"):
        import re
        import subprocess
        try:
            dem = subprocess.run(["c++filt", name], capture_output=True, text=True, timeout=10).stdout.strip()
        except (OSError, subprocess.SubprocessError):
            dem = name
        if dem and dem != name:
            name = dem
        else:  # a mangling the tool does not know (bf16 template arguments): name and first template argument
            m = re.match(r"_ZN3moe12_GLOBAL__N_1(\d+)", name)
            if m:
                n = int(m.group(1))
                ident = name[m.end():m.end() + n]
                rest = name[m.end() + n:]
                targ = "bf16" if rest.startswith("IDF16b") else "float" if rest.startswith("If") else ""
                name = ident + (f" [{targ}]" if targ else "")
    name = name.replace("moe::(anonymous namespace)::", "")
    if "_Accum" in name:  # a profiler's demangling of bf16 template arguments ("bool _Accum, int, E")
        import re
        name = re.sub(r"<[^()]*>", " [bf16]", name, count=1)
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def write_stats(trace_dir, title, out_name, command):
    """Summarise a rocprofv3 --kernel-trace --stats run (its *kernel_stats.csv)
    into profiles/<out_name>.md: calls, average, min and max duration and the
    share of GPU time of every kernel."""
    rows = _csv_rows(trace_dir, "kernel_stats.csv")
    if not rows:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"# rocprofv3 kernel statistics: {title}", "", "Command (run from the repository root on one MI355X):",
             "", "```", command, "```", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{_short_kernel_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    out = os.path.join(ROOT, "profiles", out_name + ".md")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(out)


def write_counters(pmc_dir, title, out_name, command):
    """Summarise a rocprofv3 --pmc run (its *counter_collection.csv) into
    profiles/<out_name>.md: every counter averaged over the dispatches of each
    kernel (kernels below 1% of the largest counter total are left out)."""
    rows = _csv_rows(pmc_dir, "counter_collection.csv")
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {pmc_dir}")
    acc = {}
    for r in rows:
        key = (_short_kernel_name(r["Kernel_Name"]), r["Counter_Name"])
        a = acc.setdefault(key, [0.0, 0])
        a[0] += float(r["Counter_Value"])
        a[1] += 1
    kernels = sorted({k for k, _ in acc})
    counters = sorted({c for _, c in acc})
    total = {k: max(acc[(k, c)][0] for c in counters if (k, c) in acc) for k in kernels}
    top = max(total.values())
    kernels = [k for k in kernels if total[k] >= 0.01 * top]
    lines = [f"# rocprofv3 counters: {title}", "", "Command (run from the repository root on one MI355X):", "",
             "```", command, "```", "", "Averages per dispatch.", "",
             "| counter | " + " | ".join(f"`{k}`" for k in kernels) + " |",
             "|---|" + "---|" * len(kernels)]
    for c in counters:
        vals = []
        for k in kernels:
            v = acc.get((k, c))
            vals.append(f"{v[0] / v[1]:.4g} ({v[1]})" if v else "-")
        lines.append(f"| {c} | " + " | ".join(vals) + " |")
    lines.append("")
    lines.append("(n) = dispatches averaged.")
    out = os.path.join(ROOT, "profiles", out_name + ".md")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(out)


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    sched = d.get("schedule") or schedule_of_kernel(d.get("kernel_regex", ""))
    if d.get("source_hash") != source_hash(SCHEDULE_SOURCES[sched]):
        return None
    return d.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------ GPU timing

HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class TimingEvent:
    """A hipEvent_t made with hipEventDisableSystemFence, recorded by the
    library on its own stream at a stage boundary. A default event record ends
    with a system-scope release (L2 writeback and invalidate) that slows the
    kernels after it; an event used only for its timestamp does not need it.
    Created through the HIP runtime torch has loaded, so the handles belong to
    the same runtime as torch's streams."""

    _hip = None

    @classmethod
    def runtime(cls):
        if cls._hip is None:
            paths = sorted({ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64.so" in ln})
            if not paths:
                raise RuntimeError("the HIP runtime is not loaded")
            hip = ctypes.CDLL(paths[0])
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        h = ctypes.c_void_p()
        rc = self.runtime().hipEventCreateWithFlags(ctypes.byref(h), HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.cuda_event = h.value

    def record(self, stream):
        if self.runtime().hipEventRecord(self.cuda_event, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end):
        ms = ctypes.c_float()
        rc = self.runtime().hipEventElapsedTime(ctypes.byref(ms), self.cuda_event, end.cuda_event)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if self.cuda_event and self._hip is not None:
            self._hip.hipEventDestroy(self.cuda_event)

# Routing rules other than the default softmax top-k, for the nested lines:
# extra moe_forward options (the selection bias is drawn from its own seed).
ROUTER_VARIANTS = {
    "noaux_groups": dict(score_func="sigmoid", n_group=8, topk_group=4, selection_bias=True),
    "sparsemixer": dict(score_func="sparsemixer"),
    "router_stats": dict(router_stats=True),
}
ROUTER_NESTED = (("instella_fine", "noaux_groups"), ("phimoe_prefill", "sparsemixer"),
                 ("phimoe_prefill", "router_stats"))


def run_workload(name, steps, warmup, weights="bf16", router=None):
    import torch
    import numpy as np
    import sparse_mixture_experts_logits_amd as moe
    import workloads as W

    wl = W.BY_NAME[name]
    t0 = time.time()
    inp = W.make_inputs(wl, weights_from=_INPUT_CACHE.get("weights"))
    _INPUT_CACHE.setdefault("weights", inp)
    log(f"[bench] {name}: inputs drawn in {time.time() - t0:.1f}s")
    dev = torch.device("cuda", 0)
    d = lambda a: moe.bf16_bits_to_tensor(a, dev)  # noqa: E731
    key = id(inp.gate_up)
    if key not in _DEV_CACHE:
        _DEV_CACHE.clear()
        _DEV_CACHE[key] = (d(inp.router_w), d(inp.gate_up), d(inp.down))
    router_w, gate_up, down = _DEV_CACHE[key]
    hidden = d(inp.hidden)
    scales = {}
    # low-precision weights: the routed experts are quantised once, outside the timed region
    if weights == "fp8":
        gate_up, gs = moe.quantize_fp8_rows(gate_up)
        down, ds = moe.quantize_fp8_rows(down)
        scales = dict(gate_up_scale=gs, down_scale=ds)
    elif weights == "mxfp4":
        gate_up, gs = moe.quantize_mxfp4_rows(gate_up)
        down, ds = moe.quantize_mxfp4_rows(down)
        scales = dict(gate_up_block_scale=gs, down_block_scale=ds)
    elif weights == "tile_blocks":  # the routed experts are packed once, outside the timed region
        gate_up = moe.pack_tile_blocks(gate_up, moe.PACK_GATE_UP)
        down = moe.pack_tile_blocks(down, moe.PACK_DOWN)
    sgu = sdn = None
    if inp.shared_gate_up:
        gu, dn = inp.shared_concat()
        sgu, sdn = d(gu), d(dn)
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).to(dev)
    kw = dict(routed_scale=wl.routed_scale, router_bias=bias, shared_gate_up=sgu, shared_down=sdn, **scales)
    if router:
        rv = dict(ROUTER_VARIANTS[router])
        if rv.pop("selection_bias", False):
            rng = np.random.default_rng(np.random.SeedSequence([0, 100]))
            rv["selection_bias"] = torch.from_numpy(rng.normal(0.0, 0.1, wl.E).astype(np.float32)).to(dev)
        kw.update(rv)

    out = torch.empty((wl.T, wl.H), dtype=hidden.dtype, device=dev)
    need = moe.workspace_bytes(wl.T, wl.H, wl.I, wl.E, wl.k, shared_I=sgu.shape[0] // 2 if sgu is not None else 0,
                               dtype=0 if wl.dtype == "bf16" else 1,
                               weight_layout=moe.LAYOUT_TILE_BLOCKS if weights == "tile_blocks" else moe.LAYOUT_ROWS)
    ws = torch.empty((need,), dtype=torch.uint8, device=dev)
    _, routing = moe.moe_forward(hidden, router_w, gate_up, down, wl.k, return_routing=True, out=out,
                                 workspace=ws, **kw)
    torch.cuda.synchronize()
    counts = routing["counts"].cpu().numpy().tolist()

    nev = moe.STAGE_EVENTS

    stream = torch.cuda.current_stream(dev).cuda_stream

    def event_sets(n):
        sets = [[TimingEvent() for _ in range(nev)] for _ in range(n)]
        for evs in sets:
            for e in evs:
                e.record(stream)
        torch.cuda.synchronize()
        return sets

    for _ in range(warmup):
        moe.moe_forward(hidden, router_w, gate_up, down, wl.k, out=out, workspace=ws, **kw)
    torch.cuda.synchronize()

    # pilot (untimed): every stage boundary, to find the dominant stage
    pilot = event_sets(5)
    for evs in pilot:
        h = (ctypes.c_void_p * nev)(*[e.cuda_event for e in evs])
        moe.moe_forward(hidden, router_w, gate_up, down, wl.k, out=out, workspace=ws, stage_events=h, **kw)
    torch.cuda.synchronize()
    stage_ms = np.zeros(nev - 1)
    for evs in pilot:
        for j in range(nev - 1):
            stage_ms[j] += evs[j].elapsed_time(evs[j + 1])
    stage_ms /= len(pilot)
    dom = int(np.argmax(stage_ms))

    # timed region: only the two events around the dominant stage are recorded
    events = []
    handles = []
    for _ in range(steps):
        pair = (TimingEvent(), TimingEvent())
        events.append(pair)
        arr = [None] * nev
        arr[dom], arr[dom + 1] = pair[0].cuda_event, pair[1].cuda_event
        handles.append((ctypes.c_void_p * nev)(*arr))
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()  # one rank: the barrier is the synchronize
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        moe.moe_forward(hidden, router_w, gate_up, down, wl.k, out=out, workspace=ws, stage_events=handles[i], **kw)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(end)
    dom_ms = sum(a.elapsed_time(b) for a, b in events) / steps
    stages = dict(zip(moe.STAGES, stage_ms.tolist()))
    stages[moe.STAGES[dom]] = dom_ms  # live value from the timed region
    return dict(wl=wl, counts=counts, wall_s=wall, gpu_ms=gpu_ms, steps=steps, warmup=warmup, stages=stages,
                dominant=moe.STAGES[dom], inp=inp, weights=weights, schedule=schedule_of(wl, weights), router=router)


_INPUT_CACHE = {}
_DEV_CACHE = {}


def schedule_of(wl, weights="bf16"):
    """Which expert-GEMM kernels the library runs for this workload (its
    default rule, for reporting): fp32 VALU kernels; the weight-streaming
    kernels for low-precision weights, or about 32 rows per expert or fewer
    with at most 32 tokens; "mixed" (streaming plus tiled for experts past 32
    rows) for about 32 rows per expert or fewer with more tokens; else the
    large-M tiled kernels."""
    if wl.dtype == "f32":
        return "f32"
    if weights == "tile_blocks":
        return "tiled"
    if weights != "bf16":
        return "skinny"
    if wl.T * wl.k <= 32 * wl.E:
        return "skinny" if wl.T <= 32 else "mixed"
    return "tiled"


def peak_flops(wl):
    """Dense MFMA peak of the workload's arithmetic type, FLOP/s."""
    return (BF16_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_PEAK_TFLOPS) * 1e12


def bound_of(flop, nbytes, wl):
    """The roofline bound of a piece of work: whichever of MFMA time and HBM
    time is longer. Returns (bound, roofline seconds)."""
    t_flop = flop / peak_flops(wl)
    t_bytes = nbytes / (HBM_PEAK_GBPS * 1e9)
    return ("hbm", t_bytes) if t_bytes >= t_flop else ("mfma", t_flop)


def tiled_executed_flops(wl, counts, tile_m=256, tile_xt=32, block=32, nblk_cols=128):
    """MFMA FLOPs the large-M schedule executes for the routed expert GEMMs:
    an expert's rows go to as few M-tiles as hold them at up to tile_m +
    tile_xt rows; a tile runs whole 32-row blocks (a tile with extra rows runs
    tile_m + 32), and N is padded to whole column blocks (gate_up: 128 h
    columns, i.e. 128 gate + 128 up rows; down: 256 output rows)."""
    rows_exec = 0
    for c in counts:
        c = int(c)
        if c == 0:
            continue
        n = (c + tile_m + tile_xt - 1) // (tile_m + tile_xt)
        extra = max(c - n * tile_m, 0)
        for i in range(n):
            rows = tile_m + min(max(extra - i * tile_xt, 0), tile_xt) if extra > 0 else \
                (c - i * tile_m if i == n - 1 else tile_m)
            rows_exec += tile_m + block if rows > tile_m else -(-rows // block) * block
    n_gu = -(-wl.I // nblk_cols) * nblk_cols
    n_dn = -(-wl.H // 256) * 256
    return dict(gate_up=2.0 * rows_exec * 2 * n_gu * wl.H, down=2.0 * rows_exec * n_dn * wl.I)


def roofline_of(res):
    """Roofline of the dominant expert GEMM (the stage with the largest time),
    bound by max(FLOP / peak, bytes / HBM bandwidth) of that kernel's
    algorithmic work."""
    wl = res["wl"]
    w = work(wl, res["counts"], weights=res["weights"])
    st = res["stages"]
    kernel = res["dominant"]
    if kernel not in ("gate_up", "down"):  # the expert GEMMs dominate every workload here
        kernel = "gate_up" if st["gate_up"] >= st["down"] else "down"
    dur_s = st[kernel] / 1e3
    bound, _ = bound_of(w[f"flop_{kernel}"], w[f"bytes_{kernel}"], wl)
    if bound == "hbm":
        achieved = w[f"bytes_{kernel}"] / dur_s / 1e9
        r = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                 frac=round(achieved / HBM_PEAK_GBPS, 4))
    else:
        peak = peak_flops(wl) / 1e12
        achieved = w[f"flop_{kernel}"] / dur_s / 1e12
        r = dict(bound="mfma", achieved=round(achieved, 1), peak=peak, unit="TFLOP/s",
                 frac=round(achieved / peak, 4))
    tr = measured_traffic(kernel, wl.name + ("" if res["weights"] == "bf16" else "_" + res["weights"]))
    r["traffic"] = tr
    r["kernel"] = kernel
    r["avg_launch_ms"] = round(st[kernel], 4)
    r["algorithmic"] = {"flop": w[f"flop_{kernel}"], "bytes": w[f"bytes_{kernel}"]}
    r["timing"] = "HIP events around this kernel on the library's stream, every timed step"
    if res.get("schedule") == "tiled":
        ex = tiled_executed_flops(wl, res["counts"])[kernel]
        r["mfma_flop_executed"] = ex
        r["padded_flop_frac"] = round(1.0 - w[f"flop_{kernel}"] / ex, 4)
    return r, w


def layer_summary(res, w):
    wl = res["wl"]
    ms = res["wall_s"] * 1e3 / res["steps"]
    s = ms / 1e3
    bound, t_roof = bound_of(w["flop_layer"], w["bytes_layer"], wl)
    return dict(ms_per_step=round(ms, 4), tokens_per_s=round(wl.T / s, 1),
                tflops=round(w["flop_layer"] / s / 1e12, 2), gbps=round(w["bytes_layer"] / s / 1e9, 1),
                frac_hbm=round(w["bytes_layer"] / s / 1e9 / HBM_PEAK_GBPS, 4),
                frac_mfma=round(w["flop_layer"] / s / peak_flops(wl), 4),
                bound=bound, roofline_ms=round(t_roof * 1e3, 4), roofline_frac=round(t_roof / s, 4),
                schedule=res.get("schedule"),
                experts_hit=w["hit"], stages_ms={k: round(v, 4) for k, v in res["stages"].items()})


# ------------------------------------------------------------------ CPU oracle baseline

def cpu_baseline(res, max_tokens, min_seconds=10.0):
    import numpy as np
    import oracle
    inp = res["inp"]
    wl = inp.wl
    n = min(wl.T, max_tokens)
    toks = np.arange(n, dtype=np.int32)
    shared = list(zip(inp.shared_gate_up, inp.shared_down))
    passes = 0
    t0 = time.perf_counter()
    while True:  # whole passes over the sample until at least min_seconds have passed
        logits = oracle.router_logits(inp.hidden[:n], inp.router_w, inp.bias)
        ids, wts = oracle.select_topk(logits, wl.k, wl.routed_scale)
        oracle.route(ids, wl.E)
        oracle.moe_tokens(inp.hidden[:n], inp.gate_up, inp.down, ids, wts, tokens=toks, shared=shared)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    what = "all" if n == wl.T else "the first"
    return dict(value=round(n * passes / dt, 3), unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"{what} {n} tokens of {wl.name} (routing + every selected expert FFN), "
                       f"{passes} passes in {dt:.1f} s")


# ------------------------------------------------------------------ main

# PhiMoE-shaped workloads first: they share one set of device weights
NESTED = ("phimoe_prefill", "phimoe_skewed", "phimoe_skewed_small", "instella_fine", "tiny_f32",
          "phimoe_prefill_tp8", "phimoe_prefill_ep8")
TILE_BLOCK_NESTED = ("phimoe_prefill", "phimoe_skewed", "instella_fine")


def nested_line(res):
    roof, w = roofline_of(res)
    wl = res["wl"]
    d = dict(workload=wl.name, steps=res["steps"], warmup=res["warmup"], dtype=wl.dtype,
             config={"T": wl.T, "H": wl.H, "I": wl.I, "E": wl.E, "k": wl.k, "routed_scale": wl.routed_scale,
                     "shared_I": wl.n_shared * wl.shared_I},
             roofline=roof, layer=layer_summary(res, w))
    if res["weights"] != "bf16":
        d["weights"] = WEIGHT_FORMATS[res["weights"]]
    if res.get("router"):
        d["router"] = {k: (v if not isinstance(v, bool) or k != "selection_bias" else "N(0, 0.1) per expert")
                       for k, v in ROUTER_VARIANTS[res["router"]].items()}
    return d


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="phimoe_decode")
    ap.add_argument("--router", choices=sorted(ROUTER_VARIANTS), default=None,
                    help="routing rule of the main workload (default: softmax top-k)")
    ap.add_argument("--only", action="store_true", help="measure the main workload only (no nested lines)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--skip", nargs="*", default=[], help="nested lines to leave out (workload names, "
                                                           "decode_fp8, decode_mxfp4, <workload>_tile_blocks)")
    ap.add_argument("--weights", choices=sorted(WEIGHT_FORMATS), default="bf16",
                    help="expert weight storage of the main workload (fp8 / mxfp4: decode-shaped work only)")
    ap.add_argument("--cpu-tokens", type=int, default=32)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="whole oracle passes over the CPU sample until this many seconds have passed")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a 1 GiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--write-traffic", nargs=7, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                         "COPY_WRITE_DIR", "KERNEL", "WORKLOAD", "REGEX"),
                    help="summarise rocprofv3 FETCH_SIZE/WRITE_SIZE runs into profiles/")
    ap.add_argument("--write-stats", nargs=3, metavar=("TRACE_DIR", "TITLE", "OUT_NAME"),
                    help="summarise a rocprofv3 --kernel-trace --stats run into profiles/OUT_NAME.md")
    ap.add_argument("--write-counters", nargs=3, metavar=("PMC_DIR", "TITLE", "OUT_NAME"),
                    help="summarise a rocprofv3 --pmc run (averages per kernel) into profiles/OUT_NAME.md")
    ap.add_argument("--command", default="", help="command line recorded with the --write-* modes")
    args = ap.parse_args(argv)
    if args.write_traffic:
        fd, wd, cfd, cwd, kernel, workload, regex = args.write_traffic
        write_traffic(fd, wd, cfd, cwd, kernel, workload, regex, 1 << 30, args.command)
        return 0
    if args.write_stats:
        write_stats(*args.write_stats, args.command)
        return 0
    if args.write_counters:
        write_counters(*args.write_counters, args.command)
        return 0
    if args.copy_calibration:
        copy_calibration()
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer here has no multi-GPU path (run with --gpus 1).",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2

    res = run_workload(args.workload, args.steps, args.warmup, weights=args.weights, router=args.router)
    roof, w = roofline_of(res)
    lay = layer_summary(res, w)
    wl = res["wl"]
    line = {
        "metric": METRIC,
        "value": lay["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": lay["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded normal draws; no checkpoint)",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "I": wl.I, "E": wl.E, "k": wl.k,
                   "routed_scale": wl.routed_scale, "shared_I": wl.n_shared * wl.shared_I,
                   "parallelism": "single GPU",
                   **({"expert_weights": WEIGHT_FORMATS[args.weights]} if args.weights != "bf16" else {}),
                   **({"router": args.router} if args.router else {})},
        "roofline": roof,
        "layer": lay,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(res, args.cpu_tokens, args.cpu_seconds)
    if not args.only:
        if args.weights == "bf16" and args.workload == "phimoe_decode":
            for fmt in ("fp8", "mxfp4"):
                if "decode_" + fmt not in args.skip:
                    line["decode_" + fmt] = nested_line(run_workload("phimoe_decode", args.steps, args.warmup,
                                                                     weights=fmt))
        for name in NESTED:
            if name != args.workload and name not in args.skip:
                line[name] = nested_line(run_workload(name, args.steps, args.warmup))
                log(f"[bench] {name}: {line[name]['layer']['ms_per_step']} ms per step")
        # the tiled workloads again with their routed weights packed in tile blocks
        for name in TILE_BLOCK_NESTED:
            key = name + "_tile_blocks"
            if key not in args.skip:
                line[key] = nested_line(run_workload(name, args.steps, args.warmup, weights="tile_blocks"))
                log(f"[bench] {key}: {line[key]['layer']['ms_per_step']} ms per step")
        # and with other routing rules
        for name, rv in ROUTER_NESTED:
            key = f"{name}_{rv}"
            if key not in args.skip:
                line[key] = nested_line(run_workload(name, args.steps, args.warmup, router=rv))
                log(f"[bench] {key}: {line[key]['layer']['ms_per_step']} ms per step")
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
