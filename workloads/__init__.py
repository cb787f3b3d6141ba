"""Seeded synthetic inputs for the sparse MoE feed-forward layer.

This module only draws random tensors and describes workload shapes. It holds
none of the layer's arithmetic, so both the CPU oracle (via the tests) and the
HIP library (via the tests and the benchmark) can take their inputs from it.

Generator definition (fixed, so every run and every machine sees the same bits):

* Element ``i`` of tensor ``tensor_id`` drawn under ``seed`` is element
  ``i % CHUNK`` of the float32 standard-normal stream of
  ``numpy.random.Generator(PCG64(SeedSequence([seed, tensor_id, i // CHUNK])))``,
  multiplied in float32 by the tensor's standard deviation.
* bf16 tensors are those float32 values rounded to bfloat16 with
  round-to-nearest-even and kept as ``uint16`` bit patterns.

Shapes and distributions follow the layer the pages describe: PhiMoE's
block-sparse MoE (page "深入解析 Transformers 中的 PhiMoE", section 3,
PhimoeConfig table: hidden 4096, intermediate 6400, 16 local experts, top-2,
initializer_range 0.02) and an Instella-style fine-grained MoE (page on
Instella-MoE-16B-A3B-DPO: 64 routed experts, 2 shared experts, top-6,
scaling factor 2.5).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK = 1 << 22

# Stable tensor ids; weights are keyed by tensor only, so the three PhiMoE
# workloads share one weight set, while the hidden states depend on the
# workload (hidden id = HIDDEN_BASE + workload index).
TID_ROUTER = 1
TID_GATE_UP = 2
TID_DOWN = 3
TID_SHARED_BASE = 4          # shared expert s: gate_up 4+2s, down 5+2s
HIDDEN_BASE = 100


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    T: int
    H: int
    I: int
    E: int
    k: int
    dtype: str                      # "bf16" or "f32"
    routed_scale: float = 1.0
    n_shared: int = 0
    shared_I: int = 0               # intermediate size of each shared expert
    bias: tuple = ()                # ((expert, value), ...) added to router logits
    std_hidden: float = 1.0
    std_weight: float = 0.02
    seed: int = 0
    description: str = ""

    @property
    def TK(self) -> int:
        return self.T * self.k


WORKLOADS = [
    Workload("tiny_f32", 0, T=64, H=128, I=256, E=4, k=2, dtype="f32",
             description="tiny fp32 layer, softmax top-2 with renormalisation"),
    Workload("phimoe_decode", 1, T=32, H=4096, I=6400, E=16, k=2, dtype="bf16",
             description="PhiMoE decode step, near-uniform routing, weight-bandwidth bound"),
    Workload("phimoe_prefill", 2, T=4096, H=4096, I=6400, E=16, k=2, dtype="bf16",
             description="PhiMoE prefill chunk, compute-bound grouped GEMM"),
    Workload("instella_fine", 3, T=2048, H=2048, I=1024, E=64, k=6, dtype="bf16",
             routed_scale=2.5, n_shared=2, shared_I=1024,
             description="Instella-style fine-grained MoE: top-6 of 64, scale 2.5, 2 shared experts"),
    Workload("phimoe_skewed", 4, T=16384, H=4096, I=6400, E=16, k=2, dtype="bf16",
             bias=((0, 6.0), (13, -30.0), (14, -30.0), (15, -30.0)),
             description="PhiMoE shapes with a router bias: about half of all assignments "
                         "to expert 0, experts 13-15 empty"),
    Workload("phimoe_skewed_small", 5, T=256, H=4096, I=6400, E=16, k=2, dtype="bf16",
             bias=((0, 6.0), (13, -30.0), (14, -30.0), (15, -30.0)),
             description="a decode-sized batch with the skewed router bias: about 32 rows per expert on "
                         "average, nearly every token on expert 0"),
    # One GPU's share of the prefill chunk when the layer is split over 8 GPUs.
    # Tensor parallel: each rank holds I/8 = 800 gate, up and down columns of
    # every expert and routes all tokens (the prefill's hidden stream and the
    # same router draw, so the same routing); its output is a partial sum.
    Workload("phimoe_prefill_tp8", 2, T=4096, H=4096, I=800, E=16, k=2, dtype="bf16",
             description="one rank of 8-way tensor parallelism over the prefill chunk: I/8 = 800"),
    # Expert parallel: each rank holds 2 of the 16 experts, which receive
    # about 2 * 8192 / 16 = 1024 of the chunk's assignments, 512 each. Here
    # 512 tokens each pick both of 2 experts, so the expert GEMMs are exactly
    # that share (2 experts, 512 rows each); the router and the combine run
    # over 512 tokens instead of the rank's 4096.
    Workload("phimoe_prefill_ep8", 6, T=512, H=4096, I=6400, E=2, k=2, dtype="bf16",
             description="the expert GEMMs of one rank of 8-way expert parallelism over the prefill chunk: "
                         "2 experts, 512 rows each"),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def _n_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_f32(seed: int, tensor_id: int, n: int, std: float) -> np.ndarray:
    """float32 draws of the generator defined in the module docstring."""
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id, c])))
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        out[lo:hi] *= np.float32(std)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_n_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); returns uint16 bits.

    Inputs must be finite (the generator only yields finite values)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw(seed: int, tensor_id: int, shape, std: float, dtype: str) -> np.ndarray:
    n = int(np.prod(shape))
    f = normal_f32(seed, tensor_id, n, std)
    if dtype == "bf16":
        return f32_to_bf16_bits(f).reshape(shape)
    if dtype == "f32":
        return f.reshape(shape)
    raise ValueError(dtype)


@dataclass
class Inputs:
    """Host arrays of one workload; bf16 tensors are uint16 bit patterns."""
    wl: Workload
    hidden: np.ndarray                  # [T, H]
    router_w: np.ndarray                # [E, H]
    gate_up: np.ndarray                 # [E, 2I, H]; rows [0, I) gate, [I, 2I) up
    down: np.ndarray                    # [E, H, I]
    bias: np.ndarray | None             # [E] float32 or None
    shared_gate_up: list = field(default_factory=list)   # each [2*shared_I, H]
    shared_down: list = field(default_factory=list)      # each [H, shared_I]

    def shared_concat(self):
        """The shared experts as one expert of intermediate size n_shared*shared_I:
        gate rows of every shared expert, then their up rows; down columns in
        the same order. Summing several SwiGLU experts on one input equals one
        SwiGLU expert with these concatenated weights."""
        if not self.shared_gate_up:
            return None, None
        Is = self.wl.shared_I
        gates = [g[:Is] for g in self.shared_gate_up]
        ups = [g[Is:] for g in self.shared_gate_up]
        gu = np.ascontiguousarray(np.concatenate(gates + ups, axis=0))
        dn = np.ascontiguousarray(np.concatenate(self.shared_down, axis=1))
        return gu, dn


def _same_weights(a: Workload, b: Workload) -> bool:
    return (a.seed, a.H, a.I, a.E, a.dtype, a.std_weight, a.n_shared, a.shared_I) == \
        (b.seed, b.H, b.I, b.E, b.dtype, b.std_weight, b.n_shared, b.shared_I)


def make_inputs(wl: Workload | str, T: int | None = None, weights_from: Inputs | None = None) -> Inputs:
    """Draw the inputs of a workload. ``T`` overrides the token count (hidden
    rows are a prefix of the full workload's hidden stream when smaller).
    ``weights_from`` reuses the weight arrays of another workload's inputs
    when they come from the same draws (same seed, shapes and deviation)."""
    if isinstance(wl, str):
        wl = BY_NAME[wl]
    T = wl.T if T is None else T
    dt = wl.dtype
    hidden = draw(wl.seed, HIDDEN_BASE + wl.index, (T, wl.H), wl.std_hidden, dt)
    if weights_from is not None and _same_weights(weights_from.wl, wl):
        w = weights_from
        bias = None
        if wl.bias:
            bias = np.zeros(wl.E, dtype=np.float32)
            for e, v in wl.bias:
                bias[e] = np.float32(v)
        return Inputs(wl, hidden, w.router_w, w.gate_up, w.down, bias, w.shared_gate_up, w.shared_down)
    router_w = draw(wl.seed, TID_ROUTER, (wl.E, wl.H), wl.std_weight, dt)
    gate_up = draw(wl.seed, TID_GATE_UP, (wl.E, 2 * wl.I, wl.H), wl.std_weight, dt)
    down = draw(wl.seed, TID_DOWN, (wl.E, wl.H, wl.I), wl.std_weight, dt)
    bias = None
    if wl.bias:
        bias = np.zeros(wl.E, dtype=np.float32)
        for e, v in wl.bias:
            bias[e] = np.float32(v)
    sgu, sdn = [], []
    for s in range(wl.n_shared):
        sgu.append(draw(wl.seed, TID_SHARED_BASE + 2 * s, (2 * wl.shared_I, wl.H), wl.std_weight, dt))
        sdn.append(draw(wl.seed, TID_SHARED_BASE + 2 * s + 1, (wl.H, wl.shared_I), wl.std_weight, dt))
    return Inputs(wl, hidden, router_w, gate_up, down, bias, sgu, sdn)


def custom_inputs(T, H, I, E, k, dtype="bf16", seed=0, std_hidden=1.0, std_weight=0.02,
                  n_shared=0, shared_I=0, routed_scale=1.0, bias=None, name="custom") -> Inputs:
    """Inputs of arbitrary shape from the same generator (tensor ids offset by
    1000 + seed so they never alias a named workload's tensors)."""
    wl = Workload(name, 1000 + seed, T=T, H=H, I=I, E=E, k=k, dtype=dtype,
                  routed_scale=routed_scale, n_shared=n_shared, shared_I=shared_I,
                  bias=tuple(bias or ()), std_hidden=std_hidden, std_weight=std_weight,
                  seed=1000 + seed)
    return make_inputs(wl)
