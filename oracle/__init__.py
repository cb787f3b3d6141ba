"""CPU oracle of the sparse MoE feed-forward layer (plain C, built with gcc).

TEST INFRASTRUCTURE ONLY: only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package. It shares no code
with the HIP library and never imports it.

What the C code computes, and where each step comes from, is stated in the
header of ``moe_oracle.c``. Every function here is argument marshalling
around that C code. Parity of the oracle itself is pinned by the CPU tests
against fp64 numpy evaluations, closed forms and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "moe_oracle.c")
# MOE_ORACLE_LIB may name another build of the same source (the sanitizer build)
LIB = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_HERE, "libmoe_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, fma contraction off)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        cmd = ["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-std=c11", SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def build_sanitized(out: str) -> str:
    """The same source built with AddressSanitizer and UndefinedBehaviorSanitizer
    (gcc; every finding fatal), for running the oracle's pins under them."""
    cmd = ["gcc", "-O1", "-g", "-mfma", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           SRC, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=False)
        lib = ctypes.CDLL(LIB)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        lib.oracle_router_logits.argtypes = [vp, vp, vp, i32, i64, i64, i64, vp]
        lib.oracle_select_topk.argtypes = [vp, i64, i64, i32, f32, vp, vp]
        lib.oracle_route.argtypes = [vp, i64, i32, i64, vp, vp, vp, vp]
        lib.oracle_moe_tokens.argtypes = [vp, vp, vp, i32, i64, i64, vp, vp, i32, i32,
                                          vp, vp, vp, vp, i64, vp]
        lib.oracle_num_threads.argtypes = []
        lib.oracle_router_stats.argtypes = [vp, vp, vp, i64, i64, i32, vp, vp, vp]
        lib.oracle_e4m3_values.argtypes = [vp]
        lib.oracle_quantize_e4m3_rows.argtypes = [vp, i64, i64, vp, vp]
        lib.oracle_moe_tokens_e4m3.argtypes = [vp, vp, vp, vp, vp, i64, i64, vp, vp, i32, i32,
                                               vp, vp, vp, vp, i64, vp]
        lib.oracle_exp_f32.argtypes = [vp, i64, vp]
        lib.oracle_sigmoid_scores.argtypes = [vp, i64, vp]
        lib.oracle_select_scored.argtypes = [vp, i64, i64, i32, f32, i32, vp, i32, i32, vp, vp]
        lib.oracle_select_sparsemixer.argtypes = [vp, i64, i64, i32, f32, f32, vp, vp]
        lib.oracle_e2m1_values.argtypes = [vp]
        lib.oracle_quantize_mxfp4_rows.argtypes = [vp, i64, i64, vp, vp]
        lib.oracle_dequantize_mxfp4_rows.argtypes = [vp, vp, i64, i64, vp]
        for f in (lib.oracle_e2m1_values, lib.oracle_quantize_mxfp4_rows, lib.oracle_dequantize_mxfp4_rows,
                  lib.oracle_select_sparsemixer, lib.oracle_exp_f32, lib.oracle_sigmoid_scores, lib.oracle_select_scored,
                  lib.oracle_router_logits, lib.oracle_select_topk, lib.oracle_route,
                  lib.oracle_moe_tokens, lib.oracle_num_threads, lib.oracle_e4m3_values,
                  lib.oracle_quantize_e4m3_rows, lib.oracle_moe_tokens_e4m3, lib.oracle_router_stats):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return 0          # bf16 bit patterns
    if a.dtype == np.float32:
        return 1
    raise TypeError(f"oracle takes bf16 bits (uint16) or float32, got {a.dtype}")


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments")


def num_threads() -> int:
    return _load().oracle_num_threads()


def router_logits(hidden: np.ndarray, router_w: np.ndarray, bias: np.ndarray | None = None) -> np.ndarray:
    """fp32 logits [T, E] in the canonical summation order (+ bias[e])."""
    hidden = np.ascontiguousarray(hidden)
    router_w = np.ascontiguousarray(router_w)
    assert hidden.dtype == router_w.dtype
    T, H = hidden.shape
    E = router_w.shape[0]
    assert router_w.shape == (E, H)
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        assert bias.shape == (E,)
    out = np.empty((T, E), dtype=np.float32)
    _check(_load().oracle_router_logits(_p(hidden), _p(router_w), _p(bias), _dtype_code(hidden),
                                        T, H, E, _p(out)), "router_logits")
    return out


def select_topk(logits: np.ndarray, k: int, routed_scale: float = 1.0):
    """ids [T, k] int32 (slot order = rank order) and weights [T, k] float32."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    _check(_load().oracle_select_topk(_p(logits), T, E, int(k), float(routed_scale), _p(ids), _p(w)),
           "select_topk")
    return ids, w


def exp_f32(x: np.ndarray) -> np.ndarray:
    """fp32 exp by argument reduction and a degree-8 Taylor polynomial (the
    contract's reproducible exp), elementwise."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty_like(x)
    _check(_load().oracle_exp_f32(_p(x), x.size, _p(y)), "exp_f32")
    return y


def sigmoid_scores(x: np.ndarray) -> np.ndarray:
    """fp32 sigmoid scores 1 / (1 + exp_f32(-clamp(x, -80, 80))), elementwise."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty_like(x)
    _check(_load().oracle_sigmoid_scores(_p(x), x.size, _p(y)), "sigmoid_scores")
    return y


def select_scored(logits: np.ndarray, k: int, routed_scale: float = 1.0, score_func: str = "softmax",
                  selection_bias: np.ndarray | None = None, n_group: int = 0, topk_group: int = 0):
    """Top-k under the scoring variants (sigmoid scores, selection-only bias,
    group-limited selection): ids [T, k] int32 and weights [T, k] float32."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    if selection_bias is not None:
        selection_bias = np.ascontiguousarray(selection_bias, dtype=np.float32)
        assert selection_bias.shape == (E,)
    sf = {"softmax": 0, "sigmoid": 1}[score_func]
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    _check(_load().oracle_select_scored(_p(logits), T, E, int(k), float(routed_scale), sf, _p(selection_bias),
                                        int(n_group), int(topk_group), _p(ids), _p(w)), "select_scored")
    return ids, w


def select_sparsemixer(logits: np.ndarray, k: int, routed_scale: float = 1.0, jitter_eps: float = 0.01):
    """PhiMoE's sparsemixer router at inference: ids [T, k] int32 (greedy by
    logit) and weights [T, k] float32 (each round's own softmax value)."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    _check(_load().oracle_select_sparsemixer(_p(logits), T, E, int(k), float(routed_scale), float(jitter_eps),
                                             _p(ids), _p(w)), "select_sparsemixer")
    return ids, w


def route(ids: np.ndarray, E: int):
    """counts [E], offsets [E+1], perm [T*k], inv [T*k] (all int32)."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(T * k, dtype=np.int32)
    inv = np.empty(T * k, dtype=np.int32)
    _check(_load().oracle_route(_p(ids), T, int(k), int(E), _p(counts), _p(offsets), _p(perm), _p(inv)),
           "route")
    return counts, offsets, perm, inv


def moe_tokens(hidden, gate_up, down, ids, weights, tokens=None, shared=()):
    """Layer output (fp32) for the listed tokens; ``shared`` is a sequence of
    (gate_up [2Is, H], down [H, Is]) pairs, each added unscaled."""
    hidden = np.ascontiguousarray(hidden)
    gate_up = np.ascontiguousarray(gate_up)
    down = np.ascontiguousarray(down)
    dt = _dtype_code(hidden)
    assert gate_up.dtype == hidden.dtype and down.dtype == hidden.dtype
    T, H = hidden.shape
    E, twoI, H2 = gate_up.shape
    I = twoI // 2
    assert H2 == H and down.shape == (E, H, I)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    weights = np.ascontiguousarray(weights, dtype=np.float32)
    k = ids.shape[1]
    if tokens is None:
        tokens = np.arange(T, dtype=np.int32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    n_sh = len(shared)
    keep = []
    sgu = (ctypes.c_void_p * max(1, n_sh))()
    sdn = (ctypes.c_void_p * max(1, n_sh))()
    sI = np.zeros(max(1, n_sh), dtype=np.int64)
    for s, (g, d) in enumerate(shared):
        g = np.ascontiguousarray(g)
        d = np.ascontiguousarray(d)
        assert g.dtype == hidden.dtype and d.dtype == hidden.dtype
        Is = g.shape[0] // 2
        assert g.shape == (2 * Is, H) and d.shape == (H, Is)
        keep += [g, d]
        sgu[s] = g.ctypes.data
        sdn[s] = d.ctypes.data
        sI[s] = Is
    out = np.empty((len(tokens), H), dtype=np.float32)
    _check(_load().oracle_moe_tokens(_p(hidden), _p(gate_up), _p(down), dt, H, I, _p(ids), _p(weights),
                                     int(k), n_sh, ctypes.cast(sgu, ctypes.c_void_p),
                                     ctypes.cast(sdn, ctypes.c_void_p), _p(sI), _p(tokens),
                                     len(tokens), _p(out)), "moe_tokens")
    return out


def router_stats(logits: np.ndarray, ids: np.ndarray, mask: np.ndarray | None = None):
    """Load-balancing statistics (fp64): per-expert mean router probability,
    per-expert load (assignments per counted token) and the auxiliary loss
    E * sum(load * prob_mean), over the tokens with mask != 0 (all if None)."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, E = logits.shape
    k = ids.shape[1]
    if mask is not None:
        mask = np.ascontiguousarray(mask, dtype=np.int32)
    pm = np.empty(E, dtype=np.float64)
    ld = np.empty(E, dtype=np.float64)
    aux = np.empty(1, dtype=np.float64)
    _check(_load().oracle_router_stats(_p(logits), _p(ids), _p(mask), T, E, int(k), _p(pm), _p(ld), _p(aux)),
           "router_stats")
    return dict(prob_mean=pm, load=ld, aux=float(aux[0]))


def e4m3_values() -> np.ndarray:
    """Value of each of the 256 E4M3 codes (fp64; NaN for 0x7F and 0xFF)."""
    out = np.empty(256, dtype=np.float64)
    _check(_load().oracle_e4m3_values(_p(out)), "e4m3_values")
    return out


def quantize_e4m3_rows(w: np.ndarray):
    """Per-row E4M3 quantisation of bf16 bits w [..., cols] -> (q uint8, scale fp32 [...])."""
    w = np.ascontiguousarray(w)
    assert w.dtype == np.uint16
    cols = w.shape[-1]
    rows = w.size // cols
    q = np.empty(w.shape, dtype=np.uint8)
    scale = np.empty(w.shape[:-1], dtype=np.float32)
    _check(_load().oracle_quantize_e4m3_rows(_p(w), rows, cols, _p(q), _p(scale)), "quantize_e4m3_rows")
    return q, scale


def e2m1_values() -> np.ndarray:
    """Value of each of the 16 FP4 E2M1 codes (fp64)."""
    out = np.empty(16, dtype=np.float64)
    _check(_load().oracle_e2m1_values(_p(out)), "e2m1_values")
    return out


def quantize_mxfp4_rows(w: np.ndarray):
    """MXFP4 quantisation of bf16 bits w [..., cols] (cols % 32 == 0) ->
    (q uint8 [..., cols/2] two codes per byte, scale uint8 [..., cols/32] E8M0)."""
    w = np.ascontiguousarray(w)
    assert w.dtype == np.uint16
    cols = w.shape[-1]
    rows = w.size // cols
    q = np.empty(w.shape[:-1] + (cols // 2,), dtype=np.uint8)
    scale = np.empty(w.shape[:-1] + (cols // 32,), dtype=np.uint8)
    _check(_load().oracle_quantize_mxfp4_rows(_p(w), rows, cols, _p(q), _p(scale)), "quantize_mxfp4_rows")
    return q, scale


def dequantize_mxfp4_rows(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """bf16 bits of e2m1(q) * 2^(scale - 127), the shape of q with cols doubled."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    scale = np.ascontiguousarray(scale, dtype=np.uint8)
    cols = q.shape[-1] * 2
    rows = q.size * 2 // cols
    assert scale.shape == q.shape[:-1] + (cols // 32,)
    w = np.empty(q.shape[:-1] + (cols,), dtype=np.uint16)
    _check(_load().oracle_dequantize_mxfp4_rows(_p(q), _p(scale), rows, cols, _p(w)), "dequantize_mxfp4_rows")
    return w


def moe_tokens_e4m3(hidden, gate_up_q, gu_scale, down_q, dn_scale, ids, weights, tokens=None, shared=()):
    """moe_tokens with E4M3 routed-expert weights (bf16 activations and shared experts)."""
    hidden = np.ascontiguousarray(hidden)
    assert hidden.dtype == np.uint16
    gate_up_q = np.ascontiguousarray(gate_up_q, dtype=np.uint8)
    down_q = np.ascontiguousarray(down_q, dtype=np.uint8)
    gu_scale = np.ascontiguousarray(gu_scale, dtype=np.float32)
    dn_scale = np.ascontiguousarray(dn_scale, dtype=np.float32)
    T, H = hidden.shape
    E, twoI, H2 = gate_up_q.shape
    I = twoI // 2
    assert H2 == H and down_q.shape == (E, H, I)
    assert gu_scale.shape == (E, 2 * I) and dn_scale.shape == (E, H)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    weights = np.ascontiguousarray(weights, dtype=np.float32)
    k = ids.shape[1]
    if tokens is None:
        tokens = np.arange(T, dtype=np.int32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    n_sh = len(shared)
    keep = []
    sgu = (ctypes.c_void_p * max(1, n_sh))()
    sdn = (ctypes.c_void_p * max(1, n_sh))()
    sI = np.zeros(max(1, n_sh), dtype=np.int64)
    for s, (g, d) in enumerate(shared):
        g = np.ascontiguousarray(g)
        d = np.ascontiguousarray(d)
        assert g.dtype == np.uint16 and d.dtype == np.uint16
        Is = g.shape[0] // 2
        assert g.shape == (2 * Is, H) and d.shape == (H, Is)
        keep += [g, d]
        sgu[s] = g.ctypes.data
        sdn[s] = d.ctypes.data
        sI[s] = Is
    out = np.empty((len(tokens), H), dtype=np.float32)
    _check(_load().oracle_moe_tokens_e4m3(_p(hidden), _p(gate_up_q), _p(gu_scale), _p(down_q), _p(dn_scale),
                                          H, I, _p(ids), _p(weights), int(k), n_sh,
                                          ctypes.cast(sgu, ctypes.c_void_p), ctypes.cast(sdn, ctypes.c_void_p),
                                          _p(sI), _p(tokens), len(tokens), _p(out)), "moe_tokens_e4m3")
    return out


def moe_forward_e4m3(hidden, router_w, gate_up, down, k, routed_scale=1.0, bias=None, shared=(),
                     tokens=None):
    """Whole layer with the routed experts quantised to E4M3 per row (bf16
    weights in, quantised here): routing as moe_forward, outputs for
    ``tokens``. Returns the routing, the outputs and the quantised weights."""
    logits = router_logits(hidden, router_w, bias)
    ids, w = select_topk(logits, k, routed_scale)
    counts, offsets, perm, inv = route(ids, router_w.shape[0])
    gq, gs = quantize_e4m3_rows(gate_up)
    dq, ds = quantize_e4m3_rows(down)
    out = moe_tokens_e4m3(hidden, gq, gs, dq, ds, ids, w, tokens=tokens, shared=shared)
    return dict(logits=logits, ids=ids, weights=w, counts=counts, offsets=offsets, perm=perm, inv=inv,
                out=out, gate_up_q=gq, gate_up_scale=gs, down_q=dq, down_scale=ds)


def moe_forward(hidden, router_w, gate_up, down, k, routed_scale=1.0, bias=None, shared=(),
                tokens=None, score_func="softmax", selection_bias=None, n_group=0, topk_group=0):
    """Whole layer: routing for every token, outputs for ``tokens`` (all if None)."""
    logits = router_logits(hidden, router_w, bias)
    if score_func == "softmax" and selection_bias is None and n_group <= 1:
        ids, w = select_topk(logits, k, routed_scale)
    else:
        ids, w = select_scored(logits, k, routed_scale, score_func, selection_bias, n_group, topk_group)
    counts, offsets, perm, inv = route(ids, router_w.shape[0])
    out = moe_tokens(hidden, gate_up, down, ids, w, tokens=tokens, shared=shared)
    return dict(logits=logits, ids=ids, weights=w, counts=counts, offsets=offsets,
                perm=perm, inv=inv, out=out)
