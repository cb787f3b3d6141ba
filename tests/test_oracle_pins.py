"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test checks one part of the oracle against a closed form, an invariant,
a library routine, a brute-force fp64 evaluation written independently here
(numpy), or a number the pages print (tests/golden/page_facts.json). A
plausible slip in the oracle (dropped term, swapped gate/up halves, wrong
sign, transposed down projection, unstable permutation, wrong tie order,
wrong summation order of the router logit) fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


# ---------------------------------------------------------------- helpers (fp64, numpy only)

def f64(a):
    if a.dtype == np.uint16:
        return W.bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def silu64(z):
    return z / (1.0 + np.exp(-z))


def dense_expert64(x, gu, dn):
    """SwiGLU expert in fp64: rows [0, I) of gu are gate, [I, 2I) up; dn is [H, I]."""
    I = gu.shape[0] // 2
    g = x @ gu[:I].T
    u = x @ gu[I:].T
    return (silu64(g) * u) @ dn.T


def topk_bruteforce(logits, k):
    """Order by (logit desc, index asc) with a full lexicographic sort."""
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))
        ids[t] = order[:k]
    return ids


def bf16(a):
    return W.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


# ---------------------------------------------------------------- router logits

def test_logits_exact_on_small_integers():
    # integer-valued bf16 inputs: every partial sum is an integer below 2^24,
    # so any summation order is exact and must equal the int64 dot product.
    rng = np.random.default_rng(1)
    T, H, E = 5, 1000, 7
    xi = rng.integers(-4, 5, size=(T, H))
    wi = rng.integers(-4, 5, size=(E, H))
    bias = rng.integers(-3, 4, size=E).astype(np.float32)
    for dt in ("bf16", "f32"):
        x = bf16(xi) if dt == "bf16" else xi.astype(np.float32)
        w = bf16(wi) if dt == "bf16" else wi.astype(np.float32)
        l = oracle.router_logits(x, w, bias)
        exact = (xi @ wi.T).astype(np.float64) + bias
        assert np.array_equal(l.astype(np.float64), exact)


@pytest.mark.parametrize("ones_at,expected", [
    # Hand-derived under the canonical order (partial sum of lane L takes
    # elements 8L..8L+7 of each 512-block; lanes combine by xor 32,16,8,4,2,1):
    # lanes 1 and 3 meet first (xor 2) giving 2, then 2^24 + 2 is exact.
    ((8, 24), 2.0 ** 24 + 2),
    # elements 1 and 3 share lane 0 with 2^24: each +1 is lost to rounding.
    ((1, 3), 2.0 ** 24),
    # lanes 1 and 2 reach lane 0 at different steps: each +1 is lost.
    ((8, 16), 2.0 ** 24),
    # second 512-block: element 520 is lane 1, 536 is lane 3 -> as the first case.
    ((520, 536), 2.0 ** 24 + 2),
])
def test_logit_summation_order_closed_form(ones_at, expected):
    H = 1024
    x = np.zeros((1, H), dtype=np.float32)
    w = np.zeros((1, H), dtype=np.float32)
    x[0, 0] = 2.0 ** 24
    w[0, 0] = 1.0
    for i in ones_at:
        x[0, i] = 1.0
        w[0, i] = 1.0
    l = oracle.router_logits(x, w)
    assert l[0, 0] == np.float32(expected)


def test_logits_within_fp32_bound_of_fp64():
    inp = W.custom_inputs(T=16, H=4096, I=8, E=16, k=2)
    l = oracle.router_logits(inp.hidden, inp.router_w)
    x, w = f64(inp.hidden), f64(inp.router_w)
    l64 = x @ w.T
    bound = 4096 * 2.0 ** -24 * (np.abs(x) @ np.abs(w).T)
    assert np.all(np.abs(l - l64) <= bound)


# ---------------------------------------------------------------- top-k selection and weights

def test_zero_router_closed_form():
    for k, s in ((2, 1.0), (6, 2.5), (1, 1.0)):
        inp = W.custom_inputs(T=9, H=64, I=8, E=8, k=k)
        zero = np.zeros_like(inp.router_w)
        l = oracle.router_logits(inp.hidden, zero)
        assert np.all(l == 0.0)
        ids, w = oracle.select_topk(l, k, s)
        assert np.array_equal(ids, np.tile(np.arange(k, dtype=np.int32), (9, 1)))
        assert np.all(w == np.float32(s / k))
        counts, offsets, perm, inv = oracle.route(ids, 8)
        assert list(counts) == [9] * k + [0] * (8 - k)


def test_identical_router_rows_tie_to_lower_index():
    inp = W.custom_inputs(T=64, H=128, I=8, E=8, k=3)
    wr = inp.router_w.copy()
    wr[5] = wr[2]
    wr[6] = wr[2]
    l = oracle.router_logits(inp.hidden, wr)
    assert np.all(l[:, 2] == l[:, 5]) and np.all(l[:, 2] == l[:, 6])
    ids, _ = oracle.select_topk(l, 3)
    for t in range(64):
        row = list(ids[t])
        if 5 in row:
            assert 2 in row and row.index(2) < row.index(5)
        if 6 in row:
            assert 5 in row and row.index(5) < row.index(6)
    assert np.array_equal(ids, topk_bruteforce(l, 3))


@pytest.mark.parametrize("E,k", [(4, 2), (16, 2), (64, 6), (8, 8), (1, 1), (256, 8)])
def test_topk_matches_full_sort(E, k):
    rng = np.random.default_rng(E * 100 + k)
    logits = rng.standard_normal((200, E)).astype(np.float32)
    logits[::3] = np.round(logits[::3] * 2) / 2      # many exact ties
    logits[1::7] = -0.0
    logits[2::7, 0] = 0.0
    ids, w = oracle.select_topk(logits, k)
    assert np.array_equal(ids, topk_bruteforce(logits, k))


@pytest.mark.parametrize("E,k,s", [(16, 2, 1.0), (64, 6, 2.5), (4, 4, 1.0)])
def test_weights_equal_softmax_over_all_then_renormalised(E, k, s):
    rng = np.random.default_rng(7)
    logits = (rng.standard_normal((100, E)) * 3).astype(np.float32)
    ids, w = oracle.select_topk(logits, k, s)
    l64 = logits.astype(np.float64)
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    ref = s * sel / sel.sum(axis=1, keepdims=True)
    assert np.allclose(w, ref, rtol=2e-7, atol=1e-30)
    assert np.all(np.abs(w.astype(np.float64).sum(axis=1) - s) <= 1e-6 * k * s)
    assert np.all(np.diff(w, axis=1) <= 0)       # slot order = rank order


def test_single_expert_weight_is_one():
    logits = np.random.default_rng(3).standard_normal((10, 1)).astype(np.float32)
    ids, w = oracle.select_topk(logits, 1, 1.0)
    assert np.all(ids == 0) and np.all(w == 1.0)


# ---------------------------------------------------------------- permutation

@pytest.mark.parametrize("T,k,E", [(1000, 3, 7), (64, 2, 4), (1, 1, 1), (0, 2, 4), (333, 6, 64)])
def test_route_matches_library_routines(T, k, E):
    rng = np.random.default_rng(T + k + E)
    # distinct experts per token, as top-k produces
    ids = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32).reshape(T, k)
    counts, offsets, perm, inv = oracle.route(ids, E)
    flat = ids.ravel()
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    assert np.array_equal(inv, np.argsort(perm, kind="stable"))
    # invariants: no drop, bijection, expert-major, ascending inside each segment
    assert counts.sum() == T * k and offsets[-1] == T * k
    assert np.array_equal(np.sort(perm), np.arange(T * k))
    assert np.all(np.diff(flat[perm]) >= 0)
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0) and np.all(flat[seg] == e)
    # round trip: gather rows through perm, scatter back through inv
    X = rng.standard_normal((T * k, 3)).astype(np.float32)
    assert np.array_equal(X[perm][inv], X)


# ---------------------------------------------------------------- expert FFN and combine

def dense_layer64(inp, ids_ref=None, k=None, s=None, shared=True):
    """Brute force: every expert evaluated densely for every token in fp64,
    then masked by the top-k weights of the oracle's own fp32 logits (the
    selection itself is pinned separately)."""
    wl = inp.wl
    k = wl.k if k is None else k
    s = wl.routed_scale if s is None else s
    l = oracle.router_logits(inp.hidden, inp.router_w, inp.bias).astype(np.float64)
    x = f64(inp.hidden)
    T, E = l.shape
    sel = topk_bruteforce(l.astype(np.float32), k)
    if ids_ref is not None:
        assert np.array_equal(sel, ids_ref)
    lsel = np.take_along_axis(l, sel, axis=1)
    p = np.exp(lsel - lsel[:, :1])
    wsel = s * p / p.sum(axis=1, keepdims=True)
    mask = np.zeros((T, E))
    np.put_along_axis(mask, sel, wsel, axis=1)
    out = np.zeros((T, wl.H))
    for e in range(E):
        out += mask[:, e:e + 1] * dense_expert64(x, f64(inp.gate_up[e]), f64(inp.down[e]))
    if shared:
        for g, d in zip(inp.shared_gate_up, inp.shared_down):
            out += dense_expert64(x, f64(g), f64(d))
    return out


def rel_err(a, b):
    return np.max(np.abs(a - b)) / np.max(np.abs(b))


def test_single_expert_top1_is_dense_swiglu():
    for dt in ("f32", "bf16"):
        inp = W.custom_inputs(T=40, H=96, I=160, E=1, k=1, dtype=dt, std_weight=0.1)
        r = oracle.moe_forward(inp.hidden, inp.router_w, inp.gate_up, inp.down, 1)
        assert np.all(r["ids"] == 0) and np.all(r["weights"] == 1.0)
        ref = dense_expert64(f64(inp.hidden), f64(inp.gate_up[0]), f64(inp.down[0]))
        assert rel_err(r["out"], ref) < 1e-5


def test_gate_and_up_halves_are_not_interchangeable():
    # guards the gate/up orientation: swapping the halves must change the output
    inp = W.custom_inputs(T=8, H=64, I=32, E=1, k=1, dtype="f32", std_weight=0.3)
    r = oracle.moe_forward(inp.hidden, inp.router_w, inp.gate_up, inp.down, 1)
    swapped = np.concatenate([inp.gate_up[:, 32:], inp.gate_up[:, :32]], axis=1)
    ref_swapped = dense_expert64(f64(inp.hidden), f64(swapped[0]), f64(inp.down[0]))
    assert rel_err(r["out"], ref_swapped) > 0.1


def test_tiny_workload_against_dense_masked_fp64():
    inp = W.make_inputs("tiny_f32")
    r = oracle.moe_forward(inp.hidden, inp.router_w, inp.gate_up, inp.down, 2)
    ref = dense_layer64(inp, ids_ref=r["ids"])
    assert rel_err(r["out"], ref) < 1e-5


def test_k_equals_E_is_dense_soft_mixture():
    inp = W.custom_inputs(T=24, H=64, I=48, E=5, k=5, dtype="f32", std_weight=0.1)
    r = oracle.moe_forward(inp.hidden, inp.router_w, inp.gate_up, inp.down, 5)
    l = r["logits"].astype(np.float64)
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    x = f64(inp.hidden)
    ref = sum(p[:, e:e + 1] * dense_expert64(x, f64(inp.gate_up[e]), f64(inp.down[e])) for e in range(5))
    assert rel_err(r["out"], ref) < 1e-5


def test_router_bias_shifts_selection_and_weights():
    inp = W.custom_inputs(T=50, H=64, I=32, E=6, k=2, dtype="f32",
                          bias=((0, 6.0), (4, -30.0), (5, -30.0)))
    r = oracle.moe_forward(inp.hidden, inp.router_w, inp.gate_up, inp.down, 2, bias=inp.bias)
    assert np.all(r["ids"][:, 0] == 0)
    assert r["counts"][4] == 0 and r["counts"][5] == 0
    ref = dense_layer64(inp, ids_ref=r["ids"])
    assert rel_err(r["out"], ref) < 1e-5


def test_two_shared_experts_equal_one_concatenated():
    inp = W.custom_inputs(T=32, H=64, I=32, E=8, k=3, dtype="f32", n_shared=2, shared_I=24,
                          routed_scale=2.5)
    sh = list(zip(inp.shared_gate_up, inp.shared_down))
    r2 = oracle.moe_forward(inp.hidden, inp.router_w, inp.gate_up, inp.down, 3, 2.5, shared=sh)
    gu, dn = inp.shared_concat()
    r1 = oracle.moe_forward(inp.hidden, inp.router_w, inp.gate_up, inp.down, 3, 2.5, shared=[(gu, dn)])
    assert rel_err(r1["out"], r2["out"]) < 1e-5
    ref = dense_layer64(inp, ids_ref=r2["ids"])
    assert rel_err(r2["out"], ref) < 1e-5


def test_zero_routed_scale_leaves_shared_expert_alone():
    inp = W.custom_inputs(T=16, H=64, I=32, E=4, k=2, dtype="f32", n_shared=1, shared_I=40)
    sh = list(zip(inp.shared_gate_up, inp.shared_down))
    r = oracle.moe_forward(inp.hidden, inp.router_w, inp.gate_up, inp.down, 2, 0.0, shared=sh)
    ref = dense_expert64(f64(inp.hidden), f64(sh[0][0]), f64(sh[0][1]))
    assert rel_err(r["out"], ref) < 1e-5


def test_token_subset_equals_full_rows():
    inp = W.make_inputs("tiny_f32")
    full = oracle.moe_forward(inp.hidden, inp.router_w, inp.gate_up, inp.down, 2)
    toks = np.array([63, 0, 17, 17], dtype=np.int32)
    part = oracle.moe_tokens(inp.hidden, inp.gate_up, inp.down, full["ids"], full["weights"], toks)
    assert np.array_equal(part, full["out"][toks])


@pytest.mark.slow
@pytest.mark.parametrize("name", ["phimoe_decode", "instella_fine", "phimoe_skewed"])
def test_full_size_first_tokens_against_dense_fp64(name):
    """First 4 tokens of full-size workloads (full H, I, E) against the dense
    fp64 evaluation; bf16 inputs widened exactly on both sides."""
    wl = W.BY_NAME[name]
    inp = W.make_inputs(wl, T=4)
    sh = list(zip(inp.shared_gate_up, inp.shared_down))
    r = oracle.moe_forward(inp.hidden, inp.router_w, inp.gate_up, inp.down, wl.k, wl.routed_scale,
                           inp.bias, shared=sh)
    ref = dense_layer64(inp, ids_ref=r["ids"])
    assert rel_err(r["out"], ref) < 1e-5
    if name == "phimoe_skewed":
        assert np.all(r["ids"][:, 0] == 0)
        assert np.all(r["ids"] < 13)


# ---------------------------------------------------------------- page facts

def test_workload_shapes_match_page_configs():
    g = json.load(open(GOLDEN))
    pc = g["phimoe_config"]
    for name in ("phimoe_decode", "phimoe_prefill", "phimoe_skewed"):
        wl = W.BY_NAME[name]
        assert (wl.H, wl.I, wl.E, wl.k) == (pc["hidden_size"], pc["intermediate_size"],
                                           pc["num_local_experts"], pc["num_experts_per_tok"])
        assert wl.std_weight == pc["initializer_range"]
    ic = g["instella_moe"]
    wl = W.BY_NAME["instella_fine"]
    assert (wl.E, wl.n_shared, wl.k, wl.routed_scale, wl.H) == (
        ic["routed_experts"], ic["shared_experts"], ic["experts_per_tok"],
        ic["routed_scaling_factor"], ic["hidden_size"])


def test_expert_parameter_count_matches_page():
    # 16 experts x (3 * H * I) per layer x 32 layers ~ 16 x 3.1B: the page's
    # "16 x 3.8B" counts the shared attention/embeddings in each expert model;
    # the routed-expert part of the 6.6B active parameters is 2 of 16 experts.
    pc = json.load(open(GOLDEN))["phimoe_config"]
    per_expert_layer = 3 * pc["hidden_size"] * pc["intermediate_size"]
    active_expert = per_expert_layer * pc["num_experts_per_tok"] * pc["num_hidden_layers"]
    act = json.load(open(GOLDEN))["phimoe_active_params"]["active_params_billion"] * 1e9
    assert 0.7 * act < active_expert < act          # experts are most of the active params
    assert active_expert == 5_033_164_800


def test_decode_bandwidth_model_matches_page_estimate():
    import bench
    d = json.load(open(GOLDEN))["decode_bandwidth_estimate"]
    tps = bench.decode_tokens_per_s_bound(d["bandwidth_GBps"] * 1e9,
                                          d["active_params_billion"] * 1e9 * d["bytes_per_param"])
    assert round(tps) == d["estimate_tok_per_s"]
    assert abs(d["measured_tok_per_s"] - tps) / tps < 0.05


def test_nan_keys_rank_below_every_number():
    # NaN logits rank as -inf (ties among them to the lower index), so every
    # token still gets k distinct valid experts
    nan, inf = np.float32("nan"), np.float32("inf")
    l = np.array([[nan, 1.0, nan, -inf, 0.5],
                  [nan, nan, nan, nan, nan],
                  [-inf, -inf, 2.0, nan, -inf],
                  [inf, nan, -1.0, inf, 0.0]], np.float32)
    ids, _ = oracle.select_topk(l, 3)
    assert ids.tolist() == [[1, 4, 0], [0, 1, 2], [2, 0, 1], [0, 3, 4]]
    sids, _ = oracle.select_scored(l, 3, 1.0, "softmax")
    assert np.array_equal(sids, ids)
    # sigmoid scoring: the clamp maps NaN and -inf alike to -80 (equal
    # scores, lower index first)
    g, _ = oracle.select_scored(l, 2, 1.0, "sigmoid")
    assert g.tolist()[1] == [0, 1]
    assert g.tolist()[2] == [2, 0]
