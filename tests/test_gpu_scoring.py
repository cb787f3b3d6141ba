"""GPU parity of the router scoring variants (sigmoid scores, a bias that
steers selection only, group-limited selection, PhiMoE's sparsemixer at
inference) against the oracle.

Bar: expert ids, counts, offsets and the permutation bit-exact (both sides
compute the selection keys with the same IEEE fp32 operation sequence);
weights within 2e-6 relative (fp32 sums against fp64); layer output within
max|out - ref| <= 2e-2 * max|ref|."""
import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import sparse_mixture_experts_logits_amd as moe  # noqa: E402

OUT_TOL = 2e-2


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()
    yield


def run(inp, sc, flags=0):
    d = moe.bf16_bits_to_tensor
    wl = inp.wl
    sgu = sdn = None
    if inp.shared_gate_up:
        g, dd = inp.shared_concat()
        sgu, sdn = d(g), d(dd)
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).cuda()
    sb = None if sc.get("selection_bias") is None else torch.from_numpy(sc["selection_bias"]).cuda()
    out, r = moe.moe_forward(d(inp.hidden), d(inp.router_w), d(inp.gate_up), d(inp.down), wl.k,
                             routed_scale=wl.routed_scale, router_bias=bias, shared_gate_up=sgu,
                             shared_down=sdn, flags=flags, return_routing=True, score_func=sc["score_func"],
                             selection_bias=sb, n_group=sc.get("n_group", 0), topk_group=sc.get("topk_group", 0),
                             jitter_eps=sc.get("jitter_eps"))
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), {k: v.cpu().numpy() for k, v in r.items()}


def check(inp, sc, tokens, what, flags=0):
    wl = inp.wl
    logits = oracle.router_logits(inp.hidden, inp.router_w, inp.bias)
    if sc["score_func"] == "sparsemixer":
        ids, w = oracle.select_sparsemixer(logits, wl.k, wl.routed_scale, sc.get("jitter_eps", 0.01))
    else:
        ids, w = oracle.select_scored(logits, wl.k, wl.routed_scale, sc["score_func"], sc.get("selection_bias"),
                                      sc.get("n_group", 0), sc.get("topk_group", 0))
    counts, offsets, perm, inv = oracle.route(ids, wl.E)
    out, got = run(inp, sc, flags)
    assert np.array_equal(got["logits"].view(np.uint32), logits.view(np.uint32)), f"{what}: logits differ"
    assert np.array_equal(got["ids"], ids), f"{what}: ids differ"
    for key, ref in (("counts", counts), ("offsets", offsets), ("perm", perm), ("inv", inv)):
        assert np.array_equal(got[key], ref), f"{what}: {key} differs"
    assert np.allclose(got["weights"], w, rtol=2e-6, atol=1e-7), f"{what}: weights differ"
    shared = list(zip(inp.shared_gate_up, inp.shared_down))
    ref = oracle.moe_tokens(inp.hidden, inp.gate_up, inp.down, ids, w, tokens=tokens, shared=shared)
    o = out[tokens]
    err, scale = np.max(np.abs(o - ref)), np.max(np.abs(ref))
    _say(f"  {what}: max|err|/max|ref| = {err / scale:.3e}")
    assert np.all(np.isfinite(o)) and err <= OUT_TOL * scale, f"{what}: output"


def sel_bias(E, seed, std=0.02):
    return (np.random.default_rng(seed).standard_normal(E) * std).astype(np.float32)


SMALL = [
    # name, custom_inputs kwargs, scoring
    ("sigmoid_decode", dict(T=32, H=256, I=64, E=64, k=6, routed_scale=2.5), dict(score_func="sigmoid")),
    ("sigmoid_bias", dict(T=96, H=192, I=64, E=64, k=6, routed_scale=2.5),
     dict(score_func="sigmoid", selection_bias=sel_bias(64, 1))),
    ("sigmoid_groups", dict(T=300, H=128, I=32, E=64, k=6, routed_scale=2.5),
     dict(score_func="sigmoid", selection_bias=sel_bias(64, 2), n_group=8, topk_group=3)),
    ("v3_shape_groups", dict(T=257, H=128, I=32, E=256, k=8, routed_scale=2.5),
     dict(score_func="sigmoid", selection_bias=sel_bias(256, 3), n_group=8, topk_group=4)),
    ("v3_shape_decode", dict(T=20, H=128, I=32, E=256, k=8),
     dict(score_func="sigmoid", selection_bias=sel_bias(256, 4), n_group=8, topk_group=4)),
    ("softmax_groups_bias", dict(T=129, H=128, I=64, E=16, k=2),
     dict(score_func="softmax", selection_bias=sel_bias(16, 5, 0.3), n_group=4, topk_group=2)),
    ("single_expert_groups", dict(T=70, H=128, I=32, E=16, k=4),
     dict(score_func="sigmoid", n_group=16, topk_group=4)),
    ("one_group_kept", dict(T=65, H=128, I=32, E=32, k=4),
     dict(score_func="sigmoid", selection_bias=sel_bias(32, 6), n_group=4, topk_group=1)),
    ("shared_sigmoid", dict(T=130, H=136, I=72, E=8, k=2, n_shared=2, shared_I=40),
     dict(score_func="sigmoid", selection_bias=sel_bias(8, 7))),
    # sparsemixer: small router weights put many logits within the threshold
    ("sparsemixer_decode", dict(T=32, H=512, I=64, E=16, k=2), dict(score_func="sparsemixer")),
    ("sparsemixer_wide", dict(T=300, H=128, I=32, E=64, k=4), dict(score_func="sparsemixer", jitter_eps=0.2)),
    ("sparsemixer_ties", dict(T=70, H=64, I=32, E=16, k=2),
     dict(score_func="sparsemixer", jitter_eps=0.0)),
]


@pytest.mark.parametrize("name,kw,sc", SMALL, ids=[s[0] for s in SMALL])
def test_scoring_small(name, kw, sc):
    _say(f"case scoring {name}")
    inp = W.custom_inputs(**kw, std_weight=0.05)
    if name == "sparsemixer_ties":
        # a zero router: every logit 0, so every gap is 0/0 and all experts tie
        inp.router_w[:] = 0
    check(inp, sc, np.arange(kw["T"], dtype=np.int32), name)


def test_scoring_tiled_path():
    _say("case scoring tiled")
    kw = dict(T=700, H=328, I=200, E=16, k=4)
    inp = W.custom_inputs(**kw, std_weight=0.05)
    sc = dict(score_func="sigmoid", selection_bias=sel_bias(16, 8), n_group=4, topk_group=2)
    check(inp, sc, np.arange(kw["T"], dtype=np.int32), "tiled", flags=moe.FLAG_FORCE_TILED)


@pytest.mark.parametrize("T", [32, 4096])
def test_sparsemixer_phimoe_full_size(T):
    _say(f"case sparsemixer phimoe T={T}")
    inp = W.make_inputs(W.BY_NAME["phimoe_decode"], T=T)
    tokens = np.arange(T, dtype=np.int32) if T <= 32 else np.linspace(0, T - 1, 16).astype(np.int32)
    check(inp, dict(score_func="sparsemixer"), tokens, f"sparsemixer phimoe T={T}")


@pytest.mark.parametrize("T", [32, 4096])
def test_scoring_instella_full_size(T):
    # Instella's routed experts (64, 6 per token, scale 2.5) under noaux-style routing
    _say(f"case scoring instella T={T}")
    inp = W.make_inputs(W.BY_NAME["instella_fine"], T=T)
    sc = dict(score_func="sigmoid", selection_bias=sel_bias(inp.wl.E, 9, 0.01), n_group=8, topk_group=4)
    tokens = np.arange(T, dtype=np.int32) if T <= 32 else np.linspace(0, T - 1, 24).astype(np.int32)
    check(inp, sc, tokens, f"instella T={T}")


# Routing at sizes past the small cases: hidden sizes that are not a multiple
# of the 512-element chunk a wave sums (absent slices in the last chunk),
# expert counts that leave the last group of four experts partly empty, 16k
# tokens with ragged last router blocks, and the largest k next to E.
LARGER = [
    ("h3000_e20", dict(T=1000, H=3000, I=32, E=20, k=3), dict(score_func="softmax")),
    ("t16500_groups", dict(T=16500, H=1000, I=32, E=64, k=4, routed_scale=2.5),
     dict(score_func="sigmoid", selection_bias=sel_bias(64, 10), n_group=8, topk_group=3)),
    ("t16400_k16", dict(T=16400, H=4096, I=16, E=40, k=16), dict(score_func="softmax")),
    ("t16400_k17", dict(T=16400, H=512, I=16, E=24, k=17), dict(score_func="softmax")),
    ("h2056_sparsemixer", dict(T=777, H=2056, I=32, E=16, k=2), dict(score_func="sparsemixer")),
]


@pytest.mark.parametrize("name,kw,sc", LARGER, ids=[s[0] for s in LARGER])
def test_routing_larger_shapes(name, kw, sc):
    _say(f"case routing {name}")
    inp = W.custom_inputs(**kw, std_weight=0.05)
    T = kw["T"]
    tokens = np.unique(np.concatenate([np.linspace(0, T - 1, 20).astype(np.int32),
                                       np.arange(max(0, T - 5), T, dtype=np.int32)]))
    check(inp, sc, tokens, name)
