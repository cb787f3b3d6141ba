"""GPU parity of the router statistics (load-balancing loss inputs) against
the oracle on the same logits: per-expert mean probability and the auxiliary
loss within 1e-5 relative (fp32 softmax with the fast exponential and fp32
sums against fp64), per-expert load exact up to one fp32 division."""
import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import sparse_mixture_experts_logits_amd as moe  # noqa: E402


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()
    yield


def run(inp, mask=None, flags=0):
    d = moe.bf16_bits_to_tensor
    wl = inp.wl
    sgu = sdn = None
    if inp.shared_gate_up:
        g, dd = inp.shared_concat()
        sgu, sdn = d(g), d(dd)
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).cuda()
    m = None if mask is None else torch.from_numpy(mask).cuda()
    _, r = moe.moe_forward(d(inp.hidden), d(inp.router_w), d(inp.gate_up), d(inp.down), wl.k,
                           routed_scale=wl.routed_scale, router_bias=bias, shared_gate_up=sgu, shared_down=sdn,
                           flags=flags, router_stats=True, stats_mask=m)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in r.items()}


def check(inp, mask, what):
    got = run(inp, mask)
    logits = oracle.router_logits(inp.hidden, inp.router_w, inp.bias)
    ids, _ = oracle.select_topk(logits, inp.wl.k, inp.wl.routed_scale)
    assert np.array_equal(got["ids"], ids), f"{what}: ids differ"
    ref = oracle.router_stats(logits, ids, mask)
    _say(f"  {what}: aux gpu {got['aux_loss'][0]:.7f} oracle {ref['aux']:.7f}")
    assert np.allclose(got["prob_mean"], ref["prob_mean"], rtol=1e-5, atol=1e-8), f"{what}: prob_mean"
    assert np.allclose(got["load"], ref["load"], rtol=1e-6, atol=0), f"{what}: load"
    assert abs(got["aux_loss"][0] - ref["aux"]) <= 1e-5 * max(1.0, ref["aux"]), f"{what}: aux"


CASES = [
    ("decode_shape", dict(T=32, H=512, I=64, E=16, k=2)),
    ("ragged_blocks", dict(T=257, H=256, I=64, E=16, k=2)),
    ("fine", dict(T=96, H=192, I=64, E=32, k=6, routed_scale=2.5)),
    ("many_experts", dict(T=300, H=128, I=32, E=256, k=8)),
    ("biased", dict(T=129, H=128, I=64, E=16, k=2, bias=((0, 6.0), (13, -30.0), (14, -30.0), (15, -30.0)))),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_router_stats_small(name, kw):
    _say(f"case stats {name}")
    inp = W.custom_inputs(**kw)
    check(inp, None, name)
    rng = np.random.default_rng(kw["T"])
    check(inp, (rng.random(kw["T"]) < 0.6).astype(np.int32), name + " masked")
    check(inp, np.zeros(kw["T"], dtype=np.int32), name + " all masked")


@pytest.mark.parametrize("name", ["phimoe_decode", "instella_fine", "phimoe_prefill"])
def test_router_stats_full_size(name):
    _say(f"case stats {name}")
    check(W.make_inputs(W.BY_NAME[name]), None, name)
