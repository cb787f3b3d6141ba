"""The allocation-free entry point (moe_forward_noalloc) through the C ABI,
against moe_forward with a caller workspace on the same inputs: bitwise equal
outputs and routing, and within the oracle's bar; two calls in a row, the
second with fewer tokens (the scratch keeps the first call's contents)."""
import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import sparse_mixture_experts_logits_amd as moe  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()
    yield


def _dev(a):
    return moe.bf16_bits_to_tensor(a, "cuda:0")


def _run(inp, no_alloc, **kw):
    wl = inp.wl
    sgu = sdn = None
    if inp.shared_gate_up:
        gu, dn = inp.shared_concat()
        sgu, sdn = _dev(gu), _dev(dn)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda:0")
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).to("cuda:0")
    res = moe.moe_forward(_dev(inp.hidden), _dev(inp.router_w), _dev(inp.gate_up), _dev(inp.down), wl.k,
                          routed_scale=wl.routed_scale, router_bias=bias, shared_gate_up=sgu, shared_down=sdn,
                          out=out, no_alloc=no_alloc, **kw)
    torch.cuda.synchronize()
    return res


def _oracle(inp):
    wl = inp.wl
    logits = oracle.router_logits(inp.hidden, inp.router_w, inp.bias)
    ids, w = oracle.select_topk(logits, wl.k, wl.routed_scale)
    ref = oracle.moe_tokens(inp.hidden, inp.gate_up, inp.down, ids, w, tokens=np.arange(wl.T, dtype=np.int32),
                            shared=list(zip(inp.shared_gate_up, inp.shared_down)))
    return ids, ref


@pytest.mark.parametrize("Ts,kw", [
    ((32, 5), dict(H=1024, I=768, E=8, k=2)),
    ((32, 5), dict(H=512, I=256, E=16, k=4, n_shared=1, shared_I=128, routed_scale=2.5)),
    # more than 32 tokens, few rows per expert on average: the mixed schedule
    # (streaming kernels, plus the tiled kernel for experts past 32 rows)
    ((200, 48), dict(H=512, I=256, E=16, k=2, bias=((0, 6.0),))),
], ids=["plain", "shared", "mixed"])
def test_noalloc_matches_workspace_entry_point_twice(Ts, kw):
    print(f"case noalloc {Ts} {kw}", flush=True)
    for i, T in enumerate(Ts):  # the second call is smaller
        inp = W.custom_inputs(T=T, **kw, std_weight=0.05, seed=i)
        a, ra = _run(inp, no_alloc=True, return_routing=True)
        b, rb = _run(inp, no_alloc=False, return_routing=True)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"T={T}: outputs differ"
        for key in ra:
            assert torch.equal(ra[key], rb[key]), f"T={T}: {key} differs"
        # the plain launch (no routing outputs) too
        c = _run(inp, no_alloc=True)
        assert torch.equal(c.view(torch.int16), b.view(torch.int16)), f"T={T}: plain launch differs"
        ids, ref = _oracle(inp)
        assert np.array_equal(ra["ids"].cpu().numpy(), ids)
        got = a.float().cpu().numpy()
        err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
        print(f"  T={T}: max|err|/max|ref| = {err:.2e}", flush=True)
        assert err <= 2e-2


def test_noalloc_rejects_a_workspace_and_oversized_calls():
    print("case noalloc argument checks", flush=True)
    inp = W.custom_inputs(T=8, H=64, I=32, E=4, k=2)
    args = (_dev(inp.hidden), _dev(inp.router_w), _dev(inp.gate_up), _dev(inp.down), 2)
    with pytest.raises(ValueError, match="no workspace"):
        moe.moe_forward(*args, no_alloc=True, workspace=torch.empty(1 << 20, dtype=torch.uint8, device="cuda"))
    # a large prefill call needs more scratch than the library holds
    big = W.custom_inputs(T=8192, H=4096, I=64, E=4, k=2)
    assert moe.workspace_bytes(8192, 4096, 64, 4, 2) > moe.NOALLOC_SCRATCH_BYTES
    with pytest.raises(moe.MoeError, match="scratch"):
        moe.moe_forward(_dev(big.hidden), _dev(big.router_w), _dev(big.gate_up), _dev(big.down), 2, no_alloc=True)
