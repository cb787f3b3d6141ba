"""moe_forward inside a captured HIP graph: the call allocates nothing when
given out and a workspace, makes no host synchronisation and records no
memset, so a decode loop can capture it once and replay it. Every replay is
checked bit for bit against an eager call on the same inputs, with new
inputs written into the captured buffers between replays and eager work and
synchronisations in between."""
import numpy as np
import pytest

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


def dev(a):
    return moe.bf16_bits_to_tensor(a)


CASES = [
    ("decode_direct", dict(T=32, H=512, I=256, E=8, k=2), 0, None),
    ("tiled_shared", dict(T=600, H=256, I=256, E=4, k=2, n_shared=1, shared_I=128), moe.FLAG_FORCE_TILED, None),
    ("decode_mxfp4", dict(T=16, H=512, I=256, E=8, k=2), 0, "mxfp4"),
]


@pytest.mark.parametrize("name,kw,flags,lowp", CASES, ids=[c[0] for c in CASES])
def test_captured_call_replays_like_eager(name, kw, flags, lowp):
    print(f"case graph {name} {kw}", flush=True)
    inp = W.custom_inputs(**kw)
    wl = inp.wl
    hidden = dev(inp.hidden)
    router_w, gate_up, down = dev(inp.router_w), dev(inp.gate_up), dev(inp.down)
    extra = dict(routed_scale=wl.routed_scale, flags=flags)
    if lowp == "mxfp4":
        gate_up, gs = moe.quantize_mxfp4_rows(gate_up)
        down, ds = moe.quantize_mxfp4_rows(down)
        extra.update(gate_up_block_scale=gs, down_block_scale=ds)
    shared_I = 0
    if inp.shared_gate_up:
        g, d = inp.shared_concat()
        extra.update(shared_gate_up=dev(g), shared_down=dev(d))
        shared_I = g.shape[0] // 2
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((moe.workspace_bytes(wl.T, wl.H, wl.I, wl.E, wl.k, shared_I=shared_I, flags=flags),),
                     dtype=torch.uint8, device="cuda")

    def call(o):
        return moe.moe_forward(hidden, router_w, gate_up, down, wl.k, out=o, workspace=ws, **extra)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out)  # warm-up on the capturing stream's side, as torch asks
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out)
    torch.cuda.synchronize()

    rng = np.random.default_rng(7)
    eager_out = torch.empty_like(out)
    for rep in range(4):
        if rep:
            x = (rng.standard_normal((wl.T, wl.H)) * (1.0 + rep)).astype(np.float32)
            hidden.copy_(dev(W.f32_to_bf16_bits(x)))
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        call(eager_out)  # eager work between the replays
        torch.cuda.synchronize()
        a = got.view(torch.int16).cpu().numpy()
        b = eager_out.view(torch.int16).cpu().numpy()
        assert np.array_equal(a, b), f"{name}: replay {rep} differs from the eager call"
