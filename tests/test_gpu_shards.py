"""The layer's GPU kernels at the shapes of one GPU's share when the layer is
split over G GPUs, checked by the identities the split relies on (the
expert-parallel and tensor-parallel plans of the Transformers MoE page and
the GraniteMoeSWA walkthrough): with the routing unchanged,

* the outputs counting only one group of experts' assignments (the other
  experts' weights zeroed, so they add exact zeros) sum to the layer output;
* the outputs of the G column shards of every expert (I/G matching gate and
  up rows, the same down columns) sum to the layer output.

Each partial output is a bf16 GPU result; their fp32 sum is compared with
the oracle's layer output to the parity bar (2e-2 * max|ref|), and the
routing of every shard launch is bit-exact with the full launch. Decode-sized
batches run the weight-streaming kernels, larger ones the tiled kernels."""
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


def dev(a):
    return moe.bf16_bits_to_tensor(np.ascontiguousarray(a), torch.device("cuda", 0))


def gpu_layer(inp, gate_up, down):
    out, r = moe.moe_forward(dev(inp.hidden), dev(inp.router_w), dev(gate_up), dev(down), inp.wl.k,
                             return_routing=True)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), r["ids"].cpu().numpy()


def oracle_full(inp):
    logits = oracle.router_logits(inp.hidden, inp.router_w)
    ids, w = oracle.select_topk(logits, inp.wl.k)
    return ids, oracle.moe_tokens(inp.hidden, inp.gate_up, inp.down, ids, w)


def check(total, ref, what):
    err = np.max(np.abs(total - ref))
    scale = np.max(np.abs(ref))
    _say(f"  {what}: max|err|/max|ref| = {err / scale:.3e}")
    assert np.all(np.isfinite(total)) and err <= OUT_TOL * scale, what


SHAPES = [(32, 512, 1024, 8, 2), (256, 512, 1024, 8, 2)]


@pytest.mark.parametrize("T,H,I,E,k", SHAPES)
def test_expert_parallel_shares_sum_to_the_layer(T, H, I, E, k):
    _say(f"case expert groups T={T} H={H} I={I} E={E} k={k}")
    inp = W.custom_inputs(T, H, I, E, k, seed=51)
    ids_ref, ref = oracle_full(inp)
    total = np.zeros((T, H), dtype=np.float64)
    zero_bits = np.uint16(0)  # +0.0 in bf16
    for g in np.array_split(np.arange(E), 4):
        gu = np.full_like(inp.gate_up, zero_bits)
        dn = np.full_like(inp.down, zero_bits)
        gu[g] = inp.gate_up[g]
        dn[g] = inp.down[g]
        part, ids = gpu_layer(inp, gu, dn)
        assert np.array_equal(ids, ids_ref), "routing changed"
        total += part
    check(total, ref, "sum over expert groups")


@pytest.mark.parametrize("T,H,I,E,k", SHAPES)
def test_tensor_parallel_shares_sum_to_the_layer(T, H, I, E, k):
    G = 4
    _say(f"case column shards T={T} H={H} I={I} E={E} k={k} G={G}")
    inp = W.custom_inputs(T, H, I, E, k, seed=53)
    ids_ref, ref = oracle_full(inp)
    Is = I // G
    total = np.zeros((T, H), dtype=np.float64)
    for g in range(G):
        lo, hi = g * Is, (g + 1) * Is
        gu = np.concatenate([inp.gate_up[:, lo:hi], inp.gate_up[:, I + lo:I + hi]], axis=1)
        dn = inp.down[:, :, lo:hi]
        part, ids = gpu_layer(inp, gu, dn)
        assert np.array_equal(ids, ids_ref), "routing changed"
        total += part
    check(total, ref, "sum over column shards")
