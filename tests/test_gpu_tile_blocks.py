"""Routed expert weights in tile blocks (MOE_LAYOUT_TILE_BLOCKS).

The packing entry point is checked bit for bit against the block layout the
header defines, built here with numpy from the nn.Linear arrays (ragged
shapes: rows and columns past the matrix are zeros). The layer with packed
weights runs the same arithmetic as the nn.Linear layout on the tiled
schedule, so its output must equal that launch bit for bit (the tiled launch
itself is checked against the oracle in test_gpu_parity.py); the small
shapes are also compared with the oracle directly, at the layer's bar
max|out - ref| <= 2e-2 * max|ref|.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from parity_sampling import tile_aware_positions

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


def blocks_ref(w, which, I, H):
    """The tile blocks of the header's definition, from uint16 bf16 bits."""
    E = w.shape[0]
    if which == moe.PACK_GATE_UP:
        nb, nk = -(-I // 128), -(-H // 32)
        out = np.zeros((E, nb, nk, 256, 32), np.uint16)
        for b in range(nb):
            for half in range(2):
                j0 = b * 128
                j1 = min(I, j0 + 128)
                rows = w[:, half * I + j0:half * I + j1, :]          # [E, j1-j0, H]
                pad = np.zeros((E, j1 - j0, nk * 32), np.uint16)
                pad[:, :, :H] = rows
                out[:, b, :, half * 128:half * 128 + (j1 - j0), :] = pad.reshape(E, j1 - j0, nk, 32).transpose(0, 2, 1, 3)
    else:
        nb, nk = -(-H // 256), -(-I // 32)
        out = np.zeros((E, nb, nk, 256, 32), np.uint16)
        for b in range(nb):
            r0, r1 = b * 256, min(H, b * 256 + 256)
            pad = np.zeros((E, r1 - r0, nk * 32), np.uint16)
            pad[:, :, :I] = w[:, r0:r1, :]
            out[:, b, :, :r1 - r0, :] = pad.reshape(E, r1 - r0, nk, 32).transpose(0, 2, 1, 3)
    return out.reshape(-1)


@pytest.mark.parametrize("E,I,H", [(3, 200, 328), (2, 136, 264), (4, 256, 512), (1, 8, 40)])
def test_packing_matches_the_block_layout(E, I, H):
    _say(f"case pack E={E} I={I} H={H}")
    inp = W.custom_inputs(T=4, H=H, I=I, E=E, k=1)
    for which, w in ((moe.PACK_GATE_UP, inp.gate_up), (moe.PACK_DOWN, inp.down)):
        blk = moe.pack_tile_blocks(moe.bf16_bits_to_tensor(w), which)
        torch.cuda.synchronize()
        got = blk.data.view(torch.int16).cpu().numpy().view(np.uint16)
        assert got.size * 2 == moe.tile_blocks_bytes(which, E, I, H)
        assert np.array_equal(got, blocks_ref(w, which, I, H)), f"which={which}"


def _run(inp, blocks, flags=0, tokens=None):
    wl = inp.wl
    d = moe.bf16_bits_to_tensor
    gu, dn = d(inp.gate_up), d(inp.down)
    if blocks:
        gu, dn = moe.pack_tile_blocks(gu, moe.PACK_GATE_UP), moe.pack_tile_blocks(dn, moe.PACK_DOWN)
    sgu = sdn = None
    if inp.shared_gate_up:
        g, s = inp.shared_concat()
        sgu, sdn = d(g), d(s)
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).cuda()
    out, r = moe.moe_forward(d(inp.hidden), d(inp.router_w), gu, dn, wl.k, routed_scale=wl.routed_scale,
                             router_bias=bias, shared_gate_up=sgu, shared_down=sdn, flags=flags,
                             return_routing=True)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy(), {k: v.cpu().numpy() for k, v in r.items()}


def _check_oracle(inp, out_bits, ids, w, tokens, what):
    shared = list(zip(inp.shared_gate_up, inp.shared_down))
    ref = oracle.moe_tokens(inp.hidden, inp.gate_up, inp.down, ids, w, tokens=tokens, shared=shared)
    got = (out_bits[tokens].astype(np.uint16).astype(np.uint32) << 16).view(np.float32)
    err, scale = np.max(np.abs(got - ref)), np.max(np.abs(ref))
    _say(f"  {what}: max|err|/max|ref| = {err / scale:.3e}")
    assert np.all(np.isfinite(got)) and err <= OUT_TOL * scale, what


SMALL = [
    ("ragged", dict(T=700, H=328, I=200, E=4, k=2)),             # tiles overhang N and K
    ("multi_tile", dict(T=1100, H=256, I=384, E=6, k=3)),        # several M-tiles per expert, folded tails
    ("shared", dict(T=130, H=136, I=72, E=8, k=2, n_shared=2, shared_I=40, routed_scale=0.5)),
    ("decode_sized", dict(T=32, H=512, I=256, E=16, k=2)),       # few rows: split along K
    ("one_token", dict(T=1, H=4096, I=256, E=16, k=2)),
    ("fine_grained", dict(T=96, H=192, I=64, E=32, k=6, routed_scale=2.5)),
]


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_layer_with_tile_blocks(name, kw):
    _say(f"case layer {name}")
    inp = W.custom_inputs(**kw)
    got, r = _run(inp, True)
    rows, r0 = _run(inp, False, flags=moe.FLAG_FORCE_TILED)
    for key in ("ids", "counts", "perm"):
        assert np.array_equal(r[key], r0[key]), key
    assert np.array_equal(got, rows), f"{name}: tile blocks differ from the row layout on the tiled schedule"
    _check_oracle(inp, got, r["ids"], r["weights"], np.arange(kw["T"], dtype=np.int32), name)


@pytest.mark.parametrize("name", ["phimoe_prefill", "instella_fine", "phimoe_skewed"])
def test_full_size_with_tile_blocks(name):
    _say(f"case full size {name}")
    inp = W.make_inputs(W.BY_NAME[name])
    got, r = _run(inp, True)
    rows, r0 = _run(inp, False, flags=moe.FLAG_FORCE_TILED)
    assert np.array_equal(r["ids"], r0["ids"])
    assert np.array_equal(got, rows), f"{name}: tile blocks differ from the row layout"
    # and against the oracle on a spread of the tokens whose rows open, close
    # or extend an M-tile (the tile-aware rows of the full parity test)
    pos = np.array(sorted(tile_aware_positions(r["counts"], r["offsets"])), dtype=np.int64)
    tokens = np.unique(r["perm"][pos] // inp.wl.k).astype(np.int32)
    tokens = tokens[::max(1, len(tokens) // 96)]
    _check_oracle(inp, got, r["ids"], r["weights"], tokens, name)


def test_noalloc_with_tile_blocks():
    _say("case noalloc tile blocks")
    inp = W.custom_inputs(T=300, H=256, I=128, E=8, k=2)
    d = moe.bf16_bits_to_tensor
    gu = moe.pack_tile_blocks(d(inp.gate_up), moe.PACK_GATE_UP)
    dn = moe.pack_tile_blocks(d(inp.down), moe.PACK_DOWN)
    out = torch.empty((300, 256), dtype=torch.bfloat16, device="cuda")
    a = moe.moe_forward(d(inp.hidden), d(inp.router_w), gu, dn, 2, out=out.clone())
    b = moe.moe_forward(d(inp.hidden), d(inp.router_w), gu, dn, 2, out=out, no_alloc=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
