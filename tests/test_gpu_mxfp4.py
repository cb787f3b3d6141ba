"""GPU parity of the MXFP4 expert weights (OCP MX: FP4 E2M1 codes, one E8M0
scale per 32 consecutive weights of a row) against the CPU oracle.

Bar: the quantisation kernel's codes and scales bit-exact with the oracle's
quantiser (which rounds by brute-force nearest value, the kernel by counting
boundaries); routing bit-exact; the layer output within
max|out - ref| <= 2e-2 * max|ref| of the bf16 oracle run on the oracle's
dequantised weights (every MXFP4 weight is exactly a bf16 value, so the
kernel multiplies the same numbers)."""
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
    return moe.bf16_bits_to_tensor(a)


def check_quant(bits, what):
    q, s = moe.quantize_mxfp4_rows(dev(bits))
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_mxfp4_rows(bits)
    gq, gs = q.cpu().numpy(), s.cpu().numpy()
    bad = np.argwhere(gq != rq)
    assert bad.size == 0, f"{what}: {len(bad)} code bytes differ, first at {bad[0].tolist()}"
    assert np.array_equal(gs, rs), f"{what}: block scales differ"
    return q, s, rq, rs


def crafted_rows():
    """Blocks fixed to factor 1 by a 4.0, walking every rounding boundary and
    one bf16 ulp either side of it, both signs; an all-zero block; negative
    zeros; tiny and huge blocks (factors 2^-127 and 2^125)."""
    pts = []
    for b in (0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0, 7.9):
        u = int(np.float32(b).view(np.uint32)) >> 16
        for d in (-1, 0, 1):
            pts.append(np.uint32((u + d) << 16).view(np.float32))
    rows = []
    for c in range(0, len(pts), 31):
        row = np.zeros(32, np.float32)
        row[0] = 4.0
        part = pts[c:c + 31]
        row[1:1 + len(part)] = part
        rows += [row, -row]
    rows.append(np.zeros(32, np.float32))
    rows.append(-np.zeros(32, np.float32))
    rows.append(np.full(32, 2.0 ** -125, np.float32) * np.linspace(0.5, 1.5, 32, dtype=np.float32))
    rows.append(np.full(32, 2.0 ** 126, np.float32) * np.linspace(-1.5, 1.5, 32, dtype=np.float32))
    x = np.stack(rows).reshape(-1, 64)
    return W.f32_to_bf16_bits(x)


def test_quantize_kernel_bit_exact_on_crafted_rows():
    _say("case mxfp4 crafted rows")
    check_quant(crafted_rows(), "crafted")


@pytest.mark.parametrize("rows,cols,std", [(7, 32, 1.0), (300, 96, 0.02), (64, 4096, 0.02), (33, 6400, 3.0)])
def test_quantize_kernel_bit_exact_on_random_rows(rows, cols, std):
    _say(f"case mxfp4 random rows {rows}x{cols} std {std}")
    rng = np.random.default_rng(rows * 11 + cols)
    x = (rng.standard_normal((rows, cols)) * std).astype(np.float32)
    x[rng.integers(0, rows, 9), rng.integers(0, cols, 9)] *= 30.0
    check_quant(W.f32_to_bf16_bits(x), f"{rows}x{cols}")


def run_mxfp4(inp, gq, gs, dq, ds, flags=0, routing=True):
    wl = inp.wl
    sgu = sdn = None
    if inp.shared_gate_up:
        g, d = inp.shared_concat()
        sgu, sdn = dev(g), dev(d)
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).cuda()
    res = moe.moe_forward(dev(inp.hidden), dev(inp.router_w), gq, dq, wl.k, routed_scale=wl.routed_scale,
                          router_bias=bias, shared_gate_up=sgu, shared_down=sdn, flags=flags,
                          gate_up_block_scale=gs, down_block_scale=ds, return_routing=routing)
    torch.cuda.synchronize()
    if not routing:
        return res.float().cpu().numpy(), None
    out, r = res
    return out.float().cpu().numpy(), {k: v.cpu().numpy() for k, v in r.items()}


def check_against_oracle(inp, tokens, what, flags=0):
    gq, gs, rgq, rgs = check_quant(inp.gate_up, f"{what} gate_up")
    dq, ds, rdq, rds = check_quant(inp.down, f"{what} down")
    out, got = run_mxfp4(inp, gq, gs, dq, ds, flags)
    # the launch without routing outputs (direct routing at few assignments)
    # computes the same thing bit for bit
    out_plain, _ = run_mxfp4(inp, gq, gs, dq, ds, flags, routing=False)
    assert np.array_equal(out_plain.view(np.uint32), out.view(np.uint32)), f"{what}: direct routing differs"
    wl = inp.wl
    logits = oracle.router_logits(inp.hidden, inp.router_w, inp.bias)
    ids, w = oracle.select_topk(logits, wl.k, wl.routed_scale)
    counts, offsets, perm, inv = oracle.route(ids, wl.E)
    for key, ref in (("ids", ids), ("counts", counts), ("offsets", offsets), ("perm", perm), ("inv", inv)):
        assert np.array_equal(got[key], ref), f"{what}: {key} differs"
    assert np.allclose(got["weights"], w, rtol=2e-6, atol=1e-7)
    gu_d = oracle.dequantize_mxfp4_rows(rgq, rgs)
    dn_d = oracle.dequantize_mxfp4_rows(rdq, rds)
    shared = list(zip(inp.shared_gate_up, inp.shared_down))
    ref = oracle.moe_tokens(inp.hidden, gu_d, dn_d, ids, w, tokens=tokens, shared=shared)
    got_t = out[tokens]
    err, scale = np.max(np.abs(got_t - ref)), np.max(np.abs(ref))
    _say(f"  {what}: max|err|/max|ref| = {err / scale:.3e}")
    assert np.all(np.isfinite(got_t)) and err <= OUT_TOL * scale


SMALL = [
    ("tiny", dict(T=40, H=64, I=64, E=5, k=2)),
    ("multi_pass", dict(T=100, H=256, I=128, E=8, k=2)),          # > 16 rows per expert: several passes
    ("ragged_k", dict(T=50, H=544, I=96, E=4, k=2)),               # K not a multiple of the 512-wide step
    ("fine", dict(T=96, H=192, I=64, E=32, k=6, routed_scale=2.5)),
    ("shared_bias", dict(T=70, H=128, I=64, E=16, k=2, n_shared=2, shared_I=32,
                         bias=((0, 6.0), (13, -30.0), (14, -30.0), (15, -30.0)))),
    ("one_token", dict(T=1, H=4096, I=256, E=16, k=2)),
    ("max_experts", dict(T=40, H=128, I=64, E=256, k=8)),          # the largest E the ABI takes
]


@pytest.mark.parametrize("name,kw", SMALL, ids=[c[0] for c in SMALL])
def test_mxfp4_layer_small(name, kw):
    _say(f"case mxfp4 {name} {kw}")
    inp = W.custom_inputs(**kw)
    check_against_oracle(inp, np.arange(inp.wl.T, dtype=np.int32), name)


def test_mxfp4_decode_full_size():
    _say("case mxfp4 phimoe_decode")
    inp = W.make_inputs(W.BY_NAME["phimoe_decode"])
    check_against_oracle(inp, np.arange(inp.wl.T, dtype=np.int32), "phimoe_decode mxfp4")


def test_mxfp4_layer_run_to_run_identical():
    _say("case mxfp4 run to run")
    inp = W.custom_inputs(T=100, H=256, I=128, E=8, k=2)
    gq, gs = moe.quantize_mxfp4_rows(dev(inp.gate_up))
    dq, ds = moe.quantize_mxfp4_rows(dev(inp.down))
    a, _ = run_mxfp4(inp, gq, gs, dq, ds)
    b, _ = run_mxfp4(inp, gq, gs, dq, ds)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_mxfp4_unaligned_scale_arrays():
    # block scales that start at an odd byte address take the byte-wise scale
    # loads; the result is the same bit for bit
    _say("case mxfp4 unaligned scale arrays")
    inp = W.custom_inputs(T=24, H=512, I=256, E=4, k=2)
    gq, gs = moe.quantize_mxfp4_rows(dev(inp.gate_up))
    dq, ds = moe.quantize_mxfp4_rows(dev(inp.down))
    a, _ = run_mxfp4(inp, gq, gs, dq, ds)
    gs_buf = torch.empty(gs.numel() + 1, dtype=torch.uint8, device=gs.device)
    ds_buf = torch.empty(ds.numel() + 1, dtype=torch.uint8, device=ds.device)
    gs_odd = gs_buf[1:].view(gs.shape)
    ds_odd = ds_buf[1:].view(ds.shape)
    gs_odd.copy_(gs)
    ds_odd.copy_(ds)
    assert gs_odd.data_ptr() % 4 == 1 and ds_odd.data_ptr() % 4 == 1
    b, _ = run_mxfp4(inp, gq, gs_odd, dq, ds_odd)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("score", ["sigmoid_groups", "sparsemixer"])
def test_mxfp4_with_scoring_variants_shared_expert_and_direct_routing(score):
    # the options meet: MXFP4 routed weights, a router variant, a shared
    # expert (bf16) and the launch without routing outputs (direct routing)
    _say(f"case mxfp4 + {score} + shared expert")
    inp = W.custom_inputs(T=24, H=256, I=128, E=32, k=4, routed_scale=2.5, n_shared=1, shared_I=64)
    wl = inp.wl
    gq, gs = moe.quantize_mxfp4_rows(dev(inp.gate_up))
    dq, ds = moe.quantize_mxfp4_rows(dev(inp.down))
    rgq, rgs = oracle.quantize_mxfp4_rows(inp.gate_up)
    rdq, rds = oracle.quantize_mxfp4_rows(inp.down)
    g, d = inp.shared_concat()
    kw = dict(routed_scale=wl.routed_scale, shared_gate_up=dev(g), shared_down=dev(d),
              gate_up_block_scale=gs, down_block_scale=ds)
    logits = oracle.router_logits(inp.hidden, inp.router_w, inp.bias)
    if score == "sparsemixer":
        kw.update(score_func="sparsemixer", jitter_eps=0.05)
        ids, w = oracle.select_sparsemixer(logits, wl.k, wl.routed_scale, 0.05)
    else:
        bias = (np.random.default_rng(9).standard_normal(wl.E) * 0.02).astype(np.float32)
        kw.update(score_func="sigmoid", selection_bias=torch.from_numpy(bias).cuda(), n_group=8, topk_group=3)
        ids, w = oracle.select_scored(logits, wl.k, wl.routed_scale, "sigmoid", bias, 8, 3)
    out_r, r = moe.moe_forward(dev(inp.hidden), dev(inp.router_w), gq, dq, wl.k, return_routing=True, **kw)
    out_d = moe.moe_forward(dev(inp.hidden), dev(inp.router_w), gq, dq, wl.k, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(r["ids"].cpu().numpy(), ids)
    a, b = out_r.float().cpu().numpy(), out_d.float().cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "direct routing differs"
    ref = oracle.moe_tokens(inp.hidden, oracle.dequantize_mxfp4_rows(rgq, rgs), oracle.dequantize_mxfp4_rows(rdq, rds),
                            ids, w, tokens=np.arange(wl.T, dtype=np.int32), shared=[(g, d)])
    err, scale = np.max(np.abs(b - ref)), np.max(np.abs(ref))
    _say(f"  max|err|/max|ref| = {err / scale:.3e}")
    assert np.all(np.isfinite(b)) and err <= OUT_TOL * scale
