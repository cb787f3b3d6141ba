"""GPU parity of the FP8 (OCP E4M3, one fp32 scale per weight row) expert
weights against the CPU oracle.

Bar: the quantisation kernel's codes and scales bit-exact with the oracle's
quantiser (which finds codes by a different method, bisection over the code
values); routing bit-exact as for bf16 weights; the layer output within
max|out - ref| <= 2e-2 * max|ref| of the oracle evaluated on the oracle's own
quantised weights (the GPU applies each row scale after accumulating, the
oracle before: a reordering within fp32 rounding)."""
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


def gpu_quantize(bits):
    q, s = moe.quantize_fp8_rows(dev(bits))
    torch.cuda.synchronize()
    return q, s


def check_quant(bits, what):
    q, s = gpu_quantize(bits)
    rq, rs = oracle.quantize_e4m3_rows(bits)
    gq, gs = q.cpu().numpy(), s.cpu().numpy()
    bad = np.argwhere(gq != rq)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first at {bad[0].tolist()}: gpu {gq[tuple(bad[0])]:#x} oracle {rq[tuple(bad[0])]:#x}"
    assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32)), f"{what}: scales differ"
    return q, s, rq, rs


def crafted_rows():
    """Every code value, every midpoint between neighbouring codes and one bf16
    ulp either side of it, both signs, with 448 in the row so its scale is 1;
    plus a zero row and a row too small for a normal scale."""
    v = oracle.e4m3_values()[:127]
    mids = (v[:-1] + v[1:]) / 2
    xs = list(v) + list(mids)
    for m in mids[1:]:
        u = np.float32(m).view(np.uint32)
        xs += [np.uint32(u + 0x10000).view(np.float32), np.uint32(u - 0x10000).view(np.float32)]
    xs = np.array(xs + [448.0], dtype=np.float32)
    xs = np.concatenate([xs, -xs])
    xs = xs[np.abs(xs) <= 448.0]
    n = (len(xs) + 15) // 16 * 16
    rows = np.zeros((3, n), dtype=np.float32)
    rows[0, : len(xs)] = xs
    rows[0, -1] = 448.0
    rows[2, :] = 2.0 ** -120
    u = rows.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


def test_quantize_kernel_bit_exact_on_crafted_rows():
    _say("case crafted rows")
    check_quant(crafted_rows(), "crafted")


@pytest.mark.parametrize("rows,cols,std", [(7, 16, 1.0), (300, 48, 0.02), (64, 4096, 0.02), (33, 6400, 3.0)])
def test_quantize_kernel_bit_exact_on_random_rows(rows, cols, std):
    _say(f"case random rows {rows}x{cols} std {std}")
    rng = np.random.default_rng(rows * 7 + cols)
    x = (rng.standard_normal((rows, cols)) * std).astype(np.float32)
    x[rng.integers(0, rows, 5), rng.integers(0, cols, 5)] *= 40.0  # outliers set some rows' scales
    check_quant(W.f32_to_bf16_bits(x), f"{rows}x{cols}")


def run_fp8(inp, gq, gs, dq, ds, flags=0, routing=True):
    wl = inp.wl
    sgu = sdn = None
    if inp.shared_gate_up:
        g, d = inp.shared_concat()
        sgu, sdn = dev(g), dev(d)
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).cuda()
    res = moe.moe_forward(dev(inp.hidden), dev(inp.router_w), gq, dq, wl.k, routed_scale=wl.routed_scale,
                          router_bias=bias, shared_gate_up=sgu, shared_down=sdn, flags=flags,
                          gate_up_scale=gs, down_scale=ds, return_routing=routing)
    torch.cuda.synchronize()
    if not routing:
        return res.float().cpu().numpy(), None
    out, r = res
    return out.float().cpu().numpy(), {k: v.cpu().numpy() for k, v in r.items()}


def check_against_oracle(inp, tokens, what, flags=0):
    gq, gs, rgq, rgs = check_quant(inp.gate_up, f"{what} gate_up")
    dq, ds, rdq, rds = check_quant(inp.down, f"{what} down")
    out, got = run_fp8(inp, gq, gs, dq, ds, flags)
    # the launch without routing outputs (direct routing at few assignments)
    # computes the same thing bit for bit
    out_plain, _ = run_fp8(inp, gq, gs, dq, ds, flags, routing=False)
    assert np.array_equal(out_plain.view(np.uint32), out.view(np.uint32)), f"{what}: direct routing differs"
    wl = inp.wl
    logits = oracle.router_logits(inp.hidden, inp.router_w, inp.bias)
    ids, w = oracle.select_topk(logits, wl.k, wl.routed_scale)
    counts, offsets, perm, inv = oracle.route(ids, wl.E)
    for key, ref in (("ids", ids), ("counts", counts), ("offsets", offsets), ("perm", perm), ("inv", inv)):
        assert np.array_equal(got[key], ref), f"{what}: {key} differs"
    assert np.allclose(got["weights"], w, rtol=2e-6, atol=1e-7)
    shared = [inp.shared_concat()] if inp.shared_gate_up else []
    ref = oracle.moe_tokens_e4m3(inp.hidden, rgq, rgs, rdq, rds, ids, w, tokens=tokens, shared=shared)
    got_t = out[tokens]
    err, scale = np.max(np.abs(got_t - ref)), np.max(np.abs(ref))
    _say(f"  {what}: max|err|/max|ref| = {err / scale:.3e}")
    assert np.all(np.isfinite(got_t)) and err <= OUT_TOL * scale


SMALL = [
    ("tiny", dict(T=40, H=64, I=48, E=5, k=2)),
    ("multi_pass", dict(T=100, H=256, I=128, E=8, k=2)),          # > 16 rows per expert: several passes
    ("ragged_k", dict(T=50, H=272, I=80, E=4, k=2)),               # K not a multiple of the 256-wide step
    ("fine", dict(T=96, H=192, I=64, E=32, k=6, routed_scale=2.5)),
    ("shared_bias", dict(T=70, H=128, I=64, E=16, k=2, n_shared=2, shared_I=32,
                         bias=((0, 6.0), (13, -30.0), (14, -30.0), (15, -30.0)))),
    ("one_token", dict(T=1, H=4096, I=256, E=16, k=2)),
]


@pytest.mark.parametrize("name,kw", SMALL, ids=[c[0] for c in SMALL])
def test_fp8_layer_small(name, kw):
    _say(f"case fp8 {name} {kw}")
    inp = W.custom_inputs(**kw)
    check_against_oracle(inp, np.arange(inp.wl.T, dtype=np.int32), name)


def test_fp8_decode_full_size():
    _say("case fp8 phimoe_decode")
    inp = W.make_inputs(W.BY_NAME["phimoe_decode"])
    check_against_oracle(inp, np.arange(inp.wl.T, dtype=np.int32), "phimoe_decode fp8")


def test_fp8_layer_run_to_run_identical():
    _say("case fp8 run to run")
    inp = W.custom_inputs(T=100, H=256, I=128, E=8, k=2)
    gq, gs = gpu_quantize(inp.gate_up)
    dq, ds = gpu_quantize(inp.down)
    a, _ = run_fp8(inp, gq, gs, dq, ds)
    b, _ = run_fp8(inp, gq, gs, dq, ds)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_fp8_with_sigmoid_groups_shared_expert_and_direct_routing():
    _say("case fp8 + sigmoid groups + shared expert")
    inp = W.custom_inputs(T=24, H=256, I=128, E=32, k=4, routed_scale=2.5, n_shared=1, shared_I=64)
    wl = inp.wl
    gq, gs, rgq, rgs = check_quant(inp.gate_up, "gate_up")
    dq, ds, rdq, rds = check_quant(inp.down, "down")
    g, d = inp.shared_concat()
    bias = (np.random.default_rng(11).standard_normal(wl.E) * 0.02).astype(np.float32)
    kw = dict(routed_scale=wl.routed_scale, shared_gate_up=dev(g), shared_down=dev(d), gate_up_scale=gs,
              down_scale=ds, score_func="sigmoid", selection_bias=torch.from_numpy(bias).cuda(), n_group=8,
              topk_group=3)
    out_r, r = moe.moe_forward(dev(inp.hidden), dev(inp.router_w), gq, dq, wl.k, return_routing=True, **kw)
    out_d = moe.moe_forward(dev(inp.hidden), dev(inp.router_w), gq, dq, wl.k, **kw)
    torch.cuda.synchronize()
    logits = oracle.router_logits(inp.hidden, inp.router_w, inp.bias)
    ids, w = oracle.select_scored(logits, wl.k, wl.routed_scale, "sigmoid", bias, 8, 3)
    assert np.array_equal(r["ids"].cpu().numpy(), ids)
    a, b = out_r.float().cpu().numpy(), out_d.float().cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "direct routing differs"
    ref = oracle.moe_tokens_e4m3(inp.hidden, rgq, rgs, rdq, rds, ids, w, tokens=np.arange(wl.T, dtype=np.int32),
                                 shared=[(g, d)])
    err, scale = np.max(np.abs(b - ref)), np.max(np.abs(ref))
    _say(f"  max|err|/max|ref| = {err / scale:.3e}")
    assert np.all(np.isfinite(b)) and err <= OUT_TOL * scale
