"""Pins of the oracle's FP8 (OCP E4M3, one fp32 scale per weight row) expert
weights: the code table against the format's closed forms, the quantiser
against an independent brute-force nearest-value search, and the FP8 layer
against the fp32 oracle path on the dequantised weights."""
import numpy as np
import pytest

import oracle
import workloads as W

VALS = None


def vals():
    global VALS
    if VALS is None:
        VALS = oracle.e4m3_values()
    return VALS


def f32_to_bf16_bits(x):
    """Exact conversion (the inputs below are chosen bf16-representable)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not representable in bf16"
    return (u >> 16).astype(np.uint16)


def brute_force_code(v):
    """Nearest E4M3 code to fp32 value v by scanning every finite non-negative
    code; ties go to the even code; zero is 0x00; negative values get 0x80."""
    av = abs(float(v))
    best, bestd = 0, None
    for c in range(127):
        d = abs(av - vals()[c])
        if bestd is None or d < bestd or (d == bestd and c % 2 == 0 and best % 2 == 1):
            best, bestd = c, d
    if best == 0:
        return 0
    return best | (0x80 if v < 0 else 0)


def test_code_table_closed_forms():
    v = vals()
    assert v[0x00] == 0.0 and v[0x38] == 1.0 and v[0x40] == 2.0 and v[0x3F] == 1.875
    assert v[0x7E] == 448.0 and v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.all(np.diff(v[:127]) > 0)  # codes 0..126 increase
    assert np.array_equal(v[0x81:0xFF], -v[0x01:0x7F])
    assert np.signbit(v[0x80]) and v[0x80] == 0.0
    # every normal value is (1 + m/8) 2^(e-7): 3 mantissa bits
    for c in range(8, 127):
        e, m = c >> 3, c & 7
        assert v[c] == (1 + m / 8) * 2.0 ** (e - 7)


def crafted_row():
    """448 (so the scale is exactly 1), every finite code value, every midpoint
    between neighbours, values just off the midpoints, saturation and zeros,
    with both signs; all bf16-representable."""
    v = vals()[:127]
    mids = (v[:-1] + v[1:]) / 2
    xs = list(v) + list(mids)
    # neighbours of midpoints: one bf16 ulp either side
    for m in mids:
        if m == 0:
            continue
        u = np.float32(m).view(np.uint32)
        xs += [np.uint32(u + 0x10000).view(np.float32), np.uint32(u - 0x10000).view(np.float32)]
    xs += [448.0, 0.0]
    xs = np.array(xs, dtype=np.float32)
    xs = np.concatenate([xs, -xs[1:]])
    xs = xs[np.abs(xs) <= 448.0]
    n = (len(xs) + 15) // 16 * 16
    row = np.zeros(n, dtype=np.float32)
    row[: len(xs)] = xs
    row[-1] = 448.0
    return row


def test_quantiser_matches_brute_force_on_crafted_values():
    row = crafted_row()
    q, s = oracle.quantize_e4m3_rows(f32_to_bf16_bits(row)[None, :])
    assert s[0] == np.float32(1.0)
    expect = np.array([brute_force_code(x) for x in row], dtype=np.uint8)
    assert np.array_equal(q[0], expect)
    # exact values come back exactly
    back = vals()[q[0]]
    exact = np.isin(np.abs(row), vals()[:127])
    assert np.array_equal(back[exact], row[exact].astype(np.float64))


def test_quantiser_matches_brute_force_on_random_rows():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((6, 64)) * np.array([1e-3, 0.02, 1.0, 30.0, 1e4, 1e-30])[:, None]).astype(np.float32)
    x[2, 5] = 40.0  # an outlier sets that row's scale
    bits = W.f32_to_bf16_bits(x)
    wf = W.bf16_bits_to_f32(bits)
    q, s = oracle.quantize_e4m3_rows(bits)
    for r in range(x.shape[0]):
        a = np.float32(np.max(np.abs(wf[r])))
        assert s[r] == np.float32(a / np.float32(448.0))
        v = wf[r] / s[r]  # fp32 division
        assert np.array_equal(q[r], [brute_force_code(t) for t in v])
        assert np.max(np.abs(vals()[q[r]])) == 448.0  # the row maximum maps to 448


def test_zero_tiny_and_sign_symmetric_rows():
    zero = np.zeros((1, 32), dtype=np.uint16)
    q, s = oracle.quantize_e4m3_rows(zero)
    assert s[0] == 1.0 and not q.any()
    tiny = np.full((1, 32), 2.0 ** -120, dtype=np.float32)  # max below 448 * 2^-126: stored as zeros
    q, s = oracle.quantize_e4m3_rows(W.f32_to_bf16_bits(tiny))
    assert s[0] == 1.0 and not q.any()
    rng = np.random.default_rng(3)
    x = W.f32_to_bf16_bits(rng.standard_normal((3, 48)).astype(np.float32))
    qp, sp = oracle.quantize_e4m3_rows(x)
    qn, sn = oracle.quantize_e4m3_rows(x ^ np.uint16(0x8000))
    assert np.array_equal(sp, sn)
    assert np.array_equal(qn, np.where(qp == 0, 0, qp ^ 0x80))


def dequantise(q, s):
    return (vals()[q] * s[..., None].astype(np.float64)).astype(np.float32)


def test_fp8_layer_equals_fp32_oracle_on_dequantised_weights():
    inp = W.custom_inputs(T=40, H=64, I=48, E=5, k=2, n_shared=1, shared_I=32, routed_scale=1.5)
    gq, gs = oracle.quantize_e4m3_rows(inp.gate_up)
    dq, ds = oracle.quantize_e4m3_rows(inp.down)
    logits = oracle.router_logits(inp.hidden, inp.router_w)
    ids, w = oracle.select_topk(logits, 2, 1.5)
    g, d = inp.shared_concat()
    got = oracle.moe_tokens_e4m3(inp.hidden, gq, gs, dq, ds, ids, w, shared=[(g, d)])
    f = W.bf16_bits_to_f32
    ref = oracle.moe_tokens(f(inp.hidden), dequantise(gq, gs), dequantise(dq, ds), ids, w, shared=[(f(g), f(d))])
    assert np.array_equal(got, ref)  # same fp32 arithmetic, only the weight storage differs


def test_fp8_single_expert_is_a_dense_swiglu_on_dequantised_weights():
    inp = W.custom_inputs(T=6, H=32, I=16, E=1, k=1)
    gq, gs = oracle.quantize_e4m3_rows(inp.gate_up)
    dq, ds = oracle.quantize_e4m3_rows(inp.down)
    ids = np.zeros((6, 1), dtype=np.int32)
    w = np.ones((6, 1), dtype=np.float32)
    got = oracle.moe_tokens_e4m3(inp.hidden, gq, gs, dq, ds, ids, w)
    x = W.bf16_bits_to_f32(inp.hidden).astype(np.float64)
    wg = vals()[gq[0]] * gs[0][:, None].astype(np.float32).astype(np.float64)
    wd = vals()[dq[0]] * ds[0][:, None].astype(np.float32).astype(np.float64)
    hh = x @ wg.T
    g, u = hh[:, :16], hh[:, 16:]
    ref = (g / (1 + np.exp(-g)) * u) @ wd.T
    assert np.allclose(got, ref, rtol=1e-4, atol=1e-5 * np.abs(ref).max())


def test_fp8_quantisation_error_is_within_the_format_bound():
    """|w - dequant(q)| <= half a unit in the last place of E4M3 at that
    magnitude (2^-4 relative for normals) times the scale."""
    rng = np.random.default_rng(11)
    x = W.f32_to_bf16_bits((rng.standard_normal((8, 256)) * 0.02).astype(np.float32))
    wf = W.bf16_bits_to_f32(x).astype(np.float64)
    q, s = oracle.quantize_e4m3_rows(x)
    deq = vals()[q] * s[:, None].astype(np.float64)
    v = np.abs(wf / s[:, None])
    ulp = np.where(v < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(v, 2.0 ** -6))) - 3))
    assert np.all(np.abs(wf - deq) <= 0.5 * ulp * s[:, None] * (1 + 1e-6) + 1e-30)
