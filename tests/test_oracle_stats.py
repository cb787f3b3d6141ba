"""Pins of the oracle's router statistics (the Switch Transformer
load-balancing loss inputs): closed forms at the loss's extremes, an
independent numpy evaluation, and the mask semantics."""
import numpy as np

import oracle
import workloads as W


def numpy_stats(logits, ids, mask=None):
    l = logits.astype(np.float64)
    if mask is not None:
        keep = mask != 0
        l, ids = l[keep], ids[keep]
    n, E = l.shape
    if n == 0:
        return np.zeros(E), np.zeros(E), 0.0
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    P = p.mean(axis=0)
    f = np.bincount(ids.ravel(), minlength=E) / n
    return P, f, E * float(np.dot(f, P))


def test_uniform_logits_closed_form():
    T, E, k = 24, 8, 3
    logits = np.zeros((T, E), dtype=np.float32)
    ids, _ = oracle.select_topk(logits, k)
    r = oracle.router_stats(logits, ids)
    assert np.allclose(r["prob_mean"], 1.0 / E, rtol=0, atol=1e-15)
    assert np.array_equal(r["load"], [1.0] * k + [0.0] * (E - k))  # ties pick experts 0..k-1
    assert abs(r["aux"] - k) < 1e-12


def test_confident_routing_extremes():
    E, T = 8, 64
    # every token sure of expert 0: the most unbalanced case, aux -> E
    logits = np.zeros((T, E), dtype=np.float32)
    logits[:, 0] = 50.0
    ids, _ = oracle.select_topk(logits, 1)
    assert abs(oracle.router_stats(logits, ids)["aux"] - E) < 1e-12 * E
    # tokens spread evenly and surely over the experts: the balanced optimum, aux -> 1
    logits = np.zeros((T, E), dtype=np.float32)
    logits[np.arange(T), np.arange(T) % E] = 50.0
    ids, _ = oracle.select_topk(logits, 1)
    r = oracle.router_stats(logits, ids)
    assert np.allclose(r["load"], 1.0 / E) and abs(r["aux"] - 1.0) < 1e-12


def test_matches_numpy_on_random_logits_with_mask():
    rng = np.random.default_rng(5)
    for T, E, k in [(50, 16, 2), (33, 64, 6), (7, 5, 5)]:
        logits = (rng.standard_normal((T, E)) * 1.3).astype(np.float32)
        ids, _ = oracle.select_topk(logits, k)
        mask = (rng.random(T) < 0.7).astype(np.int32)
        for m in (None, mask):
            r = oracle.router_stats(logits, ids, m)
            P, f, aux = numpy_stats(logits, ids, m)
            assert np.allclose(r["prob_mean"], P, rtol=1e-13, atol=1e-16)
            assert np.array_equal(r["load"], f)
            assert abs(r["aux"] - aux) <= 1e-13 * max(1.0, aux)
            n = T if m is None else int(m.sum())
            assert abs(r["prob_mean"].sum() - 1.0) < 1e-12 and abs(r["load"].sum() - k) < 1e-12 if n else True


def test_mask_equals_subset_and_empty_mask_gives_zeros():
    inp = W.custom_inputs(T=40, H=64, I=32, E=8, k=2)
    logits = oracle.router_logits(inp.hidden, inp.router_w)
    ids, _ = oracle.select_topk(logits, 2)
    mask = np.zeros(40, dtype=np.int32)
    mask[::3] = 1
    a = oracle.router_stats(logits, ids, mask)
    b = oracle.router_stats(logits[mask == 1], ids[mask == 1])
    assert np.array_equal(a["prob_mean"], b["prob_mean"]) and np.array_equal(a["load"], b["load"])
    z = oracle.router_stats(logits, ids, np.zeros(40, dtype=np.int32))
    assert not z["prob_mean"].any() and not z["load"].any() and z["aux"] == 0.0
