"""Pins of the oracle's router scoring variants (sigmoid scores, a bias that
steers selection only, group-limited selection: the "noaux_tc" top-k method
the Instella page names on its DeepSeek-V3 base).

The reproducible fp32 exp is pinned to the mathematics (its error against an
fp64 exp stays within one fp32 ulp, and exact points); the selection rules are
pinned by special cases that reduce to plain top-k or to numpy's sort, by
hand-worked examples whose answers follow from the rule alone, and by
invariants on random inputs."""
import math

import numpy as np
import pytest

import oracle

EPS32 = float(np.finfo(np.float32).eps)


def test_exp_within_one_ulp_of_fp64_exp():
    x = np.linspace(-80.0, 80.0, 400001).astype(np.float32)
    y = oracle.exp_f32(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    assert np.max(np.abs(y - ref) / ref) <= EPS32


def test_exp_exact_points():
    x = np.array([0.0, 1.0, -1.0, 10.0], dtype=np.float32)
    y = oracle.exp_f32(x)
    assert y[0] == 1.0                       # n = 0, r = 0: the polynomial's constant term
    assert y[1] == np.float32(math.e)        # e rounds to the nearest fp32 here
    # exp(a) exp(-a) = 1 to within two roundings
    assert abs(float(y[1]) * float(y[2]) - 1.0) < 3 * EPS32
    assert abs(float(y[3]) / math.exp(10.0) - 1.0) < EPS32


def test_sigmoid_scores_closed_forms():
    x = np.linspace(-20, 20, 4001).astype(np.float32)
    s = oracle.sigmoid_scores(x).astype(np.float64)
    ref = 1.0 / (1.0 + np.exp(-x.astype(np.float64)))
    assert np.max(np.abs(s - ref) / ref) <= 2 * EPS32
    assert oracle.sigmoid_scores(np.zeros(1, np.float32))[0] == 0.5
    # symmetry s(x) + s(-x) = 1
    assert np.max(np.abs(s + oracle.sigmoid_scores(-x).astype(np.float64) - 1.0)) <= 2 * EPS32
    # the clamp to [-80, 80]
    big = oracle.sigmoid_scores(np.array([80, 1e4, -80, -1e4], np.float32))
    assert big[0] == big[1] == 1.0 and big[2] == big[3] > 0.0


def test_softmax_without_bias_or_groups_is_plain_topk():
    rng = np.random.default_rng(1)
    logits = (rng.standard_normal((40, 16)) * 2).astype(np.float32)
    logits[3, :4] = logits[3, 4]  # ties go to the lower index in both
    for k in (1, 2, 6):
        a_ids, a_w = oracle.select_topk(logits, k, 1.5)
        b_ids, b_w = oracle.select_scored(logits, k, 1.5)
        assert np.array_equal(a_ids, b_ids) and np.array_equal(a_w, b_w)


def distinct_logits(rng, T, E, step=0.01):
    """Rows of distinct logits at least `step` apart in [-E*step/2, E*step/2]."""
    grid = (np.arange(E) - E / 2) * step
    return np.stack([rng.permutation(grid) for _ in range(T)]).astype(np.float32)


def test_sigmoid_selection_and_weights_closed_form():
    rng = np.random.default_rng(2)
    T, E, k, scale = 30, 64, 6, 2.5
    logits = distinct_logits(rng, T, E)
    ids, w = oracle.select_scored(logits, k, scale, "sigmoid")
    # sigmoid is increasing: the k largest logits, largest first
    assert np.array_equal(ids, np.argsort(-logits, axis=1, kind="stable")[:, :k])
    s = 1.0 / (1.0 + np.exp(-np.take_along_axis(logits, ids, 1).astype(np.float64)))
    assert np.allclose(w, scale * s / s.sum(1, keepdims=True), rtol=1e-6, atol=0)
    assert np.allclose(w.sum(1), scale, rtol=1e-6)


@pytest.mark.parametrize("score_func", ["softmax", "sigmoid"])
def test_selection_bias_steers_selection_not_weights(score_func):
    rng = np.random.default_rng(3)
    T, E, k = 20, 32, 4
    logits = distinct_logits(rng, T, E, 0.05)
    chosen = rng.choice(E, size=k, replace=False)
    bias = np.zeros(E, np.float32)
    bias[chosen] = 100.0 + 10.0 * np.arange(k, dtype=np.float32)  # steps above the logit range fix the order
    ids, w = oracle.select_scored(logits, k, 1.0, score_func, bias)
    order = chosen[np.argsort(-bias[chosen], kind="stable")]
    assert np.array_equal(ids, np.tile(order, (T, 1)))
    l = np.take_along_axis(logits, ids, 1).astype(np.float64)
    if score_func == "sigmoid":
        num = 1.0 / (1.0 + np.exp(-l))
    else:
        num = np.exp(l - l.max(1, keepdims=True))
    assert np.allclose(w, num / num.sum(1, keepdims=True), rtol=1e-6, atol=0)


@pytest.mark.parametrize("score_func", ["softmax", "sigmoid"])
def test_groups_that_keep_everything_change_nothing(score_func):
    rng = np.random.default_rng(4)
    T, E, k = 25, 16, 4
    logits = (rng.standard_normal((T, E)) * 1.5).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32)
    plain = oracle.select_scored(logits, k, 1.0, score_func, bias)
    for n_group, topk_group in [(4, 4), (E, E), (2, 2)]:
        g = oracle.select_scored(logits, k, 1.0, score_func, bias, n_group, topk_group)
        assert np.array_equal(plain[0], g[0]) and np.array_equal(plain[1], g[1])
    # groups of one expert each, k of them kept: the group score is the key
    g = oracle.select_scored(logits, k, 1.0, score_func, bias, E, k)
    assert np.array_equal(plain[0], g[0]) and np.array_equal(plain[1], g[1])


def test_group_limited_hand_worked_examples():
    # softmax scoring, so the keys are the logits; 4 groups of 2 experts
    l = np.array([[5.0, -5.0, 3.0, 2.5, 2.0, 2.0, 1.0, 0.5]], np.float32)
    # group scores (sum of the best two keys): 0, 5.5, 4.0, 1.5 -> groups 1, 2 kept;
    # expert 0 has the best key but its group is dropped
    ids, w = oracle.select_scored(l, 2, 1.0, "softmax", None, 4, 2)
    assert ids.tolist() == [[2, 3]]
    assert np.allclose(w, [[1 / (1 + math.exp(-0.5)), 1 / (1 + math.exp(0.5))]], rtol=1e-7)
    # third pick: experts 4 and 5 tie at 2.0, the lower index wins
    ids, _ = oracle.select_scored(l, 3, 1.0, "softmax", None, 4, 2)
    assert ids.tolist() == [[2, 3, 4]]
    # without groups the best keys win
    ids, _ = oracle.select_scored(l, 2, 1.0, "softmax")
    assert ids.tolist() == [[0, 2]]
    # one group kept: group 1 alone
    ids, _ = oracle.select_scored(l, 2, 1.0, "softmax", None, 4, 1)
    assert ids.tolist() == [[2, 3]]
    # tied group scores keep the lower group: groups 0 and 1 both sum to 3
    l2 = np.array([[2.0, 1.0, 1.5, 1.5, -1.0, -1.0]], np.float32)
    ids, _ = oracle.select_scored(l2, 1, 1.0, "softmax", None, 3, 1)
    assert ids.tolist() == [[0]]
    # a bias moves a group in: expert 7's +10 makes group 3 (score 11.5) the best
    bias = np.zeros(8, np.float32)
    bias[7] = 10.0
    ids, w = oracle.select_scored(l, 2, 1.0, "softmax", bias, 4, 1)
    assert ids.tolist() == [[7, 6]]
    # weights use the unbiased logits 0.5 and 1.0
    assert np.allclose(w, [[1 / (1 + math.exp(0.5)), 1 / (1 + math.exp(-0.5))]], rtol=1e-7)


def test_group_limited_invariants_on_random_inputs():
    rng = np.random.default_rng(6)
    T, E, k, n_group, topk_group = 200, 64, 6, 8, 3
    logits = (rng.standard_normal((T, E)) * 1.2).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.05).astype(np.float32)
    ids, w = oracle.select_scored(logits, k, 2.5, "sigmoid", bias, n_group, topk_group)
    keys = (oracle.sigmoid_scores(logits) + bias).astype(np.float64)
    gsz = E // n_group
    gs = np.sort(keys.reshape(T, n_group, gsz), axis=2)[:, :, -2:].sum(2)
    for t in range(T):
        kept = set(np.argsort(-gs[t], kind="stable")[:topk_group].tolist())
        assert len(set(ids[t].tolist())) == k
        assert all(e // gsz in kept for e in ids[t])
        allowed = [e for e in range(E) if e // gsz in kept]
        best = sorted(allowed, key=lambda e: (-keys[t, e], e))[:k]
        assert ids[t].tolist() == best
    assert np.all(w > 0) and np.allclose(w.sum(1), 2.5, rtol=1e-6)


def test_rejects_bad_group_arguments():
    l = np.zeros((2, 8), np.float32)
    for n_group, topk_group, k in [(3, 1, 1), (4, 0, 1), (4, 5, 1), (4, 1, 3)]:
        with pytest.raises(ValueError):
            oracle.select_scored(l, k, 1.0, "sigmoid", None, n_group, topk_group)


# ---------------------------------------------------------------- sparsemixer at inference


def test_sparsemixer_page_default_threshold():
    import json
    import os
    facts = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))
    assert facts["phimoe_config"]["router_jitter_noise"] == 0.01


def test_sparsemixer_ids_are_greedy_topk():
    rng = np.random.default_rng(11)
    logits = (rng.standard_normal((60, 16)) * 1.28).astype(np.float32)
    logits[5, :3] = logits[5, 7]  # ties: lower index first
    for k in (1, 2, 4):
        ids, _ = oracle.select_sparsemixer(logits, k)
        assert np.array_equal(ids, oracle.select_topk(logits, k)[0])


def test_sparsemixer_separated_logits_weigh_one():
    # gaps far above 2 * eps relative: every round's softmax holds its winner alone
    l = np.array([[4.0, 2.0, 1.0, -3.0], [-1.0, -2.0, -4.0, -8.0]], np.float32)
    for eps in (0.0, 0.01, 0.1):
        ids, w = oracle.select_sparsemixer(l, 2, 1.5, eps)
        assert np.array_equal(w, np.full((2, 2), 1.5, np.float32))


def test_sparsemixer_hand_worked_rounds():
    l = np.array([[1.0, 0.99, 0.5],      # gap 0.01 <= 0.02: expert 1 joins round 1
                  [-1.0, -1.01, -3.0],   # gap 0.01/1.01 (|l| is the larger divisor)
                  [0.0, 0.0, -1.0],      # 0/0 gaps keep the tied zero; then it wins round 2 alone
                  [2.0, 2.0, 2.0]],      # three-way tie: 1/3, then 1/2, then 1
                 np.float32)
    ids, w = oracle.select_sparsemixer(l, 3, 1.0, 0.01)
    assert ids.tolist() == [[0, 1, 2]] * 4
    a = 1 / (1 + math.exp(-0.01))
    expect = [[a, 1.0, 1.0],
              [1 / (1 + math.exp(-0.010000000000000009)), 1.0, 1.0],
              [0.5, 1.0, 1.0],
              [1 / 3, 0.5, 1.0]]
    assert np.allclose(w, expect, rtol=1e-6, atol=0)
    # a threshold just under the gap drops expert 1 from round 1
    ids, w = oracle.select_sparsemixer(l[:1], 2, 1.0, 0.004)
    assert np.allclose(w, [[1.0, 1.0]])


def test_sparsemixer_unbounded_threshold_is_full_softmax():
    # every unchosen expert passes: round j is the softmax over the experts
    # left after j removals, evaluated at its winner
    rng = np.random.default_rng(12)
    logits = (rng.standard_normal((30, 12)) * 1.5).astype(np.float32)
    ids, w = oracle.select_sparsemixer(logits, 3, 2.0, 1e30)
    l = logits.astype(np.float64)
    for t in range(30):
        left = list(range(12))
        for j in range(3):
            e = ids[t, j]
            p = np.exp(l[t, e] - np.max(l[t, left])) / np.exp(l[t, left] - np.max(l[t, left])).sum()
            assert abs(w[t, j] - 2.0 * p) <= 1e-6 * 2.0 * p
            left.remove(e)
