"""Pins of the oracle's expert FFN and combine by the two ways the layer
shards over GPUs (the expert-parallel and tensor-parallel plans of the
Transformers MoE page and the GraniteMoeSWA walkthrough):

* expert parallel: with the routing fixed, the layer output is the sum over
  disjoint groups of experts of the outputs that count only the group's
  assignments (each assignment's term w * expert(x) is linear in w);
* tensor parallel: splitting every expert's intermediate columns into G
  shards (matching gate and up rows, the same down columns) and summing the
  shard outputs gives the layer output, since silu(gate) * up is per column
  and the down product sums over columns.

Both are identities of the mathematics, exact up to fp32 reassociation, so
a wrong gate/up pairing, a transposed down matrix or weights applied in the
wrong place fails them. CPU only."""
import numpy as np
import pytest

import oracle
import workloads as W


def _routing(inp, k):
    logits = oracle.router_logits(inp.hidden, inp.router_w)
    return oracle.select_topk(logits, k)


@pytest.mark.parametrize("T,H,I,E,k", [(24, 64, 48, 6, 2), (17, 72, 40, 8, 3)])
def test_expert_groups_sum_to_the_layer(T, H, I, E, k):
    inp = W.custom_inputs(T, H, I, E, k, seed=41)
    ids, w = _routing(inp, k)
    full = oracle.moe_tokens(inp.hidden, inp.gate_up, inp.down, ids, w).astype(np.float64)
    groups = np.array_split(np.arange(E), 3)
    total = np.zeros_like(full)
    for g in groups:
        wg = np.where(np.isin(ids, g), w, np.float32(0.0)).astype(np.float32)
        total += oracle.moe_tokens(inp.hidden, inp.gate_up, inp.down, ids, wg)
    scale = np.max(np.abs(full))
    assert np.max(np.abs(total - full)) <= 1e-5 * scale
    # and the identity is not vacuous: one group alone is far from the layer
    wg = np.where(np.isin(ids, groups[0]), w, np.float32(0.0)).astype(np.float32)
    part = oracle.moe_tokens(inp.hidden, inp.gate_up, inp.down, ids, wg)
    assert np.max(np.abs(part - full)) > 0.1 * scale


def tp_shard(gate_up, down, I, G, g):
    """Shard g of G: gate rows and the matching up rows of columns
    [g I / G, (g + 1) I / G), and the same columns of down."""
    Is = I // G
    lo, hi = g * Is, (g + 1) * Is
    gu = np.ascontiguousarray(np.concatenate([gate_up[:, lo:hi], gate_up[:, I + lo:I + hi]], axis=1))
    dn = np.ascontiguousarray(down[:, :, lo:hi])
    return gu, dn


@pytest.mark.parametrize("T,H,I,E,k,G", [(24, 64, 48, 6, 2, 3), (13, 40, 64, 4, 2, 4)])
def test_column_shards_sum_to_the_layer(T, H, I, E, k, G):
    inp = W.custom_inputs(T, H, I, E, k, seed=43)
    ids, w = _routing(inp, k)
    full = oracle.moe_tokens(inp.hidden, inp.gate_up, inp.down, ids, w).astype(np.float64)
    total = np.zeros_like(full)
    for g in range(G):
        gu, dn = tp_shard(inp.gate_up, inp.down, I, G, g)
        total += oracle.moe_tokens(inp.hidden, gu, dn, ids, w)
    scale = np.max(np.abs(full))
    assert np.max(np.abs(total - full)) <= 1e-5 * scale
    # pairing gate rows of one shard with up rows of another breaks it
    gu0, dn0 = tp_shard(inp.gate_up, inp.down, I, G, 0)
    gu1, _ = tp_shard(inp.gate_up, inp.down, I, G, 1)
    Is = I // G
    bad = np.ascontiguousarray(np.concatenate([gu0[:, :Is], gu1[:, Is:]], axis=1))
    wrong = oracle.moe_tokens(inp.hidden, bad, dn0, ids, w)
    right = oracle.moe_tokens(inp.hidden, gu0, dn0, ids, w)
    assert np.max(np.abs(wrong - right)) > 0.1 * np.max(np.abs(right))
