"""Pins for ``oracle.tree`` (best-first draft-tree growth).

The heapq builder is pinned by things other than itself:

* hand-derived trees (``golden/tree_hand_examples.json``), exact fp32 values;
* brute force: enumerate every rank path, sort by the key, keep the first
  ``budget`` -- an independent formulation that a wrong push (child vs
  sibling, wrong depth row, wrong parent score) or a wrong tie order breaks;
* closed forms: top-1 lists give a chain, budget 0 gives the root only, the
  full budget gives every path, and the oracle-drafter margin puts the golden
  chain first ("The Oracle Drafter ...", section "The Oracle Drafter: A
  Deliberate 'Cheat' for Validation").
"""
import json
from pathlib import Path

import numpy as np
import pytest

from oracle import tree
from workloads import draw_drafter_topk

GOLD = Path(__file__).parent / "golden"


def _lp(seed, D, K, V=64, quant=None):
    rng = np.random.default_rng(seed)
    lp, ids = draw_drafter_topk(rng, D, K, V)
    if quant is not None:   # coarse log-probs -> many exact fp32 ties
        lp = np.minimum(np.float32(0), np.round(lp * quant) / quant).astype(np.float32)
        lp = -np.sort(-lp, axis=1)
    return lp, ids


def _same(a, b):
    assert np.array_equal(a.tokens, b.tokens)
    assert np.array_equal(a.parents, b.parents)
    assert np.array_equal(a.depths, b.depths)
    assert np.array_equal(a.scores.view(np.uint32), b.scores.view(np.uint32))
    assert list(a.rank_paths) == list(b.rank_paths)


def test_hand_examples():
    for ex in json.loads((GOLD / "tree_hand_examples.json").read_text())["examples"]:
        t = tree.build_tree(np.array(ex["lp"], np.float32), np.array(ex["ids"], np.int32),
                            ex["root"], ex["budget"])
        assert t.tokens.tolist() == ex["tokens"], ex["name"]
        assert t.parents.tolist() == ex["parents"], ex["name"]
        assert t.depths.tolist() == ex["depths"], ex["name"]
        assert t.scores.tolist() == ex["scores"], ex["name"]


@pytest.mark.parametrize("seed,D,K,B", [
    (1, 3, 2, 5), (2, 4, 3, 20), (3, 5, 2, 40), (4, 7, 4, 8), (5, 7, 4, 64), (6, 4, 4, 100),
    (7, 3, 5, 155), (8, 7, 2, 254), (9, 2, 8, 30), (10, 5, 3, 111),
])
def test_heap_equals_bruteforce(seed, D, K, B):
    lp, ids = _lp(seed, D, K)
    _same(tree.build_tree(lp, ids, 3, B), tree.build_tree_bruteforce(lp, ids, 3, B))


@pytest.mark.parametrize("seed,quant", [(11, 2), (12, 4), (13, 1), (14, 8)])
def test_heap_equals_bruteforce_with_ties(seed, quant):
    lp, ids = _lp(seed, 5, 3, quant=quant)
    B = tree.reachable(5, 3) - 7
    _same(tree.build_tree(lp, ids, 0, B), tree.build_tree_bruteforce(lp, ids, 0, B))


def test_parent_before_child_and_depth_consistency():
    lp, ids = _lp(21, 7, 8)
    t = tree.build_tree(lp, ids, 5, 64)
    for i in range(1, len(t.tokens)):
        assert 0 <= t.parents[i] < i
        assert t.depths[i] == t.depths[t.parents[i]] + 1
        assert t.tokens[i] == ids[t.depths[i] - 1, t.rank_paths[i][-1]]
        # child score = parent score + lp, in fp32
        assert t.scores[i] == np.float32(t.scores[t.parents[i]] + lp[t.depths[i] - 1, t.rank_paths[i][-1]])


def test_top1_gives_chain():
    lp, ids = _lp(31, 7, 1)
    t = tree.build_tree(lp, ids, 9, 7)
    assert t.parents.tolist() == [-1, 0, 1, 2, 3, 4, 5, 6]
    assert t.depths.tolist() == list(range(8))
    assert t.tokens.tolist() == [9] + ids[:, 0].tolist()


def test_budget_zero_is_root_only():
    lp, ids = _lp(32, 7, 4)
    t = tree.build_tree(lp, ids, 42, 0)
    assert t.tokens.tolist() == [42] and t.parents.tolist() == [-1] and t.depths.tolist() == [0]


def test_full_budget_takes_every_path():
    lp, ids = _lp(33, 3, 3)
    B = tree.reachable(3, 3)
    t = tree.build_tree(lp, ids, 0, B)
    assert sorted(t.rank_paths[1:]) == sorted(
        [(a,) for a in range(3)] + [(a, b) for a in range(3) for b in range(3)]
        + [(a, b, c) for a in range(3) for b in range(3) for c in range(3)])


def test_oracle_drafter_golden_chain_first():
    D, K = 7, 4
    golden = [101, 102, 103, 104, 105, 106, 107]
    lp = np.tile(np.float32([-0.01, -6.0, -6.5, -7.0]), (D, 1))
    ids = np.array([[g, 200 + d, 300 + d, 400 + d] for d, g in enumerate(golden)], np.int32)
    t = tree.build_tree(lp, ids, 100, 12)
    assert t.tokens[:D + 1].tolist() == [100] + golden
    assert t.parents[:D + 1].tolist() == [-1] + list(range(D))


def test_preconditions_rejected():
    lp, ids = _lp(34, 3, 2)
    with pytest.raises(ValueError):
        tree.build_tree(lp, ids, 0, tree.reachable(3, 2) + 1)
    with pytest.raises(ValueError):
        tree.build_tree(lp[:, ::-1].copy(), ids, 0, 3)          # ascending rows
    bad = lp.copy()
    bad[0, 0] = 0.5
    with pytest.raises(ValueError):
        tree.build_tree(bad, ids, 0, 3)                          # positive log-prob


def test_batch_packing():
    lp0, ids0 = _lp(41, 7, 4)
    lp1, ids1 = _lp(42, 7, 4)
    qo = np.array([0, 9, 12], np.int32)
    outs, tok, par, dep, sc = tree.build_batch(np.stack([lp0, lp1]), np.stack([ids0, ids1]),
                                               np.array([1, 2]), qo)
    assert len(tok) == 12 and par[0] == -1 and par[9] == -1
    assert np.array_equal(tok[:9], tree.build_tree(lp0, ids0, 1, 8).tokens)
    assert np.array_equal(tok[9:], tree.build_tree(lp1, ids1, 2, 2).tokens)
