"""Pins for ``oracle.accept`` (greedy root walk).

* hand-derived walks (``golden/accept_hand_examples.json``);
* the oracle-drafter case ("The Oracle Drafter ...", section "The Oracle
  Drafter: A Deliberate 'Cheat' for Validation"): when the target's argmax at
  every chain node is the next chain token, the whole chain is accepted and
  the bonus is the prediction at the leaf;
* sentinel drafts (same page, section "Reasoning About Cache Positions and
  Token Indices"): a prediction no draft carries ends acceptance at the root;
* brute force over all root paths agrees with the walk on random trees.
"""
import json
from pathlib import Path

import numpy as np
import pytest

from oracle import accept, tree
from workloads import draw_drafter_topk, draw_target_predict

GOLD = Path(__file__).parent / "golden"


def test_hand_examples():
    g = json.loads((GOLD / "accept_hand_examples.json").read_text())
    for ex in g["examples"]:
        res = accept.accept(np.array(g["tokens"]), np.array(g["parents"]), np.array(ex["pred"]), ex["depth_max"])
        assert res.path == ex["path"], ex["name"]
        assert res.accept_len == ex["accept_len"], ex["name"]
        assert res.commit_tokens == ex["commit"], ex["name"]
        assert res.bonus == ex["bonus"], ex["name"]


def _oracle_drafter_tree(D=7, extra=10):
    golden = list(range(101, 101 + D))
    lp = np.tile(np.float32([-0.01, -6.0, -6.5, -7.0]), (D, 1))
    ids = np.array([[g, 200 + d, 300 + d, 400 + d] for d, g in enumerate(golden)], np.int32)
    return golden, tree.build_tree(lp, ids, 100, D + extra)


def test_oracle_drafter_accepts_whole_chain():
    D = 7
    golden, t = _oracle_drafter_tree(D)
    pred = np.full(len(t.tokens), 999)
    for d in range(D):          # chain node d predicts the next golden token
        pred[d] = golden[d]
    pred[D] = 555               # bonus at the leaf
    res = accept.accept(t.tokens, t.parents, pred, D)
    assert res.accept_len == D + 1
    assert res.path == list(range(D + 1))
    assert res.commit_tokens == golden + [555]


def test_sentinel_stops_at_root():
    golden, t = _oracle_drafter_tree()
    pred = np.full(len(t.tokens), -1)
    res = accept.accept(t.tokens, t.parents, pred, 7)
    assert res.accept_len == 1 and res.bonus == -1 and res.commit_tokens == [-1]


def test_budget_zero_is_autoregressive():
    res = accept.accept(np.array([5]), np.array([-1]), np.array([77]), 7)
    assert res.path == [0] and res.accept_len == 1 and res.commit_tokens == [77]


@pytest.mark.parametrize("seed,K,B", [(1, 4, 8), (2, 8, 32), (3, 16, 64), (4, 2, 30), (5, 8, 16)])
def test_walk_equals_bruteforce(seed, K, B):
    rng = np.random.default_rng(seed)
    for trial in range(20):
        lp, ids = draw_drafter_topk(rng, 7, K, 16)   # tiny vocab: many matches
        t = tree.build_tree(lp, ids, int(rng.integers(0, 16)), B)
        pred = draw_target_predict(seed * 100 + trial, t.tokens, t.parents,
                                   np.array([0, len(t.tokens)]), 16, p_child=0.85)
        a = accept.accept(t.tokens, t.parents, pred, 7)
        b = accept.accept_bruteforce(t.tokens, t.parents, pred, 7)
        assert a == b


def test_batch_layout():
    g = json.loads((GOLD / "accept_hand_examples.json").read_text())
    tok = np.array(g["tokens"] * 2)
    par = np.array(g["parents"] * 2)
    pred = np.array(g["examples"][0]["pred"] + g["examples"][1]["pred"])
    nodes, alen, commit, bonus = accept.batch(tok, par, np.array([0, 6, 12]), pred, 3)
    assert nodes.tolist() == [[0, 1, 4, 5], [0, -1, -1, -1]]
    assert alen.tolist() == [4, 1]
    assert commit.tolist() == [[10, 21, 30, 99], [11, -1, -1, -1]]
    assert bonus.tolist() == [99, 11]
