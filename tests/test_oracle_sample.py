"""Pins for ``oracle.sample`` (stochastic acceptance along the tree).

* hand-derived walks (``golden/sample_hand_example.json``);
* the greedy limit: with one-hot target rows (temperature 0) the walk is the
  greedy root walk of ``oracle.accept`` with the one-hot tokens as argmax;
* the defining property of speculative sampling, by Monte Carlo over the
  uniforms: the first emitted token is distributed as the root's target
  row, and after accepting child c the next token as c's row;
* the fixed-order sums against fp64: the row mass, and the inverse-CDF token
  for thresholds away from the fp32 rounding of the boundaries.
"""
import json
from pathlib import Path

import numpy as np

from oracle import accept, sample, tree
from workloads import draw_drafter_topk

GOLD = Path(__file__).parent / "golden"


def test_hand_examples():
    g = json.loads((GOLD / "sample_hand_example.json").read_text())
    probs = np.array(g["probs"], np.float32)
    for ex in g["examples"]:
        path, n, commit, bonus = sample.sample_request(
            g["tokens"], g["parents"], probs, np.array(ex["coins"], np.float32),
            np.float32(ex["bonus_u"]), g["depth_max"])
        assert path == ex["path"], ex["name"]
        assert n == len(ex["path"]), ex["name"]
        assert bonus == ex["bonus"], ex["name"]
        assert commit == ex["commit"], ex["name"]


def test_one_hot_rows_give_the_greedy_walk():
    rng = np.random.default_rng(21)
    for trial in range(30):
        V, D = 12, 5
        lp, ids = draw_drafter_topk(rng, D, 3, V)
        t = tree.build_tree(lp, ids, 0, int(rng.integers(1, 20)))
        q = len(t.tokens)
        pred = rng.integers(0, V, size=q)
        for v in range(q):   # often follow a child
            kids = [c for c in range(q) if t.parents[c] == v]
            if kids and rng.random() < 0.7:
                pred[v] = t.tokens[kids[int(rng.integers(0, len(kids)))]]
        probs = np.zeros((q, V), np.float32)
        probs[np.arange(q), pred] = 1.0
        coins = rng.random(q).astype(np.float32)
        path, n, commit, bonus = sample.sample_request(t.tokens, t.parents, probs, coins,
                                                       np.float32(rng.random()), D)
        ref = accept.accept(t.tokens, t.parents, pred, D)
        assert path == ref.path and bonus == ref.bonus and commit == ref.commit_tokens


def _star_tree():
    # root 0 with children tokens 3, 1, 4 (nodes 1..3); node 1 has children tokens 0, 5
    tokens = [7, 3, 1, 4, 0, 5]
    parents = [-1, 0, 0, 0, 1, 1]
    return tokens, parents


def test_first_token_follows_the_target_row():
    rng = np.random.default_rng(22)
    tokens, parents = _star_tree()
    V, q = 8, 6
    probs = rng.dirichlet(np.ones(V), size=q).astype(np.float32)
    N = 30000
    counts = np.zeros(V)
    second = np.zeros(V)
    n_first3 = 0
    for i in range(N):
        coins = rng.random(q).astype(np.float32)
        path, n, commit, bonus = sample.sample_request(tokens, parents, probs, coins,
                                                       np.float32(rng.random()), 4)
        counts[commit[0]] += 1
        if len(path) > 1 and path[1] == 1:   # first token 3 (child node 1)
            n_first3 += 1
            second[commit[1]] += 1
    p0 = probs[0].astype(np.float64) / probs[0].sum()
    assert np.abs(counts / N - p0).max() < 4 * np.sqrt(0.25 / N)
    p1 = probs[1].astype(np.float64) / probs[1].sum()
    assert np.abs(second / n_first3 - p1).max() < 4 * np.sqrt(0.25 / n_first3)


def test_fixed_order_sums_against_fp64():
    rng = np.random.default_rng(23)
    for V in (5, 256, 700, 4096):
        row = rng.dirichlet(np.ones(V) * 0.5).astype(np.float32)
        assert abs(float(sample._mass(row)) - float(row.astype(np.float64).sum())) < 1e-5
        cdf = np.cumsum(row.astype(np.float64))
        for thr in rng.random(40) * float(cdf[-1]):
            j = int(np.searchsorted(cdf, thr, side="right"))
            if min(abs(cdf[j] - thr), abs(thr - (cdf[j - 1] if j else 0.0))) < 1e-5:
                continue   # too close to a boundary for fp32
            assert sample._inverse_cdf(row, np.float32(thr)) == j
