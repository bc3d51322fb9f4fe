"""Pins for ``oracle.sample`` (stochastic acceptance along the tree).

* hand-derived walks (``golden/sample_hand_example.json``);
* the greedy limit: with one-hot target rows (temperature 0) the walk is the
  greedy root walk of ``oracle.accept`` with the one-hot tokens as argmax;
* the defining property of speculative sampling, by Monte Carlo over the
  uniforms: the first emitted token is distributed as the root's target
  row, and after accepting child c the next token as c's row;
* the closed form, exactly: on dyadic rows whose acceptance ratios are
  dyadic, counting outcomes over a coin grid that never meets a boundary
  gives the target rows' probabilities as exact fractions;
* rows need not be normalised (power-of-two scaling changes nothing);
* the inverse-CDF bonus draw against exact rational arithmetic;
* the decision margin is 0 exactly on the hand-built boundary case.
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


def test_rows_need_not_be_normalised():
    """Scaling a node's row by a power of two (exact) changes no decision:
    the rule compares coin * R with res[t], both scaled alike."""
    rng = np.random.default_rng(23)
    tokens, parents = _star_tree()
    for trial in range(40):
        probs = rng.dirichlet(np.ones(8) * 0.7, size=6).astype(np.float32)
        coins = rng.random(6).astype(np.float32)
        u = np.float32(rng.random())
        base = sample.walk(tokens, parents, probs, coins, u, 4)
        scaled = probs * np.float32(2.0) ** rng.integers(-20, 20, size=(6, 1)).astype(np.float32)
        w = sample.walk(tokens, parents, scaled, coins, u, 4)
        assert (w.path, w.commit, w.bonus) == (base.path, base.commit, base.bonus)


def test_exact_distribution_on_a_dyadic_grid():
    """Closed form of speculative sampling: the first emitted token follows
    the root's row exactly, and after accepting a child the next token
    follows that child's row.  With dyadic rows whose acceptance ratios are
    dyadic too, the midpoints of a fine coin grid never sit on a boundary, so
    counting the walk's outcomes over the whole grid gives the probabilities
    exactly (no sampling error)."""
    from fractions import Fraction as Fr
    # root (token 7) with children: node 1 (token 0) and node 2 (token 1);
    # node 1 has one child, node 3 (token 2)
    tokens, parents = [7, 0, 1, 2], [-1, 0, 0, 1]
    probs = np.zeros((4, 4), np.float32)
    probs[0] = [0.5, 0.25, 0.125, 0.125]   # accept 0: 1/2; then 1: 1/2; bonus over {2, 3}
    probs[1] = [0.25, 0.25, 0.5, 0.0]      # accept 2: 1/2; else bonus over {0, 1}
    probs[2] = [0.0, 0.0, 1.0, 0.0]
    probs[3] = [0.5, 0.0, 0.0, 0.5]
    N = 8                                  # grid midpoints (i + 1/2) / N
    grid = [(i + 0.5) / N for i in range(N)]
    first = {}
    second_after_0 = {}
    for c1 in grid:
        for c2 in grid:
            for c3 in grid:
                for u in grid:
                    w = sample.walk(tokens, parents, probs, np.float32([0, c1, c2, c3]),
                                    np.float32(u), 3)
                    assert w.margin > 0 and w.bonus_margin > 0
                    first[w.commit[0]] = first.get(w.commit[0], 0) + 1
                    if len(w.path) > 1 and w.path[1] == 1:
                        t = w.commit[1]
                        second_after_0[t] = second_after_0.get(t, 0) + 1
    tot = N ** 4
    assert {t: Fr(n, tot) for t, n in first.items()} == {0: Fr(1, 2), 1: Fr(1, 4), 2: Fr(1, 8),
                                                          3: Fr(1, 8)}
    tot0 = sum(second_after_0.values())
    assert {t: Fr(n, tot0) for t, n in second_after_0.items()} == {0: Fr(1, 4), 1: Fr(1, 4),
                                                                  2: Fr(1, 2)}


def test_inverse_cdf_against_exact_rationals():
    """The bonus draw against a brute-force definition in exact rational
    arithmetic: token j is drawn iff the mass before it is <= the threshold
    and the mass up to it is larger."""
    from fractions import Fraction as Fr
    rng = np.random.default_rng(24)
    for trial in range(200):
        V = int(rng.integers(1, 12))
        row = (rng.integers(0, 5, size=V) / 8.0).astype(np.float32)   # dyadic, some zero
        if row.sum() == 0:
            row[0] = 0.25
        R = sum(Fr(float(x)) for x in row)
        thr = Fr(int(rng.integers(0, 64)), 64) * R
        exact = next(j for j in range(V)
                     if sum(Fr(float(x)) for x in row[:j]) <= thr < sum(Fr(float(x)) for x in row[:j + 1]))
        j, m = sample._inverse_cdf(row.astype(np.float64), float(thr))
        assert j == exact
        assert row[j] > 0


def test_margin_marks_the_boundary_case():
    """The hand example whose coin sits exactly on the acceptance boundary has
    margin 0 (an fp32 implementation must take the same strict comparison);
    the others are clear of every boundary."""
    import json
    g = json.loads((GOLD / "sample_hand_example.json").read_text())
    probs = np.array(g["probs"], np.float32)
    for ex in g["examples"]:
        w = sample.walk(g["tokens"], g["parents"], probs, np.array(ex["coins"], np.float32),
                        np.float32(ex["bonus_u"]), g["depth_max"])
        if ex["name"] == "boundary_coin_rejects":
            assert w.margin == 0.0
        else:
            assert w.margin > 0.0 and w.bonus_margin > 0.0
        lo, hi = w.bonus_bounds(w.bonus)
        assert lo <= w.threshold < hi
