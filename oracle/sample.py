"""Oracle: stochastic (temperature) acceptance along the draft tree.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

Source: "The DDTree CUDA Graph Fix ...", section "Temperature Support:
Already Working for Linear, Planned for DDTree": with temperature, the tree
is walked by tree-structured rejection sampling against the target's
(temperature-, top-k-, top-p-filtered) distribution at every node, the
draft being the tree's tokens themselves (no draft distribution).

Reading: the standard speculative-sampling rule for a draft that puts all
its mass on one token, walked from the root:

* at node ``cur`` the residual distribution ``res`` starts as the target row
  ``P[cur]``; its total mass is ``R``;
* the children of ``cur`` are tried in ascending node order; child ``c`` with
  token ``t`` is accepted iff ``coins[c] * R < res[t]`` (probability
  ``res[t] / R``); on rejection the draft's point mass on ``t`` is removed
  from the residual, ``res <- max(res - onehot(t) * res[t], 0)``, i.e.
  ``res[t] = 0``, and ``R`` becomes the residual's new mass;
* an accepted child becomes ``cur``; the walk stops when no child is
  accepted or after ``depth_max + 1`` path nodes;
* the bonus token is drawn from the residual at the last node by inverse
  CDF: the first token ``j`` whose cumulative residual mass (tokens in
  vocabulary order) exceeds ``bonus_u * R``; ``-1`` if the residual has no
  mass.

Arithmetic is plain fp64 on the exactly widened fp32 inputs: masses are
``math.fsum`` of the residual (correctly rounded), cumulative masses a
sequential fp64 running sum in token order.  Nothing here follows any
particular blocking or summation order of a fast implementation: an fp32
implementation takes the same decisions whenever they are not within its
rounding error of a boundary, which ``margin`` measures (see ``walk``).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass
class Walk:
    path: list           # accepted nodes, root first
    commit: list         # accepted draft tokens, then the bonus
    bonus: int           # -1 if the residual at the last node has no mass
    margin: float        # smallest distance of an accept/reject decision from its boundary / row mass
    bonus_margin: float  # distance of the bonus threshold from the drawn token's bounds / row mass
    residual: np.ndarray  # the residual at the last node (fp64)
    threshold: float     # the bonus threshold (fp64)
    row_mass: float      # mass of the last node's row

    @property
    def accept_len(self) -> int:
        return len(self.path)

    def bonus_bounds(self, token: int):
        """Running residual masses (token order) just before and just after
        ``token``: the draw picks ``token`` iff the threshold lies in between."""
        run = np.cumsum(self.residual)
        return (float(run[token - 1]) if token > 0 else 0.0), float(run[token])


def _mass(res: np.ndarray) -> float:
    return math.fsum(res.tolist())


def _inverse_cdf(res: np.ndarray, threshold: float):
    """(token, margin) of the inverse-CDF draw: the first token whose running
    mass in token order exceeds ``threshold``; ``margin`` is the distance of
    the threshold to the two running masses that bound the chosen token."""
    run = np.cumsum(res)              # fp64, sequential in token order
    hit = np.nonzero(run > threshold)[0]
    if len(hit) == 0:                 # only if rounding put the threshold at the total
        nz = np.nonzero(res > 0)[0]
        return (int(nz[-1]) if len(nz) else -1), 0.0
    j = int(hit[0])
    below = float(run[j - 1]) if j > 0 else 0.0
    return j, min(float(run[j]) - threshold, threshold - below)


def walk(tokens, parents, probs, coins, bonus_u, depth_max: int) -> Walk:
    """One request.  tokens, parents [Q]; probs [Q, V] (non-negative target
    rows of every node, any total); coins [Q] in [0, 1) (the coin of a node,
    used when it is tried as a child); bonus_u in [0, 1).

    ``margin`` is the smallest |coin * R - res[t]| over the accept/reject
    decisions taken, ``bonus_margin`` the bonus threshold's distance to the
    running masses around the drawn token, each divided by the mass of the
    row it was taken on: an implementation whose mass and running-mass errors
    stay below that fraction of the row mass takes those decisions the same
    way.  A request whose last residual has no mass has a bonus of -1 and an
    infinite bonus margin (nothing to decide)."""
    tokens = [int(t) for t in tokens]
    parents = [int(p) for p in parents]
    probs = np.asarray(probs, dtype=np.float32).astype(np.float64)
    coins = np.asarray(coins, dtype=np.float32).astype(np.float64)
    V = probs.shape[1]
    q = len(tokens)
    margin = math.inf
    cur, path = 0, [0]
    while True:
        res = probs[cur].copy()
        R0 = R = _mass(res)
        nxt = None
        if len(path) < depth_max + 1:
            for c in range(1, q):
                if parents[c] != cur:
                    continue
                t = tokens[c]
                pt = res[t] if 0 <= t < V else 0.0
                if R0 > 0:
                    margin = min(margin, abs(coins[c] * R - pt) / R0)
                if coins[c] * R < pt:
                    nxt = c
                    break
                if 0 <= t < V:
                    res[t] = 0.0
                R = _mass(res)
        if nxt is None:
            break
        cur = nxt
        path.append(cur)
    threshold = float(np.float64(np.float32(bonus_u))) * R
    if R > 0:
        bonus, m = _inverse_cdf(res, threshold)
        bonus_margin = m / R0
    else:
        bonus, bonus_margin = -1, math.inf
    commit = [tokens[n] for n in path[1:]] + [bonus]
    return Walk(path, commit, bonus, margin, bonus_margin, res, threshold, R0)


def sample_request(tokens, parents, probs, coins, bonus_u, depth_max: int):
    """(path, accept_len, commit_tokens, bonus) of one request (see ``walk``)."""
    w = walk(tokens, parents, probs, coins, bonus_u, depth_max)
    return w.path, w.accept_len, w.commit, w.bonus


def batch(node_tokens, node_parents, qo_indptr, probs, coins, bonus_u, depth_max: int,
          with_walks: bool = False):
    """Arrays shaped like ddtree_tree_sample's outputs (and, with
    ``with_walks``, each request's ``Walk``, None for requests without
    nodes)."""
    qo = np.asarray(qo_indptr)
    bs = len(qo) - 1
    nodes = np.full((bs, depth_max + 1), -1, np.int32)
    alen = np.zeros(bs, np.int32)
    commit = np.full((bs, depth_max + 1), -1, np.int32)
    bonus = np.full(bs, -1, np.int32)
    walks = [None] * bs
    for r in range(bs):
        a, b = int(qo[r]), int(qo[r + 1])
        if b - a < 1:
            continue
        w = walk(node_tokens[a:b], node_parents[a:b], probs[a:b], coins[a:b], bonus_u[r],
                 depth_max)
        n = w.accept_len
        nodes[r, :n] = w.path
        alen[r] = n
        commit[r, :n] = w.commit
        bonus[r] = w.bonus
        walks[r] = w
    if with_walks:
        return nodes, alen, commit, bonus, walks
    return nodes, alen, commit, bonus
