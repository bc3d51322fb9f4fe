"""Oracle: stochastic (temperature) acceptance along the draft tree.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

Source: "The DDTree CUDA Graph Fix ...", section "Temperature Support:
Already Working for Linear, Planned for DDTree": with temperature, the tree
is walked by tree-structured rejection sampling against the target's
(temperature-, top-k-, top-p-filtered) distribution at every node, the
draft being the tree's tokens themselves (no draft distribution).

Reading: the standard speculative-sampling rule for a
deterministic draft, walked from the root:

* at node ``cur`` the residual distribution starts as the target row
  ``P[cur]`` with total mass ``R``; the children of ``cur`` are tried in
  ascending node order; child ``c`` with token ``t`` is accepted iff
  ``coins[c] * R < res[t]``; on rejection ``R -= res[t]`` and ``res[t] = 0``
  (the draft put all its mass on ``t``, so ``max(p - q, 0)`` removes ``t``);
* an accepted child becomes ``cur``; the walk stops when no child is
  accepted or after ``depth_max + 1`` path nodes;
* the bonus token is drawn from the residual at the last node by inverse
  CDF at ``bonus_uniform * R`` (``_inverse_cdf``).

Everything is fp32, and the order of every sum is fixed, because these
comparisons decide integers and the kernel must take them identically: a
row is cut into ``NT = 256`` contiguous blocks of ``ceil(V / 256)`` tokens;
a block's mass is summed token by token; the row's mass is the block masses
summed block by block; the running mass at token ``j`` is the masses of the
blocks before its block, summed block by block, plus its block's tokens up
to ``j`` summed token by token.
"""
from __future__ import annotations

import numpy as np

NT = 256  # blocks per row (the kernel's threads)


def _blocks(vocab: int):
    per = -(-vocab // NT)
    return [(b * per, min(vocab, (b + 1) * per)) for b in range(NT)]


def _seq(values) -> np.ndarray:
    """Running sums of fp32 values, added one by one from 0 (numpy's cumsum
    accumulates in order, in the array's dtype)."""
    return np.cumsum(np.asarray(values, dtype=np.float32), dtype=np.float32)


def _block_masses(row: np.ndarray) -> list:
    return [(_seq(row[lo:hi])[-1] if hi > lo else np.float32(0.0)) for lo, hi in _blocks(len(row))]


def _mass(row: np.ndarray) -> np.float32:
    """Row mass in the fixed order (fp32)."""
    return _seq(_block_masses(row))[-1]


def _inverse_cdf(row: np.ndarray, threshold: np.float32) -> int:
    """Token drawn at ``threshold`` (fixed order, fp32): the first block b
    with run_b + mass_b > threshold (run_b: the masses of the blocks before
    b, summed block by block), then in it the first token j with
    run_b + (its tokens up to j, summed token by token) > threshold.  If
    rounding leaves the threshold unreached inside that block, its last token
    with mass; if no block reaches it, the row's last token with mass."""
    blocks = _blocks(len(row))
    masses = _block_masses(row)
    run = np.float32(0.0)
    for (lo, hi), bs in zip(blocks, masses):
        if np.float32(run + bs) > threshold:
            acc, last = run, -1
            for j in range(lo, hi):
                acc = np.float32(acc + row[j])
                if acc > threshold:
                    return j
                if row[j] > 0:
                    last = j
            return last
        run = np.float32(run + bs)
    nz = np.nonzero(row > 0)[0]
    return int(nz[-1]) if len(nz) else -1


def sample_request(tokens, parents, probs, coins, bonus_u, depth_max: int):
    """(path, accept_len, commit_tokens, bonus) of one request.

    tokens, parents [Q]; probs [Q, V] float32 (non-negative target
    probabilities of every node); coins [Q] float32 in [0, 1) (coin of a
    node, used when it is tried as a child); bonus_u float32 in [0, 1).
    """
    tokens = np.asarray(tokens)
    parents = np.asarray(parents)
    probs = np.asarray(probs, dtype=np.float32)
    coins = np.asarray(coins, dtype=np.float32)
    q = len(tokens)
    cur, path = 0, [0]
    res = probs[0].copy()
    R = _mass(res)
    while True:
        nxt = None
        if len(path) < depth_max + 1:
            for c in range(1, q):
                if int(parents[c]) != cur:
                    continue
                t = int(tokens[c])
                if np.float32(coins[c] * R) < res[t]:
                    nxt = c
                    break
                R = np.float32(R - res[t])
                res[t] = np.float32(0.0)
        if nxt is None:
            break
        cur = nxt
        path.append(cur)
        res = probs[cur].copy()
        R = _mass(res)
    bonus = _inverse_cdf(res, np.float32(np.float32(bonus_u) * R))
    commit = [int(tokens[n]) for n in path[1:]] + [bonus]
    return path, len(path), commit, bonus


def batch(node_tokens, node_parents, qo_indptr, probs, coins, bonus_u, depth_max: int):
    """Arrays shaped like ddtree_tree_sample's outputs."""
    qo = np.asarray(qo_indptr)
    bs = len(qo) - 1
    nodes = np.full((bs, depth_max + 1), -1, np.int32)
    alen = np.zeros(bs, np.int32)
    commit = np.full((bs, depth_max + 1), -1, np.int32)
    bonus = np.full(bs, -1, np.int32)
    for r in range(bs):
        a, b = int(qo[r]), int(qo[r + 1])
        if b - a < 1:
            continue
        path, n, com, bo = sample_request(node_tokens[a:b], node_parents[a:b], probs[a:b],
                                          coins[a:b], bonus_u[r], depth_max)
        nodes[r, :n] = path
        alen[r] = n
        commit[r, :n] = com
        bonus[r] = bo
    return nodes, alen, commit, bonus
