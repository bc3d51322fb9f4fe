"""Oracle: greedy tree acceptance along the target argmax.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

Sources:

* "The DDTree CUDA Graph Fix ...", section "The DDTree Architecture:
  Confirming Multiple-Path Evaluation": starting at the root, follow the
  target's argmax at each node, stepping to the child whose token matches,
  until no child matches; the result is the longest accepted chain plus one
  bonus token.
* "The Oracle Drafter: ...", section "The Engine Interface Design": the
  accept step reports the accepted path, the accept length, the proposed
  tokens, the commit length and the bonus token; section "Reasoning About
  Cache Positions and Token Indices": the bonus is the target's prediction
  at the deepest accepted node; sentinel drafts that never equal the argmax
  end acceptance.
* "The Architecture of a Speculative Decoding Engine ...", section "The
  Final Resolution: A Concrete Trace": accepted nodes including the root are
  committed, so the cache grows by accept_len; autoregressive decoding is
  the budget-0 tree with accept_len = 1.

Readings: accept_len counts the root; commit tokens are the
accepted draft tokens followed by the bonus (accept_len tokens in all); if
two children of one node carried the same token the lower node index wins;
the walk stops after ``depth_max + 1`` path nodes.
"""
from __future__ import annotations

from typing import NamedTuple

import numpy as np


class Accepted(NamedTuple):
    path: list          # node indices, root first
    accept_len: int
    commit_tokens: list
    bonus: int


def accept(tokens: np.ndarray, parents: np.ndarray, target_predict: np.ndarray,
           depth_max: int) -> Accepted:
    tokens = np.asarray(tokens)
    parents = np.asarray(parents)
    pred = np.asarray(target_predict)
    q = len(tokens)
    cur, path = 0, [0]
    while len(path) < depth_max + 1:
        t = int(pred[cur])
        nxt = None
        for c in range(1, q):
            if int(parents[c]) == cur and int(tokens[c]) == t:
                nxt = c
                break
        if nxt is None:
            break
        cur = nxt
        path.append(cur)
    bonus = int(pred[cur])
    commit = [int(tokens[n]) for n in path[1:]] + [bonus]
    return Accepted(path, len(path), commit, bonus)


def accept_bruteforce(tokens, parents, target_predict, depth_max: int) -> Accepted:
    """Pin: among all root paths whose every step matches the target argmax of
    the step's parent, take the longest (lowest node indices on ties)."""
    tokens = np.asarray(tokens)
    parents = np.asarray(parents)
    pred = np.asarray(target_predict)
    best = [0]
    for leaf in range(len(tokens)):
        path, j = [], leaf
        while j >= 0:
            path.append(j)
            j = int(parents[j])
        path.reverse()
        if len(path) > depth_max + 1:
            continue
        if all(int(tokens[path[k]]) == int(pred[path[k - 1]]) for k in range(1, len(path))):
            if len(path) > len(best) or (len(path) == len(best) and path < best):
                best = path
    bonus = int(pred[best[-1]])
    return Accepted(best, len(best), [int(tokens[n]) for n in best[1:]] + [bonus], bonus)


def batch(node_tokens, node_parents, qo_indptr, target_predict, depth_max: int):
    """Packed outputs as the library lays them out: [bs, D+1] rows padded with -1."""
    bs = len(qo_indptr) - 1
    acc_nodes = np.full((bs, depth_max + 1), -1, np.int32)
    acc_len = np.zeros(bs, np.int32)
    commit = np.full((bs, depth_max + 1), -1, np.int32)
    bonus = np.zeros(bs, np.int32)
    for r in range(bs):
        a, b = int(qo_indptr[r]), int(qo_indptr[r + 1])
        res = accept(node_tokens[a:b], node_parents[a:b], target_predict[a:b], depth_max)
        acc_nodes[r, :res.accept_len] = res.path
        acc_len[r] = res.accept_len
        commit[r, :len(res.commit_tokens)] = res.commit_tokens
        bonus[r] = res.bonus
    return acc_nodes, acc_len, commit, bonus
