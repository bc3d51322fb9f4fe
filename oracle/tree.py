"""Oracle: best-first draft-tree growth from per-depth top-k log-probabilities.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

Source: "The DDTree CUDA Graph Fix: Unlocking Speculative Decoding at 109
tok/s on PCIe Blackwell", section "The DDTree Architecture: Confirming
Multiple-Path Evaluation" -- one drafter forward gives block_size hidden
states; each depth position yields its top-k candidates with log-probs; a
heap expansion repeatedly takes the candidate with the highest cumulative
log-prob, adds it to the tree, and offers that candidate's best child and its
next-ranked sibling, until ``budget`` draft nodes have been added, so the
tree has budget + 1 nodes with the root.  "The Oracle Drafter: Validating a
Custom DDTree Speculative Decoding Engine", section "The Engine Interface
Design": the root node carries the last verified token; section "The Context:
A Native DDTree Engine Built from Scratch": the reference builder was a
per-request CPU heapq.

Readings where the pages are silent:

* depth d = 1..D uses top-k list d-1; D = block_size - 1 = 7;
* scores are fp32, accumulated root-to-leaf as ``f32(parent + lp)``; a
  sibling's score is ``f32(parent_score + lp[d][rank+1])`` (never derived by
  subtracting the current lp);
* heap key = ``(-score, depth, rank_path)`` compared as a Python tuple, so
  ties go to the shallower node, then the lexicographically smaller rank path;
* node index = pop order with the root as node 0, hence parent < child;
* preconditions: each depth's lp row is non-increasing and <= 0;
  ``budget`` may not exceed the number of distinct rank paths
  ``sum_{d=1..D} K^d`` (a shorter tree is never produced).
"""
from __future__ import annotations

import heapq
import itertools
from typing import NamedTuple

import numpy as np


class Tree(NamedTuple):
    tokens: np.ndarray   # [budget+1] int32; node 0 = root token
    parents: np.ndarray  # [budget+1] int32; root -1
    depths: np.ndarray   # [budget+1] int32
    scores: np.ndarray   # [budget+1] float32; root 0
    rank_paths: list     # per node tuple of ranks (root: ())


def reachable(depth: int, topk: int) -> int:
    """Number of distinct rank paths of length 1..depth."""
    return sum(topk ** d for d in range(1, depth + 1))


def check_preconditions(lp: np.ndarray, budget: int) -> None:
    lp = np.asarray(lp, dtype=np.float32)
    D, K = lp.shape
    if budget < 0:
        raise ValueError("budget must be >= 0")
    if budget > 0 and (D < 1 or K < 1):
        raise ValueError("a non-empty tree needs depth >= 1 and topk >= 1")
    if budget > reachable(D, K):
        raise ValueError(f"budget {budget} exceeds the {reachable(D, K)} reachable paths")
    if not np.all(lp <= 0):
        raise ValueError("log-probs must be <= 0")
    if K > 1 and not np.all(lp[:, :-1] >= lp[:, 1:]):
        raise ValueError("each depth's top-k row must be non-increasing")


def build_tree(lp: np.ndarray, ids: np.ndarray, root_token: int, budget: int) -> Tree:
    """heapq best-first growth for one request (lp, ids: [D, K])."""
    lp = np.asarray(lp, dtype=np.float32)
    ids = np.asarray(ids, dtype=np.int32)
    check_preconditions(lp, budget)
    D, K = lp.shape
    f32 = np.float32

    tokens, parents, depths, scores, paths = [int(root_token)], [-1], [0], [f32(0.0)], [()]
    heap = []
    if budget > 0:
        s = f32(f32(0.0) + lp[0, 0])
        # entry: (-score, depth, rank_path, parent_node, parent_score)
        heapq.heappush(heap, (-float(s), 1, (0,), 0, f32(0.0)))
    while len(tokens) < budget + 1:
        neg, d, path, par, par_score = heapq.heappop(heap)
        score = f32(-neg)
        k = len(tokens)
        tokens.append(int(ids[d - 1, path[-1]]))
        parents.append(par)
        depths.append(d)
        scores.append(score)
        paths.append(path)
        if d < D:  # best child of the node just added
            cs = f32(score + lp[d, 0])
            heapq.heappush(heap, (-float(cs), d + 1, path + (0,), k, score))
        if path[-1] + 1 < K:  # next-ranked sibling, same parent
            ss = f32(par_score + lp[d - 1, path[-1] + 1])
            heapq.heappush(heap, (-float(ss), d, path[:-1] + (path[-1] + 1,), par, par_score))
    return Tree(np.array(tokens, np.int32), np.array(parents, np.int32),
                np.array(depths, np.int32), np.array(scores, np.float32), paths)


def build_tree_bruteforce(lp: np.ndarray, ids: np.ndarray, root_token: int, budget: int) -> Tree:
    """Enumerate every rank path, score it fp32 left to right, sort by the heap key.

    Pin for ``build_tree``: with lp <= 0 and sorted rows, every node's pusher
    (parent, or previous sibling) has a key no larger than its own, so the
    best-first pop order equals the first ``budget`` paths of the global
    ascending key order.  Cost is sum K^d, so keep inputs tiny.
    """
    lp = np.asarray(lp, dtype=np.float32)
    ids = np.asarray(ids, dtype=np.int32)
    check_preconditions(lp, budget)
    D, K = lp.shape
    f32 = np.float32
    cands = []
    for d in range(1, D + 1):
        for path in itertools.product(range(K), repeat=d):
            s = f32(0.0)
            for j, rk in enumerate(path):
                s = f32(s + lp[j, rk])
            cands.append((-float(s), d, path))
    cands.sort()
    chosen = cands[:budget]
    index = {(): 0}
    tokens, parents, depths, scores, paths = [int(root_token)], [-1], [0], [f32(0.0)], [()]
    for neg, d, path in chosen:
        if path[:-1] not in index:
            raise AssertionError("selected set is not closed under prefixes")
        index[path] = len(tokens)
        tokens.append(int(ids[d - 1, path[-1]]))
        parents.append(index[path[:-1]])
        depths.append(d)
        scores.append(f32(-neg))
        paths.append(path)
    return Tree(np.array(tokens, np.int32), np.array(parents, np.int32),
                np.array(depths, np.int32), np.array(scores, np.float32), paths)


def build_batch(topk_logprobs, topk_ids, root_tokens, qo_indptr):
    """Apply ``build_tree`` per request; budgets come from ``qo_indptr`` (Q_r - 1)."""
    outs = []
    for r in range(len(root_tokens)):
        q_len = int(qo_indptr[r + 1] - qo_indptr[r])
        outs.append(build_tree(topk_logprobs[r], topk_ids[r], int(root_tokens[r]), q_len - 1))
    cat = lambda f: np.concatenate([getattr(t, f) for t in outs]) if outs else np.zeros(0)
    return outs, cat("tokens").astype(np.int32), cat("parents").astype(np.int32), \
        cat("depths").astype(np.int32), cat("scores").astype(np.float32)
