"""Pins for ``oracle.commit`` (committing the accepted path into the cache).

* hand-derived commits of one small tree (``golden/commit_hand_example.json``);
* the autoregressive case ("The Architecture of a Speculative Decoding
  Engine ...", section "The Final Resolution: A Concrete Trace"): a budget-0
  tree accepts only its root, the cache grows by one and nothing moves;
* a fully accepted chain (same page, section "The First Attempt: Temporary
  Buffers and Post-Verify Compaction": when every appended token is accepted
  no compaction is needed): the index form returns the slot list unchanged
  and the move form leaves the pool unchanged;
* consistency with the accept step and the positions rule: with a toy model
  whose latent is a function of (token, position), each tree node's row
  holding the latent of its token at position P + depth, the committed cache
  read in order equals the latents an autoregressive decode of the root
  token and the accepted drafts would have written at P, P + 1, ..., and the
  bonus token is not among them (section "The Off-by-One Labyrinth");
* every root path of random trees: the list has P + len(path) entries,
  rejected nodes' slots never appear in the index form, and the move form
  changes no row outside the path's destination slots.
"""
import json
from pathlib import Path

import numpy as np

from oracle import accept, commit, tree, visibility
from workloads import draw_drafter_topk

GOLD = Path(__file__).parent / "golden"


def _toy_latent(token: int, pos: int, width: int = 6) -> np.ndarray:
    # any injective-enough function of (token, position) serves
    return np.array([token, pos, token * 31 + pos, (token ^ pos) & 0xff, token % 7, pos % 5],
                    dtype=np.float64)[:width]


def _path_to(parents, v):
    path = [v]
    while parents[path[-1]] >= 0:
        path.append(int(parents[path[-1]]))
    return path[::-1]


def test_hand_example():
    g = json.loads((GOLD / "commit_hand_example.json").read_text())
    pre, nodes = g["prefix_slots"], g["node_slots"]
    for ex in g["examples"]:
        got = commit.commit_request(pre, nodes, ex["path"], move=False)
        assert got.tolist() == ex["index_list"], ex["name"]
        got = commit.commit_request(pre, nodes, ex["path"], move=True)
        assert got.tolist() == ex["move_list"], ex["name"]
        pool = np.arange(32, dtype=np.float64)[:, None] * np.ones((1, 3))
        new = commit.compact_request(pool, nodes, ex["path"])
        expect = pool.copy()
        for dst, src in ex["moves"]:
            expect[dst] = pool[src]
        assert np.array_equal(new, expect), ex["name"]


def test_autoregressive_budget_zero():
    # one request, P = 5 prefix slots, a 1-node tree: accept_len 1
    kv = np.array([7, 3, 9, 1, 4, 8])
    out = commit.batch([0, 6], kv, [0, 1], np.array([[0, -1]]), np.array([1]))
    assert out.kv_indptr.tolist() == [0, 6]
    assert out.kv_indices.tolist() == kv.tolist()
    pool = np.random.default_rng(0).normal(size=(12, 4))
    out = commit.batch([0, 6], kv, [0, 1], np.array([[0, -1]]), np.array([1]), pool=pool)
    assert np.array_equal(out.pool, pool)


def test_fully_accepted_chain_needs_no_compaction():
    q, p = 6, 4
    kv = np.array([40, 41, 42, 43, 50, 51, 52, 53, 54, 55])
    path = np.arange(q)[None, :]
    out = commit.batch([0, p + q], kv, [0, q], path, np.array([q]))
    assert out.kv_indices.tolist() == kv.tolist()
    pool = np.random.default_rng(1).normal(size=(60, 3))
    out = commit.batch([0, p + q], kv, [0, q], path, np.array([q]), pool=pool)
    assert np.array_equal(out.pool, pool)
    assert out.kv_indices.tolist() == kv.tolist()


def test_commit_equals_autoregressive_cache():
    rng = np.random.default_rng(7)
    D, K = 5, 3
    for trial in range(30):
        lp, ids = draw_drafter_topk(rng, D, K, 40)
        root = int(rng.integers(0, 40))
        budget = int(rng.integers(1, 20))
        t = tree.build_tree(lp, ids, root, budget)
        q = len(t.tokens)
        p = int(rng.integers(0, 6))
        pos = visibility.positions(t.depths, p)
        # target predictions: mostly follow some child, else a fresh token
        pred = np.array([int(rng.integers(0, 40)) for _ in range(q)])
        for v in range(q):
            kids = [c for c in range(q) if t.parents[c] == v]
            if kids and rng.random() < 0.7:
                pred[v] = t.tokens[kids[int(rng.integers(0, len(kids)))]]
        acc = accept.accept(t.tokens, t.parents, pred, D)
        # slots: prefix then nodes, scattered in a pool of 64 rows
        slots = rng.permutation(64)[:p + q]
        pool = np.zeros((64, 6))
        prefix_tokens = rng.integers(0, 40, size=p)
        for j in range(p):
            pool[slots[j]] = _toy_latent(int(prefix_tokens[j]), j)
        for i in range(q):
            pool[slots[p + i]] = _toy_latent(int(t.tokens[i]), int(pos[i]))
        # what decoding root, then the accepted drafts, one by one would cache
        seq = [int(t.tokens[0])] + acc.commit_tokens[:-1]   # the bonus is not cached
        want = [_toy_latent(int(prefix_tokens[j]), j) for j in range(p)]
        want += [_toy_latent(tok, p + k) for k, tok in enumerate(seq)]
        nodes = np.array([acc.path + [-1] * (D + 1 - acc.accept_len)])
        for move in (False, True):
            out = commit.batch([0, p + q], slots, [0, q], nodes, np.array([acc.accept_len]),
                               pool=pool if move else None)
            cache = (out.pool if move else pool)[out.kv_indices]
            assert out.kv_indptr[1] == p + acc.accept_len
            assert np.array_equal(cache, np.array(want)), (trial, move)


def test_every_root_path():
    rng = np.random.default_rng(11)
    for trial in range(10):
        lp, ids = draw_drafter_topk(rng, 4, 3, 30)
        t = tree.build_tree(lp, ids, 0, int(rng.integers(3, 15)))
        q, p = len(t.tokens), int(rng.integers(0, 5))
        slots = rng.permutation(100)[:p + q]
        pool = rng.normal(size=(100, 2))
        for v in range(q):
            path = _path_to(t.parents, v)
            lst = commit.commit_request(slots[:p], slots[p:], path, move=False)
            assert len(lst) == p + len(path)
            rejected = set(slots[p:].tolist()) - {int(slots[p + n]) for n in path}
            assert not rejected & set(lst.tolist())
            new = commit.compact_request(pool, slots[p:], path)
            dest = {int(slots[p + i]) for i in range(len(path))}
            untouched = [s for s in range(100) if s not in dest]
            assert np.array_equal(new[untouched], pool[untouched])
