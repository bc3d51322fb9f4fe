"""Pins for ``oracle.visibility``.

* hand-derived mask, bitset words and positions (``golden/mask_hand_example.json``);
* the page's printed shapes (``golden/p5_debug_shapes.json``): a 9-node tree
  over a 21-token prefix gives a 9 x 30 = 270-entry mask, columns 0..20 the
  prefix, 21..29 the tree; the stride-21 misread is a different mask;
* closed forms: a chain is the lower triangle; the root column and the
  diagonal are all ones; row i = row parent(i) plus bit i; row sums equal
  prefix + depth + 1.
"""
import json
from pathlib import Path

import numpy as np

from oracle import tree, visibility
from workloads import draw_drafter_topk

GOLD = Path(__file__).parent / "golden"


def test_hand_example():
    g = json.loads((GOLD / "mask_hand_example.json").read_text())
    par = np.array(g["parents"])
    assert [sorted(s) for s in visibility.ancestors(par)] == g["ancestor_sets"]
    assert visibility.full_mask(par, g["prefix"]).tolist() == g["dense_rows"]
    assert visibility.vis_bits(par, 1)[:, 0].tolist() == g["vis_words"]
    assert visibility.vis_bits(par, 3)[:, 1:].sum() == 0
    assert visibility.positions(np.array(g["depths"]), g["prefix"]).tolist() == g["positions"]


def _c1_tree():
    rng = np.random.default_rng(1001)
    lp, ids = draw_drafter_topk(rng, 7, 4, 512)
    return tree.build_tree(lp, ids, 0, 8)


def test_page_shapes_9x30():
    g = json.loads((GOLD / "p5_debug_shapes.json").read_text())
    t = _c1_tree()
    assert len(t.tokens) == g["q_len"]
    P = g["kv_len_max"]
    m = visibility.full_mask(t.parents, P)
    assert m.shape == (g["q_len"], g["mask_stride"]) and m.size == g["mask_numel"]
    lo, hi = g["prefix_columns"]
    assert m[:, lo:hi + 1].all()                      # prefix visible to every node
    tlo, thi = g["tree_columns"]
    tail = m[:, tlo:thi + 1]
    assert tail[:, 0].all()                           # every node sees the root
    assert np.diag(tail).all()                        # and itself
    assert m.sum(axis=1).tolist() == (P + t.depths + 1).tolist()
    # row i = row parent(i) | bit i
    for i in range(1, len(t.parents)):
        expect = tail[t.parents[i]].copy()
        expect[i] = 1
        assert np.array_equal(tail[i], expect)
    # the stride bug: reading row i at flat[i*21 + c] gives a different mask
    flat = m.ravel()
    wrong = np.array([[flat[i * g["wrong_stride"] + c] for c in range(g["mask_stride"])]
                      for i in range(g["q_len"])])
    assert not np.array_equal(wrong, m)


def test_chain_is_lower_triangle():
    par = np.array([-1, 0, 1, 2, 3, 4, 5, 6])
    m = visibility.full_mask(par, 5)
    assert m[:, :5].all()
    assert np.array_equal(m[:, 5:], np.tril(np.ones((8, 8), np.uint8)))


def test_root_only():
    assert visibility.full_mask(np.array([-1]), 4).tolist() == [[1, 1, 1, 1, 1]]
    assert visibility.full_mask(np.array([-1]), 0).tolist() == [[1]]


def test_bits_match_matrix_for_wide_trees():
    rng = np.random.default_rng(7)
    lp, ids = draw_drafter_topk(rng, 7, 16, 512)
    t = tree.build_tree(lp, ids, 0, 64)
    vis = visibility.visibility_matrix(t.parents)
    bits = visibility.vis_bits(t.parents, 3)
    for i in range(65):
        for j in range(65):
            assert bool((int(bits[i, j // 32]) >> (j % 32)) & 1) == bool(vis[i, j])


def test_batch_flat_mask_uses_per_request_stride():
    par = [np.array([-1, 0, 0]), np.array([-1, 0])]
    qo = np.array([0, 3, 5])
    P = np.array([2, 4])
    bits, pos, dense = visibility.batch(np.concatenate(par), np.array([0, 1, 1, 0, 1]), qo, P, 1)
    assert dense.size == 3 * 5 + 2 * 6
    assert dense[:15].reshape(3, 5).tolist() == [[1, 1, 1, 0, 0], [1, 1, 1, 1, 0], [1, 1, 1, 0, 1]]
    assert dense[15:].reshape(2, 6).tolist() == [[1, 1, 1, 1, 1, 0], [1, 1, 1, 1, 1, 1]]
    assert pos.tolist() == [2, 3, 3, 4, 5]
