"""Oracle: tree visibility, the full verify mask, and node positions.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

Sources:

* "The DDTree CUDA Graph Fix ...", section "The DDTree Architecture:
  Confirming Multiple-Path Evaluation": the compiled visibility is a
  ``[q_len, q_len]`` matrix in which a node sees only its ancestors (and,
  plain reading, itself); the full mask marks every prefix column visible to
  every tree node, so the prefix is read once and shared.
* "The Architecture of a Speculative Decoding Engine ...", section "The Final
  Resolution: A Concrete Trace": the cache holds positions 0..L-1, the root
  (last verified token) sits at position L and sees cache[0:L] plus itself;
  a draft node sees cache[0:L] plus its ancestor chain.  Hence a depth-d node
  sits at position L + d.
* "The 30-Column Mask: ...", sections "The Message: Tensor Shapes as Evidence"
  and "Mask Stride Formula": the flattened mask is row-major over a logical
  ``[q_len, prefix_len + q_len]`` matrix whose first prefix_len columns are the
  prefix and whose last q_len columns are the tree nodes in node order; the
  row stride is prefix_len + q_len (9 x 30 = 270 for prefix 21).

Reading where the final-scheme formula was lost: full mask row i =
``[1] * P ++ vis[i]`` with kv_len = P + q_len.
"""
from __future__ import annotations

import numpy as np


def ancestors(parents: np.ndarray) -> list:
    """anc(i) = {i} + anc(parent(i)); the root's set is {0}."""
    parents = np.asarray(parents)
    out = []
    for i in range(len(parents)):
        s, j, steps = set(), i, 0
        while j >= 0:
            s.add(j)
            j = int(parents[j])
            steps += 1
            if steps > len(parents):
                raise ValueError("parent pointers form a cycle")
        out.append(s)
    return out


def visibility_matrix(parents: np.ndarray) -> np.ndarray:
    """``vis[i, j]`` is True iff tree node j is node i or one of its ancestors."""
    anc = ancestors(parents)
    q = len(parents)
    vis = np.zeros((q, q), dtype=bool)
    for i, s in enumerate(anc):
        for j in s:
            vis[i, j] = True
    return vis


def full_mask(parents: np.ndarray, prefix_len: int) -> np.ndarray:
    """Logical ``[q_len, prefix_len + q_len]`` mask: prefix all visible ++ visibility."""
    vis = visibility_matrix(parents)
    q = len(parents)
    m = np.zeros((q, prefix_len + q), dtype=np.uint8)
    m[:, :prefix_len] = 1
    m[:, prefix_len:] = vis
    return m


def positions(depths: np.ndarray, prefix_len: int) -> np.ndarray:
    """Sequence position of each node: cache length + depth (root at prefix_len)."""
    return np.asarray(depths, dtype=np.int64) + int(prefix_len)


def vis_bits(parents: np.ndarray, words_per_row: int) -> np.ndarray:
    """Pack ``visibility_matrix`` as uint32 words: bit j%32 of word j//32 = node j."""
    vis = visibility_matrix(parents)
    q = vis.shape[0]
    out = np.zeros((q, words_per_row), dtype=np.uint32)
    for i in range(q):
        for j in range(q):
            if vis[i, j]:
                out[i, j // 32] |= np.uint32(1) << np.uint32(j % 32)
    return out


def batch(node_parents, node_depths, qo_indptr, prefix_lens, words_per_row):
    """Per-request visibility for a packed batch: bits, positions, flat dense mask."""
    bits, pos, dense = [], [], []
    for r in range(len(prefix_lens)):
        a, b = int(qo_indptr[r]), int(qo_indptr[r + 1])
        par = node_parents[a:b]
        bits.append(vis_bits(par, words_per_row))
        pos.append(positions(node_depths[a:b], int(prefix_lens[r])))
        dense.append(full_mask(par, int(prefix_lens[r])).ravel())
    return (np.concatenate(bits) if bits else np.zeros((0, words_per_row), np.uint32),
            np.concatenate(pos) if pos else np.zeros(0, np.int64),
            np.concatenate(dense) if dense else np.zeros(0, np.uint8))
