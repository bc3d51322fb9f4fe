"""Oracle: tree-verify attention in absorbed-MLA form, fp64.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

Sources:

* "The Architecture of a Speculative Decoding Engine ...", section "The
  Forward Pass Pseudocode": the verify attention takes the absorbed query
  (q_nope pushed through the key up-projection into latent space) and the
  roped q_pe, attends over the cached c_kv and k_pe under an ``[M, kv_len]``
  mask with a softmax scale, and returns a latent-space output that is only
  afterwards projected by the value up-projection.  So the score is the dot
  product over the whole latent (c_kv part + rope part) and the output is a
  softmax-weighted sum of c_kv rows.
* "The 30-Column Mask: ...", sections "The Message: Tensor Shapes as
  Evidence" and "Multi-Head Latent Attention (MLA)": per token one 576-wide
  latent row shared by all heads, 512 c_kv + 64 rope; queries are
  ``[q_len, heads, 576]``; the scale is the literal 0.14468.
* "The DDTree CUDA Graph Fix ...", section "The DDTree Architecture:
  Confirming Multiple-Path Evaluation": all budget+1 nodes are verified in
  one pass, each seeing the shared prefix plus its own ancestors.

This is the plain definition: for query row (node i, head h) and its visible
columns c, ``s_c = scale * sum_{d<576} q[i,h,d] * kv[c,d]``,
``out = sum_c softmax(s)_c * kv[c, :512]``, ``lse = ln sum_c exp(s_c)``,
computed in fp64 from the exactly widened fp32/bf16 inputs.  A KV split
(partial softmax + log-sum-exp merge) reaches the same result up to rounding
order, so the oracle does not split.
"""
from __future__ import annotations

import numpy as np

from . import visibility

DL = 512


def attend(q: np.ndarray, kv: np.ndarray, mask: np.ndarray, scale: float):
    """Masked softmax attention for ``n`` query nodes.

    q: [n, H, 576]; kv: [m, 576] latent rows in logical column order;
    mask: [n, m] (nonzero = visible).  Returns out [n, H, 512] and lse [n, H]
    in fp64.  Every row must see at least one column.
    """
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    mask = np.asarray(mask).astype(bool)
    n, H, _ = q.shape
    out = np.zeros((n, H, DL), dtype=np.float64)
    lse = np.zeros((n, H), dtype=np.float64)
    v = kv[:, :DL]
    for i in range(n):
        if not mask[i].any():
            raise ValueError(f"query node {i} sees no column")
        # scores of every column; an invisible column's score is -inf, so its
        # softmax weight is exactly 0
        s = np.where(mask[i][None, :], float(scale) * (q[i] @ kv.T), -np.inf)   # [H, m]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        out[i] = (e @ v) / l
        lse[i] = (m + np.log(l))[:, 0]
    return out, lse


def verify_request(q_r: np.ndarray, kv_r: np.ndarray, prefix_len: int,
                   parents: np.ndarray, scale: float, nodes=None):
    """One request: q_r [Q, H, 576], kv_r [P+Q, 576] (prefix rows then node rows).

    ``nodes`` optionally restricts the computation to a subset of query nodes
    (used to sample outputs of large workloads one by one).
    """
    mask = visibility.full_mask(parents, prefix_len)
    if nodes is None:
        nodes = np.arange(len(parents))
    nodes = np.asarray(nodes, dtype=np.int64)
    return attend(np.asarray(q_r)[nodes], kv_r, mask[nodes], scale)


def verify_request_layers(q_layers, kv_layers, prefix_len: int, parents: np.ndarray, scale: float,
                          nodes=None):
    """One request over L layers: q_layers[l] [Q, H, 576], kv_layers[l]
    [P+Q, 576] (layer l's latents gathered through the request's slot list).

    "The 30-Column Mask ...", sections "The Fix: Building Combined Indices"
    and "Layer-Invariant Slot Optimization": within a step the slot
    positions are the same in every layer and only the stored latents
    differ, so the mask (hence the visible columns) is built once and every
    layer attends through it; layer l's result is the single-layer verify of
    its own queries and latents.  Returns a list of (out, lse) per layer.
    """
    mask = visibility.full_mask(parents, prefix_len)
    if nodes is None:
        nodes = np.arange(len(parents))
    nodes = np.asarray(nodes, dtype=np.int64)
    return [attend(np.asarray(q)[nodes], kv, mask[nodes], scale)
            for q, kv in zip(q_layers, kv_layers)]
