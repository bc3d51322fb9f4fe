"""Oracle: per-depth top-k log-probabilities of the drafter's logits.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

Source: "The DDTree CUDA Graph Fix ...", section "The DDTree Architecture:
Confirming Multiple-Path Evaluation": one draft forward yields a hidden state
per depth position, and from each the vocabulary head gives the top-k
candidate tokens with their log-probabilities; the best-first builder
consumes them.

Readings: the log-probability is the log-softmax over the whole
vocabulary, computed here in fp64 from the exactly widened inputs; the top-k
are the k largest log-probabilities in descending order, equal values in
ascending token id; the values are returned rounded to fp32.  Since the
log-softmax subtracts one constant from every logit of a row, the order is
the order of the logits themselves.
"""
from __future__ import annotations

import numpy as np


def log_softmax(logits_row) -> np.ndarray:
    """fp64 log-softmax of one row: x - (max + log sum exp(x - max))."""
    x = np.asarray(logits_row, dtype=np.float64)
    m = x.max()
    return x - (m + np.log(np.exp(x - m).sum()))


def topk_row(logits_row, k: int):
    """(values fp32 [k], ids int32 [k]) of one row."""
    lp = log_softmax(logits_row)
    ids = np.arange(len(lp))
    order = np.lexsort((ids, -lp))[:k]   # by -lp, then by id
    return lp[order].astype(np.float32), order.astype(np.int32)


def batch(logits, k: int):
    """Rows of ``logits`` [rows, V] -> (values [rows, k] fp32, ids [rows, k] int32)."""
    logits = np.asarray(logits)
    vals = np.zeros((logits.shape[0], k), np.float32)
    ids = np.zeros((logits.shape[0], k), np.int32)
    for i in range(logits.shape[0]):
        vals[i], ids[i] = topk_row(logits[i], k)
    return vals, ids
