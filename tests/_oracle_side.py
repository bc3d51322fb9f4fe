"""Test helpers that run the oracle on a generated workload (CPU only).

Only inputs flow in (the workload and, for accept, predictions drawn from the
oracle's own tree); nothing here reads results of the HIP path.
"""
from __future__ import annotations

import numpy as np

from oracle import accept, attention, drafter, tree, visibility
from workloads import draw_target_predict


def oracle_tables(wl):
    """The builder's per-depth top-k tables [bs, D, K] on the oracle side: the
    workload's drawn tables, or the oracle drafter's top-k of its logits."""
    if wl.drafter_logits is None:
        return wl.topk_logprobs, wl.topk_ids
    bs, D, V = wl.drafter_logits.shape
    lp, ids = drafter.batch(wl.drafter_logits.reshape(bs * D, V), wl.topk)
    return lp.reshape(bs, D, wl.topk), ids.reshape(bs, D, wl.topk)


class OracleRun:
    def __init__(self, wl):
        self.wl = wl
        self.topk_logprobs, self.topk_ids = oracle_tables(wl)
        self.trees, self.tokens, self.parents, self.depths, self.scores = tree.build_batch(
            self.topk_logprobs, self.topk_ids, wl.root_tokens, wl.qo_indptr)
        self.words = (wl.max_q_len + 31) // 32
        self.bits, self.positions, self.dense = visibility.batch(
            self.parents, self.depths, wl.qo_indptr, wl.prefix_lens, self.words)
        self.target_predict = draw_target_predict(wl.seed, self.tokens, self.parents,
                                                  wl.qo_indptr, wl.vocab)
        self.accept = accept.batch(self.tokens, self.parents, wl.qo_indptr, self.target_predict,
                                   wl.depth)

    def mask_indptr(self) -> np.ndarray:
        wl = self.wl
        q = np.diff(wl.qo_indptr).astype(np.int64)
        sizes = q * (wl.prefix_lens.astype(np.int64) + q)
        return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)

    def attention_rows(self, r: int, nodes=None):
        """fp64 oracle output [n, H, 512] and lse [n, H] for request r's nodes."""
        wl = self.wl
        a, b = int(wl.qo_indptr[r]), int(wl.qo_indptr[r + 1])
        q = wl.q_f32()[a:b]
        kv = wl.kv_rows_f32(wl.request_slots(r))
        return attention.verify_request(q, kv, int(wl.prefix_lens[r]), self.parents[a:b],
                                        float(np.float32(wl.scale)), nodes=nodes)

