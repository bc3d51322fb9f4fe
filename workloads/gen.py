"""Seeded input generator shared by the oracle tests, the GPU tests and the bench.

Recipe (one ``numpy.random.default_rng(seed)`` stream, drawn in this order):

1. ragged configs only: per-request prefix lengths ``P_r ~ U{lo..hi}``, then
   per-request budgets ``B_r`` uniform over the allowed choices;
2. per request r, in request order: the drafter's output -- for configs
   whose drafter is "logits", raw per-depth logits ``N(0, 1)[depth, vocab]``
   drawn as fp32 (their log-softmax top-k is a stage of the method); for the
   others the per-depth top-``k`` table drawn directly
   (``draw_drafter_topk``: a first log-probability ``-(3 + Exp(1))``, then
   ``Exp(0.3)`` gaps, rounded to fp32; distinct token ids uniform over the
   vocabulary); then the root token ``U[0, vocab)``;
3. one permutation of the slot pool: the first ``sum(P_r + Q_r)`` slots are
   dealt out request by request, ``P_r`` prefix slots then ``Q_r`` node slots
   (so ``kv_indices`` is the combined prefix ++ tree-node slot list);
4. q ``[total_q, H, 576]`` ~ N(0, 0.5^2) drawn as fp32;
5. the used latent rows ``[sum(P_r + Q_r), 576]`` ~ N(0, 0.5^2) drawn as fp32,
   in ``kv_indices`` order, written into the pool at their slots.

bf16 workloads round q and the latent rows to bf16 with round-to-nearest-even
and keep them as raw uint16 bit patterns.  Pool rows no request uses are NaN
by default, so a stray read shows up in the output.

The top-k tables are drawn, not computed: log-softmax and top-k selection
over logits are a stage of the method (``ddtree_drafter_topk``), whose
inputs are raw logits (``draw_drafter_logits``).  The module contains no
log-softmax, selection, tree search, mask, attention or acceptance.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

from .configs import LATENT, Config


# ----------------------------------------------------------------------------
# bf16 bit helpers (storage format only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even), returned as uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    bits = ((u + r) >> 16).astype(np.uint16)
    if nan.any():
        bits = np.where(nan, np.uint16(0x7FC0), bits)
    return bits


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
@dataclass
class Workload:
    name: str
    seed: int
    bs: int
    heads: int
    depth: int
    topk: int
    vocab: int
    scale: float
    dtype: str                       # "f32" | "bf16"
    budgets: np.ndarray              # [bs] int64
    prefix_lens: np.ndarray          # [bs] int32
    qo_indptr: np.ndarray            # [bs+1] int32
    kv_indptr: np.ndarray            # [bs+1] int32
    topk_logprobs: Optional[np.ndarray]  # [bs, depth, topk] float32 (None: from drafter_logits)
    topk_ids: Optional[np.ndarray]       # [bs, depth, topk] int32 (None: from drafter_logits)
    root_tokens: np.ndarray          # [bs] int32
    kv_indices: np.ndarray           # [sum(P_r+Q_r)] int32
    q: np.ndarray                    # [total_q, H, 576] float32 or uint16 bf16 bits
    kv_pool: np.ndarray              # [num_slots, 576] float32 or uint16 bf16 bits
    extra: dict = field(default_factory=dict)
    drafter_logits: Optional[np.ndarray] = None  # [bs, depth, vocab] float32 raw logits

    # -- derived sizes ------------------------------------------------------
    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.qo_indptr)

    @property
    def total_q(self) -> int:
        return int(self.qo_indptr[-1])

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.bs else 0

    @property
    def max_kv_len(self) -> int:
        return int(np.diff(self.kv_indptr).max()) if self.bs else 0

    @property
    def max_budget(self) -> int:
        return int(self.budgets.max()) if self.bs else 0

    @property
    def num_slots(self) -> int:
        return int(self.kv_pool.shape[0])

    # -- value views (exact) ------------------------------------------------
    def q_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.q) if self.dtype == "bf16" else self.q

    def kv_rows_f32(self, slots: np.ndarray) -> np.ndarray:
        rows = self.kv_pool[np.asarray(slots, dtype=np.int64)]
        return bf16_bits_to_f32(rows) if self.dtype == "bf16" else rows

    def request_slots(self, r: int) -> np.ndarray:
        return self.kv_indices[self.kv_indptr[r]:self.kv_indptr[r + 1]]


def draw_drafter_topk(rng: np.random.Generator, depth: int, topk: int, vocab: int):
    """Per-depth top-k tables shaped like a drafter's, drawn directly: the
    first log-probability is -(3 + Exp(1)), each next one lower by an Exp(0.3)
    gap (non-increasing after rounding to fp32), and the token ids are
    distinct, uniform over the vocabulary.  No softmax and no selection: those
    are a stage of the method (ddtree_drafter_topk), whose inputs are the raw
    logits of draw_drafter_logits."""
    first = -(3.0 + rng.exponential(1.0, size=(depth, 1)))
    gaps = rng.exponential(0.3, size=(depth, topk - 1))
    vals = np.concatenate([first, first - np.cumsum(gaps, axis=1)], axis=1).astype(np.float32)
    ids = np.stack([rng.choice(vocab, size=topk, replace=False) for _ in range(depth)])
    return vals, ids.astype(np.int32)


def draw_target_probs(seed: int, node_tokens: np.ndarray, node_parents: np.ndarray,
                      qo_indptr: np.ndarray, vocab: int, p_child: float = 0.7) -> np.ndarray:
    """Synthetic target distributions [total_q, vocab] fp32 for stochastic
    acceptance: each node's row is a Dirichlet(0.3) spread over the
    vocabulary; with probability p_child a share U(0.3, 0.9) of its mass is
    moved onto the token of one of its children (chosen uniformly), so that
    walks go deep.  Drawn, not computed from logits."""
    rng = np.random.default_rng(int(seed) + 0xACCE)
    total = int(qo_indptr[-1])
    out = np.zeros((total, vocab), np.float32)
    for r in range(len(qo_indptr) - 1):
        a, b = int(qo_indptr[r]), int(qo_indptr[r + 1])
        par = np.asarray(node_parents[a:b])
        for i in range(b - a):
            row = rng.dirichlet(np.full(vocab, 0.3))
            kids = np.nonzero(par == i)[0]
            if len(kids) and rng.random() < p_child:
                w = rng.uniform(0.3, 0.9)
                row = row * (1.0 - w)
                row[int(node_tokens[a + int(kids[rng.integers(0, len(kids))])])] += w
            out[a + i] = row.astype(np.float32)
    return out


def draw_drafter_logits(rng: np.random.Generator, rows: int, vocab: int, std: float = 2.0,
                        dtype: str = "f32") -> np.ndarray:
    """Raw drafter logits N(0, std) [rows, vocab]: fp32, or bf16 bits (RNE)."""
    x = (rng.standard_normal((rows, vocab)) * std).astype(np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def make_workload(cfg: Config, *, seed: Optional[int] = None, unused: str = "nan",
                  bs: Optional[int] = None, heads: Optional[int] = None,
                  topk: Optional[int] = None, depth: Optional[int] = None,
                  budgets: Optional[Sequence[int]] = None,
                  prefixes: Optional[Sequence[int]] = None,
                  pool_slots: Optional[int] = None, dtype: Optional[str] = None,
                  q_std: float = 0.5, kv_std: float = 0.5,
                  drafter: Optional[str] = None) -> Workload:
    """Draw one seeded workload for ``cfg``; keyword overrides shrink or reshape it
    (``drafter``: "logits" or "tables", see ``Config.drafter``)."""
    seed = cfg.seed if seed is None else int(seed)
    rng = np.random.default_rng(seed)
    bs = cfg.bs if bs is None else int(bs)
    H = cfg.heads if heads is None else int(heads)
    K = cfg.topk if topk is None else int(topk)
    D = cfg.depth if depth is None else int(depth)
    dtype = cfg.dtype if dtype is None else dtype
    V = cfg.vocab

    # 1. per-request lengths
    if prefixes is None and cfg.prefix is None:
        lo, hi = cfg.prefix_range
        P = rng.integers(lo, hi + 1, size=bs)
    elif prefixes is None:
        P = np.full(bs, cfg.prefix, dtype=np.int64)
    else:
        P = np.asarray(prefixes, dtype=np.int64)
    if budgets is None and cfg.budget is None:
        B = rng.choice(np.asarray(cfg.budget_choices), size=bs)
    elif budgets is None:
        B = np.full(bs, cfg.budget, dtype=np.int64)
    else:
        B = np.asarray(budgets, dtype=np.int64)
    assert P.shape == (bs,) and B.shape == (bs,)
    Q = B + 1

    # 2. drafter output (raw logits, or top-k tables) and root tokens
    drafter = cfg.drafter if drafter is None else drafter
    if drafter not in ("logits", "tables"):
        raise ValueError(drafter)
    lps = ids = logits = None
    if drafter == "logits":
        logits = np.zeros((bs, D, V), np.float32)
    else:
        lps = np.zeros((bs, D, K), np.float32)
        ids = np.zeros((bs, D, K), np.int32)
    roots = np.zeros(bs, np.int32)
    for r in range(bs):
        if drafter == "logits":
            logits[r] = rng.standard_normal((D, V), dtype=np.float32)
        else:
            lps[r], ids[r] = draw_drafter_topk(rng, D, K, V)
        roots[r] = rng.integers(0, V)

    qo_indptr = np.zeros(bs + 1, np.int32)
    qo_indptr[1:] = np.cumsum(Q)
    kv_indptr = np.zeros(bs + 1, np.int32)
    kv_indptr[1:] = np.cumsum(P + Q)
    n_used = int(kv_indptr[-1])
    total_q = int(qo_indptr[-1])

    if pool_slots is None:
        pool_slots = cfg.pool_slots if cfg.pool_slots is not None else int(np.ceil(1.25 * n_used))
    if pool_slots < n_used:
        raise ValueError(f"pool of {pool_slots} slots cannot hold {n_used} rows")

    # 3. slots
    kv_indices = rng.permutation(pool_slots)[:n_used].astype(np.int32)

    # 4. queries, 5. latent rows
    q = rng.standard_normal((total_q, H, LATENT), dtype=np.float32) * np.float32(q_std)
    rows = rng.standard_normal((n_used, LATENT), dtype=np.float32) * np.float32(kv_std)

    fill = np.nan if unused == "nan" else 0.0
    if dtype == "bf16":
        q = f32_to_bf16_bits(q)
        pool = np.full((pool_slots, LATENT), f32_to_bf16_bits(np.float32([fill]))[0], np.uint16)
        pool[kv_indices] = f32_to_bf16_bits(rows)
    elif dtype == "f32":
        pool = np.full((pool_slots, LATENT), fill, np.float32)
        pool[kv_indices] = rows
    else:
        raise ValueError(dtype)

    return Workload(name=cfg.name, seed=seed, bs=bs, heads=H, depth=D, topk=K, vocab=V,
                    scale=cfg.scale, dtype=dtype, budgets=B.astype(np.int64),
                    prefix_lens=P.astype(np.int32), qo_indptr=qo_indptr, kv_indptr=kv_indptr,
                    topk_logprobs=lps, topk_ids=ids, root_tokens=roots, kv_indices=kv_indices,
                    q=q, kv_pool=pool, drafter_logits=logits)


def draw_target_predict(seed: int, node_tokens: np.ndarray, node_parents: np.ndarray,
                        qo_indptr: np.ndarray, vocab: int, p_child: float = 0.8) -> np.ndarray:
    """Synthetic target argmax per tree node.

    With probability ``p_child`` a node's prediction is the token of one of its
    children chosen uniformly (so acceptance can proceed), otherwise a uniform
    vocabulary draw.  Uses its own stream ``default_rng([seed, 7])``; three
    draws per node in node order, whatever the branch, so the stream layout
    does not depend on the tree.
    """
    rng = np.random.default_rng([int(seed), 7])
    node_tokens = np.asarray(node_tokens)
    node_parents = np.asarray(node_parents)
    out = np.zeros(len(node_tokens), np.int32)
    bs = len(qo_indptr) - 1
    for r in range(bs):
        a, b = int(qo_indptr[r]), int(qo_indptr[r + 1])
        par = node_parents[a:b]
        tok = node_tokens[a:b]
        children = [[] for _ in range(b - a)]
        for j in range(1, b - a):
            p = int(par[j])
            if 0 <= p < b - a:
                children[p].append(j)
        for i in range(b - a):
            u = rng.random()
            c = int(rng.integers(0, max(1, len(children[i]))))
            t = int(rng.integers(0, vocab))
            out[a + i] = int(tok[children[i][c]]) if (children[i] and u < p_child) else t
    return out


def sensitize_tree_columns(wl: Workload, c: float = 9.0) -> Workload:
    """Twin of ``wl`` in which every visible tree column carries a large score.

    Rope dimension 0 (column 512) is set to ``c`` in every query row and in
    every tree-node latent row, and to 0 in every prefix row, which adds
    ``scale * c * c`` (about 11.7 for c = 9) to each query-to-tree-node score.
    Over long prefixes the tree columns then hold a large share of the softmax
    mass, so a wrong tree mask moves the output far beyond the parity
    tolerance.  ``c`` and 0 are exact in bf16.  Returns a new workload.
    """
    import copy
    out = copy.copy(wl)
    q = wl.q.copy()
    pool = wl.kv_pool.copy()
    if wl.dtype == "bf16":
        cv, zv = f32_to_bf16_bits(np.float32([c, 0.0]))
    else:
        cv, zv = np.float32(c), np.float32(0.0)
    q[:, :, 512] = cv
    for r in range(wl.bs):
        slots = wl.request_slots(r)
        P = int(wl.prefix_lens[r])
        pool[slots[:P], 512] = zv
        pool[slots[P:], 512] = cv
    out.q, out.kv_pool = q, pool
    out.name = wl.name + "+sensitized"
    return out


def draw_layer(wl: Workload, layer: int, q_std: float = 0.5, kv_std: float = 0.5) -> Workload:
    """The same step for another layer: tree inputs, lengths, slot lists and
    pool size unchanged; fresh seeded queries and latent rows (same
    distributions as make_workload) in the same slots; unused rows keep the
    fill of ``wl``'s pool."""
    import dataclasses

    rng = np.random.default_rng([int(wl.seed), 1000 + int(layer)])
    n_used = len(wl.kv_indices)
    q = rng.standard_normal(wl.q.shape, dtype=np.float32) * np.float32(q_std)
    rows = rng.standard_normal((n_used, LATENT), dtype=np.float32) * np.float32(kv_std)
    pool = wl.kv_pool.copy()
    if wl.dtype == "bf16":
        q = f32_to_bf16_bits(q)
        pool[wl.kv_indices] = f32_to_bf16_bits(rows)
    else:
        pool[wl.kv_indices] = rows
    return dataclasses.replace(wl, q=q, kv_pool=pool)
