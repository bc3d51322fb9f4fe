"""Oracle: committing the accepted path into the paged KV cache.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

Source: "The Architecture of a Speculative Decoding Engine ...",
* section "The First Attempt: Temporary Buffers and Post-Verify Compaction":
  the verify forward appends the tree nodes' latents to the request's cache,
  attention runs over prefix plus appended region, and afterwards the
  accepted latents are gathered from their scattered places in the appended
  region into contiguous positions; the cache length moves accordingly, and
  when every appended token is accepted nothing needs to move;
* section "The Off-by-One Labyrinth": the bonus token is not cached; the
  cache after the step holds the old positions plus the accepted ones;
* section "The Final Resolution: A Concrete Trace": the accepted nodes,
  root included, are what is committed, so the cache grows by accept_len;
  autoregressive decoding is the budget-0 case (accept_len 1, growth 1).

Paged form used here: request r's slot list (``kv_indices`` between
``kv_indptr[r]`` and ``kv_indptr[r+1]``) is its P_r prefix slots followed by
the slots of its Q_r tree nodes in node order (``qo_indptr``).  The accepted
path is ``accepted_nodes[r, :accept_len[r]]`` (request-local node ids, root
first), as the accept step reports it.

Two forms of the commit:

* index form -- no latent moves; the new slot list is the prefix slots
  followed by the slots of the path's nodes, in path order;
* move form (the compaction the page describes) -- the latent row of the
  path's i-th node is copied into the request's i-th node slot, every row
  read from the pool as it was before the commit; the new slot list is the
  prefix slots followed by the first accept_len node slots.

Either way, reading the new list gives the prefix latents followed by the
accepted nodes' latents in path order, and the list is accept_len entries
longer than the prefix.
"""
from __future__ import annotations

from typing import List, NamedTuple, Optional

import numpy as np


class Committed(NamedTuple):
    kv_indptr: np.ndarray         # [bs + 1] int64, starts at 0
    kv_indices: np.ndarray        # [kv_indptr[bs]] int64
    pool: Optional[np.ndarray]    # the pool after the move form, else None


def split_request(kv_indices_r: np.ndarray, q_len: int):
    """(prefix slots, node slots) of one request's slot list."""
    kv_indices_r = np.asarray(kv_indices_r)
    p = len(kv_indices_r) - q_len
    if p < 0:
        raise ValueError("slot list shorter than the request's tree")
    return kv_indices_r[:p], kv_indices_r[p:]


def commit_request(prefix_slots, node_slots, path: List[int], move: bool) -> np.ndarray:
    """New slot list of one request (index form, or move form's list)."""
    prefix_slots = [int(s) for s in prefix_slots]
    node_slots = [int(s) for s in node_slots]
    if move:
        tail = node_slots[:len(path)]
    else:
        tail = [node_slots[n] for n in path]
    return np.array(prefix_slots + tail, dtype=np.int64)


def compact_request(pool: np.ndarray, node_slots, path: List[int]) -> np.ndarray:
    """Pool after the move form for one request: row node_slots[i] receives
    the old row node_slots[path[i]], for every i on the path."""
    old = pool.copy()
    new = pool.copy()
    for i, n in enumerate(path):
        new[int(node_slots[i])] = old[int(node_slots[n])]
    return new


def batch(kv_indptr, kv_indices, qo_indptr, accepted_nodes, accept_len,
          pool: Optional[np.ndarray] = None) -> Committed:
    """The commit of a whole batch.  With ``pool`` given, the move form runs
    (requests own disjoint slots, so their moves are independent)."""
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    qo_indptr = np.asarray(qo_indptr, dtype=np.int64)
    kv_indices = np.asarray(kv_indices)
    accepted_nodes = np.asarray(accepted_nodes)
    accept_len = np.asarray(accept_len)
    bs = len(qo_indptr) - 1
    lists = []
    new_pool = None if pool is None else pool.copy()
    for r in range(bs):
        q = int(qo_indptr[r + 1] - qo_indptr[r])
        prefix, nodes = split_request(kv_indices[kv_indptr[r]:kv_indptr[r + 1]], q)
        path = [int(n) for n in accepted_nodes[r, :int(accept_len[r])]]
        lists.append(commit_request(prefix, nodes, path, move=pool is not None))
        if pool is not None:
            new_pool = compact_request(new_pool, nodes, path)
    indptr = np.zeros(bs + 1, dtype=np.int64)
    for r in range(bs):
        indptr[r + 1] = indptr[r] + len(lists[r])
    indices = np.concatenate(lists) if lists else np.zeros(0, dtype=np.int64)
    return Committed(indptr, indices.astype(np.int64), new_pool)
