"""Upload a generated workload to device tensors (layout only, no arithmetic)."""
from __future__ import annotations

import numpy as np
import torch

from .gen import Workload


def _i32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def to_device(wl: Workload, device="cuda", target_predict=None):
    """Return ``tree_verify_mla_amd.step.StepInputs`` for ``wl`` on ``device``."""
    from tree_verify_mla_amd.step import StepInputs

    if wl.dtype == "bf16":
        q = torch.from_numpy(wl.q.view(np.int16)).to(device).view(torch.bfloat16)
        pool = torch.from_numpy(wl.kv_pool.view(np.int16)).to(device).view(torch.bfloat16)
    else:
        q = torch.from_numpy(np.ascontiguousarray(wl.q, np.float32)).to(device)
        pool = torch.from_numpy(np.ascontiguousarray(wl.kv_pool, np.float32)).to(device)
    if wl.drafter_logits is not None:   # the tables are the step's own drafter stage's output
        bs, D, V = wl.drafter_logits.shape
        logits = torch.from_numpy(np.ascontiguousarray(wl.drafter_logits, np.float32)).to(device)
        lp = torch.empty(bs, D, wl.topk, dtype=torch.float32, device=device)
        ids = torch.empty(bs, D, wl.topk, dtype=torch.int32, device=device)
    else:
        logits = None
        lp = torch.from_numpy(np.ascontiguousarray(wl.topk_logprobs, np.float32)).to(device)
        ids = _i32(wl.topk_ids, device)
    return StepInputs(
        topk_logprobs=lp,
        topk_ids=ids,
        root_tokens=_i32(wl.root_tokens, device),
        qo_indptr=_i32(wl.qo_indptr, device),
        kv_indptr=_i32(wl.kv_indptr, device),
        kv_indices=_i32(wl.kv_indices, device),
        prefix_lens=_i32(wl.prefix_lens, device),
        q=q.contiguous(),
        kv_pool=pool.contiguous(),
        total_q=wl.total_q,
        max_q_len=wl.max_q_len,
        max_kv_len=wl.max_kv_len,
        max_budget=wl.max_budget,
        scale=float(np.float32(wl.scale)),
        target_predict=None if target_predict is None else _i32(target_predict, device),
        drafter_logits=logits,
    )
