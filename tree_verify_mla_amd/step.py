"""One DDTree verify step on device tensors: build + visibility -> attention -> accept
(-> commit of the accepted paths into the KV slot lists).

``VerifyStep`` owns the output and workspace tensors (torch allocations, made
once) and enqueues the four library calls on the current stream with no host
synchronisation, so a step can be timed with events or captured in a graph.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib

LATENT = 576
DV = 512


@dataclass
class StepInputs:
    """Device tensors and host-known sizes of one batch (request order = index order)."""
    topk_logprobs: torch.Tensor   # [bs, D, K] f32
    topk_ids: torch.Tensor        # [bs, D, K] i32
    root_tokens: torch.Tensor     # [bs] i32
    qo_indptr: torch.Tensor       # [bs+1] i32
    kv_indptr: torch.Tensor       # [bs+1] i32
    kv_indices: torch.Tensor      # [sum(P_r+Q_r)] i32
    prefix_lens: torch.Tensor     # [bs] i32
    q: torch.Tensor               # [total_q, H, 576] bf16 | f32
    kv_pool: torch.Tensor         # [num_slots, 576] bf16 | f32
    total_q: int
    max_q_len: int
    max_kv_len: int
    max_budget: int
    scale: float
    target_predict: Optional[torch.Tensor] = None  # [total_q] i32
    # [bs, D, V] f32 drafter logits: when given, the step's drafter stage
    # (ddtree_drafter_topk) writes topk_logprobs / topk_ids from them
    drafter_logits: Optional[torch.Tensor] = None

    @property
    def bs(self) -> int:
        return self.qo_indptr.numel() - 1

    @property
    def heads(self) -> int:
        return self.q.shape[1]

    @property
    def depth(self) -> int:
        return self.topk_logprobs.shape[1]


class VerifyStep:
    def __init__(self, x: StepInputs, num_splits: int = 0, want_lse: bool = True,
                 want_positions: bool = True):
        dev = x.q.device
        i32 = dict(dtype=torch.int32, device=dev)
        self.x = x
        self.num_splits = int(num_splits)
        self.words = (x.max_q_len + 31) // 32
        self.node_tokens = torch.empty(x.total_q, **i32)
        self.node_parents = torch.empty(x.total_q, **i32)
        self.node_depths = torch.empty(x.total_q, **i32)
        self.node_scores = torch.empty(x.total_q, dtype=torch.float32, device=dev)
        self.vis_bits = torch.empty(x.total_q, self.words, **i32)
        self.positions = torch.empty(x.total_q, dtype=torch.int64, device=dev) if want_positions else None
        self.out = torch.empty(x.total_q, x.heads, DV, dtype=x.q.dtype, device=dev)
        self.lse = torch.empty(x.total_q, x.heads, dtype=torch.float32, device=dev) if want_lse else None
        dt = _lib.DDTREE_BF16 if x.q.dtype == torch.bfloat16 else _lib.DDTREE_F32
        ws = _lib.ddtree_verify_attn_workspace_size(x.bs, x.heads, x.max_q_len, x.max_kv_len,
                                                    self.num_splits, dt)
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
        D = x.depth
        self.accepted_nodes = torch.empty(x.bs, D + 1, **i32)
        self.accept_len = torch.empty(x.bs, **i32)
        self.commit_tokens = torch.empty(x.bs, D + 1, **i32)
        self.bonus_tokens = torch.empty(x.bs, **i32)
        self.drafter_ws = None
        if x.drafter_logits is not None:
            rows = x.drafter_logits.shape[0] * x.drafter_logits.shape[1]
            self.drafter_ws = torch.empty(max(1, _lib.ddtree_drafter_topk_workspace_size(
                rows, x.drafter_logits.shape[2], x.topk_logprobs.shape[2])), dtype=torch.uint8,
                device=dev)
        # the committed slot lists (never longer than the verify lists)
        self.new_kv_indptr = torch.empty(x.bs + 1, **i32)
        self.new_kv_indices = torch.empty(max(x.kv_indices.numel(), 1), **i32)

    def drafter(self, stream=None):
        """Per-depth top-k log-probs of the drafter logits (when the inputs
        carry logits; otherwise the tables are inputs and this does nothing)."""
        x = self.x
        if x.drafter_logits is None:
            return
        bs, D, V = x.drafter_logits.shape
        K = x.topk_logprobs.shape[2]
        _lib.ddtree_drafter_topk(x.drafter_logits.view(bs * D, V), x.topk_logprobs.view(bs * D, K),
                                 x.topk_ids.view(bs * D, K), workspace=self.drafter_ws,
                                 stream=stream)

    def build(self, stream=None):
        """The draft trees (after the drafter stage, when the inputs carry logits)."""
        x = self.x
        self.drafter(stream)
        _lib.ddtree_build_tree(x.topk_logprobs, x.topk_ids, x.root_tokens, x.qo_indptr,
                               x.max_budget, self.node_tokens, self.node_parents,
                               self.node_depths, self.node_scores, stream=stream)

    def visibility(self, stream=None):
        x = self.x
        _lib.ddtree_compile_visibility(self.node_parents, self.node_depths, x.qo_indptr,
                                       x.prefix_lens, x.max_q_len, self.vis_bits,
                                       positions=self.positions, stream=stream)

    def build_visibility(self, stream=None):
        """build + visibility in one library call (one launch for trees up to
        64 draft nodes), after the drafter stage when the inputs carry logits."""
        x = self.x
        self.drafter(stream)
        _lib.ddtree_build_tree_visibility(x.topk_logprobs, x.topk_ids, x.root_tokens, x.qo_indptr,
                                          x.prefix_lens, x.max_budget, x.max_q_len,
                                          self.node_tokens, self.node_parents, self.node_depths,
                                          self.vis_bits, node_scores=self.node_scores,
                                          positions=self.positions, stream=stream)

    def attention(self, stream=None):
        x = self.x
        _lib.ddtree_verify_attn(x.q, x.kv_pool, x.kv_indptr, x.kv_indices, x.qo_indptr,
                                self.vis_bits, x.max_q_len, x.max_kv_len, x.scale, self.out,
                                lse=self.lse, num_splits=self.num_splits,
                                workspace=self.workspace, stream=stream)

    def accept(self, target_predict=None, stream=None):
        x = self.x
        tp = x.target_predict if target_predict is None else target_predict
        _lib.ddtree_accept(self.node_tokens, self.node_parents, x.qo_indptr, tp, x.depth,
                           self.accepted_nodes, self.accept_len, self.commit_tokens,
                           self.bonus_tokens, stream=stream)

    def commit(self, kv_pool=None, stream=None):
        """Commit the accepted paths into new slot lists: index form, or with
        ``kv_pool`` the move form (accepted rows compacted in that pool, in place)."""
        x = self.x
        _lib.ddtree_commit_kv(x.kv_indptr, x.kv_indices, x.qo_indptr, self.accepted_nodes,
                              self.accept_len, x.max_kv_len, self.new_kv_indptr,
                              self.new_kv_indices, kv_pool=kv_pool, stream=stream)

    def run(self, stream=None):
        """All four stages (accept needs ``target_predict`` in the inputs)."""
        self.build_visibility(stream)
        self.attention(stream)
        self.accept(stream=stream)
