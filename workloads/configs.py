"""The five verify-step workloads, by shape.

Shapes follow the pages' verify step: 576-d absorbed-MLA latents (512 c_kv +
64 rope) in a paged slot pool, 8 heads per tensor-parallel shard of a 64-head
model, draft trees grown from block_size-8 drafter output (depths 1..7) with
budget/top-k pairs of the sizes the pages sweep, and the literal softmax scale
0.14468 printed with the 9-node debug shapes ("The 30-Column Mask", section
"The Message: Tensor Shapes as Evidence").
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

LATENT = 576      # absorbed q / latent KV width: 512 c_kv + 64 k_pe
DL = 512          # c_kv width (value / output width)
DR = 64           # rope width
VOCAB = 512       # synthetic vocabulary for drafter logits
DEPTH = 7         # tree depth cap = block_size - 1 with block_size 8
SCALE = 0.14468   # softmax scale applied to the full 576-d dot product


@dataclass(frozen=True)
class Config:
    index: int                 # 1..5
    name: str
    bs: int
    heads: int
    topk: int
    dtype: str                 # "f32" or "bf16"
    budget: Optional[int]      # fixed budget (q_len = budget + 1); None -> ragged
    prefix: Optional[int]      # fixed prefix length; None -> ragged
    pool_slots: Optional[int]  # None -> ceil(1.25 * sum(P_r + Q_r))
    budget_choices: tuple = ()
    prefix_range: tuple = ()   # inclusive (lo, hi) for a uniform integer draw
    depth: int = DEPTH
    vocab: int = VOCAB
    scale: float = SCALE
    # "logits": the drafter's raw per-depth logits N(0, 1) over the vocabulary
    # (its log-softmax top-k is a stage of the method); "tables": per-depth
    # top-k log-prob tables drawn directly
    drafter: str = "tables"

    @property
    def seed(self) -> int:
        return 1000 + self.index


CONFIGS = {
    1: Config(1, "tiny_fp32_q9_p21", bs=1, heads=8, topk=4, dtype="f32",
              budget=8, prefix=21, pool_slots=64, drafter="logits"),
    2: Config(2, "shard8_bf16_q33_p4096", bs=1, heads=8, topk=8, dtype="bf16",
              budget=32, prefix=4096, pool_slots=200_000),
    3: Config(3, "h64_bs8_q33_p8192", bs=8, heads=64, topk=8, dtype="bf16",
              budget=32, prefix=8192, pool_slots=300_000),
    4: Config(4, "long_h64_q65_p131072", bs=1, heads=64, topk=16, dtype="bf16",
              budget=64, prefix=131072, pool_slots=262_144),
    5: Config(5, "ragged_bs32_h64", bs=32, heads=64, topk=8, dtype="bf16",
              budget=None, prefix=None, pool_slots=None,
              budget_choices=(16, 32, 64), prefix_range=(1024, 32768)),
}


def get_config(i: int) -> Config:
    return CONFIGS[int(i)]
