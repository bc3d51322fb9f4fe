"""GPU parity of ddtree_tree_sample (through the C ABI) against ``oracle.sample``.

Bar: bit-exact (accepted path, accept length, commit tokens, bonus).  Both
sides take every decision in fp32 with the same fixed order of sums, so the
integers agree exactly.  The HIP side samples along its own tree
(ddtree_build_tree), the oracle along its own (bit-exact, see
test_gpu_parity.py); target rows, coins and bonus uniforms come from the
seeded generator.  Covered: budget 0 (root only: the bonus is a plain draw
from the root's row), ragged trees up to 65 nodes, the headline batch, a
vocabulary whose blocks are ragged (5000 = 256 x 20 - 120), a vocabulary of
163,840 tokens, several uniform draws per workload, and a zero row (every
token rejected: no mass left, bonus -1), blocks wider than one staging
tile (vocabulary 1,279,983: 5000 tokens a block, staged one at a time),
a vocabulary that leaves most blocks empty (513), and a caller-provided workspace reused across
calls.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import sample
from tests._oracle_side import OracleRun
from tree_verify_mla_amd import _lib
from tree_verify_mla_amd.step import VerifyStep
from workloads import draw_target_probs, get_config, make_workload
from workloads.device import to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(wl, vocab, draws=3, zero_root_of=None, workspace=False):
    orc = OracleRun(wl)
    x = to_device(wl, "cuda")
    st = VerifyStep(x)
    st.build()
    torch.cuda.synchronize()
    probs = draw_target_probs(wl.seed, orc.tokens, orc.parents, wl.qo_indptr, vocab)
    if zero_root_of is not None:   # a request whose root row has mass only on drafted tokens
        a = int(wl.qo_indptr[zero_root_of])
        kids = [int(orc.tokens[a + c]) for c in range(1, int(wl.qo_indptr[zero_root_of + 1]) - a)
                if orc.parents[a + c] == 0]
        probs[a] = 0.0
        probs[a, kids] = 1.0 / max(len(kids), 1)
    probs_d = torch.from_numpy(probs).cuda()
    D = wl.depth
    bs = wl.bs
    rng = np.random.default_rng(wl.seed + 99)
    out = [torch.empty(bs, D + 1, dtype=torch.int32, device="cuda"),
           torch.empty(bs, dtype=torch.int32, device="cuda"),
           torch.empty(bs, D + 1, dtype=torch.int32, device="cuda"),
           torch.empty(bs, dtype=torch.int32, device="cuda")]
    ws = None
    if workspace:   # stale contents must not matter
        ws = torch.full((_lib.ddtree_tree_sample_workspace_size(wl.total_q),), 0x7F,
                        dtype=torch.uint8, device="cuda")
    for d in range(draws):
        coins = rng.random(wl.total_q).astype(np.float32)
        bonus_u = rng.random(bs).astype(np.float32)
        _lib.ddtree_tree_sample(st.node_tokens, st.node_parents, x.qo_indptr, probs_d,
                                torch.from_numpy(coins).cuda(), torch.from_numpy(bonus_u).cuda(),
                                D, *out, workspace=ws)
        torch.cuda.synchronize()
        ref = sample.batch(orc.tokens, orc.parents, wl.qo_indptr, probs, coins, bonus_u, D)
        for got, want in zip(out, ref):
            assert np.array_equal(got.cpu().numpy(), want), d
    return ref


def test_sample_ragged_trees():
    _say("test_sample_ragged_trees")
    wl = make_workload(get_config(3), bs=6, heads=1, budgets=[0, 1, 8, 16, 64, 33],
                       prefixes=[0, 1, 31, 33, 700, 5000], pool_slots=20000)
    ref = _case(wl, 512, draws=4)
    assert ref[1][0] == 1            # budget 0: root only


def test_sample_headline_batch_and_ragged_blocks():
    _say("test_sample_headline_batch_and_ragged_blocks")
    wl = make_workload(get_config(3), heads=1, pool_slots=80000)
    _case(wl, 512, draws=3)
    _case(wl, 5000, draws=2)


def test_sample_large_vocabulary():
    _say("test_sample_large_vocabulary")
    wl = make_workload(get_config(3), bs=2, heads=1, budgets=[32, 16], prefixes=[10, 20],
                       pool_slots=1000)
    _case(wl, 163840, draws=2)


def test_sample_all_mass_on_rejected_tokens():
    _say("test_sample_all_mass_on_rejected_tokens")
    wl = make_workload(get_config(3), bs=3, heads=1, budgets=[8, 8, 8], prefixes=[5, 5, 5],
                       pool_slots=1000)
    _case(wl, 512, draws=6, zero_root_of=1)


def test_sample_wide_and_empty_blocks():
    _say("test_sample_wide_and_empty_blocks")
    wl = make_workload(get_config(3), bs=2, heads=1, budgets=[8, 4], prefixes=[3, 4],
                       pool_slots=1000)
    _case(wl, 256 * 5000 - 17, draws=2, workspace=True)
    _case(wl, 513, draws=3, workspace=True)   # 3 tokens a block, 171 blocks in use
