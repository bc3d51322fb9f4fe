"""ddtree_tree_sample_noalloc (through the C ABI) against ddtree_tree_sample.

The allocation-free entry point runs the same kernels on the library's
static scratch, so its outputs must equal the workspace entry point's bit
for bit.  Two calls in a row, the second with a smaller input (the scratch
keeps the first call's contents, which must not matter), and a size above
the built-in limit is rejected on the host.
"""
import sys

import numpy as np
import pytest
import torch

from tree_verify_mla_amd import _lib
from tree_verify_mla_amd.step import VerifyStep
from workloads import draw_target_probs, get_config, make_workload
from workloads.device import to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _outputs(bs, D):
    return [torch.full((bs, D + 1), -7, dtype=torch.int32, device="cuda"),
            torch.full((bs,), -7, dtype=torch.int32, device="cuda"),
            torch.full((bs, D + 1), -7, dtype=torch.int32, device="cuda"),
            torch.full((bs,), -7, dtype=torch.int32, device="cuda")]


def _compare(wl, vocab, seed):
    x = to_device(wl, "cuda")
    st = VerifyStep(x)
    st.build()
    torch.cuda.synchronize()
    tok, par = st.node_tokens.cpu().numpy(), st.node_parents.cpu().numpy()
    probs = torch.from_numpy(draw_target_probs(wl.seed, tok, par, wl.qo_indptr, vocab)).cuda()
    rng = np.random.default_rng(seed)
    coins = torch.from_numpy(rng.random(wl.total_q).astype(np.float32)).cuda()
    bonus_u = torch.from_numpy(rng.random(wl.bs).astype(np.float32)).cuda()
    D = wl.depth
    ref, got = _outputs(wl.bs, D), _outputs(wl.bs, D)
    ws = torch.empty(_lib.ddtree_tree_sample_workspace_size(wl.total_q), dtype=torch.uint8,
                     device="cuda")
    _lib.ddtree_tree_sample(st.node_tokens, st.node_parents, x.qo_indptr, probs, coins, bonus_u,
                            D, *ref, workspace=ws)
    _lib.ddtree_tree_sample_noalloc(st.node_tokens, st.node_parents, x.qo_indptr, probs, coins,
                                    bonus_u, D, *got)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    return ref


def test_noalloc_matches_workspace_entry_point():
    _say("test_noalloc_matches_workspace_entry_point: headline batch, vocab 5000")
    big = make_workload(get_config(3), heads=1, pool_slots=80000)
    r1 = _compare(big, 5000, 1)
    assert int(r1[1].min()) >= 1
    _say("  second call: 3 ragged requests, vocab 700")
    small = make_workload(get_config(3), bs=3, heads=1, budgets=[0, 16, 5], prefixes=[1, 2, 3],
                          pool_slots=1000)
    _compare(small, 700, 2)


def test_noalloc_rejects_sizes_above_its_scratch():
    _say("test_noalloc_rejects_sizes_above_its_scratch")
    q = 4097
    i32 = dict(dtype=torch.int32, device="cuda")
    tok = torch.zeros(q, **i32)
    par = torch.full((q,), -1, **i32)
    qo = torch.tensor([0, q], **i32)
    probs = torch.ones(q, 4, dtype=torch.float32, device="cuda")
    coins = torch.zeros(q, dtype=torch.float32, device="cuda")
    u = torch.zeros(1, dtype=torch.float32, device="cuda")
    with pytest.raises(_lib.DDTreeError) as e:
        _lib.ddtree_tree_sample_noalloc(tok, par, qo, probs, coins, u, 7, *_outputs(1, 7))
    assert e.value.code == -2 and "4096" in str(e.value)
