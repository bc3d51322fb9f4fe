"""ddtree_validate_inputs (through the C ABI) on crafted inputs.

Only the validator runs on these arrays: they are exactly the kinds of
broken marshalling the checker exists for ("The 30-Column Mask ...",
sections "The Fix: Building Combined Indices" and "Mistakes and Incorrect
Assumptions"; "The Mask Bug That Changed Everything ...", section "The
Context: A Cascade of Infrastructure and Algorithm Challenges"), and no
other kernel is given them.  Each case states the expected count and first
offending index of every check; a well-formed step reports nothing.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import tree
from tree_verify_mla_amd import _lib
from workloads import get_config, make_workload

pytestmark = pytest.mark.gpu

NAMES = _lib.CHECK_NAMES


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _validate(qo, total_q, kvp, kvi, num_slots, prefix_lens=None, parents=None):
    rep = torch.full((2 * _lib.DDTREE_NUM_CHECKS,), 12345, dtype=torch.int32, device="cuda")
    _lib.ddtree_validate_inputs(_i32(qo), total_q, _i32(kvp), _i32(kvi), num_slots, rep,
                                prefix_lens=None if prefix_lens is None else _i32(prefix_lens),
                                node_parents=None if parents is None else _i32(parents))
    torch.cuda.synchronize()
    r = rep.cpu().numpy()
    return {NAMES[k]: (int(r[2 * k]), int(r[2 * k + 1])) for k in range(len(NAMES))}


def _clean():
    return {n: (0, -1) for n in NAMES}


@pytest.fixture(scope="module")
def step():
    wl = make_workload(get_config(3), bs=4, heads=1, budgets=[32, 8, 0, 16],
                       prefixes=[21, 0, 40, 7], pool_slots=500)
    _, _, parents, _, _ = tree.build_batch(wl.topk_logprobs, wl.topk_ids, wl.root_tokens,
                                           wl.qo_indptr)
    return wl, parents


def test_well_formed_step_reports_nothing(step):
    _say("test_well_formed_step_reports_nothing")
    wl, par = step
    got = _validate(wl.qo_indptr, wl.total_q, wl.kv_indptr, wl.kv_indices, wl.num_slots,
                    wl.prefix_lens, par)
    assert got == _clean()


def test_prefix_only_kv_list(step):
    """The index list holds the prefix slots only (the tree nodes' own slots
    were left out): every request with nodes has P_r columns, not P_r + Q_r."""
    _say("test_prefix_only_kv_list")
    wl, par = step
    kvp = np.concatenate([[0], np.cumsum(wl.prefix_lens)]).astype(np.int32)
    kvi = np.concatenate([wl.request_slots(r)[:wl.prefix_lens[r]] for r in range(wl.bs)])
    got = _validate(wl.qo_indptr, wl.total_q, kvp, kvi, wl.num_slots, wl.prefix_lens, par)
    want = _clean()
    want["KV_LEN"] = (wl.bs, 0)
    assert got == want


def test_qo_offsets_from_block_size(step):
    """qo_indptr stepped by the drafter block size (8) instead of budget + 1."""
    _say("test_qo_offsets_from_block_size")
    wl, par = step
    qo = (np.arange(wl.bs + 1) * 8).astype(np.int32)
    got = _validate(qo, wl.total_q, wl.kv_indptr, wl.kv_indices, wl.num_slots, wl.prefix_lens)
    # Q_r = 8 for all; request 0 has N = 21 + 33 != 21 + 8, request 1: 9 != 8,
    # request 2: 41 != 48, request 3: 24 != 15
    assert got["KV_LEN"] == (4, 0)
    assert got["QO_INDPTR"] == (0, -1)


def test_slots_outside_the_pool_and_bad_offsets(step):
    _say("test_slots_outside_the_pool_and_bad_offsets")
    wl, par = step
    kvi = wl.kv_indices.copy()
    kvi[17] = wl.num_slots        # one past the end
    kvi[5] = -1
    kvp = wl.kv_indptr.copy()
    kvp[2] = kvp[3] + 1           # request 1 ends after request 2 starts... and goes backwards
    got = _validate(wl.qo_indptr, wl.total_q, kvp, kvi, wl.num_slots)
    assert got["KV_INDEX"] == (2, 5)
    assert got["KV_INDPTR"] == (1, 2)     # request 2: kv[3] < kv[2]
    assert got["KV_LEN"][0] >= 1
    qo = wl.qo_indptr.copy()
    qo[-1] = wl.total_q + 5       # past the node arrays
    got = _validate(qo, wl.total_q, wl.kv_indptr, wl.kv_indices, wl.num_slots, parents=par)
    assert got["QO_INDPTR"] == (1, wl.bs - 1)


def test_bad_parents(step):
    _say("test_bad_parents")
    wl, par = step
    p = par.copy()
    a = int(wl.qo_indptr[0])
    p[a + 5] = 5                  # a node its own parent
    p[a + 9] = 30                 # a later node as parent
    b = int(wl.qo_indptr[3])
    p[b] = 0                      # a root with a parent
    got = _validate(wl.qo_indptr, wl.total_q, wl.kv_indptr, wl.kv_indices, wl.num_slots,
                    wl.prefix_lens, p)
    want = _clean()
    want["PARENT"] = (3, a + 5)
    assert got == want


def test_empty_batch():
    _say("test_empty_batch")
    got = _validate(np.zeros(1), 0, np.zeros(1), np.zeros(0), 10)
    assert got == _clean()
