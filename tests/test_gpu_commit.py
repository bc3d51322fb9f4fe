"""GPU parity of ddtree_commit_kv (through the C ABI) against ``oracle.commit``.

Bar: bit-exact -- the new slot lists, and in the move form every pool row
(the compacted rows and all others).  The HIP side commits its own tree and
accept results; the oracle commits the path its own tree and accept oracles
give on the same generated inputs (tree and accept are bit-exact, see
test_gpu_parity.py).  Covered: budget 0 (autoregressive, nothing moves),
empty and odd prefixes, trees up to 65 nodes, the headline batch, the
131k-prefix batch (17 chunks of prefix slot ids per request), an fp32 pool,
and hand-built deep paths whose compaction spans several move batches.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import commit
from tests._oracle_side import OracleRun
from tree_verify_mla_amd import _lib
from tree_verify_mla_amd.step import VerifyStep
from workloads import get_config, make_workload
from workloads.device import to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bits(pool: torch.Tensor) -> np.ndarray:
    if pool.dtype == torch.bfloat16:
        return pool.view(torch.int16).cpu().numpy().view(np.uint16)
    return pool.cpu().numpy().view(np.uint32)


def _ref_bits(wl_pool: np.ndarray) -> np.ndarray:
    return wl_pool if wl_pool.dtype == np.uint16 else wl_pool.view(np.uint32)


def _case(wl, check_all_rows=True):
    orc = OracleRun(wl)
    x = to_device(wl, "cuda", target_predict=orc.target_predict)
    st = VerifyStep(x)
    st.build()
    st.accept()
    nodes, alen, _, _ = orc.accept
    # index form
    st.commit()
    torch.cuda.synchronize()
    ref = commit.batch(wl.kv_indptr, wl.kv_indices, wl.qo_indptr, nodes, alen)
    n = int(ref.kv_indptr[-1])
    assert np.array_equal(st.new_kv_indptr.cpu().numpy(), ref.kv_indptr)
    assert np.array_equal(st.new_kv_indices.cpu().numpy()[:n], ref.kv_indices)
    index_list = st.new_kv_indices[:n].clone()
    # move form on a copy of the pool
    pool = x.kv_pool.clone()
    st.commit(kv_pool=pool)
    torch.cuda.synchronize()
    refm = commit.batch(wl.kv_indptr, wl.kv_indices, wl.qo_indptr, nodes, alen,
                        pool=_ref_bits(wl.kv_pool))
    assert np.array_equal(st.new_kv_indptr.cpu().numpy(), refm.kv_indptr)
    assert np.array_equal(st.new_kv_indices.cpu().numpy()[:n], refm.kv_indices)
    got = _bits(pool)
    if check_all_rows:
        assert np.array_equal(got, refm.pool)
    else:  # every node slot, every prefix slot, and a sample of the rest
        rng = np.random.default_rng(0)
        rows = np.unique(np.concatenate([wl.kv_indices.astype(np.int64),
                                         rng.integers(0, wl.num_slots, 4096)]))
        assert np.array_equal(got[rows], refm.pool[rows])
    # both forms' lists read the same latents
    move_list = st.new_kv_indices[:n].long()
    assert torch.equal(pool[move_list], x.kv_pool[index_list.long()])
    return alen


def test_commit_ragged_edges_bf16():
    _say("test_commit_ragged_edges_bf16")
    wl = make_workload(get_config(3), bs=6, heads=2, budgets=[0, 1, 8, 16, 64, 33],
                       prefixes=[0, 1, 31, 33, 700, 5000], pool_slots=20000)
    alen = _case(wl)
    assert alen[0] == 1          # budget 0: the root only


def test_commit_fp32_pool():
    _say("test_commit_fp32_pool")
    wl = make_workload(get_config(1), bs=4, heads=2, budgets=[0, 5, 8, 31], prefixes=[0, 2, 33, 100],
                       pool_slots=400)
    _case(wl)


def test_commit_headline_full_size():
    _say("test_commit_headline_full_size")
    _case(make_workload(get_config(3)), check_all_rows=False)


def test_commit_long_context_chunks():
    _say("test_commit_long_context_chunks")
    _case(make_workload(get_config(4)), check_all_rows=False)


def test_commit_deep_paths_multiple_move_batches():
    """Paths of up to 20 nodes with spaced node ids (n_i = 2i, 3i, ...)."""
    _say("test_commit_deep_paths_multiple_move_batches")
    rng = np.random.default_rng(5)
    D = 19
    q_lens = [1, 40, 60, 25, 20]
    p_lens = [3, 0, 9000, 17, 1]
    strides = [1, 2, 3, 1, 1]
    alens = [1, 20, 20, 13, 20]
    bs = len(q_lens)
    qo = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    kvp = np.concatenate([[0], np.cumsum(np.add(q_lens, p_lens))]).astype(np.int32)
    num_slots = int(kvp[-1]) + 500
    kvi = rng.permutation(num_slots)[:kvp[-1]].astype(np.int32)
    nodes = np.full((bs, D + 1), -1, np.int32)
    for r in range(bs):
        path = [min(i * strides[r], q_lens[r] - 1) for i in range(alens[r])]
        path = sorted(set(path))
        alens[r] = len(path)
        nodes[r, :len(path)] = path
    alen = np.array(alens, np.int32)
    pool_np = rng.integers(0, 2**16, size=(num_slots, 576), dtype=np.uint16)
    dev = "cuda"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    pool = t(pool_np.view(np.int16)).view(torch.bfloat16)
    new_p = torch.empty(bs + 1, dtype=torch.int32, device=dev)
    new_i = torch.empty(int(kvp[-1]), dtype=torch.int32, device=dev)
    for move in (False, True):
        _lib.ddtree_commit_kv(t(kvp), t(kvi), t(qo), t(nodes), t(alen), int(np.diff(kvp).max()),
                              new_p, new_i, kv_pool=pool if move else None)
        torch.cuda.synchronize()
        ref = commit.batch(kvp, kvi, qo, nodes, alen, pool=pool_np if move else None)
        n = int(ref.kv_indptr[-1])
        assert np.array_equal(new_p.cpu().numpy(), ref.kv_indptr)
        assert np.array_equal(new_i.cpu().numpy()[:n], ref.kv_indices)
        if move:
            assert np.array_equal(_bits(pool), ref.pool)
