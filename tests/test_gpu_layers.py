"""GPU parity of ddtree_verify_attn_layers (one launch over L layers).

Bars: each layer of the layered call equals the single-layer
ddtree_verify_attn call on that layer's inputs bit for bit (same kernels,
same schedule, same arithmetic), and the oracle's per-layer result within
the single-layer tolerances (1e-2 * max|out| bf16, 1e-5 fp32).  Covered:
bf16 persistent and forced splits (lane-layout and row merges), fp32 with
and without split, a pool shared by every layer (stride 0), no lse, the
8-head shard at full size, L = 1, and the 64-head batch whose layers
get one launch each.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import attention
from tests._oracle_side import OracleRun
from tree_verify_mla_amd import _lib
from tree_verify_mla_amd.step import VerifyStep
from workloads import draw_layer, get_config, make_workload
from workloads.device import to_device

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f32": 1e-5}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _layered(wl0, L, num_splits=0, shared_pool=False, with_lse=True, oracle_check=True):
    wls = [wl0] + [draw_layer(wl0, l) for l in range(1, L)]
    if shared_pool:
        import dataclasses
        wls = [dataclasses.replace(w, kv_pool=wl0.kv_pool) for w in wls]
    xs = [to_device(w, "cuda") for w in wls]
    st = VerifyStep(xs[0], num_splits=num_splits)
    st.build()
    st.visibility()
    torch.cuda.synchronize()
    x0 = xs[0]
    q = torch.stack([x.q for x in xs]).contiguous()
    pool = x0.kv_pool.unsqueeze(0) if shared_pool else torch.stack([x.kv_pool for x in xs]).contiguous()
    total_q, H = x0.q.shape[0], x0.q.shape[1]
    out = torch.empty(L, total_q, H, 512, dtype=x0.q.dtype, device="cuda")
    lse = torch.empty(L, total_q, H, dtype=torch.float32, device="cuda") if with_lse else None
    dt = _lib.DDTREE_BF16 if x0.q.dtype == torch.bfloat16 else _lib.DDTREE_F32
    ws = torch.empty(max(1, _lib.ddtree_verify_attn_layers_workspace_size(
        L, wl0.bs, H, wl0.max_q_len, wl0.max_kv_len, num_splits, dt)), dtype=torch.uint8, device="cuda")
    _lib.ddtree_verify_attn_layers(q, pool, x0.kv_indptr, x0.kv_indices, x0.qo_indptr, st.vis_bits,
                                   wl0.max_q_len, wl0.max_kv_len, float(np.float32(wl0.scale)), out,
                                   lse, num_splits=num_splits, workspace=ws)
    torch.cuda.synchronize()
    # each layer against the single-layer call: bit-exact
    for l in range(L):
        o1 = torch.empty_like(out[l])
        l1 = torch.empty_like(lse[l]) if with_lse else None
        ws1 = torch.empty(max(1, _lib.ddtree_verify_attn_workspace_size(
            wl0.bs, H, wl0.max_q_len, wl0.max_kv_len, num_splits, dt)), dtype=torch.uint8, device="cuda")
        _lib.ddtree_verify_attn(xs[l].q, pool[0] if shared_pool else pool[l], x0.kv_indptr,
                                x0.kv_indices, x0.qo_indptr, st.vis_bits, wl0.max_q_len,
                                wl0.max_kv_len, float(np.float32(wl0.scale)), o1, l1,
                                num_splits=num_splits, workspace=ws1)
        torch.cuda.synchronize()
        assert torch.equal(out[l].view(torch.int16) if dt == _lib.DDTREE_BF16 else out[l],
                           o1.view(torch.int16) if dt == _lib.DDTREE_BF16 else o1), l
        if with_lse:
            assert torch.equal(lse[l], l1), l
    if not oracle_check:
        return
    # each layer against the oracle
    orc = OracleRun(wl0)
    outs = out.float().cpu().numpy().astype(np.float64)
    worst = 0.0
    for r in range(wl0.bs):
        a, b = int(wl0.qo_indptr[r]), int(wl0.qo_indptr[r + 1])
        nodes = list(range(b - a)) if b - a <= 40 else sorted({0, (b - a) // 2, b - a - 1})
        qs = [w.q_f32()[a:b] for w in wls]
        kvs = [w.kv_rows_f32(wl0.request_slots(r)) for w in wls]
        refs = attention.verify_request_layers(qs, kvs, int(wl0.prefix_lens[r]),
                                               orc.parents[a:b], float(np.float32(wl0.scale)),
                                               nodes=nodes)
        for l, (ref, _) in enumerate(refs):
            got = outs[l, a + np.array(nodes)]
            worst = max(worst, np.abs(got - ref).max() / np.abs(ref).max())
    _say(f"  {wl0.name} L={L}: max|err|/max|out| = {worst:.3e}")
    assert worst <= TOL[wl0.dtype]


@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_layers_bf16(num_splits):
    _say(f"test_layers_bf16 splits={num_splits}")
    _layered(make_workload(get_config(1), dtype="bf16"), 3, num_splits)


@pytest.mark.parametrize("num_splits", [0, 2])
def test_layers_fp32(num_splits):
    _say(f"test_layers_fp32 splits={num_splits}")
    _layered(make_workload(get_config(1)), 3, num_splits)


def test_layers_shared_pool_no_lse():
    _say("test_layers_shared_pool_no_lse")
    _layered(make_workload(get_config(1), dtype="bf16"), 4, 0, shared_pool=True, with_lse=False)


def test_layers_shard_full_size():
    _say("test_layers_shard_full_size")
    _layered(make_workload(get_config(2)), 4, 0)


def test_layers_single_layer():
    _say("test_layers_single_layer")
    _layered(make_workload(get_config(1), dtype="bf16"), 1, 0)


def test_layers_headline_one_launch_per_layer():
    # 64 heads, 8k context: each layer fills the device, so the call enqueues
    # one launch per layer; still bit-exact against single-layer calls (which
    # the single-layer parity tests hold to the oracle)
    _say("test_layers_headline_one_launch_per_layer")
    _layered(make_workload(get_config(3)), 2, 0, oracle_check=False)
