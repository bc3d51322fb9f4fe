"""GPU parity of the small-problem verify kernel (32-row tiles, a fixed split
of each tile's KV range, log-sum-exp merge of the parts) against the fp64
oracle, through the C ABI.  Bars as in test_gpu_parity: every output row,
max|err| <= 1e-2 * max|out| (bf16), lse within 2e-3; unused pool rows are NaN.

ddtree_verify_attn_plan reports the path each case takes, so the cases below
are known to run this kernel: the 8-head shard (and its sensitized twin, on
which a wrong tree mask exceeds the tolerance), a ragged batch whose short
requests leave most of their tile's parts empty, one part per tile (the
kernel writes the output itself), rows that do not fill the last tile, trees
past 128 nodes, and the layer-batched call."""
import pytest
import torch

from tests.test_gpu_parity import _check_attention, _check_integer_stages, _run, _say
from tree_verify_mla_amd import _lib
from workloads import get_config, make_workload, sensitize_tree_columns

pytestmark = pytest.mark.gpu


def _plan(wl, num_splits=0):
    """The path VerifyStep's call takes (it passes the workload's own bounds)."""
    dt = _lib.DDTREE_BF16 if wl.dtype == "bf16" else _lib.DDTREE_F32
    return _lib.ddtree_verify_attn_plan(wl.bs, wl.heads, wl.max_q_len, wl.max_kv_len, num_splits, dt)


def test_plan_picks_the_narrow_kernel_for_small_calls():
    _say("test_plan_picks_the_narrow_kernel_for_small_calls")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows, S = _lib.ddtree_verify_attn_plan(1, 8, 33, 4129, 0, _lib.DDTREE_BF16)
    assert rows == 32 and S >= 2
    # every workgroup fits on the device at once (9 tiles of 32 rows)
    assert 9 * S <= cus
    assert _lib.ddtree_verify_attn_plan(8, 64, 33, 8225, 0, _lib.DDTREE_BF16) == (128, 0)
    # a forced split keeps the 128-row kernel
    assert _lib.ddtree_verify_attn_plan(1, 8, 33, 4129, 7, _lib.DDTREE_BF16) == (128, 7)
    # an empty batch is a valid call (the attention call returns at once)
    assert _lib.ddtree_verify_attn_plan(0, 8, 33, 4129, 0, _lib.DDTREE_BF16) == (128, 0)


@pytest.mark.parametrize("twin", [False, True])
def test_shard_narrow(twin):
    _say(f"test_shard_narrow twin={twin}")
    wl = make_workload(get_config(2))
    if twin:
        wl = sensitize_tree_columns(wl)
    assert _plan(wl)[0] == 32
    orc, st = _run(wl)
    _check_integer_stages(orc, st)
    _check_attention(orc, st)


def test_narrow_ragged_batch_with_empty_parts():
    """Requests of 1, 41 and 2065 columns under one split count: the short
    ones have fewer KV blocks than parts, so most of their parts are empty
    and the merge must skip them; an autoregressive request (budget 0)."""
    _say("test_narrow_ragged_batch_with_empty_parts")
    wl = make_workload(get_config(3), bs=3, heads=4, budgets=[0, 7, 64], prefixes=[0, 33, 2000],
                       pool_slots=9000, seed=321)
    rows, S = _plan(wl)
    assert rows == 32 and S > 2
    orc, st = _run(wl)
    _check_integer_stages(orc, st)
    _check_attention(orc, st)


def test_narrow_single_part():
    """KV ranges of one block: one part per tile, output written directly."""
    _say("test_narrow_single_part")
    wl = make_workload(get_config(3), bs=2, heads=8, budgets=[8, 3], prefixes=[21, 5],
                       pool_slots=500, seed=77)
    assert _plan(wl) == (32, 1)
    orc, st = _run(wl)
    _check_integer_stages(orc, st)
    _check_attention(orc, st)


def test_narrow_odd_heads_and_long_trees():
    """3 heads (tiles start mid-node), trees of 150 and 40 nodes (ancestor
    words past the fourth read from memory in the tail blocks)."""
    _say("test_narrow_odd_heads_and_long_trees")
    wl = make_workload(get_config(3), bs=2, heads=3, budgets=[149, 39], prefixes=[900, 64],
                       pool_slots=4000, seed=99)
    assert _plan(wl)[0] == 32
    orc, st = _run(wl)
    _check_integer_stages(orc, st)
    _check_attention(orc, st)


def test_narrow_without_lse_and_repeatable():
    """No lse requested (the merge's lse store is skipped), and two calls on
    the same inputs give the same bits: the parts are folded in a fixed
    order, whatever order the workgroups finish in."""
    _say("test_narrow_without_lse_and_repeatable")
    from tests._oracle_side import OracleRun
    from tree_verify_mla_amd.step import VerifyStep
    from workloads.device import to_device
    import numpy as np
    wl = make_workload(get_config(2), seed=2024)
    orc = OracleRun(wl)
    x = to_device(wl, "cuda", target_predict=orc.target_predict)
    st = VerifyStep(x, want_lse=False)
    st.run()
    torch.cuda.synchronize()
    first = st.out.clone()
    st.attention()
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), st.out.view(torch.int16))
    out = st.out.float().cpu().numpy().astype(np.float64)
    ref, _ = orc.attention_rows(0)
    err = np.abs(out - ref).max() / np.abs(ref).max()
    _say(f"  max|err|/max|out| = {err:.3e}")
    assert err <= 1e-2
