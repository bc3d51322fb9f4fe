"""The seeded generator: determinism, shapes and the builder's input preconditions."""
import numpy as np
import pytest

from workloads import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, get_config, make_workload


def test_bf16_rounding_is_rne():
    x = np.float32([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5, np.inf])
    got = bf16_bits_to_f32(f32_to_bf16_bits(x))
    assert got.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5, np.inf]
    assert np.isnan(bf16_bits_to_f32(f32_to_bf16_bits(np.float32([np.nan]))))[0]


def test_deterministic_and_seeded():
    a = make_workload(get_config(1))
    b = make_workload(get_config(1))
    c = make_workload(get_config(1), seed=5)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.kv_indices, b.kv_indices)
    assert not np.array_equal(a.q, c.q)


@pytest.mark.parametrize("i,drafter", [(1, "tables"), (2, None)])
def test_shapes_and_preconditions(i, drafter):
    cfg = get_config(i)
    wl = make_workload(cfg, drafter=drafter)
    Q = cfg.budget + 1
    assert wl.qo_indptr.tolist() == [0, Q]
    assert wl.kv_indptr.tolist() == [0, cfg.prefix + Q]
    assert wl.q.shape == (Q, cfg.heads, 576)
    assert wl.kv_pool.shape == (cfg.pool_slots, 576)
    assert len(np.unique(wl.kv_indices)) == len(wl.kv_indices)
    lp = wl.topk_logprobs
    assert lp.shape == (1, 7, cfg.topk) and (lp <= 0).all() and (lp[..., :-1] >= lp[..., 1:]).all()
    for d in range(7):
        assert len(set(wl.topk_ids[0, d].tolist())) == cfg.topk
    used = np.zeros(cfg.pool_slots, bool)
    used[wl.kv_indices] = True
    vals = wl.kv_rows_f32(np.nonzero(~used)[0][:50])
    assert np.isnan(vals).all()


def test_ragged_config_draws():
    cfg = get_config(5)
    wl = make_workload(cfg, bs=6, prefixes=None)
    assert set(wl.budgets.tolist()) <= {16, 32, 64}
    assert ((wl.prefix_lens >= 1024) & (wl.prefix_lens <= 32768)).all()
    assert wl.num_slots == int(np.ceil(1.25 * wl.kv_indptr[-1]))


def test_all_configs_named():
    assert sorted(CONFIGS) == [1, 2, 3, 4, 5]
    assert CONFIGS[3].heads == 64 and CONFIGS[3].bs == 8 and CONFIGS[3].budget == 32 and CONFIGS[3].prefix == 8192


def test_tiny_config_draws_drafter_logits():
    """The tiny configuration's trees start from N(0, 1) drafter logits over
    the 512-token vocabulary; the tables are left to the method."""
    wl = make_workload(get_config(1))
    assert wl.topk_logprobs is None and wl.topk_ids is None
    assert wl.drafter_logits.shape == (1, 7, 512) and wl.drafter_logits.dtype == np.float32
    x = wl.drafter_logits.astype(np.float64)
    assert abs(x.mean()) < 0.1 and abs(x.std() - 1.0) < 0.05
