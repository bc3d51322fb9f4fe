"""The benchmark's algorithmic work, checked against the method's own
objects on the CPU: the attention flops of a batch are 2 * 576 + 2 * 512 per
visible (node, head, column) pair, and the visible pairs are exactly the
ones of the oracle's dense [q_len, prefix + q_len] visibility mask
("The 30-Column Mask ...", section "Mask Stride Formula")."""
import numpy as np

import bench
from tests._oracle_side import OracleRun
from workloads import get_config, make_workload


def test_attention_flops_count_the_visible_pairs_of_the_mask():
    wl = make_workload(get_config(3), bs=4, heads=5, budgets=[8, 0, 33, 64],
                       prefixes=[5, 0, 100, 31], pool_slots=2000)
    orc = OracleRun(wl)
    flops, nbytes = bench.algorithmic_work(wl, orc.depths)
    pairs = int(np.asarray(orc.dense, dtype=np.int64).sum())  # ones of every request's mask
    assert flops == (2 * 576 + 2 * 512) * wl.heads * pairs
    # each request's KV rows are counted once, whatever its node count
    alone = [bench.algorithmic_work(make_workload(get_config(3), bs=1, heads=5, budgets=[b],
                                                  prefixes=[p], pool_slots=400),
                                    np.zeros(b + 1, np.int32))[1]
             for b, p in ((0, 7), (0, 8))]
    assert alone[1] - alone[0] == 576 * 2 + 4  # one more prefix row: one latent row and one slot id


def test_tiny_configuration_mask_is_the_pages_9_by_30():
    wl = make_workload(get_config(1))
    orc = OracleRun(wl)
    assert wl.max_q_len == 9 and int(wl.prefix_lens[0]) == 21
    assert np.asarray(orc.dense).size == 9 * 30
