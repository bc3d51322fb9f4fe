"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: tree, visibility, positions, dense mask and accept bit-exact;
attention max|err| <= 1e-2 * max|out| for bf16 and <= 1e-5 * max|out| for
fp32; lse within 2e-3 (bf16) / 1e-5 (fp32) absolute.  Every output row is
compared at every configuration, the full-size ones included, in the
bench's launch configuration (persistent split, num_splits = 0), so every
split tile's log-sum-exp merge is checked.  The full-size configurations
also run on their sensitized twin, where a mask error would exceed the
tolerance (tests/test_oracle_attention.py shows a leak is invisible at 131k
prefix otherwise).  Unused pool rows are NaN, so a stray read poisons the
output.  The whole step is also captured in a HIP graph and replayed, on the
8-head shard and on the ragged 32-request batch.
"""
import sys

import numpy as np
import pytest
import torch

import functools

from tests._oracle_side import OracleRun
from tree_verify_mla_amd import _lib
from tree_verify_mla_amd.step import VerifyStep
from workloads import get_config, make_workload, sensitize_tree_columns
from workloads.device import to_device

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f32": 1e-5}
LSE_TOL = {"bf16": 2e-3, "f32": 1e-5}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(wl, num_splits=0):
    orc = OracleRun(wl)
    x = to_device(wl, "cuda", target_predict=orc.target_predict)
    st = VerifyStep(x, num_splits=num_splits)
    st.run()
    torch.cuda.synchronize()
    return orc, st


def _out_f64(st):
    return st.out.float().cpu().numpy().astype(np.float64)


def _check_integer_stages(orc, st):
    wl = orc.wl
    if wl.drafter_logits is not None:
        # the drafter stage (ddtree_drafter_topk against oracle.drafter): ids
        # exact, log-probs within 1e-5 (fp32 against fp64, see
        # tests/test_gpu_drafter.py); the scores built from them then agree to
        # the same order, the trees exactly (no two candidates within 1e-5)
        assert np.array_equal(st.x.topk_ids.cpu().numpy(), orc.topk_ids)
        assert np.abs(st.x.topk_logprobs.cpu().numpy() - orc.topk_logprobs).max() <= 1e-5
        assert np.abs(st.node_scores.cpu().numpy() - orc.scores).max() <= 1e-5 * (wl.depth + 1)
    else:
        assert np.array_equal(st.node_scores.cpu().numpy().view(np.uint32),
                              orc.scores.view(np.uint32))
    assert np.array_equal(st.node_tokens.cpu().numpy(), orc.tokens)
    assert np.array_equal(st.node_parents.cpu().numpy(), orc.parents)
    assert np.array_equal(st.node_depths.cpu().numpy(), orc.depths)
    assert np.array_equal(st.vis_bits.cpu().numpy().view(np.uint32), orc.bits)
    assert np.array_equal(st.positions.cpu().numpy(), orc.positions)
    nodes, alen, commit, bonus = orc.accept
    assert np.array_equal(st.accepted_nodes.cpu().numpy(), nodes)
    assert np.array_equal(st.accept_len.cpu().numpy(), alen)
    assert np.array_equal(st.commit_tokens.cpu().numpy(), commit)
    assert np.array_equal(st.bonus_tokens.cpu().numpy(), bonus)


def _check_attention(orc, st):
    """Every output row and lse of every request against the fp64 oracle."""
    wl = orc.wl
    out = _out_f64(st)
    lse = st.lse.cpu().numpy().astype(np.float64)
    worst, worst_lse = 0.0, 0.0
    for r in range(wl.bs):
        a, b = int(wl.qo_indptr[r]), int(wl.qo_indptr[r + 1])
        ref, ref_lse = orc.attention_rows(r)
        got = out[a:b]
        assert np.isfinite(got).all(), f"request {r}: non-finite output"
        err = np.abs(got - ref).max() / np.abs(ref).max()
        worst = max(worst, err)
        worst_lse = max(worst_lse, np.abs(lse[a:b] - ref_lse).max())
    _say(f"  {wl.name}: max|err|/max|out| = {worst:.3e}, max|lse err| = {worst_lse:.3e} "
         f"over {wl.total_q} nodes x {wl.heads} heads")
    assert worst <= TOL[wl.dtype]
    assert worst_lse <= LSE_TOL[wl.dtype]


@functools.lru_cache(maxsize=2)
def _full_size(index: int, twin: bool):
    """The full-size workload of a configuration (drawn once per process)."""
    wl = make_workload(get_config(index))
    return sensitize_tree_columns(wl) if twin else wl


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("num_splits", [0, 1, 2, 3])
def test_c1_tiny_fp32(num_splits):
    _say(f"test_c1_tiny_fp32 splits={num_splits}")
    orc, st = _run(make_workload(get_config(1)), num_splits)
    _check_integer_stages(orc, st)
    _check_attention(orc, st)


@pytest.mark.parametrize("num_splits", [0, 1, 2])
def test_c1_shape_bf16(num_splits):
    _say(f"test_c1_shape_bf16 splits={num_splits}")
    orc, st = _run(make_workload(get_config(1), dtype="bf16"), num_splits)
    _check_integer_stages(orc, st)
    _check_attention(orc, st)


@pytest.mark.parametrize("num_splits", [0, 1, 2, 7])
def test_c2_shard_bf16_full_compare(num_splits):
    _say(f"test_c2 splits={num_splits}")
    orc, st = _run(make_workload(get_config(2)), num_splits)
    _check_integer_stages(orc, st)
    _check_attention(orc, st)


@pytest.mark.parametrize("shift", [20, -40])
def test_partials_any_magnitude(shift):
    """c_kv scaled by 2^shift and the queries' c_kv part by 2^-shift: the
    scores are unchanged (powers of two are exact in bf16) and every output
    scales by 2^shift.  2^20 puts |c_kv| far above the largest fp16 (65504)
    and 2^-40 far below its smallest normal, so the split tiles' fp16
    partials must carry their per-row scale to match the oracle."""
    _say(f"test_partials_any_magnitude shift={shift}")
    import copy
    from workloads.gen import bf16_bits_to_f32, f32_to_bf16_bits
    wl = copy.copy(make_workload(get_config(2)))
    pool = bf16_bits_to_f32(wl.kv_pool)
    q = bf16_bits_to_f32(wl.q)
    pool[:, :512] *= np.float32(2.0 ** shift)
    q[:, :, :512] *= np.float32(2.0 ** -shift)
    wl.kv_pool = f32_to_bf16_bits(pool)
    wl.q = f32_to_bf16_bits(q)
    assert np.array_equal(bf16_bits_to_f32(wl.kv_pool)[:, :512], pool[:, :512], equal_nan=True)  # exact (unused rows hold NaN)
    for num_splits in (0, 7):
        orc, st = _run(wl, num_splits)
        _check_attention(orc, st)


def test_one_tile_over_the_whole_device_bf16():
    """A single 34-row tile over a 60,000-column prefix: the persistent
    schedule splits it over about 220 workgroups and the merge folds that
    many segments of one tile; a second request (one 2-row tile, no tree
    nodes) takes the remaining workgroups."""
    _say("test_one_tile_over_the_whole_device_bf16")
    wl = make_workload(get_config(3), bs=2, heads=2, budgets=[16, 0], prefixes=[60000, 9000],
                       pool_slots=80000, seed=4242)
    orc, st = _run(wl)
    _check_integer_stages(orc, st)
    _check_attention(orc, st)


def test_ragged_edges_bf16():
    """Empty and odd prefixes, budget 0 (autoregressive), ragged tails across tiles."""
    _say("test_ragged_edges_bf16")
    wl = make_workload(get_config(3), bs=6, heads=16, budgets=[0, 1, 8, 16, 64, 33],
                       prefixes=[0, 1, 31, 33, 700, 5000], pool_slots=20000)
    orc, st = _run(wl)
    _check_integer_stages(orc, st)
    _check_attention(orc, st)
    for S in (1, 5):
        orc2, st2 = _run(wl, S)
        _check_attention(orc2, st2)


def test_many_requests_bf16():
    """More requests than the attention kernel's request table holds (64):
    the schedule falls back to reading the offsets from memory."""
    _say("test_many_requests_bf16")
    rng = np.random.default_rng(70)
    bs = 70
    wl = make_workload(get_config(3), bs=bs, heads=4, budgets=rng.choice([0, 3, 8, 32], size=bs),
                       prefixes=rng.integers(0, 300, size=bs), pool_slots=40000)
    orc, st = _run(wl)
    _check_integer_stages(orc, st)
    _check_attention(orc, st)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_trees_past_128_nodes(dtype):
    """Trees of more than 128 nodes: the attention reads the rows' ancestor
    words past the fourth from memory in its tail blocks (W = 7 here)."""
    _say(f"test_trees_past_128_nodes {dtype}")
    wl = make_workload(get_config(3), bs=3, heads=2, budgets=[200, 129, 3], prefixes=[50, 0, 700],
                       pool_slots=5000, dtype=dtype)
    orc, st = _run(wl)
    _check_integer_stages(orc, st)
    _check_attention(orc, st)


def test_maximum_budget_end_to_end():
    """The largest tree the builder takes (2048 draft nodes, 2049-node rows of
    65 bitset words), a mid-size one and an autoregressive request, through
    the whole step: the LDS-frontier builder, bitsets and positions, the
    attention's mask from ancestor words in memory, and accept."""
    _say("test_maximum_budget_end_to_end")
    wl = make_workload(get_config(3), bs=3, heads=2, depth=8, topk=32, budgets=[2048, 1000, 0],
                       prefixes=[0, 100, 7], pool_slots=5000, seed=2048)
    orc, st = _run(wl)
    _check_integer_stages(orc, st)
    _check_attention(orc, st)


def test_pool_past_4gib():
    """A bf16 pool of 5M slots (5.8 GB): byte offsets past 2^32 take the
    kernel's 64-bit global gathers instead of the buffer-resource ones."""
    _say("test_pool_past_4gib")
    wl = make_workload(get_config(3), bs=2, heads=4, budgets=[32, 16], prefixes=[3000, 500],
                       pool_slots=5_000_000)
    assert int(wl.kv_indices.max()) * 1152 > 2 ** 32  # some rows lie past the first 4 GiB
    orc, st = _run(wl)
    _check_integer_stages(orc, st)
    _check_attention(orc, st)


def test_ragged_edges_fp32():
    _say("test_ragged_edges_fp32")
    wl = make_workload(get_config(1), bs=4, heads=3, budgets=[0, 5, 8, 31], prefixes=[0, 2, 33, 100],
                       pool_slots=400)
    orc, st = _run(wl)
    _check_integer_stages(orc, st)
    _check_attention(orc, st)


@pytest.mark.parametrize("twin", [False, True])
def test_c3_headline_full_size(twin):
    _say(f"test_c3_headline_full_size twin={twin}")
    orc, st = _run(_full_size(3, twin))
    _check_integer_stages(orc, st)
    _check_attention(orc, st)


@pytest.mark.parametrize("twin", [False, True])
def test_c4_long_context_full_size(twin):
    _say(f"test_c4_long_context_full_size twin={twin}")
    orc, st = _run(_full_size(4, twin))
    _check_integer_stages(orc, st)
    _check_attention(orc, st)


def test_c4_forced_splits_agree():
    """Split count must not change the result beyond rounding."""
    _say("test_c4_forced_splits_agree")
    orc, st = _run(_full_size(4, True), num_splits=64)
    _check_attention(orc, st)


@pytest.mark.parametrize("twin", [False, True])
def test_c5_ragged_e2e_full_size(twin):
    _say(f"test_c5_ragged_e2e_full_size twin={twin}")
    orc, st = _run(_full_size(5, twin))
    _check_integer_stages(orc, st)
    _check_attention(orc, st)


def test_dense_mask_matches_oracle():
    _say("test_dense_mask_matches_oracle")
    wl = make_workload(get_config(3), bs=3, heads=2, budgets=[8, 32, 64], prefixes=[21, 0, 333],
                       pool_slots=2000)
    orc = OracleRun(wl)
    x = to_device(wl, "cuda")
    st = VerifyStep(x)
    st.build()
    mi = orc.mask_indptr()
    dense = torch.full((int(mi[-1]),), 7, dtype=torch.uint8, device="cuda")
    _lib.ddtree_compile_visibility(st.node_parents, st.node_depths, x.qo_indptr, x.prefix_lens,
                                   x.max_q_len, st.vis_bits, positions=st.positions,
                                   dense_mask=dense,
                                   mask_indptr=torch.from_numpy(mi).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(dense.cpu().numpy(), orc.dense)


def test_build_tree_exact_many_shapes():
    """Bit-exact trees over depth/top-k/budget combinations, incl. ties."""
    _say("test_build_tree_exact_many_shapes")
    # budgets up to 64 (depth x top-k up to 256) take the lean register
    # builder, which also forms the bitsets in the one-call form; budgets up
    # to 126 the two-slot register builder; above that the LDS-frontier one;
    # depth x top-k above 256 keeps the top-k table in LDS
    for (D, K, budgets) in [(7, 4, [8, 0, 3]), (7, 8, [32, 16, 64]), (7, 16, [64, 1, 40]),
                            (3, 2, [14, 7, 1]), (1, 5, [5, 2, 0]), (7, 8, [126, 125, 2]),
                            (7, 8, [200, 127, 9]), (7, 40, [100, 12, 3]), (8, 32, [64, 63, 5]),
                            (2, 64, [64, 33, 1]), (6, 1, [6, 3, 0])]:
        wl = make_workload(get_config(3), bs=3, heads=1, depth=D, topk=K, budgets=budgets,
                           prefixes=[4, 4, 4], pool_slots=400, seed=77 + D * K)
        # coarse log-probs give exact fp32 ties in the scores
        lp = np.minimum(0, np.round(wl.topk_logprobs * 2) / 2).astype(np.float32)
        wl.topk_logprobs = -np.sort(-lp, axis=2)
        orc = OracleRun(wl)
        x = to_device(wl, "cuda")
        st = VerifyStep(x)
        st.build()
        torch.cuda.synchronize()
        assert np.array_equal(st.node_tokens.cpu().numpy(), orc.tokens), (D, K)
        assert np.array_equal(st.node_parents.cpu().numpy(), orc.parents), (D, K)
        assert np.array_equal(st.node_depths.cpu().numpy(), orc.depths), (D, K)
        sc = st.node_scores.cpu().numpy().view(np.uint32)
        assert np.array_equal(sc, orc.scores.view(np.uint32)), (D, K)
        # the same tree, bitsets and positions from the one-call form
        st2 = VerifyStep(x)
        for t in (st2.node_tokens, st2.node_parents, st2.node_depths, st2.vis_bits, st2.positions):
            t.fill_(-7)
        st2.build_visibility()
        torch.cuda.synchronize()
        for a, b in ((st2.node_tokens, orc.tokens), (st2.node_parents, orc.parents),
                     (st2.node_depths, orc.depths)):
            assert np.array_equal(a.cpu().numpy(), b), (D, K, "one-call form")
        assert np.array_equal(st2.node_scores.cpu().numpy().view(np.uint32), sc), (D, K)
        assert np.array_equal(st2.vis_bits.cpu().numpy().view(np.uint32), orc.bits), (D, K)
        assert np.array_equal(st2.positions.cpu().numpy(), orc.positions), (D, K)


def test_accept_sentinel_and_full_chain():
    _say("test_accept_sentinel_and_full_chain")
    wl = make_workload(get_config(3), bs=2, heads=1, budgets=[32, 32], prefixes=[4, 4], pool_slots=200)
    orc = OracleRun(wl)
    x = to_device(wl, "cuda")
    st = VerifyStep(x)
    st.build()
    from oracle import accept as oacc
    # request 0: sentinel everywhere; request 1: follow the best path to the deepest node
    tok, par = orc.tokens, orc.parents
    pred = np.full(len(tok), -1, np.int32)
    a = int(wl.qo_indptr[1])
    t1 = orc.trees[1]
    deepest = int(np.argmax(t1.depths))
    path, j = [], deepest
    while j >= 0:
        path.append(j)
        j = int(t1.parents[j])
    path.reverse()
    for u, v in zip(path[:-1], path[1:]):
        pred[a + u] = t1.tokens[v]
    pred[a + deepest] = 4242
    tp = torch.from_numpy(pred).cuda()
    st.accept(target_predict=tp)
    torch.cuda.synchronize()
    ref = oacc.batch(tok, par, wl.qo_indptr, pred, wl.depth)
    assert np.array_equal(st.accept_len.cpu().numpy(), ref[1])
    assert st.accept_len.cpu().numpy().tolist() == [1, len(path)]
    assert np.array_equal(st.commit_tokens.cpu().numpy(), ref[2])
    assert st.bonus_tokens.cpu().numpy().tolist() == [-1, 4242]


def _accept_case(rng, Q, kind):
    """(tokens, parents, predictions) of one request.  "bushy": parents among
    the three previous nodes, three token values, random predictions (many
    siblings share a token: the smaller index must win).  "deep": mostly a
    chain; the predictions lead from the root to the last node, whose path
    carries tokens no other node has.  "star0"/"star1": every node a child of
    the root, two of them carrying the predicted token, both in the first 64
    nodes or the first at 64 or beyond."""
    if kind == "bushy":
        par = [-1] + [int(rng.integers(max(0, j - 3), j)) for j in range(1, Q)]
        tok = rng.integers(0, 3, size=Q)
        pred = rng.integers(0, 3, size=Q)
    elif kind == "deep":
        par = [-1] + [j - 1 if rng.random() < 0.7 else int(rng.integers(0, j)) for j in range(1, Q)]
        tok = rng.integers(0, 8, size=Q)
        pred = rng.integers(0, 8, size=Q)
        j, k = Q - 1, 0
        while j > 0:
            tok[j] = 1000 + k
            pred[par[j]] = tok[j]
            j, k = par[j], k + 1
    else:
        par = [-1] + [0] * (Q - 1)
        tok = rng.integers(0, 6, size=Q)
        pred = rng.integers(0, 6, size=Q)
        a, b = (10, 40) if kind == "star0" else (70, 100)
        tok[a] = tok[b] = pred[0] = 7
    return (np.asarray(tok, np.int32)[:Q], np.asarray(par, np.int32)[:Q],
            np.asarray(pred, np.int32)[:Q])


def test_accept_random_trees_both_walks():
    """Requests of 0..300 nodes on both sides of the 128-node register walk,
    against the oracle bit for bit, at a depth limit the walks never reach
    and at one that cuts them; an empty request gets the sentinel rows."""
    _say("test_accept_random_trees_both_walks")
    from oracle import accept as oacc
    rng = np.random.default_rng(11)
    cases = [(1, "bushy"), (2, "deep"), (63, "bushy"), (64, "deep"), (65, "bushy"),
             (127, "bushy"), (128, "deep"), (0, None), (128, "star0"), (128, "star1"),
             (129, "deep"), (200, "bushy"), (300, "deep"), (90, "deep")]
    parts = [_accept_case(rng, Q, kind) if Q else (np.zeros(0, np.int32),) * 3 for Q, kind in cases]
    sizes = [Q for Q, _ in cases]
    qo = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    tok, par, pred = (np.concatenate([c[i] for c in parts]) for i in range(3))
    bs = len(cases)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    reached = 0
    for D in (300, 5):
        outs = [torch.full(shape, 77, dtype=torch.int32, device="cuda")
                for shape in ((bs, D + 1), (bs,), (bs, D + 1), (bs,))]
        _lib.ddtree_accept(dev(tok), dev(par), dev(qo), dev(pred), D, *outs)
        torch.cuda.synchronize()
        nodes, alen, commit, bonus = (t.cpu().numpy() for t in outs)
        for r, Q in enumerate(sizes):
            if Q == 0:
                assert alen[r] == 0 and bonus[r] == -1
                assert (nodes[r] == -1).all() and (commit[r] == -1).all()
                continue
            a, b = qo[r], qo[r + 1]
            ref = oacc.accept(tok[a:b], par[a:b], pred[a:b], D)
            case = (D, cases[r])
            assert alen[r] == ref.accept_len, (case, alen[r], ref.accept_len)
            assert nodes[r, :ref.accept_len].tolist() == ref.path, case
            assert (nodes[r, ref.accept_len:] == -1).all(), case
            assert commit[r, :ref.accept_len].tolist() == ref.commit_tokens, case
            assert (commit[r, ref.accept_len:] == -1).all(), case
            assert bonus[r] == ref.bonus, case
            reached = max(reached, int(nodes[r].max()))
        if D == 300:
            star0, star1 = cases.index((128, "star0")), cases.index((128, "star1"))
            assert nodes[star0, 1] == 10 and nodes[star1, 1] == 70
    # the walks pass node 64 and node 128, so both register slots and the
    # walk through memory are exercised
    assert reached == 299


def _graph_replay(wl):
    """The whole step captured in one graph, replayed with eager work between
    the replays; every replay must equal the eager run bit for bit."""
    orc = OracleRun(wl)
    x = to_device(wl, "cuda", target_predict=orc.target_predict)
    st = VerifyStep(x)
    st.run()
    torch.cuda.synchronize()
    outs = (st.node_tokens, st.vis_bits, st.out, st.lse, st.accept_len, st.commit_tokens)
    eager = [t.clone() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        st.run(stream=s)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        st.run(stream=s)
    for rep in range(4):
        for t in outs:
            t.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for a, b in zip(eager, outs):
            assert torch.equal(a, b), f"replay {rep} differs from eager"
    return orc, st


def test_graph_replay_matches_eager():
    _say("test_graph_replay_matches_eager")
    _graph_replay(make_workload(get_config(2)))


def test_graph_replay_ragged_batch():
    """The ragged 32-request batch (budgets 16/32/64, prefixes 1k-32k) under
    capture: replays equal the eager run, and the replayed step is oracle-exact
    on the integer stages."""
    _say("test_graph_replay_ragged_batch")
    orc, st = _graph_replay(_full_size(5, False))
    _check_integer_stages(orc, st)
