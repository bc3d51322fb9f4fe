"""GPU parity of ddtree_tree_sample (through the C ABI) against ``oracle.sample``.

The oracle walks the tree in plain fp64; the kernel in fp32 with its own
fixed order of sums.  Both take the same decisions except where a decision
lies within the kernel's rounding of a boundary: its masses and running
masses are sums over 256 blocks of ceil(V / 256) tokens (the tokens of a
block one by one, then the blocks), each off by at most about
(ceil(V / 256) + 256) * 2^-24 of the row's mass, plus one rounding per
rejected child and one per product.  The bar: for every request whose
accept/reject margin (``oracle.sample.walk``: the distance of each coin
product from its boundary, over the row's mass) exceeds MARGIN_FACTOR times
that bound, the accepted path, accept length and accepted tokens are
bit-exact; the bonus is bit-exact where its threshold lies further than that
from the drawn token's bounds, and otherwise (large vocabularies: a token's
mass is then below the rounding) must be a token with mass whose running
masses bracket the threshold to within the bound -- one of the draws fp32
rounding allows.  Coins and uniforms are seeded draws; a
request whose margin does not clear the bound gets the next draws of the
same stream for its coins and uniform until it does (at a 512-token
vocabulary a token holds about 2e-3 of a row's mass and the bound is about
3e-5 of it, so about one request in ten is redrawn).  Hand-built cases with
dyadic rows, where every sum is exact on both sides, run with coins exactly
on a boundary (a strict comparison must reject).

The HIP side samples along its own tree (ddtree_build_tree), the oracle along
its own (bit-exact, see test_gpu_parity.py); target rows come from the
seeded generator.  Covered: budget 0 (root only: the bonus is a plain draw
from the root's row), ragged trees up to 65 nodes, the headline batch, a
vocabulary whose blocks are ragged (5000 = 256 x 20 - 120), a vocabulary of
163,840 tokens, several draws per workload, a root row with mass only on
drafted tokens, blocks wider than one staging tile (vocabulary 1,279,983:
5000 tokens a block, staged one at a time), a vocabulary that leaves most
blocks empty (513), and a caller-provided workspace reused across calls.
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

MARGIN_FACTOR = 2.0
GOLD = __import__("pathlib").Path(__file__).parent / "golden"


def _bound(vocab: int, q_len: int) -> float:
    """Decision margin (fraction of the row mass) beyond which the kernel's
    fp32 sums cannot change a decision."""
    return MARGIN_FACTOR * (-(-vocab // 256) + 256 + q_len + 2) * 2.0 ** -24


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
    if ws is None:
        ws = torch.empty(max(1, _lib.ddtree_tree_sample_workspace_size(wl.total_q)),
                         dtype=torch.uint8, device="cuda")
    bound = _bound(vocab, wl.max_q_len)
    redrawn = near = exact = 0
    qo = wl.qo_indptr
    for d in range(draws):
        coins = rng.random(wl.total_q).astype(np.float32)
        bonus_u = rng.random(bs).astype(np.float32)
        for attempt in range(50):
            *ref, walks = sample.batch(orc.tokens, orc.parents, qo, probs, coins, bonus_u, D,
                                       with_walks=True)
            bad = [r for r in range(bs) if walks[r] is not None and walks[r].margin <= bound]
            if not bad:
                break
            for r in bad:   # the next draws of the stream for those requests only
                coins[qo[r]:qo[r + 1]] = rng.random(int(qo[r + 1] - qo[r])).astype(np.float32)
                bonus_u[r] = np.float32(rng.random())
            redrawn += len(bad)
        else:
            raise AssertionError("no draw clears the fp32 margin")
        _lib.ddtree_tree_sample(st.node_tokens, st.node_parents, x.qo_indptr, probs_d,
                                torch.from_numpy(coins).cuda(), torch.from_numpy(bonus_u).cuda(),
                                D, *out, workspace=ws)
        torch.cuda.synchronize()
        nodes, alen, commit, bonus = (t.cpu().numpy() for t in out)
        # the walk: exact
        assert np.array_equal(nodes, ref[0]), d
        assert np.array_equal(alen, ref[1]), d
        for r in range(bs):
            n = int(ref[1][r])
            assert np.array_equal(commit[r, :max(n - 1, 0)], ref[2][r, :max(n - 1, 0)]), (d, r)
            assert np.array_equal(commit[r, n:], ref[2][r, n:]), (d, r)
            w = walks[r]
            if w is None or w.bonus < 0 or w.bonus_margin > bound:
                assert bonus[r] == ref[3][r], (d, r)    # decided beyond the fp32 rounding
            else:
                # within the fp32 rounding of a boundary: any token whose
                # running masses bracket the threshold up to that rounding
                j = int(bonus[r])
                tol = bound * w.row_mass
                lo, hi = w.bonus_bounds(j)
                assert 0 <= j < vocab and w.residual[j] > 0, (d, r, j)
                assert lo - tol <= w.threshold <= hi + tol, (d, r, j)
                exact += bonus[r] == ref[3][r]
                near += 1
            if n >= 1:
                assert commit[r, n - 1] == bonus[r]
    assert redrawn <= bs * draws, f"{redrawn} request draws fell within the fp32 margin"
    _say(f"  vocab {vocab}: {redrawn} requests redrawn; {near} bonus draws within the fp32 "
         f"margin of a boundary ({exact} equal to the fp64 draw)")
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


def test_sample_hand_examples_exact_boundaries():
    """Dyadic rows and coins: every sum is exact in fp32 and fp64, including
    a coin exactly on the acceptance boundary (strict comparison rejects)."""
    _say("test_sample_hand_examples_exact_boundaries")
    import json
    g = json.loads((GOLD / "sample_hand_example.json").read_text())
    tok = torch.tensor(g["tokens"], dtype=torch.int32, device="cuda")
    par = torch.tensor(g["parents"], dtype=torch.int32, device="cuda")
    q = len(g["tokens"])
    qo = torch.tensor([0, q], dtype=torch.int32, device="cuda")
    probs = np.array(g["probs"], np.float32)
    D = g["depth_max"]
    out = [torch.empty(1, D + 1, dtype=torch.int32, device="cuda"),
           torch.empty(1, dtype=torch.int32, device="cuda"),
           torch.empty(1, D + 1, dtype=torch.int32, device="cuda"),
           torch.empty(1, dtype=torch.int32, device="cuda")]
    ws = torch.empty(_lib.ddtree_tree_sample_workspace_size(q), dtype=torch.uint8, device="cuda")
    for ex in g["examples"]:
        coins = np.array(ex["coins"], np.float32)
        u = np.array([ex["bonus_u"]], np.float32)
        _lib.ddtree_tree_sample(tok, par, qo, torch.from_numpy(probs).cuda(),
                                torch.from_numpy(coins).cuda(), torch.from_numpy(u).cuda(), D, *out,
                                workspace=ws)
        torch.cuda.synchronize()
        n = len(ex["path"])
        assert out[1].item() == n, ex["name"]
        assert out[0].cpu().numpy()[0, :n].tolist() == ex["path"], ex["name"]
        assert out[2].cpu().numpy()[0, :n].tolist() == ex["commit"], ex["name"]
        assert out[3].item() == ex["bonus"], ex["name"]
