"""Model of the 32-row verify kernel's plan and block order.

The host takes the 32-row kernel (attn_narrow_kernel) for bf16 calls of at
most NARROW_UNITS_PER_CU units of 128 rows x 32 columns per compute unit and
cuts every 32-row tile's KV blocks into S parts; workgroup i runs on XCD
i % 8 and takes part x + 8 * ((i >> 3) // tiles) of tile (i >> 3) % tiles.
Inside a part of n blocks, wave w takes position q = 4k + (w == 3 ? -1 : w)
in step k (position q is block (q + 3t) % n), so the queries can be staged
through wave 3's buffer during the first step.  This model restates those
integer formulas in Python, with the constants read from the kernel's
header, and checks on many shapes that the plan keeps every XCD's
workgroups resident at once, that every (tile, block) is taken exactly once,
and that the merge's two loads per part stay within one wave's 63
outstanding loads for the batch the host picks.  The GPU parity tests
(tests/test_gpu_narrow.py) check the same end to end on the shapes they run.
"""
import itertools
import re
from pathlib import Path

CSRC = Path(__file__).resolve().parents[1] / "tree_verify_mla_amd" / "csrc"
HDR = (CSRC / "attn_common.h").read_text()
NARROW = (CSRC / "verify_attn_narrow.hip").read_text()


def _const(name, text=HDR):
    return int(re.search(rf"constexpr int {name} = (\d+);", text).group(1))


KB, MT128, MT32 = _const("KB"), _const("MT_BF16"), _const("MT_NARROW")
UNITS_PER_CU, STEP = _const("NARROW_UNITS_PER_CU"), _const("NARROW_STEP")
NW, NMW = _const("NW", NARROW), _const("NMW", NARROW)


def plan(bs, H, max_q, max_kv, G):
    """(T32, S) as narrow_plan computes them, or None for the 128-row kernel."""
    nb = (max_kv + KB - 1) // KB
    t128 = (max_q * H + MT128 - 1) // MT128
    if bs * t128 * nb > UNITS_PER_CU * G:
        return None
    t32 = (max_q * H + MT32 - 1) // MT32
    tiles = bs * t32
    per_xcd = max(1, (G // 8) // tiles)
    S = 1 if nb <= STEP else (nb + 1) // 2
    return t32, min(S, 8 * per_xcd)


def workgroups(bs, T, S):
    """(blockIdx, xcd, r, t, s) of every live workgroup of the grid."""
    tiles = bs * T
    grid = 8 * ((S + 7) // 8) * tiles
    out = []
    for i in range(grid):
        x, k8 = i & 7, i >> 3
        s = x + 8 * (k8 // tiles)
        r, t = (k8 % tiles) // T, (k8 % tiles) % T
        if s < S:
            out.append((i, x, r, t, s))
    return out


def blocks_taken(n, t):
    """Blocks of a part of n blocks (tile t) in the order the waves take them."""
    nsteps = 1 if n <= 3 else 1 + (n - 3 + NW - 1) // NW
    rot = (3 * t) % n
    got = []
    for k in range(nsteps):
        for w in range(NW):
            q = NW * k + (-1 if w == 3 else w)
            if 0 <= q < n:
                got.append((q + rot) % n)
    return got


def test_shard_plan():
    # one 8-head shard on 256 compute units: 9 tiles of 32 rows, 24 parts
    assert plan(1, 8, 33, 4129, 256) == (9, 24)
    # the 64-head batch keeps the 128-row kernel
    assert plan(8, 64, 33, 8225, 256) is None


def test_every_block_once_and_xcds_resident():
    shapes = itertools.product([1, 2, 3, 8], [1, 3, 8, 16], [1, 9, 33, 65], [1, 30, 700, 4129, 20000],
                               [80, 256])
    checked = 0
    for bs, H, Q, P, G in shapes:
        N = P + Q
        pl = plan(bs, H, Q, N, G)
        if pl is None:
            continue
        T, S = pl
        wgs = workgroups(bs, T, S)
        # every XCD holds all of its workgroups at once (one per compute unit)
        per_x = [sum(1 for w in wgs if w[1] == x) for x in range(8)]
        assert max(per_x) <= max(1, G // 8) or S <= 8, (bs, H, Q, P, G, per_x)
        NB = (N + KB - 1) // KB
        R = Q * H
        taken = {}
        for _, _, r, t, s in wgs:
            if t * MT32 >= R:
                continue
            b0, b1 = s * NB // S, (s + 1) * NB // S
            if b0 >= b1:
                continue
            for b in blocks_taken(b1 - b0, t):
                key = (r, t, b0 + b)
                taken[key] = taken.get(key, 0) + 1
        T_real = (R + MT32 - 1) // MT32
        want = {(r, t, b) for r in range(bs) for t in range(T_real) for b in range(NB)}
        assert set(taken) == want and all(v == 1 for v in taken.values()), (bs, H, Q, P, G)
        checked += 1
    assert checked > 50


def test_merge_loads_fit_a_wave():
    # the host picks batch 2 for S <= 8, else 6; a wave folds ceil(S / NMW)
    # parts in batches, two loads per part, all of a batch in flight at once
    batches = [int(b) for b in re.findall(r"merge_narrow_kernel<(\d+)>, mgrid", NARROW)]
    assert sorted(batches) == [2, 6]
    assert 2 * max(batches) <= 63
    assert NMW * 2 >= 8  # S <= 8 fits one batch per wave
