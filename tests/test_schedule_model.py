"""Model of the persistent schedule of the matrix-core verify kernel.

The kernel (attn_bf16_kernel) gives workgroup v the virtual-unit range
[v V / Ge, (v+1) V / Ge) of a list in which every (row tile, KV block) unit
is preceded per tile by KAPPA virtual units, maps the ends to real units,
and runs the range as segments inside one tile each (a range that starts
mid-tile runs that first segment last); a segment that does not cover its
whole tile writes partial slot 2 v (the range's first segment) or 2 v + 1.
The merge finds a tile's segments from the virtual ids that hold its first
and last units.  This model restates those integer formulas in Python,
with the constants read from the kernel's header, and checks on random
batch shapes that every unit is covered exactly once and that the merge
expects exactly the partial slots the kernel writes.  The GPU parity tests
check the same end to end on the shapes they run.
"""
import re
from pathlib import Path

import numpy as np

HDR = (Path(__file__).resolve().parents[1] / "tree_verify_mla_amd" / "csrc" / "attn_common.h").read_text()


def _const(name):
    return int(re.search(rf"constexpr int {name} = (\d+);", HDR).group(1))


KB, KAPPA, MIN_UNITS, MT = _const("KB"), _const("KAPPA"), _const("MIN_UNITS"), _const("MT_BF16")


def schedule(Qs, Ps, H, G):
    """(coverage count per unit, {(r, t): slots written}, {(r, t): slots the merge reads}, segments per group)"""
    gs = [(((Q * H + MT - 1) // MT), (P + Q + KB - 1) // KB) if Q >= 1 else (0, 0) for Q, P in zip(Qs, Ps)]
    U = sum(T * NB for T, NB in gs)
    if U <= 0:
        return np.zeros(0, int), {}, {}, []
    Ge = max(1, min(G, U // MIN_UNITS))
    V = sum(T * (NB + KAPPA) for T, NB in gs)
    ustart = np.cumsum([0] + [T * NB for T, NB in gs])
    vstart = np.cumsum([0] + [T * (NB + KAPPA) for T, NB in gs])

    def real_of(x):
        for r, (T, NB) in enumerate(gs):
            if x < vstart[r + 1]:
                t, off = divmod(x - vstart[r], NB + KAPPA)
                return ustart[r] + t * NB + max(off - KAPPA, 0)
        return U

    def locate(u):
        for r in range(len(gs)):
            if u < ustart[r + 1]:
                return r, ustart[r]
        return len(gs), U

    cover, writes, nsegs = np.zeros(U, int), {}, []
    for v in range(Ge):
        u0, u1 = real_of(v * V // Ge), real_of((v + 1) * V // Ge)
        if u0 >= u1:
            nsegs.append(0)
            continue
        r0, s0 = locate(u0)
        cursor = s0 + min(((u0 - s0) // gs[r0][1] + 1) * gs[r0][1], u1 - s0)
        first_done, n = False, 0
        while True:
            if cursor < u1:
                useg = cursor
            elif not first_done:
                useg, first_done = u0, True
            else:
                break
            r, st = locate(useg)
            NB = gs[r][1]
            t, bb = divmod(useg - st, NB)
            seg_end = min((t + 1) * NB, u1 - st)
            be = seg_end - t * NB
            cover[st + t * NB + bb: st + t * NB + be] += 1
            n += 1
            if not (bb == 0 and be == NB):
                writes.setdefault((r, t), set()).add(2 * v + (0 if useg == u0 else 1))
            if useg != u0:
                cursor = st + seg_end
        nsegs.append(n)

    def group_of(x):
        return ((x + 1) * Ge + V - 1) // V - 1

    reads = {}
    for r, (T, NB) in enumerate(gs):
        for t in range(T):
            vtile = vstart[r] + t * (NB + KAPPA)
            wf, wl = group_of(vtile + KAPPA), group_of(vtile + KAPPA + NB - 1)
            if wl != wf:
                reads[(r, t)] = {2 * w + (0 if w * V // Ge >= vtile else 1) for w in range(wf, wl + 1)}
    return cover, writes, reads, nsegs


def test_headline_batch():
    cover, writes, reads, nsegs = schedule([33] * 8, [8192] * 8, 64, 256)
    assert (cover == 1).all()
    assert writes == reads
    assert max(nsegs) <= 3


def test_random_batches_cover_once_and_merge_reads_what_is_written():
    rng = np.random.default_rng(11)
    for _ in range(150):
        bs = int(rng.integers(1, 24))
        H = int(rng.choice([1, 8, 64, 128]))
        Qs = [int(q) for q in rng.integers(0, 130, bs)]
        Ps = [int(p) for p in rng.integers(0, int(rng.choice([40, 3000, 40000])), bs)]
        G = int(rng.choice([256, 304, 80, 8]))
        cover, writes, reads, _ = schedule(Qs, Ps, H, G)
        assert (cover == 1).all(), (Qs, Ps, H, G)
        assert writes == reads, (Qs, Ps, H, G)
