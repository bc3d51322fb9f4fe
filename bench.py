#!/usr/bin/env python3
"""Benchmark of one DDTree verify step on one MI355X.

A step = build the draft trees -> compile visibility (bitsets + positions)
-> tree-verify attention -> greedy accept, over one batch of the workload
"64 heads, 33-node trees, 8k context": bs 8, 64 heads, budget 32 (q_len
33), prefix 8192 per request, bf16 latents in a 300k-slot pool, top-8
per-depth log-probs, seeded synthetic inputs.

Timing: W untimed warm-up steps, then exactly K steps between two
synchronisations, bracketed by HIP events on the stream every stage is
launched on.  Steps rotate over R independent instances (separate pools) so
more than 512 MB is touched between two uses of one instance, i.e. the
numbers are not served from the 256 MB last-level cache.  A first pass of K
steps records an event between the stages (the per-stage times and the
attention call's duration); ``ms_per_step`` comes from a second pass of K
steps with no event inside a step, since each event is a marker in the
launch queue that keeps the next small kernel's launch from overlapping
the previous kernel.

Prints one JSON line.  ``value`` = algorithmic attention TFLOP/s of the whole
step (attention flops / step time); ``roofline`` = the verify-attention call
(matrix-core kernel + partial merge) against the bf16 MFMA peak;
``cpu_baseline`` = the CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector ALUs (the fp32 path is not a matrix-core kernel)
FLOP_PER_PAIR = 2 * 576 + 2 * 512  # score dot product + value accumulation per (row, column)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=400.0,
                    help="untimed full steps run first, for this long, so that the timed steps "
                         "see the GPU's steady-state clocks")
    ap.add_argument("--config", type=int, default=3, help="workload 1..5 (default: the headline, 3)")
    ap.add_argument("--instances", type=int, default=8, help="rotated independent instances")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle sample budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the verify step (no commit, drafter top-k, tree sampling or "
                         "layer-batched lines), e.g. for a trace of the step's kernels alone")
    ap.add_argument("--ragged-instances", type=int, default=2,
                    help="instances of the ragged 32-request batch timed among the extras (0: skip)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run 5 device-to-device copies of this many MiB (counter calibration)")
    return ap.parse_args()


def copy_probe(mib: int) -> None:
    """Plain copies of known size: FETCH_SIZE / WRITE_SIZE of these dispatches
    give the factor that turns the counters into bytes."""
    import torch

    src = torch.ones(mib << 18, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": mib << 20, "copies": 5}), flush=True)


ATTN_SOURCES = ("tree_verify_mla_amd/csrc/verify_attn_bf16.hip", "tree_verify_mla_amd/csrc/verify_attn.hip",
                "tree_verify_mla_amd/csrc/attn_common.h", "tree_verify_mla_amd/csrc/attn_device.h")
COUNTERS = os.path.join(ROOT, "profiles", "verify_attn_h64_bs8_q33_p8192_counters.txt")


def attn_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per attention call from the committed counter summary, or None.

    The summary holds FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the two
    kernels of one call and of a plain copy of known size; the copy turns
    the counters into bytes.  The figures count only while the attention
    sources are the ones they were taken from."""
    try:
        with open(COUNTERS) as fh:
            kv = dict(l.strip().split("=", 1) for l in fh if "=" in l and not l.startswith("#"))
    except OSError:
        return None
    if kv.get("source_sha256") != attn_source_hash() or kv.get("workload") != workload:
        return None
    copy_kib = float(kv["copy_bytes"]) / 1024.0
    f_fac = copy_kib / float(kv["copy.FETCH_SIZE"])
    w_fac = copy_kib / float(kv["copy.WRITE_SIZE"])
    fetch = sum(float(kv[f"{k}.FETCH_SIZE"]) for k in ("attn_bf16_kernel", "merge_lanes_kernel"))
    write = sum(float(kv[f"{k}.WRITE_SIZE"]) for k in ("attn_bf16_kernel", "merge_lanes_kernel"))
    return {"fetch_bytes": fetch * 1024.0 * f_fac, "write_bytes": write * 1024.0 * w_fac,
            "fetch_factor": f_fac, "write_factor": w_fac}


def algorithmic_work(wl, depths):
    """(attention flops, attention bytes) the method itself needs for this batch."""
    H = wl.heads
    flops = 0
    nbytes = 0
    elt = 2 if wl.dtype == "bf16" else 4
    W = (wl.max_q_len + 31) // 32
    for r in range(wl.bs):
        a, b = int(wl.qo_indptr[r]), int(wl.qo_indptr[r + 1])
        P = int(wl.prefix_lens[r])
        Q = b - a
        visible = Q * P + int((np.asarray(depths[a:b]) + 1).sum())
        flops += FLOP_PER_PAIR * H * visible
        nbytes += (P + Q) * 576 * elt + (P + Q) * 4          # latent rows once + slot indices
        nbytes += Q * H * (576 + 512) * elt + Q * H * 4      # q in, out + lse
        nbytes += Q * W * 4                                   # ancestor bitsets
    return flops, nbytes


def commit_bytes(wl, accept_len, move: bool) -> int:
    """Bytes ddtree_commit_kv needs: the prefix slot ids read and written, the
    path entries, node slots and new entries, the per-request scalars, and in
    the move form each moved latent row read and written once."""
    row = 576 * (2 if wl.dtype == "bf16" else 4)
    n = 0
    for r in range(wl.bs):
        P, a = int(wl.prefix_lens[r]), int(accept_len[r])
        n += 8 * P + 12 * a + 5 * 4
        if move:
            n += 2 * row * max(a - 1, 0)
    return n + 4 * (wl.bs + 1)


def time_commit(steps, K, stream, move: bool):
    """Average duration (ms) of ddtree_commit_kv over K calls (HIP events on
    the launch stream), rotating the instances like the main loop."""
    import torch

    R = len(steps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for i in range(3):
        st = steps[i % R]
        st.commit(kv_pool=st.x.kv_pool if move else None, stream=stream)
    torch.cuda.synchronize()
    for i in range(K):
        st = steps[i % R]
        ev[i][0].record(stream)
        st.commit(kv_pool=st.x.kv_pool if move else None, stream=stream)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return sum(e[0].elapsed_time(e[1]) for e in ev) / K


DRAFTER_VOCAB = 163840  # the pages give no vocabulary size: a large-model vocabulary


def time_drafter_topk(wl, R: int, K: int, stream):
    """Average duration (ms) of ddtree_drafter_topk on bs * depth rows of
    DRAFTER_VOCAB fp32 logits (R rotated instances), and its bytes."""
    import torch

    from tree_verify_mla_amd import _lib
    from workloads import draw_drafter_logits

    rows, k = wl.bs * wl.depth, wl.topk
    xs = [torch.from_numpy(draw_drafter_logits(np.random.default_rng(wl.seed + 7919 * (i + 1)), rows,
                                               DRAFTER_VOCAB)).cuda() for i in range(R)]
    vals = torch.empty(rows, k, dtype=torch.float32, device="cuda")
    ids = torch.empty(rows, k, dtype=torch.int32, device="cuda")
    ws = torch.empty(_lib.ddtree_drafter_topk_workspace_size(rows, DRAFTER_VOCAB, k),
                     dtype=torch.uint8, device="cuda")
    for i in range(3):
        _lib.ddtree_drafter_topk(xs[i % R], vals, ids, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        _lib.ddtree_drafter_topk(xs[i % R], vals, ids, workspace=ws, stream=stream)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    nbytes = rows * DRAFTER_VOCAB * 4 + rows * k * 8
    return ms, rows, k, nbytes


def time_tree_sample(st, wl, K: int, stream, vocab: int = DRAFTER_VOCAB):
    """Average duration (ms) of ddtree_tree_sample over K calls on the step's
    tree (drawn target rows of `vocab` tokens for every node; four rotated sets
    of coins), the mean accepted length, and the bytes: every node's target
    row read once (the block masses of all rows are formed before the walk)."""
    import torch

    from tree_verify_mla_amd import _lib
    from workloads import draw_target_probs

    x = st.x
    tok, par = st.node_tokens.cpu().numpy(), st.node_parents.cpu().numpy()
    probs = torch.from_numpy(draw_target_probs(wl.seed, tok, par, wl.qo_indptr, vocab)).cuda()
    rng = np.random.default_rng(wl.seed + 31337)
    coins = [torch.from_numpy(rng.random(wl.total_q).astype(np.float32)).cuda() for _ in range(4)]
    bonus_u = [torch.from_numpy(rng.random(wl.bs).astype(np.float32)).cuda() for _ in range(4)]
    D = wl.depth
    outs = [[torch.empty(wl.bs, D + 1, dtype=torch.int32, device="cuda"),
             torch.empty(wl.bs, dtype=torch.int32, device="cuda"),
             torch.empty(wl.bs, D + 1, dtype=torch.int32, device="cuda"),
             torch.empty(wl.bs, dtype=torch.int32, device="cuda")] for _ in range(4)]

    ws = torch.empty(_lib.ddtree_tree_sample_workspace_size(wl.total_q), dtype=torch.uint8,
                     device="cuda")

    def run(i):
        _lib.ddtree_tree_sample(st.node_tokens, st.node_parents, x.qo_indptr, probs, coins[i % 4],
                                bonus_u[i % 4], D, *outs[i % 4], workspace=ws, stream=stream)

    for i in range(4):
        run(i)
    torch.cuda.synchronize()
    alen = float(np.mean([o[1].cpu().numpy().mean() for o in outs]))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        run(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    # the method reads the target row of every node on the accepted paths
    # (accept_len rows per request) and the children's probabilities; the
    # kernels read every node's row to form the block masses beforehand
    alg = sum(int(o[1].cpu().numpy().sum()) for o in outs) / len(outs) * vocab * 4
    return ms, alen, alg, wl.total_q * vocab * 4


def measured_peaks(stream) -> dict:
    """The device's own side of the roofline ratios: compute units and peak
    clock as the runtime reports them, the rate of a loop of nothing but
    bf16 32x32x16 matrix-core instructions (one workgroup of four waves per
    compute unit, eight independent accumulators per wave), and the rate of
    a 512 MiB device-to-device copy (bytes read + written).  Medians of 10
    timed launches after 3 untimed."""
    import torch
    from tree_verify_mla_amd import _lib

    cus, khz = _lib.ddtree_device_info()
    grid = cus
    out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")

    def med(fn, n=10):
        for _ in range(3):
            fn()
        ts = []
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    flops = grid * 4 * 4096 * 8 * 32768
    t_mfma = med(lambda: _lib.ddtree_probe_mfma_loop(grid, 4096, out, stream=stream))
    src = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t_copy = med(lambda: dst.copy_(src))
    copy_bytes = 2 * src.numel() * 4
    del src, dst
    mfma = flops / t_mfma / 1e12
    copy = copy_bytes / t_copy / 1e9
    return {"compute_units": cus, "peak_clock_MHz": round(khz / 1e3),
            "mfma_bf16_loop_TFLOPs": round(mfma, 1), "mfma_loop_frac_of_published": round(mfma / PEAK_BF16_TFLOPS, 4),
            "copy_GBps": round(copy, 1), "copy_frac_of_published": round(copy / PEAK_HBM_GBPS, 4)}


def time_layers(cfg_index: int, L: int, K: int, stream):
    """ddtree_verify_attn_layers over L layers (seeded latents per layer, one
    slot list) against L back-to-back ddtree_verify_attn calls: average ms of
    one layered call and of the L single calls."""
    import torch

    from tree_verify_mla_amd import _lib
    from tree_verify_mla_amd.step import VerifyStep
    from workloads import draw_layer, get_config, make_workload
    from workloads.device import to_device

    wl0 = make_workload(get_config(cfg_index))
    xs = [to_device(w, "cuda") for w in [wl0] + [draw_layer(wl0, l) for l in range(1, L)]]
    st = VerifyStep(xs[0])
    st.build(stream)
    st.visibility(stream)
    q = torch.stack([x.q for x in xs]).contiguous()
    pool = torch.stack([x.kv_pool for x in xs]).contiguous()
    del xs[1:]
    x0 = xs[0]
    T, H = x0.q.shape[0], x0.q.shape[1]
    out = torch.empty(L, T, H, 512, dtype=q.dtype, device="cuda")
    lse = torch.empty(L, T, H, dtype=torch.float32, device="cuda")
    dt = _lib.DDTREE_BF16 if q.dtype == torch.bfloat16 else _lib.DDTREE_F32
    ws = torch.empty(max(1, _lib.ddtree_verify_attn_layers_workspace_size(
        L, wl0.bs, H, wl0.max_q_len, wl0.max_kv_len, 0, dt)), dtype=torch.uint8, device="cuda")
    sc = float(np.float32(wl0.scale))
    args = (x0.kv_indptr, x0.kv_indices, x0.qo_indptr, st.vis_bits, wl0.max_q_len, wl0.max_kv_len, sc)

    def layered():
        _lib.ddtree_verify_attn_layers(q, pool, *args, out, lse, workspace=ws, stream=stream)

    def singles():
        for l in range(L):
            _lib.ddtree_verify_attn(q[l], pool[l], *args, out[l], lse[l], workspace=ws, stream=stream)

    # warm both up together for at least 200 ms, so neither is timed at low clocks
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.2:
        layered()
        singles()
        torch.cuda.synchronize()
    res = []
    for fn in (layered, singles):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(K):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) / K)
    return {"workload": wl0.name, "layers": L, "layered_call_us": round(res[0] * 1e3, 2),
            "single_calls_us": round(res[1] * 1e3, 2),
            "per_layer_us": {"layered": round(res[0] * 1e3 / L, 2), "single": round(res[1] * 1e3 / L, 2)},
            "speedup": round(res[1] / res[0], 3)}


def dist_us(ms) -> dict:
    """Median, 10th and 90th percentile (us) and count of per-call durations (ms)."""
    a = np.asarray(ms, dtype=np.float64) * 1e3
    return {"median_us": round(float(np.median(a)), 2), "p10_us": round(float(np.percentile(a, 10)), 2),
            "p90_us": round(float(np.percentile(a, 90)), 2), "mean_us": round(float(a.mean()), 2),
            "calls": int(a.size)}


def attention_modes(steps, stream, n: int) -> dict:
    """The attention call timed two more ways beside the cold rotation:
    warm = one instance called back to back (its data stays in the caches);
    graph = n calls over the rotated instances captured in one HIP graph and
    replayed (no launch gaps), per call = replay time / n."""
    import torch

    st = steps[0]
    for _ in range(20):
        st.attention(stream)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
    for i in range(n):
        ev[i][0].record(stream)
        st.attention(stream)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    warm = dist_us([e[0].elapsed_time(e[1]) for e in ev])

    R = len(steps)
    s = torch.cuda.Stream()
    s.wait_stream(stream)
    with torch.cuda.stream(s):
        for i in range(R):
            steps[i].attention(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(n):
            steps[i % R].attention(s)
    torch.cuda.synchronize()
    reps = []
    for _ in range(4):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        reps.append(e0.elapsed_time(e1) / n)
    del g
    graph = {"per_call_us": round(float(np.median(reps[1:])) * 1e3, 2), "calls_per_replay": n,
             "replays": len(reps) - 1}
    return {"warm": warm, "graph": graph}


def ragged_batch_line(instances: int, K: int, stream) -> dict:
    """The ragged end-to-end workload (32 requests, 64 heads, prefixes
    1k-32k, budgets 16/32/64): whole verify steps (build + visibility ->
    attention -> accept) over rotated instances, tree-steps/s from the median
    step, the attention call against the bf16 MFMA peak, and the histogram of
    accepted lengths (root included) under the synthetic target predictions."""
    import torch

    from tree_verify_mla_amd.step import VerifyStep
    from workloads import draw_target_predict, get_config, make_workload
    from workloads.device import to_device

    cfg = get_config(5)
    wls, steps = [], []
    for k in range(instances):
        wl = make_workload(cfg, seed=cfg.seed + 1000 * k, unused="zero")
        st = VerifyStep(to_device(wl, "cuda"))
        st.build_visibility()
        torch.cuda.synchronize()
        tok, par = st.node_tokens.cpu().numpy(), st.node_parents.cpu().numpy()
        st.x.target_predict = torch.from_numpy(
            draw_target_predict(wl.seed, tok, par, wl.qo_indptr, wl.vocab)).cuda()
        wls.append(wl)
        steps.append(st)
    flops = [algorithmic_work(w, s.node_depths.cpu().numpy())[0] for w, s in zip(wls, steps)]
    R = len(steps)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.3:
        for st in steps:
            st.run(stream)
        torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    for i in range(K):
        st = steps[i % R]
        ev[i][0].record(stream)
        st.build_visibility(stream)
        ev[i][1].record(stream)
        st.attention(stream)
        ev[i][2].record(stream)
        st.accept(stream=stream)
        ev[i][3].record(stream)
    torch.cuda.synchronize()
    step_ms = np.array([e[0].elapsed_time(e[3]) for e in ev])
    attn_tflops = [flops[i % R] / (ev[i][1].elapsed_time(ev[i][2]) * 1e-3) / 1e12 for i in range(K)]
    alen = np.concatenate([st.accept_len.cpu().numpy() for st in steps])
    hist = {int(v): int(c) for v, c in zip(*np.unique(alen, return_counts=True))}
    bs = wls[0].bs
    return {"workload": wls[0].name, "instances": R, "steps": K,
            "total_q": [w.total_q for w in wls], "step": dist_us(step_ms),
            "tree_steps_per_s": round(bs / (float(np.median(step_ms)) * 1e-3), 1),
            "attention_TFLOPs_median": round(float(np.median(attn_tflops)), 1),
            "mfma_frac_median": round(float(np.median(attn_tflops)) / PEAK_BF16_TFLOPS, 4),
            "accept_len_histogram": hist, "mean_accept_len": round(float(alen.mean()), 3)}


def cpu_baseline(wls, budget_s: float):
    """The CPU oracle as it stands, on whole requests of the workload (cycling
    through the rotated instances) until about budget_s seconds are used."""
    from threadpoolctl import threadpool_info

    from oracle import accept, attention, drafter, tree, visibility
    from workloads import draw_target_predict

    done, flops, t0 = 0, 0, time.perf_counter()
    for wl in wls:
        for r in range(wl.bs):
            a, b = int(wl.qo_indptr[r]), int(wl.qo_indptr[r + 1])
            if wl.drafter_logits is not None:   # the drafter stage first
                lp, ids = drafter.batch(wl.drafter_logits[r], wl.topk)
            else:
                lp, ids = wl.topk_logprobs[r], wl.topk_ids[r]
            t = tree.build_tree(lp, ids, int(wl.root_tokens[r]), b - a - 1)
            P = int(wl.prefix_lens[r])
            visibility.vis_bits(t.parents, (wl.max_q_len + 31) // 32)
            visibility.positions(t.depths, P)
            attention.verify_request(wl.q_f32()[a:b], wl.kv_rows_f32(wl.request_slots(r)), P,
                                     t.parents, float(np.float32(wl.scale)))
            pred = draw_target_predict(wl.seed, t.tokens, t.parents, np.array([0, b - a]), wl.vocab)
            accept.accept(t.tokens, t.parents, pred, wl.depth)
            flops += FLOP_PER_PAIR * wl.heads * ((b - a) * P + int((t.depths + 1).sum()))
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    total = sum(w.bs for w in wls)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {total} requests of the {len(wls)} rotated instances (tree + "
                      f"visibility + fp64 attention + accept, whole requests), {dt:.1f} s wall, "
                      f"{len(os.sched_getaffinity(0))} host cores visible",
            "tree_steps_per_s": done / dt}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the verify path is built and timed on a single MI355X; "
              "run it with --gpus 1 (sharding across GPUs is not built).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib)
        return

    from tree_verify_mla_amd.step import VerifyStep
    from workloads import draw_target_predict, get_config, make_workload
    from workloads.device import to_device

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    cfg = get_config(args.config)

    # ---- instances (rotated so the timed steps do not run out of cache) ----
    R = max(1, args.instances)
    wls, steps = [], []
    for k in range(R):
        wl = make_workload(cfg, seed=cfg.seed + 1000 * k, unused="zero")
        x = to_device(wl, "cuda")
        st = VerifyStep(x, num_splits=args.num_splits)
        st.build()
        torch.cuda.synchronize()
        tok = st.node_tokens.cpu().numpy()
        par = st.node_parents.cpu().numpy()
        x.target_predict = torch.from_numpy(
            draw_target_predict(wl.seed, tok, par, wl.qo_indptr, wl.vocab)).cuda()
        wls.append(wl)
        steps.append(st)
        print(f"instance {k}: {wl.name} bs={wl.bs} H={wl.heads} total_q={wl.total_q} "
              f"max_kv={wl.max_kv_len}", file=sys.stderr, flush=True)
    depths = steps[0].node_depths.cpu().numpy()
    flops, nbytes = algorithmic_work(wls[0], depths)

    stream = torch.cuda.current_stream()
    # Clock settle: a GPU that was idle through the set-up above needs on the
    # order of a hundred milliseconds of load before its clocks reach their
    # steady state; the W warmup steps alone can be far shorter.
    settle_steps = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(20):
            steps[settle_steps % R].run(stream)
            settle_steps += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        steps[i % R].run(stream)
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(K):
        st = steps[i % R]
        e = ev[i]
        e[0].record(stream)
        st.build_visibility(stream)
        e[1].record(stream)
        st.attention(stream)
        e[2].record(stream)
        st.accept(stream=stream)
        e[3].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    staged_step_ms = t_start.elapsed_time(t_end) / K
    tv_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    # The same K steps again with no event inside a step (the events above
    # give the per-stage times; each one is a marker in the launch queue).
    for i in range(args.warmup):
        steps[i % R].run(stream)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(K):
        steps[i % R].run(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    step_ms = t_start.elapsed_time(t_end) / K
    attn_calls = np.array([e[1].elapsed_time(e[2]) for e in ev])
    attn_ms = float(attn_calls.mean())
    acc_ms = sum(e[2].elapsed_time(e[3]) for e in ev) / K
    modes = {"cold": dist_us(attn_calls)}
    if not args.no_extras:
        modes.update(attention_modes(steps, stream, max(K, 100)))

    extras = None
    if not args.no_extras:
        # the KV commit after acceptance (not part of a step): index form, then
        # the move form, last, since it compacts the instances' pools in place
        alens = [st.accept_len.cpu().numpy() for st in steps]
        cb_i = sum(commit_bytes(wls[k], alens[k], False) for k in range(R)) / R
        cb_m = sum(commit_bytes(wls[k], alens[k], True) for k in range(R)) / R
        commit_i_ms = time_commit(steps, K, stream, move=False)
        commit_m_ms = time_commit(steps, K, stream, move=True)
        # the drafter's per-depth top-k (the stage before the tree build; not part of a step)
        dk_ms, dk_rows, dk_k, dk_bytes = time_drafter_topk(wls[0], R, K, stream)
        # stochastic acceptance along the tree (the alternative to greedy accept)
        ts_ms, ts_alen, ts_bytes, ts_read = time_tree_sample(steps[0], wls[0], K, stream)
        ragged = ragged_batch_line(args.ragged_instances, max(20, K // 5), stream) \
            if args.ragged_instances > 0 else None
        # one launch over several layers against one launch per layer
        layers = [time_layers(2, 16, K, stream), time_layers(3, 4, max(5, K // 5), stream)]
        peaks = measured_peaks(stream)
        extras = {
              "measured_peaks": peaks,
              "commit_kv": {
                  "index_form_us": round(commit_i_ms * 1e3, 2),
                  "index_form_bytes": round(cb_i),
                  "index_form_GBps": round(cb_i / (commit_i_ms * 1e-3) / 1e9, 1),
                  "move_form_us": round(commit_m_ms * 1e3, 2),
                  "move_form_bytes": round(cb_m),
                  "move_form_GBps": round(cb_m / (commit_m_ms * 1e-3) / 1e9, 1),
                  "hbm_peak_GBps": PEAK_HBM_GBPS},
              "drafter_topk": {
                  "rows": dk_rows, "vocab": DRAFTER_VOCAB, "k": dk_k, "dtype": "f32",
                  "us": round(dk_ms * 1e3, 2), "bytes": dk_bytes,
                  "GBps": round(dk_bytes / (dk_ms * 1e-3) / 1e9, 1),
                  "hbm_frac": round(dk_bytes / (dk_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)},
              "tree_sample": {
                  "vocab": DRAFTER_VOCAB, "us": round(ts_ms * 1e3, 2),
                  "mean_accept_len": round(ts_alen, 3),
                  "algorithmic_bytes": round(ts_bytes),
                  "GBps": round(ts_bytes / (ts_ms * 1e-3) / 1e9, 1),
                  "hbm_frac": round(ts_bytes / (ts_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                  "kernel_read_bytes": ts_read,
                  "kernel_read_GBps": round(ts_read / (ts_ms * 1e-3) / 1e9, 1)},
              "ragged_batch": ragged,
              "verify_attn_layers": layers}

    achieved = flops / (attn_ms * 1e-3) / 1e12
    bf16 = wls[0].dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    traffic = measured_traffic(wls[0].name)
    value = flops / (step_ms * 1e-3) / 1e12
    gbps = nbytes / (attn_ms * 1e-3) / 1e9
    line = {
        "metric": "verify-attn TFLOP/s + % of MFMA/HBM roofline, 33-node tree, 64 heads, 8k ctx",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle": {"ms": args.settle_ms, "steps": settle_steps},
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wls[0].dtype == "bf16" else "f32",
        "data": "synthetic (seeded; random latents, " + (
            "drafter top-k from N(0,1) logits)" if wls[0].drafter_logits is not None
            else "drawn drafter top-k tables)"),
        "config": {"workload": wls[0].name, "bs": wls[0].bs, "heads": wls[0].heads,
                   "q_len": int(wls[0].max_q_len), "prefix": int(wls[0].prefix_lens.max()),
                   "topk": wls[0].topk, "pool_slots": wls[0].num_slots, "instances": R,
                   "num_splits": args.num_splits, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma" if bf16 else "alu",
                     "kernel": "ddtree_verify_attn (attn_bf16_kernel + merge_lanes_kernel)" if bf16
                     else "ddtree_verify_attn (attn_f32_kernel)",
                     "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": None if traffic is None else round(traffic["fetch_bytes"] + traffic["write_bytes"]),
                     "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": nbytes,
                     "traffic_detail": traffic},
        "attention_call": modes,
        "extra": {"step_us_with_stage_events": round(staged_step_ms * 1e3, 2),
                  "attn_ms": round(attn_ms, 5), "build_visibility_ms": round(tv_ms, 5),
                  "accept_ms": round(acc_ms, 5),
                  "attn_GBps": round(gbps, 1), "attn_hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
                  "tree_steps_per_s": round(wls[0].bs / (step_ms * 1e-3), 1),
                  **(extras or {})},
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(wls, args.cpu_seconds)
        # the same step on the GPU against the oracle on the host cores
        cb["gpu_speedup"] = {"flops_rate": round(value / cb["value"], 1),
                             "tree_steps": round(line["extra"]["tree_steps_per_s"] / cb["tree_steps_per_s"], 1)}
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
