"""Pins for ``oracle.attention.verify_request_layers`` (layer-batched verify).

The layered oracle shares one mask across layers; what could go wrong is
mixing layers (a layer read with another layer's queries or latents, a
stride error, the mask of one layer reused with the wrong columns).  Pinned
by invariants that do not restate it:

* locality: changing layer j's queries or latents changes layer j's output
  and leaves every other layer's output bit-identical;
* equivariance: permuting the layers permutes the outputs;
* a layer whose latents put one column far above the others (a spike
  visible to a node) returns that column's value row (the softmax limit),
  whatever the other layers hold;
* identical layers give identical outputs, equal to the single-layer
  oracle's.
"""
import numpy as np

from oracle import attention, tree
from workloads import draw_layer, get_config, make_workload


def _request(wl, r, parents):
    a, b = int(wl.qo_indptr[r]), int(wl.qo_indptr[r + 1])
    return wl.q_f32()[a:b], wl.kv_rows_f32(wl.request_slots(r)), int(wl.prefix_lens[r]), parents[a:b]


def _setup(L=3):
    wl0 = make_workload(get_config(1), bs=2, heads=2, budgets=[6, 3], prefixes=[5, 9],
                        pool_slots=64, dtype="f32")
    from tests._oracle_side import oracle_tables
    lp, ids = oracle_tables(wl0)
    _, _, parents, _, _ = tree.build_batch(lp, ids, wl0.root_tokens, wl0.qo_indptr)
    wls = [wl0] + [draw_layer(wl0, l) for l in range(1, L)]
    return wls, parents


def _layers(wls, parents, r):
    qs, kvs = [], []
    for w in wls:
        q, kv, P, par = _request(w, r, parents)
        qs.append(q)
        kvs.append(kv)
    return qs, kvs, P, par


def test_locality():
    wls, parents = _setup()
    scale = float(np.float32(wls[0].scale))
    qs, kvs, P, par = _layers(wls, parents, 0)
    base = attention.verify_request_layers(qs, kvs, P, par, scale)
    for j in range(len(wls)):
        q2, kv2 = list(qs), list(kvs)
        kv2[j] = kv2[j] * 1.5 + 0.25
        q2[j] = q2[j][::-1].copy()
        got = attention.verify_request_layers(q2, kv2, P, par, scale)
        for l in range(len(wls)):
            same = np.array_equal(got[l][0], base[l][0]) and np.array_equal(got[l][1], base[l][1])
            assert same == (l != j), (j, l)


def test_permutation_equivariance():
    wls, parents = _setup(4)
    scale = float(np.float32(wls[0].scale))
    qs, kvs, P, par = _layers(wls, parents, 1)
    base = attention.verify_request_layers(qs, kvs, P, par, scale)
    perm = [2, 0, 3, 1]
    got = attention.verify_request_layers([qs[i] for i in perm], [kvs[i] for i in perm], P, par,
                                          scale)
    for k, i in enumerate(perm):
        assert np.array_equal(got[k][0], base[i][0]) and np.array_equal(got[k][1], base[i][1])


def test_spike_layer_returns_the_spiked_row():
    wls, parents = _setup()
    scale = float(np.float32(wls[0].scale))
    qs, kvs, P, par = _layers(wls, parents, 0)
    kv = kvs[1].copy()
    # column 2 (a prefix column, visible to every node) aligned with each query: make it dominate
    kv[2, :512] = np.linspace(-1.0, 1.0, 512)
    kv[2, 512:] = 400.0
    q = qs[1].copy()
    q[..., 512:] = np.abs(q[..., 512:]) + 1.0
    kvs2, qs2 = list(kvs), list(qs)
    kvs2[1], qs2[1] = kv, q
    out = attention.verify_request_layers(qs2, kvs2, P, par, scale)
    assert np.allclose(out[1][0], kv[2, :512][None, None, :], atol=1e-9)
    ref = attention.verify_request_layers(qs, kvs, P, par, scale)
    assert np.array_equal(out[0][0], ref[0][0]) and np.array_equal(out[2][0], ref[2][0])


def test_identical_layers_match_single_layer():
    wls, parents = _setup()
    scale = float(np.float32(wls[0].scale))
    q, kv, P, par = _request(wls[0], 1, parents)
    got = attention.verify_request_layers([q, q, q], [kv, kv, kv], P, par, scale)
    one = attention.verify_request(q, kv, P, par, scale)
    for o, lse in got:
        assert np.array_equal(o, one[0]) and np.array_equal(lse, one[1])
