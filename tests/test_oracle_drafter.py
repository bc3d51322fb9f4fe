"""Pins for ``oracle.drafter`` (per-depth top-k log-probabilities).

* closed forms: equal logits give -log V for every token and ids 0 .. k-1
  (ties in ascending id); one logit L above V - 1 zeros gives
  L - log(e^L + V - 1) for it and -log(e^L + V - 1) for the rest;
* an independent library routine: scipy.special.log_softmax on random rows,
  and numpy's stable argsort for the order;
* invariants: adding a constant to a row changes nothing; the exponentials
  of a row's log-probabilities sum to 1;
* brute force on small rows: every token left out has a log-probability no
  larger than the k-th kept one, and equal values are kept lowest id first.
"""
import numpy as np
import pytest
from scipy.special import log_softmax as sp_log_softmax

from oracle import drafter


def test_uniform_row():
    V, k = 1000, 8
    vals, ids = drafter.topk_row(np.zeros(V, np.float32), k)
    assert np.allclose(vals, -np.log(V), atol=1e-6)
    assert ids.tolist() == list(range(k))


def test_single_spike():
    V, k, L, j = 5000, 6, 7.5, 4321
    x = np.zeros(V, np.float32)
    x[j] = L
    vals, ids = drafter.topk_row(x, k)
    z = np.log(np.exp(L) + V - 1)
    assert ids.tolist() == [j, 0, 1, 2, 3, 4]
    assert abs(vals[0] - (L - z)) < 1e-6
    assert np.allclose(vals[1:], -z, atol=1e-6)


def test_against_scipy():
    rng = np.random.default_rng(3)
    for V in (7, 512, 4097, 65536):
        x = (rng.standard_normal(V) * 3).astype(np.float32)
        ref = sp_log_softmax(x.astype(np.float64))
        assert np.allclose(drafter.log_softmax(x), ref, atol=1e-12)
        k = min(16, V)
        order = np.argsort(-ref, kind="stable")[:k]
        vals, ids = drafter.topk_row(x, k)
        assert ids.tolist() == order.tolist()
        assert np.array_equal(vals, ref[order].astype(np.float32))


def test_shift_invariance_and_normalisation():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(3000).astype(np.float32)
    a = drafter.topk_row(x, 10)
    b = drafter.topk_row(x + np.float32(123.0), 10)
    assert a[1].tolist() == b[1].tolist()
    assert np.allclose(a[0], b[0], atol=1e-5)
    assert abs(np.exp(drafter.log_softmax(x)).sum() - 1.0) < 1e-12


@pytest.mark.parametrize("V,k", [(1, 1), (5, 5), (9, 3), (40, 16)])
def test_bruteforce_small_rows_with_ties(V, k):
    rng = np.random.default_rng(V * 31 + k)
    for trial in range(20):
        x = rng.integers(-3, 4, size=V).astype(np.float32)   # many equal values
        vals, ids = drafter.topk_row(x, k)
        lp = drafter.log_softmax(x)
        kept = set(ids.tolist())
        kth = lp[ids[-1]]
        for j in range(V):
            if j not in kept:
                assert lp[j] < kth or (lp[j] == kth and j > ids[-1])
        for a, b in zip(ids[:-1], ids[1:]):
            assert lp[a] > lp[b] or (lp[a] == lp[b] and a < b)
