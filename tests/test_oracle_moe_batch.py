"""Pins of the prompt-batch routed-expert oracle: sort_by_expert (slots
grouped by expert) and ref_moe_batch (each token's routed products).

sort_by_expert is checked against examples worked by hand, against numpy's
stable argsort (a library routine that orders the same keys by another
algorithm), and against the invariants of a grouping.  ref_moe_batch is
checked against the one-token routed product and the multi-column product,
both pinned in test_oracle_products.py.
"""
import numpy as np

import oracle
from test_oracle_products import _tiny_matrix


def test_sort_by_expert_hand_examples():
    # slots 0..3 = (token 0: experts 2, 0), (token 1: experts 0, 1)
    # expert 0 <- slots 1, 2; expert 1 <- slot 3; expert 2 <- slot 0
    off, order = oracle.sort_by_expert(np.array([[2, 0], [0, 1]]), 3)
    assert off.tolist() == [0, 2, 3, 4]
    assert order.tolist() == [1, 2, 3, 0]
    # ids outside [0, E) are left out; an expert nobody chose has an empty range
    off, order = oracle.sort_by_expert(np.array([5, -1, 2, 2, 0]), 4)
    assert off.tolist() == [0, 1, 1, 3, 3]
    assert order.tolist() == [4, 2, 3]
    off, order = oracle.sort_by_expert(np.array([], np.int32), 2)
    assert off.tolist() == [0, 0, 0] and order.size == 0


def test_sort_by_expert_matches_stable_argsort():
    rng = np.random.default_rng(21)
    for trial in range(30):
        E = int(rng.integers(1, 40))
        S = int(rng.integers(0, 300))
        ids = rng.integers(-3, E + 3, S)
        off, order = oracle.sort_by_expert(ids, E)
        valid = np.flatnonzero((ids >= 0) & (ids < E))
        want = valid[np.argsort(ids[valid], kind="stable")]
        assert np.array_equal(order, want)
        counts = np.bincount(ids[valid], minlength=E)
        assert np.array_equal(off, np.concatenate([[0], np.cumsum(counts)]))


def test_sort_by_expert_invariants():
    rng = np.random.default_rng(22)
    E = 16
    ids = np.stack([rng.choice(E, 4, replace=False) for _ in range(50)]).reshape(-1)
    off, order = oracle.sort_by_expert(ids, E)
    assert sorted(order.tolist()) == list(range(ids.size))       # every slot once
    for e in range(E):
        seg = order[off[e]:off[e + 1]]
        assert (ids[seg] == e).all()
        assert (np.diff(seg) > 0).all()                           # slot order kept


def test_moe_batch_is_each_tokens_routed_product():
    E, N, K, T, top_k = 4, 3, 64, 5, 3
    bank = np.stack([_tiny_matrix(N, K, seed=70 + e) for e in range(E)])
    a = np.random.default_rng(23).standard_normal((T, K)).astype(np.float32)
    q, d = oracle.quantize_acts(a)
    ids = np.array([[0, 1, 2], [3, 3, 0], [2, 9, 1], [1, 0, -2], [0, 1, 2]], np.int32)
    y = oracle.ref_moe_batch(bank.reshape(-1), E, N, K, ids, q, d)
    assert y.shape == (T * top_k, N)
    for t in range(T):
        one = oracle.ref_moe_gemv(bank.reshape(-1), E, N, K, ids[t], q[t:t + 1], d[t:t + 1])
        assert np.array_equal(y[t * top_k:(t + 1) * top_k], one, equal_nan=True)
    assert np.isnan(y[7]).all() and np.isnan(y[11]).all()


def test_moe_batch_one_expert_is_the_multi_column_product():
    E, N, K, T = 3, 4, 96, 6
    bank = np.stack([_tiny_matrix(N, K, seed=80 + e) for e in range(E)])
    a = np.random.default_rng(24).standard_normal((T, K)).astype(np.float32)
    q, d = oracle.quantize_acts(a)
    y = oracle.ref_moe_batch(bank.reshape(-1), E, N, K, np.full((T, 1), 2), q, d)
    assert np.allclose(y, oracle.ref_gemv(bank[2], N, K, q, d), rtol=1e-15, atol=0)
