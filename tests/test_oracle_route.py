"""Pins of the oracle's routing: block means, block softmax, Top-p, the Top-k floor and Eq. 1.

Fixed independently of the oracle's code by:
  * block means: a constant block pools to that constant; pooling a grid tensor
    through the Hilbert gather equals the mean over the block's cells taken
    straight from the grid by explicit loops;
  * softmax: rows sum to one; adding one vector to every key summary leaves P
    unchanged (a per-row constant shift of the scores);
  * Top-p (FVAttn explainer, "Key Concepts"): minimality CDF_{c-1} < p <= CDF_c;
    nested sets and monotone counts in p; p = 1 keeps all; uniform scores give
    c = ceil(p * nb) lowest ids; brute force over all subsets for nb <= 10 gives
    the same smallest size reaching p; hand-derived golden rows
    (tests/golden/topp_cases.json);
  * floor: every tile keeps at least min(k, nb) blocks, and the floor only
    extends the same importance order;
  * Eq. 1 (xllm-io review of FVAttn, 核心公式): L_h = sum_i count'_{h,i} / nb.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import absh_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- block means

def test_constant_block_pools_to_constant():
    xh = np.full((1, 2, 37, 8), 0.375, dtype=np.float32)
    xh[0, 1] = -2.5
    m = O.block_means(xh, 16)
    assert m.shape == (1, 2, 3, 8)
    assert (m[0, 0] == np.float32(0.375)).all() and (m[0, 1] == np.float32(-2.5)).all()


def test_pooling_equals_direct_cell_mean():
    rng = np.random.default_rng(3)
    T, Y, X, H, d, b = 3, 5, 6, 2, 4, 8
    N = T * Y * X
    x = rng.standard_normal((1, N, H, d)).astype(np.float32)
    perm, _ = O.hilbert_perm(T, Y, X)
    got = O.block_means(O.to_hilbert(x, perm), b)
    for h in range(H):
        for j in range(-(-N // b)):
            cells = perm[j * b: min((j + 1) * b, N)]
            acc = [0.0] * d
            for n in cells:
                for c in range(d):
                    acc[c] += float(x[0, n, h, c])
            want = np.array([a / len(cells) for a in acc], dtype=np.float32)
            assert np.allclose(got[0, h, j], want, rtol=0, atol=1e-6)


def test_partial_tail_block_uses_true_count():
    xh = np.ones((1, 1, 20, 2), dtype=np.float32)
    xh[0, 0, 16:] = 3.0
    m = O.block_means(xh, 16)
    assert (m[0, 0, 1] == 3.0).all()          # 4 tokens of value 3, not 3*4/16
    assert list(O.block_sizes(20, 16)) == [16, 4]


# ---------------------------------------------------------------- softmax

def test_softmax_rows_sum_to_one_and_shift_invariance():
    rng = np.random.default_rng(5)
    qbar = rng.standard_normal((3, 11, 16)).astype(np.float32)
    kbar = rng.standard_normal((3, 11, 16)).astype(np.float32)
    P = O.block_softmax(O.block_scores(qbar, kbar))
    assert np.allclose(P.sum(-1), 1.0, atol=1e-12)
    u = rng.standard_normal(16).astype(np.float32)
    P2 = O.block_softmax(O.block_scores(qbar, kbar + u))
    assert np.allclose(P, P2, atol=1e-5)


def test_scores_are_scaled_dot_products():
    qbar = np.array([[[1.0, 2.0, 0.0, 0.0]]], dtype=np.float32)
    kbar = np.array([[[3.0, 0.5, 0.0, 0.0], [0.0, 0.0, 0.0, 0.0]]], dtype=np.float32)
    s = O.block_scores(qbar, kbar)
    assert s.dtype == np.float32 and s[0, 0, 0] == np.float32(2.0) and s[0, 0, 1] == 0.0


# ---------------------------------------------------------------- Top-p

def test_golden_rows():
    with open(os.path.join(GOLDEN, "topp_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        s = np.array(c["scores"], dtype=np.float32)
        r = O.route_row(s, c["p"], c["k"])
        assert r.count_topp == c["count_topp"], c["why"]
        assert sorted(r.order[: r.count].tolist()) == c["retained"], c["why"]


@settings(max_examples=60, deadline=None)
@given(st.integers(2, 40), st.floats(0.05, 0.99), st.integers(0, 2 ** 31 - 1), st.floats(0.1, 8.0))
def test_minimality_nested_monotone(nb, p, seed, spread):
    rng = np.random.default_rng(seed)
    s = (rng.standard_normal(nb) * spread).astype(np.float32)
    r = O.route_row(s, p, 0)
    c = r.count_topp
    assert r.cdf[c - 1] >= p or c == nb
    if c > 1:
        assert r.cdf[c - 2] < p
    for p2 in (p * 0.5, p * 0.9, min(0.999, p + 0.05)):
        r2 = O.route_row(s, p2, 0)
        if p2 <= p:
            assert r2.count_topp <= c
            assert set(r2.order[: r2.count_topp]) <= set(r.order[:c])
        else:
            assert r2.count_topp >= c


def test_p_one_keeps_all():
    rng = np.random.default_rng(0)
    s = (rng.standard_normal((4, 9, 9)) * 30).astype(np.float32)
    P = O.block_softmax(s)
    cdf = np.cumsum(np.take_along_axis(P, O.importance_order(P), -1), -1)
    assert (O.topp_count(cdf, 1.0) == 9).all()


@pytest.mark.parametrize("nb,p", [(16, 0.9), (16, 0.5), (10, 0.33), (64, 0.9), (1182, 0.9)])
def test_uniform_scores_closed_form(nb, p):
    r = O.route_row(np.zeros(nb, dtype=np.float32), p, 0)
    want = math.ceil(p * nb - 1e-9)
    assert r.count_topp == want
    assert sorted(r.order[: r.count].tolist()) == list(range(want))


def test_dominant_block_then_floor():
    s = np.full(12, -40.0, dtype=np.float32)
    s[7] = 40.0
    r = O.route_row(s, 0.95, 4)
    assert r.count_topp == 1 and r.count == 4
    assert sorted(r.order[:4].tolist()) == [0, 1, 2, 7]


@settings(max_examples=40, deadline=None)
@given(st.integers(2, 10), st.floats(0.05, 0.98), st.integers(0, 2 ** 31 - 1))
def test_brute_force_smallest_subset(nb, p, seed):
    rng = np.random.default_rng(seed)
    s = (rng.standard_normal(nb) * 2).astype(np.float32)
    P = O.block_softmax(s[None])[0]
    sums = {}
    best = None
    for size in range(1, nb + 1):
        for sub in itertools.combinations(range(nb), size):
            tot = math.fsum(P[list(sub)])
            if abs(tot - p) < 1e-9:
                return  # too close to the threshold for a rounding-free comparison
            if tot >= p and best is None:
                best = size
    r = O.route_row(s, p, 0)
    assert r.count_topp == best


@settings(max_examples=30, deadline=None)
@given(st.integers(1, 30), st.integers(0, 40), st.integers(0, 2 ** 31 - 1))
def test_floor_keeps_at_least_k(nb, k, seed):
    rng = np.random.default_rng(seed)
    s = (rng.standard_normal(nb) * 6).astype(np.float32)
    r = O.route_row(s, 0.5, k)
    assert r.count == max(r.count_topp, min(k, nb))
    assert r.count >= min(k, nb)


# ---------------------------------------------------------------- full route + Eq. 1

def test_route_shapes_and_eq1():
    rng = np.random.default_rng(9)
    qh = rng.standard_normal((1, 3, 100, 8)).astype(np.float32)
    kh = rng.standard_normal((1, 3, 100, 8)).astype(np.float32)
    R = O.route(qh, kh, 16, 0.8, 2)
    assert R.counts.shape == (1, 3, 7) and R.nb == 7
    work, L = O.workloads(R.counts)
    for h in range(3):
        assert work[0, h] == sum(int(c) for c in R.counts[0, h])
        assert L[0, h] == np.float32(work[0, h]) / np.float32(7)
    # per-row routing agrees with the batched route
    for h in range(3):
        for i in range(7):
            rr = O.route_row(R.scores[0, h, i], 0.8, 2)
            assert rr.count == R.counts[0, h, i]
            assert (np.sort(rr.order[: rr.count]) == R.retained(0, h, i)).all()


def test_imbalance_eq2():
    assert O.imbalance([1, 1, 1, 1]) == 1.0
    assert abs(O.imbalance([2, 1, 1, 0]) - 2.0) < 1e-12
