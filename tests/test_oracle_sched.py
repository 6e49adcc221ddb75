"""Pins of the oracle's one-GPU scheduling: slack fill (SASA reading) and the LPT tile queue (RLB reading).

Fixed independently of the oracle's code by:
  * slack fill: the heap loop equals an independent closed form (water level plus
    a remainder by tile id); beta = 0 is the identity; the blocks added equal
    min(E, capacity); no count ever drops; the fill never raises a tile above
    the level the lightest tiles reach, so the heaviest tile is unchanged unless
    every tile reaches it (the slack never lengthens the critical path, the
    review's condition B_r <= Delta L_r in the SASA steps);
  * a single extra block goes to the smallest (count, tile id) below nb (brute force);
  * LPT queue: a permutation, non-increasing in cost, ties by ascending id;
  * list scheduling: Graham's bound makespan <= sum/W + max for any order, and
    LPT <= (4/3 - 1/(3W)) OPT, OPT by brute force over all assignments (R. L.
    Graham, "Bounds on multiprocessing timing anomalies", 1969);
  * Eq. 2: rho = max / mean of the per-worker loads.
"""
import itertools

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import absh_oracle as O


@settings(max_examples=80, deadline=None)
@given(st.integers(1, 6), st.integers(1, 30), st.integers(0, 2 ** 31 - 1), st.floats(0.0, 0.9))
def test_heap_equals_closed_form(H, nb, seed, beta):
    rng = np.random.default_rng(seed)
    counts = rng.integers(1, nb + 1, size=(1, H, nb))
    a = O.slack_fill(counts, beta)
    b = O.slack_fill_level(counts, beta)
    assert (a == b).all()
    E = O.slack_budget(counts, beta)
    cap = int((nb - counts).sum())
    assert int((a - counts).sum()) == min(E, cap)
    assert (a >= counts).all() and (a <= nb).all()
    if (a - counts).sum() and (a < nb).any():
        assert a.max() == counts.max() or a.min() >= counts.max() - 1


def test_beta_zero_identity_and_single_block():
    counts = np.array([[[3, 1, 4, 1, 5]]])
    assert (O.slack_fill(counts, 0.0) == counts).all()
    # E = floor(0.08 * 14) = 1: the smallest (count, id) is tile 1
    out = O.slack_fill(counts, 0.08)
    assert out.tolist() == [[[3, 2, 4, 1, 5]]]


def test_full_tiles_are_skipped():
    counts = np.array([[[3, 3, 1]]])   # nb = 3: two full tiles
    out = O.slack_fill(counts, 0.5)    # E = floor(0.5 * 7) = 3, capacity 2
    assert out.tolist() == [[[3, 3, 3]]]


def test_lpt_queue_properties():
    rng = np.random.default_rng(1)
    counts = rng.integers(1, 9, size=(2, 3, 7))
    q = O.lpt_queue(counts)
    flat = counts.reshape(-1)
    assert sorted(q.tolist()) == list(range(flat.size))
    c = flat[q]
    assert (np.diff(c) <= 0).all()
    for a, b in zip(q[:-1], q[1:]):
        if flat[a] == flat[b]:
            assert a < b


def brute_opt(costs, W):
    best = None
    for assign in itertools.product(range(W), repeat=len(costs)):
        loads = [0] * W
        for c, w in zip(costs, assign):
            loads[w] += c
        m = max(loads)
        best = m if best is None else min(best, m)
    return best


@settings(max_examples=40, deadline=None)
@given(st.integers(1, 3), st.lists(st.integers(1, 20), min_size=1, max_size=8))
def test_graham_bounds(W, costs):
    costs = np.array(costs, dtype=np.int64)
    ident = np.arange(costs.size)
    _, any_ms = O.list_schedule(costs, ident, W)
    assert any_ms <= costs.sum() / W + costs.max() + 1e-9
    _, lpt_ms = O.list_schedule(costs, O.lpt_queue(costs[None]), W)
    opt = brute_opt(costs.tolist(), W)
    assert lpt_ms <= (4.0 / 3.0 - 1.0 / (3 * W)) * opt + 1e-9
    assert lpt_ms >= opt


def test_list_schedule_eq2():
    loads, ms = O.list_schedule([5, 3, 3, 1], [0, 1, 2, 3], 2)
    # 5 -> w0, 3 -> w1, 3 -> w1 (free at 3), 1 -> w0 (free at 5 vs 6)
    assert loads.tolist() == [6.0, 6.0] and ms == 6.0
    assert O.imbalance(loads) == 1.0
