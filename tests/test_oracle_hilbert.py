"""Pins of the oracle's Hilbert order (xllm-io review of FVAttn, 3.1: blocks follow a Hilbert curve).

What fixes the answer here, independently of the oracle's own code:
  * the order is a bijection of the grid cells;
  * on a full 2^m cube consecutive cells are face neighbours (L1 distance 1) and
    the curve starts at the origin (defining properties of a Hilbert curve);
  * every aligned 2^k sub-cube is visited in one contiguous run (the recursive
    octant structure), which a snake or Z-order curve fails;
  * the order-1 curve is the reflected Gray code (golden fixture);
  * in 2-D the same transform reproduces the textbook quadrant-recursion curve
    (the distance-to-coordinates construction of the Hilbert curve article,
    re-derived here independently);
  * a cropped grid is the cube order with the out-of-grid cells dropped.
"""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import absh_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def cube_order(m):
    n = 1 << m
    perm, _ = O.hilbert_perm(n, n, n)
    return np.stack(np.unravel_index(perm, (n, n, n)), axis=1)


@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_full_cube_unit_steps_from_origin(m):
    cells = cube_order(m)
    assert cells.shape[0] == 8 ** m
    assert (cells[0] == 0).all()
    steps = np.abs(np.diff(cells, axis=0)).sum(axis=1)
    assert (steps == 1).all()


@pytest.mark.parametrize("m", [2, 3, 4])
def test_subcubes_are_contiguous_runs(m):
    cells = cube_order(m)
    for k in range(1, m):
        key = cells >> k                      # which aligned 2^k sub-cube
        flat = (key[:, 0] * (1 << (m - k)) + key[:, 1]) * (1 << (m - k)) + key[:, 2]
        run = 8 ** k
        chunks = flat.reshape(-1, run)
        assert (chunks == chunks[:, :1]).all(), f"sub-cubes of side 2^{k} are split"
        assert len(np.unique(chunks[:, 0])) == chunks.shape[0]


def test_order1_is_gray_code():
    with open(os.path.join(GOLDEN, "hilbert_m1.json")) as f:
        want = np.array(json.load(f)["cells_t_y_x"])
    assert (cube_order(1) == want).all()


def textbook_d2xy(m, dist):
    """Quadrant recursion: peel two bits of the distance per level, rotate/reflect the lower levels."""
    x = y = 0
    t = dist
    s = 1
    while s < (1 << m):
        rx = 1 & (t // 2)
        ry = 1 & (t ^ rx)
        if ry == 0:
            if rx == 1:
                x, y = s - 1 - x, s - 1 - y
            x, y = y, x
        x += s * rx
        y += s * ry
        t //= 4
        s *= 2
    return x, y


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 6])
def test_2d_matches_textbook_curve(m):
    n = 1 << m
    g = np.stack(np.meshgrid(np.arange(n), np.arange(n), indexing="ij"), -1).reshape(-1, 2)
    ours = g[np.argsort(O.hilbert_index(g, m))]
    ref = np.array([textbook_d2xy(m, dd) for dd in range(n * n)])
    assert (ours == ref).all()


@settings(max_examples=30, deadline=None)
@given(st.integers(1, 19), st.integers(1, 19), st.integers(1, 19))
def test_bijection_and_cropped_cube(T, Y, X):
    perm, inv = O.hilbert_perm(T, Y, X)
    N = T * Y * X
    assert sorted(perm.tolist()) == list(range(N))
    assert (perm[inv] == np.arange(N)).all()
    m = O.hilbert_bits(T, Y, X)
    assert (1 << m) >= max(T, Y, X) and (m == 1 or (1 << (m - 1)) < max(T, Y, X))
    cells = cube_order(m)
    keep = (cells[:, 0] < T) & (cells[:, 1] < Y) & (cells[:, 2] < X)
    want = (cells[keep, 0] * Y + cells[keep, 1]) * X + cells[keep, 2]
    assert (perm == want).all()


def test_workload_grids_are_bijections():
    for (T, Y, X) in [(4, 8, 8), (21, 30, 52)]:
        perm, inv = O.hilbert_perm(T, Y, X)
        assert np.bincount(perm, minlength=T * Y * X).max() == 1
