"""Pins of the oracle's structured router (LVSA note: local window plus rotating global anchors).

Fixed independently of the oracle's code by:
  * closed form of the count: the clipped window length plus the anchors outside it;
  * no anchors (stride 0) gives the band |i - j| <= window; a window covering all
    blocks gives every block; window 0 and stride 1 give every block;
  * the anchors rotate: the offset at step t is (t * shift) mod stride, so after
    stride / gcd(shift, stride) steps the pattern repeats, and in between every
    key block is an anchor at some step;
  * lists are ascending and inside [0, nb).
"""
import math

import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import absh_oracle as O


@settings(max_examples=200, deadline=None)
@given(st.integers(1, 80), st.integers(0, 10), st.integers(0, 12), st.integers(0, 7), st.integers(0, 30), st.data())
def test_count_closed_form(nb, window, stride, shift, step, data):
    i = data.draw(st.integers(0, nb - 1))
    lst = O.window_anchor_list(nb, i, window, stride, shift, step)
    assert np.all(np.diff(lst) > 0) and lst.min() >= 0 and lst.max() < nb
    lo, hi = max(0, i - window), min(nb - 1, i + window)
    n = hi - lo + 1
    if stride:
        o = (step * shift) % stride
        n += sum(1 for j in range(o, nb, stride) if not lo <= j <= hi)
    assert lst.size == n


def test_special_cases():
    nb = 20
    for i in range(nb):
        assert list(O.window_anchor_list(nb, i, 2, 0, 0, 0)) == [j for j in range(nb) if abs(i - j) <= 2]
        assert list(O.window_anchor_list(nb, i, nb, 5, 1, 3)) == list(range(nb))
        assert list(O.window_anchor_list(nb, i, 2 ** 31 - 1, 0, 0, 0)) == list(range(nb))
        assert list(O.window_anchor_list(nb, i, 0, 1, 0, 0)) == list(range(nb))
    assert list(O.window_anchor_list(10, 0, 0, 4, 1, 1)) == [0, 1, 5, 9]   # window {0}, anchors 1, 5, 9


def test_anchors_rotate():
    nb, stride, shift = 40, 6, 4
    period = stride // math.gcd(shift, stride)
    seen = set()
    for t in range(period):
        seen |= set(O.window_anchor_list(nb, 20, 0, stride, shift, t).tolist())
    assert O.anchor_offset(stride, shift, period) == O.anchor_offset(stride, shift, 0)
    # over a period the anchors visit every residue reachable from shift: all of them when gcd = 1
    want = {j for j in range(nb) if (j % math.gcd(shift, stride)) == 0} | {20}
    assert seen == want
