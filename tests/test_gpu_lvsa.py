"""GPU parity of the structured router (LVSA note: local window plus rotating global anchors).

Bars: counts and lists bit-exact against the oracle's window_anchor_list for
every tile; work and L follow from the counts; attention on these lists (the
same sparse kernel) within the attention bar on sampled tiles.
"""
import numpy as np
import pytest
import torch

import adaptive_block_sparse_hilbert_amd as absh
from oracle import absh_oracle as O
from test_gpu_parity import ATOL_MAX, ATOL_MEAN, attention_errors, case, check_lists_valid

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("index,window,stride,shift,step,schedule", [
    (4, 24, 32, 5, 3, "xcd"), (4, 6, 0, 0, 0, "order"), (1, 3, 7, 2, 11, "lpt"), (0, 1, 3, 1, 1, "xcd"),
    (0, 2 ** 31 - 1, 0, 0, 0, "xcd")])  # a window past int range: every block, no overflow
def test_window_anchor_lists(index, window, stride, shift, step, schedule):
    c = case(index)
    w = c.w
    r = absh.route(c.ctx, c.qh, c.kh, 0.9, 0, schedule=schedule, router="window-anchor", window=window,
                   anchor_stride=stride, anchor_shift=shift, step=step)
    counts, kv, _ = check_lists_valid(r, w.nb)
    want = O.window_anchor_counts(w.nb, window, stride, shift, step)
    assert np.array_equal(counts.reshape(-1, w.nb), np.broadcast_to(want, (w.B * w.H, w.nb)))
    flat_kv = kv.reshape(-1, w.nb)
    for i in range(w.nb):
        lst = O.window_anchor_list(w.nb, i, window, stride, shift, step)
        for bh in range(w.B * w.H):
            assert np.array_equal(flat_kv[bh * w.nb + i, : lst.size], lst)
    assert np.array_equal(r.work.cpu().numpy().reshape(-1), np.full(w.B * w.H, want.sum()))
    print(f"[window-anchor] {w.name}: density {want.sum() / w.nb ** 2:.4f}")


@pytest.mark.parametrize("index,schedule", [(4, "xcd"), (4, "lpt"), (2, "xcd")])
def test_attention_window_anchor(index, schedule):
    c = case(index)
    w = c.w
    r = absh.route(c.ctx, c.qh, c.kh, 0.9, 0, schedule=schedule, router="window-anchor", window=12,
                   anchor_stride=24, anchor_shift=7, step=2)
    check_lists_valid(r, w.nb)
    rng = np.random.default_rng(300 + index)
    pick = {0, w.nb - 1, w.tiles - 1} | set(rng.choice(w.tiles, size=10, replace=False).tolist())
    mx, mean = attention_errors(c, r, sorted(pick))
    print(f"[attn window-anchor] {w.name} {schedule}: max {mx:.3e} mean {mean:.3e}")
    assert mx <= ATOL_MAX and mean <= ATOL_MEAN


def test_window_anchor_rejects_bad_options():
    c = case(0)
    with pytest.raises(absh.AbshError):
        absh.route(c.ctx, c.qh, c.kh, 0.9, 0, schedule="xcd", router="window-anchor", window=-1)
    with pytest.raises(absh.AbshError):
        absh.route(c.ctx, c.qh, c.kh, 0.9, 0, schedule="ranks", router="window-anchor", window=2)
    with pytest.raises(absh.AbshError):
        absh.route(c.ctx, c.qh, c.kh, 0.9, 0, slack_frac=0.1, schedule="xcd", router="window-anchor", window=2)
    torch.cuda.synchronize()
