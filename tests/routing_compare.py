"""Comparison of GPU routing with the oracle's, under the excusal rule for float noise.

A retained-set mismatch at block j of a tile is excused iff, in the oracle's
importance order, (i) the cumulative probability just before or at j's rank lies
within 1e-5 of p (the threshold rule of the routing tolerance), or (ii) j's
score ties the score of the oracle's cut-off block within 5e-7 relative (two
float codes need not agree on the order of scores that equal to the last bits).
A tile is excused when every block in its symmetric difference is; anything else
is a failure. Integer outputs derived from the counts must then match exactly.
"""
from __future__ import annotations

import numpy as np

CDF_TOL = 1e-5
TIE_TOL = 5e-7


def compare_routing(R, counts_g, kv_g, p, flat_tiles=None):
    """R: oracle Routing; counts_g [B,H,nb]; kv_g [B,H,nb,nb] (GPU, numpy).

    Returns (n_excused_tiles, failures list).
    """
    B, H, nb = counts_g.shape
    excused, failures = 0, []
    co = R.counts
    tiles = range(B * H * nb) if flat_tiles is None else flat_tiles
    for t in tiles:
        b, h, i = np.unravel_index(t, (B, H, nb))
        cg, cor = int(counts_g[b, h, i]), int(co[b, h, i])
        gset = kv_g[b, h, i, :cg]
        if cg == cor:
            oset = R.retained(b, h, i)
            if np.array_equal(gset, oset):
                continue
        oset = R.retained(b, h, i)
        if np.any(np.diff(gset) <= 0) or gset.min(initial=0) < 0 or gset.max(initial=0) >= nb:
            failures.append((t, "GPU list not strictly ascending / out of range"))
            continue
        diff = np.setxor1d(gset, oset)
        order = R.order[b, h, i]
        rank = np.empty(nb, dtype=np.int64)
        rank[order] = np.arange(nb)
        cdf = R.cdf[b, h, i]
        s = R.scores[b, h, i].astype(np.float64)
        cut = order[cor - 1]
        ok = True
        for j in diff:
            r = rank[j]
            near_p = abs(cdf[r] - p) <= CDF_TOL or (r > 0 and abs(cdf[r - 1] - p) <= CDF_TOL)
            near_cut = abs(s[j] - s[cut]) <= TIE_TOL * max(1.0, abs(s[cut]))
            if not (near_p or near_cut):
                ok = False
                break
        if ok:
            excused += 1
        else:
            failures.append((t, f"count gpu {cg} oracle {cor}; diff {diff[:8].tolist()}"))
    return excused, failures
