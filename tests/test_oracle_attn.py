"""Pins of the oracle's block-sparse attention.

Fixed independently of the oracle's code by:
  * a token-level brute force: expand the block mask to a token mask and compute
    softmax(QK^T/sqrt(d)) V with explicit Python loops and math.fsum;
  * every block retained: torch's CPU scaled_dot_product_attention in float64
    (a library routine) reproduces the dense result;
  * a single retained block whose V rows are one constant vector returns that
    vector for every query row;
  * retained FLOPs: 4 n_i n_j d summed over retained pairs, checked against a
    hand count with a partial tail block.
"""
import math

import numpy as np
import pytest
import torch

from oracle import absh_oracle as O


def brute_force_masked(q, k, v, perm, block, keep):
    """keep(b, h, i) -> key block ids; token masks built from the Hilbert positions."""
    B, N, H, d = q.shape
    pos = np.empty(N, dtype=np.int64)
    pos[perm] = np.arange(N)              # Hilbert position of each grid token
    out = np.zeros((B, N, H, d))
    for b in range(B):
        for h in range(H):
            for n in range(N):
                i = pos[n] // block
                allowed = set(keep(b, h, i))
                keys = [m for m in range(N) if pos[m] // block in allowed]
                logits = [sum(float(q[b, n, h, c]) * float(k[b, m, h, c]) for c in range(d)) / math.sqrt(d)
                          for m in keys]
                top = max(logits)
                w = [math.exp(x - top) for x in logits]
                z = math.fsum(w)
                for c in range(d):
                    out[b, n, h, c] = math.fsum(w[t] * float(v[b, keys[t], h, c]) for t in range(len(keys))) / z
    return out


def small_problem(seed=0, T=2, Y=3, X=5, H=2, d=4):
    rng = np.random.default_rng(seed)
    N = T * Y * X
    q = rng.standard_normal((1, N, H, d)).astype(np.float32)
    k = rng.standard_normal((1, N, H, d)).astype(np.float32)
    v = rng.standard_normal((1, N, H, d)).astype(np.float32)
    perm, _ = O.hilbert_perm(T, Y, X)
    return q, k, v, perm


def test_block_sparse_matches_token_brute_force():
    q, k, v, perm = small_problem()
    block = 4
    nb = -(-q.shape[1] // block)
    rng = np.random.default_rng(1)
    sets = {(0, h, i): sorted(rng.choice(nb, size=rng.integers(1, nb + 1), replace=False).tolist())
            for h in range(2) for i in range(nb)}
    keep = lambda b, h, i: sets[(b, h, i)]
    got = O.attention(q, k, v, perm, block, keep)
    want = brute_force_masked(q, k, v, perm, block, keep)
    assert np.abs(got - want).max() < 1e-12


def test_routed_sets_match_token_brute_force():
    q, k, v, perm = small_problem(seed=4, T=2, Y=4, X=4, H=1, d=4)
    block = 4
    R = O.route(O.to_hilbert(q, perm), O.to_hilbert(k, perm), block, 0.6, 1)
    keep = lambda b, h, i: R.retained(b, h, i)
    got = O.attention(q, k, v, perm, block, keep)
    want = brute_force_masked(q, k, v, perm, block, keep)
    assert np.abs(got - want).max() < 1e-12


def test_dense_equals_library_sdpa():
    q, k, v, perm = small_problem(seed=2, T=3, Y=4, X=6, H=3, d=8)
    got = O.attention(q, k, v, perm, 16, None)
    t = lambda a: torch.from_numpy(a.astype(np.float64)).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v)).permute(0, 2, 1, 3).numpy()
    assert np.abs(got - ref).max() < 1e-12


def test_p_one_route_is_dense():
    q, k, v, perm = small_problem(seed=3, T=2, Y=4, X=5, H=2, d=8)
    R = O.route(O.to_hilbert(q, perm), O.to_hilbert(k, perm), 8, 1.0, 0)
    assert (R.counts == R.nb).all()
    sparse = O.attention(q, k, v, perm, 8, lambda b, h, i: R.retained(b, h, i))
    dense = O.attention(q, k, v, perm, 8, None)
    assert np.abs(sparse - dense).max() < 1e-12


def test_single_block_constant_v():
    q, k, v, perm = small_problem(seed=5)
    block = 4
    vh = O.to_hilbert(v, perm)
    const = np.array([0.5, -1.25, 3.0, 0.0], dtype=np.float32)
    # make every V row of Hilbert block 2 equal to const (in grid order)
    v = v.copy()
    v[0, perm[8:12], :, :] = const
    out = O.attention(q, k, v, perm, block, lambda b, h, i: [2])
    assert np.abs(out - const).max() < 1e-12


def test_retained_flops_counts_true_tokens():
    sizes = O.block_sizes(20, 8)          # [8, 8, 4]
    flops = O.retained_flops(sizes, 16, [(0, [0, 2]), (2, [1])])
    assert flops == 4 * 8 * (8 + 4) * 16 + 4 * 4 * 8 * 16
