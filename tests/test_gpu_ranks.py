"""GPU parity of the rank-level stages (RLB head migration, SASA budgets) with the XCDs as ranks.

The GPU's plan is checked against the oracle's rank stage run on the GPU's own
pre-stage counts (the route of the "order" schedule on the same inputs, which
the two schedules share up to that point):
  * rho before / after migration / after augmentation, policy, moves, rank loads,
    budgets E_r, head order and queue segment bounds: exact (integers, and the
    same float64 operations on the same integers);
  * counts after the fill: exact; the extended lists are importance-order
    prefixes (checked against the oracle's routing with the shared excuse rule);
    work and L follow from the counts;
  * attention under the rank schedule, strict or not: the attention bar on
    sampled tiles; with the policy forced to 'none' and no strictness, outputs
    equal the "order" schedule's bit for bit (same units, same lists).
"""
import numpy as np
import pytest
import torch

import adaptive_block_sparse_hilbert_amd as absh
from oracle import absh_oracle as O
from routing_compare import compare_routing
from test_gpu_parity import ATOL_MAX, ATOL_MEAN, attention_errors, case, check_lists_valid

pytestmark = pytest.mark.gpu


def gpu_rank_report(r):
    info = r.rank_info.cpu().numpy()
    moves = [tuple(int(x) for x in info[37 + 3 * i: 40 + 3 * i]) for i in range(int(info[4]))]
    return dict(rho0=info[0], rho_rlb=info[1], rho_final=info[2], policy=["none", "sasa", "rlb+sasa", "rlb"][int(info[3])],
                moves=moves, W0=info[5:13].astype(np.int64), W1=info[13:21].astype(np.int64),
                W2=info[21:29].astype(np.int64), E=info[29:37].astype(np.int64), space=info[61], reserved=info[62])


@pytest.mark.parametrize("index,policy", [(1, "auto"), (2, "auto"), (3, "auto"), (2, "rlb+sasa"), (3, "sasa"),
                                          (3, "rlb"), (1, "none")])
def test_rank_stage_matches_oracle(index, policy):
    c = case(index)
    w = c.w
    base = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor, slack_frac=w.slack_frac, schedule="order")
    ranked = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor, slack_frac=w.slack_frac, schedule="ranks",
                        rank_policy=policy)
    torch.cuda.synchronize()
    c0, _, _ = check_lists_valid(base, w.nb)
    c1, kv1, _ = check_lists_valid(ranked, w.nb)
    want = O.rank_stage(c0, policy=None if policy == "auto" else policy)
    got = gpu_rank_report(ranked)
    print(f"[ranks] {w.name} {policy}: rho {got['rho0']:.4f} -> {got['rho_rlb']:.4f} -> {got['rho_final']:.4f}, "
          f"policy {got['policy']}, moves {got['moves']}, E {list(got['E'])}")
    assert got["reserved"] == 0
    assert got["policy"] == want["policy"]
    if want["policy"] in ("rlb+sasa", "rlb"):
        owner0 = O.rank_of_heads(w.B * w.H)
        assert got["space"] == O.rlb_space(c0.reshape(w.B * w.H, -1).sum(-1), owner0)
    assert got["rho0"] == want["rho0"] and got["rho_rlb"] == want["rho_rlb"] and got["rho_final"] == want["rho_final"]
    assert got["moves"] == [(h, s, d) for h, s, d in want["moves"]]
    for k in ("W0", "W1", "W2", "E"):
        assert np.array_equal(got[k], want[k]), k
    assert np.array_equal(c1, want["counts"])
    assert np.array_equal(ranked.head_order.cpu().numpy(), want["head_order"])
    per_head = (w.nb + 3) // 4 if w.block <= 64 else (w.nb + 1) // 2
    bounds = np.concatenate([[0], np.cumsum(want["heads_per_rank"])]) * per_head
    sched = ranked.sched.cpu().numpy()
    assert np.array_equal(sched[:9], bounds)
    assert np.array_equal(ranked.work.cpu().numpy(), c1.sum(-1))
    if policy != "none":
        R = c.oracle_route()
        R.counts = c1.astype(np.int64)
        excused, failures = compare_routing(R, c1, kv1, w.p)
        assert not failures, failures[:5]


@pytest.mark.parametrize("index,strict", [(2, False), (3, True), (4, True)])
def test_attention_ranks(index, strict):
    c = case(index)
    w = c.w
    r = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor, slack_frac=w.slack_frac, schedule="ranks",
                   strict_ranks=strict)
    counts, _, _ = check_lists_valid(r, w.nb)
    rng = np.random.default_rng(200 + index)
    flat = counts.reshape(-1)
    pick = {int(np.argmax(flat)), w.nb - 1, w.tiles - 1}
    pick |= set(rng.choice(w.tiles, size=10, replace=False).tolist())
    mx, mean = attention_errors(c, r, sorted(pick))
    print(f"[attn ranks] {w.name} strict={strict}: max {mx:.3e} mean {mean:.3e}")
    assert mx <= ATOL_MAX and mean <= ATOL_MEAN


@pytest.mark.parametrize("index", [1, 3])
def test_ranks_without_stages_equal_order(index):
    c = case(index)
    w = c.w
    a = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor, schedule="order")
    oa = absh.unpermute(c.ctx, absh.sparse_attn(c.ctx, c.qh, c.kh, c.vt, a))
    b = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor, schedule="ranks", rank_policy="none")
    ob = absh.unpermute(c.ctx, absh.sparse_attn(c.ctx, c.qh, c.kh, c.vt, b))
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))
