"""absh_route_static (routing with the library's static device scratch, no allocation)
against absh_route with a caller workspace, on the same inputs, bit for bit: calls in a
row, each with a smaller input than the last (fewer heads, smaller grids), and the
rejection of a shape whose workspace exceeds the static maximum."""
import ctypes

import numpy as np
import pytest
import torch

import adaptive_block_sparse_hilbert_amd as absh
import workloads as W

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
EWORKSPACE = -3


def inputs(index, heads=None, seed=None):
    w = W.workload(index)
    d = W.generate(w, seed=seed)
    H = w.H if heads is None else heads
    to_dev = lambda b: torch.from_numpy(np.ascontiguousarray(b[:, :, :H]).view(np.int16)).view(torch.bfloat16).to(DEV)
    ctx = absh.create(w.T, w.Y, w.X, w.block)
    qh, kh = absh.permute(ctx, to_dev(d["q16"])), absh.permute(ctx, to_dev(d["k16"]))
    return w, ctx, qh, kh, H


def route_static(ctx, qh, kh, opts, out):
    B, H, _, d = qh.shape
    lists = out.lists()
    st = absh.lib().absh_route_static(ctx.handle, ctypes.c_void_p(qh.data_ptr()), ctypes.c_void_p(kh.data_ptr()),
                                      absh.ABSH_BF16, B, H, d, ctypes.byref(opts), ctypes.byref(lists),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    out.schedule = lists.schedule
    return st


def same(a, b, units, schedule):
    """Every field the call defines: counts, work, L, the queue and run bounds whole, each list
    up to its count (entries past it are unspecified), the unit queue for the longest-first
    schedule."""
    for f in ("counts", "work", "L", "queue", "sched"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
    nb = a.kv_idx.shape[-1]
    keep = torch.arange(nb, device=DEV) < a.counts.unsqueeze(-1)
    assert torch.equal(torch.where(keep, a.kv_idx, -1), torch.where(keep, b.kv_idx, -1)), "kv_idx"
    if int(a.sched[9]) == 1:  # single tiles: no unit lists
        return
    assert torch.equal(a.unit_cnt[:units], b.unit_cnt[:units]), "unit_cnt"
    if schedule == "lpt":
        assert torch.equal(a.unit_queue[:units], b.unit_queue[:units])
    ucnt = a.unit_cnt[:units]
    keep = torch.arange(nb, device=DEV) < ucnt.unsqueeze(-1)
    assert torch.equal(torch.where(keep, a.unit_list[:units], -1), torch.where(keep, b.unit_list[:units], -1)), "unit_list"


@pytest.mark.parametrize("schedule", ["xcd", "lpt"])
def test_static_route_equals_workspace_route(schedule):
    print(f"[no-alloc] schedule {schedule}", flush=True)
    # 720p at 40 heads, then 480p at 12 heads, at 5 heads, and the tiny grid
    cases = [(2, None, 0.9, 0.0), (1, None, 0.9, 0.05), (1, 5, 0.8, 0.0), (0, None, 0.9, 0.3)]
    for index, heads, p, beta in cases:
        w, ctx, qh, kh, H = inputs(index, heads)
        print(f"[no-alloc] {w.name} heads {H} p {p} slack {beta}", flush=True)
        ref = absh.route(ctx, qh, kh, p, w.k_floor, slack_frac=beta, schedule=schedule)
        out = absh.alloc_routing(ctx, w.B, H)
        opts = absh.RouteOpts(p, w.k_floor, beta, absh.SCHEDULES[schedule], 0)
        assert route_static(ctx, qh, kh, opts, out) == 0, absh.lib().absh_last_error()
        torch.cuda.synchronize()
        same(ref, out, absh.lists_units(ctx, w.B, H, schedule), schedule)


def test_static_route_rejects_large_shapes():
    w = W.workload(2)
    H = 64  # 720p at 64 heads: about 78 MB of workspace
    ctx = absh.create(w.T, w.Y, w.X, w.block)
    qh = kh = torch.zeros((w.B, H, ctx.n_pad, w.d), dtype=torch.bfloat16, device=DEV)
    # the block means alone (two float32 [B, H, nb, d]) exceed the maximum
    assert 2 * 4 * w.B * H * ctx.nb * w.d > absh.STATIC_SCRATCH_BYTES
    out = absh.alloc_routing(ctx, w.B, H)
    out.counts.fill_(-7)
    opts = absh.RouteOpts(0.9, 4, 0.0, absh.SCHEDULES["xcd"], 0)
    assert route_static(ctx, qh, kh, opts, out) == EWORKSPACE
    assert b"maximum" in absh.lib().absh_last_error()
    torch.cuda.synchronize()
    assert (out.counts == -7).all()


@pytest.mark.parametrize("grid,block,d,H,p,k,beta", [
    ((16, 128, 128), 128, 64, 1, 0.9, 4, 0.1),    # nb = 2048, the router's maximum
    ((5, 20, 40), 16, 128, 2, 0.8, 2, 0.0),       # nb = 250, blocks of 16
    ((3, 9, 10), 128, 128, 2, 0.99, 1, 0.2),      # ragged tail of 14 tokens
])
def test_static_route_at_other_block_counts(grid, block, d, H, p, k, beta):
    """The on-chip score path at every staged row width (up to nb = 2048, 128 KB of LDS per
    workgroup), with and without slack fill, against absh_route bit for bit."""
    T, Y, X = grid
    N = T * Y * X
    print(f"[no-alloc] grid {grid} block {block} d {d} H {H}", flush=True)
    rng = np.random.default_rng(17)
    ctx = absh.create(T, Y, X, block)
    x = [torch.from_numpy((rng.standard_normal((1, N, H, d)) * 2).astype(np.float32)).to(DEV) for _ in range(2)]
    qh, kh = (absh.permute(ctx, t) for t in x)
    for schedule in ("xcd", "lpt"):
        ref = absh.route(ctx, qh, kh, p, k, slack_frac=beta, schedule=schedule)
        out = absh.alloc_routing(ctx, 1, H)
        opts = absh.RouteOpts(p, k, beta, absh.SCHEDULES[schedule], 0)
        assert route_static(ctx, qh, kh, opts, out) == 0, absh.lib().absh_last_error()
        torch.cuda.synchronize()
        same(ref, out, absh.lists_units(ctx, 1, H, schedule), schedule)
