"""The permute fused with the block pooling (absh_permute_pool) and routing from the
block means it writes (absh_route_means): rows bit-identical to absh_permute, means
bit-identical to absh_pool over those rows and to the oracle's block means, and the
routing lists bit-identical to absh_route on the rows."""
import numpy as np
import pytest
import torch

import adaptive_block_sparse_hilbert_amd as absh
import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def check_fused(ctx, x, layout, block, host_rows=None):
    """permute_pool against permute + pool on the GPU, and (if given) the oracle's block
    means of the host rows in Hilbert order."""
    xh, xbar = absh.permute_pool(ctx, x, layout=layout)
    ref_rows = absh.permute(ctx, x, layout=layout)
    ref_bar = absh.pool(ctx, ref_rows) if layout == absh.ABSH_ROWS else None
    torch.cuda.synchronize()
    assert torch.equal(xh.view(torch.int16 if xh.dtype == torch.bfloat16 else torch.int32),
                       ref_rows.view(torch.int16 if xh.dtype == torch.bfloat16 else torch.int32)), "rows"
    if ref_bar is not None:
        assert torch.equal(xbar.view(torch.int32), ref_bar.view(torch.int32)), "means vs absh_pool"
    if host_rows is not None:
        want = O.block_means(host_rows, block)
        assert np.array_equal(xbar.cpu().numpy(), want), "means vs oracle"
    return xh, xbar


@pytest.mark.parametrize("index", [0, 1, 2, 4])
def test_permute_pool_bf16_rows(index):
    w = W.workload(index)
    print(f"[permute-pool] {w.name}", flush=True)
    d = W.generate(w)
    ctx = absh.create(w.T, w.Y, w.X, w.block)
    perm, _ = O.hilbert_perm(w.T, w.Y, w.X)
    host = O.to_hilbert(W.bf16_to_f32(d["q16"]), perm) if index in (0, 1) else None
    check_fused(ctx, bf16_dev(d["q16"]), absh.ABSH_ROWS, w.block, host)


def test_permute_pool_float_inputs():
    """float32 inputs: bf16 rows (rounded; the means are of the rounded values) and
    float32 rows (the means of the float32 values, against the oracle)."""
    w = W.workload(0)
    d = W.generate(w, want_fp32=True)
    ctx = absh.create(w.T, w.Y, w.X, w.block)
    perm, _ = O.hilbert_perm(w.T, w.Y, w.X)
    x = torch.from_numpy(d["q32"]).to(DEV)
    rounded = W.bf16_to_f32(W.bf16_bits(d["q32"]))
    check_fused(ctx, x, absh.ABSH_ROWS, w.block, O.to_hilbert(rounded, perm))
    check_fused(ctx, x, absh.ABSH_ROWS_F32, w.block, O.to_hilbert(d["q32"], perm))


@pytest.mark.parametrize("grid,block,d,H", [
    ((3, 9, 10), 128, 128, 2),   # ragged tail of 14 tokens in a 128-token block
    ((5, 20, 40), 16, 64, 3),    # blocks of 16, d = 64
    ((2, 7, 9), 64, 64, 1),      # one partial block per 64 (126 tokens)
])
def test_permute_pool_other_shapes(grid, block, d, H):
    T, Y, X = grid
    N = T * Y * X
    print(f"[permute-pool] grid {grid} block {block} d {d} H {H}", flush=True)
    rng = np.random.default_rng(5)
    ctx = absh.create(T, Y, X, block)
    perm, _ = O.hilbert_perm(T, Y, X)
    bits = W.bf16_bits((rng.standard_normal((2, N, H, d)) * 3).astype(np.float32))
    host = O.to_hilbert(W.bf16_to_f32(bits), perm)
    check_fused(ctx, bf16_dev(bits), absh.ABSH_ROWS, block, host)
    xf = torch.from_numpy((rng.standard_normal((2, N, H, d))).astype(np.float32)).to(DEV)
    check_fused(ctx, xf, absh.ABSH_ROWS_F32, block, O.to_hilbert(xf.cpu().numpy(), perm))


def same_routing(a, b, ctx, B, H, schedule):
    for f in ("counts", "work", "L", "queue", "sched"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
    nb = ctx.nb
    keep = torch.arange(nb, device=DEV) < a.counts.unsqueeze(-1)
    assert torch.equal(torch.where(keep, a.kv_idx, -1), torch.where(keep, b.kv_idx, -1)), "kv_idx"
    units = absh.lists_units(ctx, B, H, schedule)
    if schedule == "ranks":
        assert torch.equal(a.head_order, b.head_order), "head order"
        assert torch.equal(a.rank_info.view(torch.int64), b.rank_info.view(torch.int64)), "rank report"
    if int(a.sched[9]) == 1:  # single tiles: no unit lists
        return
    assert torch.equal(a.unit_cnt[:units], b.unit_cnt[:units]), "unit_cnt"
    if schedule == "lpt":
        assert torch.equal(a.unit_queue[:units], b.unit_queue[:units]), "unit_queue"
    ucnt = a.unit_cnt[:units]
    keep = torch.arange(nb, device=DEV) < ucnt.unsqueeze(-1)
    assert torch.equal(torch.where(keep, a.unit_list[:units], -1), torch.where(keep, b.unit_list[:units], -1))


@pytest.mark.parametrize("index,schedule", [(2, "xcd"), (3, "lpt"), (1, "lpt"), (4, "xcd"), (3, "ranks")])
def test_route_from_means_equals_route(index, schedule):
    w = W.workload(index)
    print(f"[route-means] {w.name} {schedule}", flush=True)
    d = W.generate(w)
    ctx = absh.create(w.T, w.Y, w.X, w.block)
    q, k = bf16_dev(d["q16"]), bf16_dev(d["k16"])
    qh, qbar = absh.permute_pool(ctx, q)
    kh, kbar = absh.permute_pool(ctx, k)
    ref = absh.route(ctx, qh, kh, w.p, w.k_floor, slack_frac=w.slack_frac, schedule=schedule)
    got = absh.route(ctx, None, None, w.p, w.k_floor, slack_frac=w.slack_frac, schedule=schedule,
                     qbar=qbar, kbar=kbar)
    torch.cuda.synchronize()
    same_routing(ref, got, ctx, w.B, w.H, schedule)


def test_route_means_rejects_the_structured_router():
    w = W.workload(0)
    ctx = absh.create(w.T, w.Y, w.X, w.block)
    bar = torch.zeros((w.B, w.H, ctx.nb, w.d), dtype=torch.float32, device=DEV)
    with pytest.raises(absh.AbshError, match="Top-p router"):
        absh.route(ctx, None, None, 0.9, 1, schedule="xcd", router="window-anchor", window=2, qbar=bar, kbar=bar)


@pytest.mark.parametrize("index,schedule", [(1, "xcd"), (3, "lpt"), (0, "xcd")])
def test_forward_equals_the_separate_calls(index, schedule):
    """absh_forward (permute with pooling, route from the means, sparse attention,
    unpermute in one call) against the same calls made one by one: lists and output
    bit for bit."""
    w = W.workload(index)
    print(f"[forward] {w.name} {schedule}", flush=True)
    d = W.generate(w, want_fp32=index == 0)
    ctx = absh.create(w.T, w.Y, w.X, w.block)
    if index == 0:  # float32 inputs, rounded to bf16 by the permutes
        q, k, v = (torch.from_numpy(d[n]).to(DEV) for n in ("q32", "k32", "v32"))
    else:
        q, k, v = (bf16_dev(d[n]) for n in ("q16", "k16", "v16"))
    o, got = absh.forward(ctx, q, k, v, w.p, w.k_floor, slack_frac=w.slack_frac, schedule=schedule)
    qh, qbar = absh.permute_pool(ctx, q)
    kh, kbar = absh.permute_pool(ctx, k)
    vt = absh.permute(ctx, v, layout=absh.ABSH_VT)
    ref = absh.route(ctx, None, None, w.p, w.k_floor, slack_frac=w.slack_frac, schedule=schedule,
                     qbar=qbar, kbar=kbar)
    o_ref = absh.unpermute(ctx, absh.sparse_attn(ctx, qh, kh, vt, ref))
    torch.cuda.synchronize()
    same_routing(ref, got, ctx, w.B, w.H, schedule)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))


@pytest.mark.parametrize("schedule", ["xcd", "lpt"])
def test_route_from_float_means_equals_float_route(schedule):
    """Routing from float32 rows: the means absh_permute_pool writes with the float32 rows
    route exactly as absh_route does from those rows."""
    w = W.workload(0)
    d = W.generate(w, want_fp32=True)
    ctx = absh.create(w.T, w.Y, w.X, w.block)
    q, k = (torch.from_numpy(d[n]).to(DEV) for n in ("q32", "k32"))
    qr, qbar = absh.permute_pool(ctx, q, layout=absh.ABSH_ROWS_F32)
    kr, kbar = absh.permute_pool(ctx, k, layout=absh.ABSH_ROWS_F32)
    ref = absh.route(ctx, qr, kr, w.p, w.k_floor, schedule=schedule)
    got = absh.route(ctx, None, None, w.p, w.k_floor, schedule=schedule, qbar=qbar, kbar=kbar)
    torch.cuda.synchronize()
    same_routing(ref, got, ctx, w.B, w.H, schedule)


def test_forward_rejects_bad_options_before_launching():
    """A bad routing option makes absh_forward return ABSH_EINVAL before its first launch:
    the output and the workspace keep their contents."""
    import ctypes
    w = W.workload(0)
    d = W.generate(w)
    ctx = absh.create(w.T, w.Y, w.X, w.block)
    q, k, v = (bf16_dev(d[n]) for n in ("q16", "k16", "v16"))
    o = torch.full((w.B, w.N, w.H, w.d), 7.0, dtype=torch.bfloat16, device=DEV)
    ws = torch.full((absh.forward_workspace_bytes(ctx, w.B, w.H, w.d),), 0x5A, dtype=torch.uint8, device=DEV)
    out = absh.alloc_routing(ctx, w.B, w.H)
    out.counts.fill_(-3)
    for p, k_floor, slack in ((1.5, 4, 0.0), (0.9, -1, 0.0), (0.9, 4, 1.0)):
        with pytest.raises(absh.AbshError) as e:
            absh.forward(ctx, q, k, v, p, k_floor, slack_frac=slack, schedule="xcd", routing=out, out=o, workspace=ws)
        assert e.value.status == -1
    torch.cuda.synchronize()
    assert (o == 7.0).all() and (ws == 0x5A).all() and (out.counts == -3).all()
