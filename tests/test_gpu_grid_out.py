"""absh_sparse_attn_grid: the attention writing its output in the caller's grid order.
Every element must be bit-identical to absh_unpermute of the Hilbert-order output of
absh_sparse_attn (bf16 values) or absh_sparse_attn_v8 (8-bit values). The cases cover
both kernels (the tile kernel for blocks of 16, the union kernel for 64 and 128), every
schedule, dense mode, and shapes whose last block is partial (its pad rows must not be
written anywhere)."""
import numpy as np
import pytest
import torch

import adaptive_block_sparse_hilbert_amd as absh
import workloads as W

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
SENTINEL = 0x7FC1  # a NaN bit pattern no attention output takes


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def inputs_for(grid, block, d, H, B=1, seed=3):
    T, Y, X = grid
    N = T * Y * X
    rng = np.random.default_rng(seed)
    # a smooth part over the grid so that routing keeps neighbours, plus noise
    t, y, x = np.meshgrid(np.arange(T), np.arange(Y), np.arange(X), indexing="ij")
    base = np.stack([np.sin(0.3 * t + 0.2 * y + 0.1 * x + f) for f in range(d)], axis=-1).reshape(N, 1, d)
    out = []
    for _ in range(3):
        a = (base[None] * 2.0 + rng.standard_normal((B, N, H, d))).astype(np.float32)
        out.append(bf16_dev(W.bf16_bits(a)))
    return out


def hilbert_side(ctx, q, k, v, fp8):
    qh = absh.permute(ctx, q)
    kh = absh.permute(ctx, k)
    if fp8:
        vt, vscale = absh.quantize_v(ctx, absh.permute(ctx, v))
    else:
        vt, vscale = absh.permute(ctx, v, layout=absh.ABSH_VT), None
    return qh, kh, vt, vscale


def check(ctx, q, qh, kh, vt, vscale, routing):
    if vscale is None:
        ref = absh.unpermute(ctx, absh.sparse_attn(ctx, qh, kh, vt, routing))
    else:
        ref = absh.unpermute(ctx, absh.sparse_attn_v8(ctx, qh, kh, vt, vscale, routing))
    o = torch.full_like(q, 0).view(torch.int16).fill_(SENTINEL).view(torch.bfloat16)
    got = absh.sparse_attn_grid(ctx, qh, kh, vt, routing, vscale=vscale, out=o)
    torch.cuda.synchronize()
    assert got.data_ptr() == o.data_ptr()
    assert not (got.view(torch.int16) == SENTINEL).any(), "an output row was not written"
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("index,schedule,fp8", [
    (0, "xcd", False),   # blocks of 16: the tile kernel on group units
    (0, "lpt", False),   # blocks of 16: the tile kernel on single tiles
    (1, "xcd", False),   # 480p, blocks of 64: the union kernel
    (1, "lpt", True),    # 8-bit values, longest-first group units
    (3, "lpt", False),   # the head-skew workload on its own schedule, with slack fill
    (4, "order", False),  # blocks of 128 (two members), 196,560 tokens
    (4, "xcd", True),
])
def test_grid_output_equals_unpermuted_output(index, schedule, fp8):
    w = W.workload(index)
    print(f"[grid-out] {w.name} {schedule} fp8={fp8}", flush=True)
    d = W.generate(w)
    ctx = absh.create(w.T, w.Y, w.X, w.block)
    q, k, v = (bf16_dev(d[n]) for n in ("q16", "k16", "v16"))
    qh, kh, vt, vscale = hilbert_side(ctx, q, k, v, fp8)
    routing = absh.route(ctx, qh, kh, w.p, w.k_floor, slack_frac=w.slack_frac, schedule=schedule)
    check(ctx, q, qh, kh, vt, vscale, routing)


@pytest.mark.parametrize("grid,block,d,H,B,fp8", [
    ((3, 9, 10), 128, 128, 2, 2, False),   # 270 tokens: last block of 14
    ((3, 9, 10), 128, 128, 2, 1, True),
    ((2, 7, 9), 64, 64, 3, 2, False),      # 126 tokens: last block of 62
    ((2, 7, 9), 64, 64, 3, 1, True),
    ((5, 11, 13), 16, 64, 2, 2, False),    # 715 tokens: last block of 11, tile kernel
    ((4, 30, 31), 64, 128, 5, 1, False),   # 3,720 tokens: last block of 8
])
def test_grid_output_ragged_shapes(grid, block, d, H, B, fp8):
    print(f"[grid-out] grid {grid} block {block} d {d} H {H} B {B} fp8={fp8}", flush=True)
    ctx = absh.create(*grid, block)
    q, k, v = inputs_for(grid, block, d, H, B)
    qh, kh, vt, vscale = hilbert_side(ctx, q, k, v, fp8)
    for schedule in ("xcd", "lpt"):
        routing = absh.route(ctx, qh, kh, 0.8, 2, schedule=schedule)
        check(ctx, q, qh, kh, vt, vscale, routing)


@pytest.mark.parametrize("index,fp8", [(0, False), (1, False), (1, True)])
def test_grid_output_dense(index, fp8):
    w = W.workload(index)
    print(f"[grid-out dense] {w.name} fp8={fp8}", flush=True)
    d = W.generate(w)
    ctx = absh.create(w.T, w.Y, w.X, w.block)
    q, k, v = (bf16_dev(d[n]) for n in ("q16", "k16", "v16"))
    qh, kh, vt, vscale = hilbert_side(ctx, q, k, v, fp8)
    check(ctx, q, qh, kh, vt, vscale, None)


def test_grid_output_rejects_8bit_values_on_blocks_of_16():
    w = W.workload(0)
    ctx = absh.create(w.T, w.Y, w.X, w.block)
    z = torch.zeros((w.B, w.H, ctx.n_pad, w.d), dtype=torch.bfloat16, device=DEV)
    sc = torch.ones((w.B, w.H, w.d), dtype=torch.float32, device=DEV)
    with pytest.raises(absh.AbshError, match="8-bit values"):
        absh.sparse_attn_grid(ctx, z, z, z, None, vscale=sc)
