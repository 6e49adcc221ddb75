"""GPU parity of the 8-bit value path: V quantization and the fp8 value product.

Bars (written here):
  * absh_quantize_v: bit-exact against the oracle's quantize_v (E4M3 codes of every
    key and channel, read back through the documented ABSH_VT8 layout, and the
    per-channel scales 2^e), pad keys coded 0;
  * absh_sparse_attn_v8 on the GPU's own mask, against the oracle's exact attention
    with the dequantized values O8 (float64), element by element:
        |O_gpu - O8| <= 2e-2 + u / (1 - u) * A1 + 2^-16 / (1 - u) * As
    and over the checked elements
        mean |O_gpu - O8| <= 2e-3 + mean(u * A2),
    with u = 2^-4 the relative rounding error of an E4M3 probability and A1, A2,
    As the oracle's spreads (attention_tile_spread, small = 2^-12 / (1 - u)). The
    derivation: the kernel scales each row's probabilities so that its reference
    maximum maps to at least 2^6, so the row sum is at least 2^6 (1 - u); a
    normal E4M3 value is off by at most u relative, and a probability below 2^-6
    (normalised weight below 2^-12 / (1 - u)) by at most 2^-10 absolute, i.e.
    2^-16 / (1 - u) in normalised weight. Renormalisation by the sum of the same
    rounded values gives the u / (1 - u) factor. The 2e-2 / 2e-3 terms are the
    bf16 path's own bar (scores, exponentials, bf16 output);
  * invariants of the same kernel: p = 1 sparse == dense, the order, xcd and
    longest-first schedules, bit-identical; constant values per channel come back as the
    constant (the row sum adds exactly the probabilities the MFMA multiplies).
"""
import numpy as np
import pytest
import torch

import adaptive_block_sparse_hilbert_amd as absh
import workloads as W
from oracle import absh_oracle as O
from test_gpu_parity import ATOL_MAX, ATOL_MEAN, DEV, Case, case, check_lists_valid

pytestmark = pytest.mark.gpu

U = 2.0 ** -4
SMALL = 2.0 ** -12 / (1 - U)


def vt8_to_codes(img, d):
    """ABSH_VT8 bytes [B, H, steps, 64 * d] -> codes [B, H, steps * 64, d] (the header's layout)."""
    key = np.arange(64)[:, None]
    c = np.arange(d)[None, :]
    eta, a, g, i = key >> 5, (key >> 4) & 1, (key >> 3) & 1, key & 7
    off = eta * 32 * d + 32 * c + 16 * (g ^ ((c >> 3) & 1)) + 8 * a + i      # [64, d]
    B, H, steps, _ = img.shape
    return img[:, :, :, off].reshape(B, H, steps * 64, d)


def quantized(c):
    """GPU quantization of a case's values (cached on the case)."""
    if not hasattr(c, "_q8"):
        vh = absh.permute(c.ctx, c.v)
        c._q8 = absh.quantize_v(c.ctx, vh)
        torch.cuda.synchronize()
    return c._q8


def hv8(c, b, h):
    """The oracle's dequantized Hilbert-order values [N, d] of one head (cached on the case)."""
    if not hasattr(c, "_hv8"):
        c._hv8 = {}
    if (b, h) not in c._hv8:
        codes, e = O.quantize_v(c.hv[b, h])
        c._hv8[(b, h)] = O.dequantize_v(codes, e)
    return c._hv8[(b, h)]


def check_quantization(c, heads):
    w = c.w
    vt8, vscale = quantized(c)
    codes = vt8_to_codes(vt8.cpu().numpy(), w.d)
    scales = vscale.cpu().numpy()
    for b, h in heads:
        want, e = O.quantize_v(c.hv[b, h])
        assert np.array_equal(codes[b, h, : w.N], want), (b, h)
        assert (codes[b, h, w.N:] == 0).all()
        assert np.array_equal(scales[b, h], np.ldexp(1.0, e).astype(np.float32)), (b, h)


@pytest.mark.parametrize("index", [1, 4])
def test_quantize_bit_exact_all_heads(index):
    c = case(index)
    check_quantization(c, [(b, h) for b in range(c.w.B) for h in range(c.w.H)])


def test_quantize_bit_exact_720p_sampled_heads():
    c = case(2)
    check_quantization(c, [(0, 0), (0, 17), (0, c.w.H - 1)])


def test_quantize_small_ragged_d64():
    # d = 64, a ragged tail (N = 2 * 3 * 37 = 222 keys: 3 full 64-key steps + 30),
    # channels of very different magnitudes and one all-zero channel
    w = W.Workload(90, "ragged-d64", 2, 3, 64, 2, 3, 37, 64, 0.9, 2)
    rng = np.random.default_rng(90)
    v = rng.standard_normal((w.B, w.N, w.H, w.d)).astype(np.float32)
    v *= np.exp(rng.uniform(-12, 12, w.d)).astype(np.float32)[None, None, None, :]
    v[..., 5] = 0.0
    bits = W.bf16_bits(v)
    ctx = absh.create(w.T, w.Y, w.X, w.block)
    vd = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    vh = absh.permute(ctx, vd)
    vt8, vscale = absh.quantize_v(ctx, vh)
    torch.cuda.synchronize()
    codes = vt8_to_codes(vt8.cpu().numpy(), w.d)
    perm, _ = O.hilbert_perm(w.T, w.Y, w.X)
    hv = O.to_hilbert(W.bf16_to_f32(bits), perm)
    for b in range(w.B):
        for h in range(w.H):
            want, e = O.quantize_v(hv[b, h])
            assert np.array_equal(codes[b, h, : w.N], want)
            assert (codes[b, h, w.N:] == 0).all()
            assert np.array_equal(vscale[b, h].cpu().numpy(), np.ldexp(1.0, e).astype(np.float32))
            assert e[5] == 0


def fp8_attention_check(c, r, tiles, label):
    w = c.w
    vt8, vscale = quantized(c)
    oh = absh.sparse_attn_v8(c.ctx, c.qh, c.kh, vt8, vscale, r)
    o = absh.unpermute(c.ctx, oh).float().cpu().numpy()
    if r is not None:
        counts = r.counts.cpu().numpy().reshape(-1)
        kv = r.kv_idx.cpu().numpy().astype(np.int64).reshape(counts.size, -1)
    errs, slack, a2 = [], [], []
    for t in tiles:
        bh, i = divmod(int(t), w.nb)
        b, h = divmod(bh, w.H)
        blocks = range(w.nb) if r is None else kv[t, : counts[t]]
        ref, A1, A2, As = O.attention_tile_spread(c.hq[b, h], c.hk[b, h], hv8(c, b, h), w.block, i, blocks,
                                                  small=SMALL)
        rows = c.perm[i * w.block: min((i + 1) * w.block, w.N)]
        err = np.abs(o[b, rows, h, :] - ref)
        bound = ATOL_MAX + U / (1 - U) * A1 + 2.0 ** -16 / (1 - U) * As
        errs.append(err.ravel())
        slack.append((bound - err).ravel())
        a2.append((U * A2).ravel())
    e, sl, a2 = np.concatenate(errs), np.concatenate(slack), np.concatenate(a2)
    print(f"[attn v8] {label}: max {e.max():.3e} mean {e.mean():.3e}, min slack {sl.min():.3e}, "
          f"mean bar {ATOL_MEAN + a2.mean():.3e}", flush=True)
    assert sl.min() >= 0
    assert e.mean() <= ATOL_MEAN + a2.mean()


@pytest.mark.parametrize("index,schedule", [(1, "xcd"), (2, "xcd"), (3, "xcd"), (4, "xcd"), (3, "order"),
                                            (3, "lpt"), (4, "lpt")])
def test_attention_v8_sampled_tiles(index, schedule):
    c = case(index)
    w = c.w
    r = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor, slack_frac=w.slack_frac, schedule=schedule)
    counts, _, _ = check_lists_valid(r, w.nb)
    rng = np.random.default_rng(300 + index)
    flat = counts.reshape(-1)
    pick = {int(np.argmax(flat)), w.nb - 1, w.tiles - 1}
    pick |= set(rng.choice(w.tiles, size=5, replace=False).tolist())
    fp8_attention_check(c, r, sorted(pick), f"{w.name} {schedule}")


def test_attention_v8_dense_sampled_tiles():
    c = case(1)
    w = c.w
    rng = np.random.default_rng(310)
    pick = sorted({w.nb - 1, w.tiles - 1} | set(rng.choice(w.tiles, size=4, replace=False).tolist()))
    fp8_attention_check(c, None, pick, f"{w.name} dense")


@pytest.mark.parametrize("index", [1, 4])
def test_v8_invariants(index):
    c = case(index)
    w = c.w
    vt8, vscale = quantized(c)
    dense = absh.sparse_attn_v8(c.ctx, c.qh, c.kh, vt8, vscale, None)
    full = absh.route(c.ctx, c.qh, c.kh, 1.0, w.k_floor, schedule="xcd")
    o_full = absh.sparse_attn_v8(c.ctx, c.qh, c.kh, vt8, vscale, full)
    r1 = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor, schedule="order")
    r2 = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor, schedule="xcd")
    r3 = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor, schedule="lpt")
    a = absh.sparse_attn_v8(c.ctx, c.qh, c.kh, vt8, vscale, r1)
    b = absh.sparse_attn_v8(c.ctx, c.qh, c.kh, vt8, vscale, r2)
    b2 = absh.sparse_attn_v8(c.ctx, c.qh, c.kh, vt8, vscale, r2)
    l3 = absh.sparse_attn_v8(c.ctx, c.qh, c.kh, vt8, vscale, r3)
    torch.cuda.synchronize()
    n = w.N
    assert torch.equal(dense[:, :, :n].view(torch.int16), o_full[:, :, :n].view(torch.int16))
    assert torch.equal(a[:, :, :n].view(torch.int16), b[:, :, :n].view(torch.int16))
    assert torch.equal(a[:, :, :n].view(torch.int16), l3[:, :, :n].view(torch.int16))
    assert torch.equal(b.view(torch.int16), b2.view(torch.int16))


def test_v8_constant_values():
    c = case(1)
    w = c.w
    rng = np.random.default_rng(320)
    const = rng.uniform(-3, 3, (w.B, w.H, w.d)).astype(np.float32)
    v = np.broadcast_to(const[:, None, :, :], (w.B, w.N, w.H, w.d)).copy()
    bits = W.bf16_bits(v)
    vd = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    vt8, vscale = absh.quantize_v(c.ctx, absh.permute(c.ctx, vd))
    r = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor, schedule="xcd")
    o = absh.unpermute(c.ctx, absh.sparse_attn_v8(c.ctx, c.qh, c.kh, vt8, vscale, r)).float().cpu().numpy()
    # the quantized constant of each channel, from the oracle
    want = np.empty_like(const, dtype=np.float64)
    for b in range(w.B):
        for h in range(w.H):
            codes, e = O.quantize_v(W.bf16_to_f32(bits)[b, :1, h, :])
            want[b, h] = O.dequantize_v(codes, e)[0]
    err = np.abs(o - want[:, None, :, :])
    print(f"[attn v8] constant values: max {err.max():.3e}", flush=True)
    assert (err <= 2.0 ** -8 * np.abs(want[:, None, :, :]) + 1e-6).all()


@pytest.mark.parametrize("grid,block,d,H,B", [
    ((1, 1, 1), 64, 64, 1, 1),       # one token: one partial block
    ((2, 3, 37), 64, 64, 3, 2),      # d = 64, ragged tail of 30, batch of 2
    ((4, 4, 4), 64, 128, 2, 1),      # exactly one full block
    ((5, 6, 7), 64, 128, 2, 1),      # ragged tail of 18
    ((3, 9, 10), 128, 128, 2, 1),    # block 128, tail of 14: the last block's second half is empty
    ((2, 5, 13), 128, 64, 2, 2),     # block 128, d = 64, tail of 2
])
@pytest.mark.parametrize("schedule", ["xcd", "order", "lpt", "dense"])
def test_v8_edge_shapes(grid, block, d, H, B, schedule):
    T, Y, X = grid
    N = T * Y * X
    rng = np.random.default_rng(11)
    q32 = rng.standard_normal((B, N, H, d)).astype(np.float32) * 2
    k32 = rng.standard_normal((B, N, H, d)).astype(np.float32) * 2
    v32 = rng.standard_normal((B, N, H, d)).astype(np.float32) * rng.uniform(0.1, 4.0, d).astype(np.float32)
    bits = [W.bf16_bits(a) for a in (q32, k32, v32)]
    ctx = absh.create(T, Y, X, block)
    qd, kd, vd = (torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(DEV) for b in bits)
    qh, kh, vh = absh.permute(ctx, qd), absh.permute(ctx, kd), absh.permute(ctx, vd)
    vt8, vscale = absh.quantize_v(ctx, vh)
    r = None if schedule == "dense" else absh.route(ctx, qh, kh, 0.7, 2, schedule=schedule)
    if r is not None:
        counts, kv, _ = check_lists_valid(r, ctx.nb)
    o = absh.unpermute(ctx, absh.sparse_attn_v8(ctx, qh, kh, vt8, vscale, r)).float().cpu().numpy()
    perm, _ = O.hilbert_perm(T, Y, X)
    hq, hk, hv = (O.to_hilbert(W.bf16_to_f32(b), perm) for b in bits)
    nb = ctx.nb
    for b in range(B):
        for h in range(H):
            codes, e = O.quantize_v(hv[b, h])
            v8 = O.dequantize_v(codes, e)
            for i in range(nb):
                blocks = range(nb) if r is None else kv[b, h, i, : counts[b, h, i]]
                ref, A1, A2, As = O.attention_tile_spread(hq[b, h], hk[b, h], v8, block, i, blocks, small=SMALL)
                rows = perm[i * block: min((i + 1) * block, N)]
                err = np.abs(o[b, rows, h, :] - ref)
                bound = ATOL_MAX + U / (1 - U) * A1 + 2.0 ** -16 / (1 - U) * As
                assert (err <= bound).all(), (b, h, i, float((err - bound).max()))
                assert err.mean() <= ATOL_MEAN + (U * A2).mean()



@pytest.mark.parametrize("schedule", ["xcd", "dense"])
def test_v8_rising_logits(schedule):
    """Logits rising by about 2.5 per key block along the walk: with the 8-bit
    path's lazy threshold of 2^2 the reference maximum moves at almost every
    block, and each move rescales O and re-bases the E4M3 probabilities. Every
    tile meets the derived bound (ragged tail of 9 tokens)."""
    T, Y, X, block, H, d = 3, 17, 19, 64, 2, 128   # N = 969: 16 blocks
    N = T * Y * X
    rng = np.random.default_rng(5)
    perm, _ = O.hilbert_perm(T, Y, X)
    qh = np.zeros((1, H, N, d), np.float32)
    kh = (rng.standard_normal((1, H, N, d)) * 0.25).astype(np.float32)
    qh[..., 0] = 1.0
    blk = np.arange(N) // block
    kh[..., 0] = (2.5 * np.sqrt(d) * blk)[None, None, :] + rng.standard_normal((1, H, N)).astype(np.float32)
    vh = (rng.standard_normal((1, H, N, d)) * rng.uniform(0.1, 4.0, d)).astype(np.float32)
    q = np.empty((1, N, H, d), np.float32)
    k = np.empty_like(q)
    v = np.empty_like(q)
    for dst, src in ((q, qh), (k, kh), (v, vh)):
        dst[:, perm] = np.transpose(src, (0, 2, 1, 3))
    bits = [W.bf16_bits(a) for a in (q, k, v)]
    ctx = absh.create(T, Y, X, block)
    qd, kd, vd = (torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(DEV) for b in bits)
    qhd, khd, vhd = absh.permute(ctx, qd), absh.permute(ctx, kd), absh.permute(ctx, vd)
    vt8, vscale = absh.quantize_v(ctx, vhd)
    r = None if schedule == "dense" else absh.route(ctx, qhd, khd, 1.0, 0, schedule=schedule)
    o = absh.unpermute(ctx, absh.sparse_attn_v8(ctx, qhd, khd, vt8, vscale, r)).float().cpu().numpy()
    hq, hk, hv = (O.to_hilbert(W.bf16_to_f32(b), perm) for b in bits)
    nb = ctx.nb
    worst = 0.0
    for h in range(H):
        codes, e = O.quantize_v(hv[0, h])
        v8 = O.dequantize_v(codes, e)
        for i in range(nb):
            ref, A1, A2, As = O.attention_tile_spread(hq[0, h], hk[0, h], v8, block, i, range(nb), small=SMALL)
            rows = perm[i * block: min((i + 1) * block, N)]
            err = np.abs(o[0, rows, h, :] - ref)
            bound = ATOL_MAX + U / (1 - U) * A1 + 2.0 ** -16 / (1 - U) * As
            worst = max(worst, float((err / bound).max()))
            assert (err <= bound).all(), (h, i, float((err - bound).max()))
            assert err.mean() <= ATOL_MEAN + (U * A2).mean()
    print(f"[v8 rising] {schedule}: worst error / bound {worst:.3f}", flush=True)


def test_v8_rejects_unsupported_shapes():
    # block 16 has no 64-key steps
    ctx16 = absh.create(2, 3, 5, 16)
    x = torch.zeros((1, 30, 1, 64), dtype=torch.bfloat16, device=DEV)
    vh16 = absh.permute(ctx16, x)
    with pytest.raises(absh.AbshError) as e:
        absh.quantize_v(ctx16, vh16, out=torch.empty(64 * 64, dtype=torch.uint8, device=DEV),
                        scale=torch.empty(64, dtype=torch.float32, device=DEV))
    assert e.value.status == -2
    torch.cuda.synchronize()


@pytest.mark.parametrize("index,strict,policy", [(2, False, "auto"), (3, True, "auto"), (3, False, "rlb")])
def test_attention_v8_rank_schedule(index, strict, policy):
    # the rank schedule: segment positions map to heads through head_order (after migration)
    c = case(index)
    w = c.w
    r = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor, slack_frac=w.slack_frac, schedule="ranks",
                   strict_ranks=strict, rank_policy=policy)
    counts, _, _ = check_lists_valid(r, w.nb)
    rng = np.random.default_rng(330 + index)
    flat = counts.reshape(-1)
    pick = {int(np.argmax(flat)), w.nb - 1, w.tiles - 1} | set(rng.choice(w.tiles, size=5, replace=False).tolist())
    fp8_attention_check(c, r, sorted(pick), f"{w.name} ranks strict={strict} {policy}")


def test_attention_v8_window_anchor():
    c = case(4)
    w = c.w
    r = absh.route(c.ctx, c.qh, c.kh, 0.9, 0, schedule="xcd", router="window-anchor", window=12,
                   anchor_stride=24, anchor_shift=7, step=2)
    check_lists_valid(r, w.nb)
    rng = np.random.default_rng(340)
    pick = {0, w.nb - 1, w.tiles - 1} | set(rng.choice(w.tiles, size=5, replace=False).tolist())
    fp8_attention_check(c, r, sorted(pick), f"{w.name} window-anchor")
