"""GPU parity: every step of the HIP path against the CPU oracle, through the C ABI.

Bars (written here, per step):
  * Hilbert perm, permutes, pooling, LPT queue, slack-fill counts: bit-exact;
  * block scores: within one float32 ulp (float64 sums in a different order,
    rounded once), at most a 1e-5 share of entries off;
  * routing sets and counts: exact, except tiles excused by the rule in
    routing_compare (threshold within 1e-5 of p, or a score tie within 5e-7);
    work and L then follow exactly from the counts;
  * attention on the GPU's own mask: max-abs <= 2e-2 and mean-abs <= 2e-3 against
    the float64 oracle (bf16 inputs, bf16 probabilities in the value product);
  * same-kernel invariants: p = 1 sparse == dense, the three schedules (order,
    xcd, longest-first) against each other, and two runs, all bit-identical:
    with blocks of 64 and 128 every schedule runs the same group units on the
    union kernel, with blocks of 16 the same single tiles on the tile kernel.
"""
import functools

import numpy as np
import pytest
import torch

import adaptive_block_sparse_hilbert_amd as absh
import workloads as W
from oracle import absh_oracle as O
from routing_compare import compare_routing

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
ATOL_MAX, ATOL_MEAN = 2e-2, 2e-3


def to_dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def bf16_bits_of(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class Case:
    """Inputs of one workload on the GPU and on the host (exact float32 of the bf16 values)."""

    def __init__(self, w, seed=None):
        self.w = w
        d = W.generate(w, seed=seed)
        self.bits = d
        self.s = d["s"]
        self.ctx = absh.create(w.T, w.Y, w.X, w.block)
        self.q, self.k, self.v = (to_dev_bf16(d[n]) for n in ("q16", "k16", "v16"))
        self.qh = absh.permute(self.ctx, self.q)
        self.kh = absh.permute(self.ctx, self.k)
        self.vt = absh.permute(self.ctx, self.v, layout=absh.ABSH_VT)
        torch.cuda.synchronize()
        self.perm, _ = O.hilbert_perm(w.T, w.Y, w.X)
        self._routes = {}

    def host(self, name):
        return W.bf16_to_f32(self.bits[name + "16"])

    @functools.cached_property
    def hq(self):
        return O.to_hilbert(self.host("q"), self.perm)

    @functools.cached_property
    def hk(self):
        return O.to_hilbert(self.host("k"), self.perm)

    @functools.cached_property
    def hv(self):
        return O.to_hilbert(self.host("v"), self.perm)

    def oracle_route(self, p=None, k=None):
        w = self.w
        key = (w.p if p is None else p, w.k_floor if k is None else k)
        if key not in self._routes:
            self._routes[key] = O.route(self.hq, self.hk, w.block, *key)
        R = self._routes[key]
        return O.Routing(R.nb, R.sizes, R.scores, R.P, R.order, R.cdf, R.count_topp, R.counts.copy())


@functools.lru_cache(maxsize=None)
def case(index):
    print(f"[gpu-parity] building case {W.workload(index).name}", flush=True)
    return Case(W.workload(index))


def check_lists_valid(r, nb):
    """Host-side validity of lists and queue before any kernel consumes them."""
    counts = r.counts.cpu().numpy()
    kv = r.kv_idx.cpu().numpy().astype(np.int64)
    queue = r.queue.cpu().numpy()
    assert counts.min() >= 1 and counts.max() <= nb
    assert np.array_equal(np.sort(queue), np.arange(queue.size))
    flat_c = counts.reshape(-1)
    flat_kv = kv.reshape(-1, nb)
    for t in range(flat_c.size):
        row = flat_kv[t, : flat_c[t]]
        assert row.min() >= 0 and row.max() < nb and np.all(np.diff(row) > 0), f"tile {t} list invalid"
    return counts, kv, queue


# ---------------------------------------------------------------- Hilbert permutation

@pytest.mark.parametrize("grid,block", [((4, 8, 8), 16), ((21, 30, 52), 64), ((21, 45, 80), 64),
                                        ((126, 30, 52), 128), ((1, 1, 1), 16), ((3, 5, 7), 16),
                                        ((2, 1, 9), 64), ((17, 2, 33), 128), ((64, 64, 64), 64)])
def test_perm_matches_oracle(grid, block):
    ctx = absh.create(*grid, block)
    perm, inv = absh.perm_copy(ctx)
    want, want_inv = O.hilbert_perm(*grid)
    assert np.array_equal(perm.cpu().numpy(), want)
    assert np.array_equal(inv.cpu().numpy(), want_inv)
    N = grid[0] * grid[1] * grid[2]
    assert (ctx.N, ctx.nb, ctx.n_pad) == (N, -(-N // block), -(-N // block) * block)


# ---------------------------------------------------------------- permute / unpermute

def test_permute_f32_rounds_to_nearest_even():
    w = W.workload(0)
    d = W.generate(w, want_fp32=True)
    ctx = absh.create(w.T, w.Y, w.X, w.block)
    x = torch.from_numpy(d["q32"]).to(DEV)
    xh = absh.permute(ctx, x)
    perm, _ = O.hilbert_perm(w.T, w.Y, w.X)
    want = np.transpose(W.bf16_bits(d["q32"])[:, perm], (0, 2, 1, 3))
    got = bf16_bits_of(xh)
    assert np.array_equal(got[:, :, : w.N], want)
    assert (got[:, :, w.N:] == 0).all()


@pytest.mark.parametrize("index", [0, 1])
def test_permute_rows_and_vt_bit_exact(index):
    c = case(index)
    w = c.w
    want = np.transpose(c.bits["k16"][:, c.perm], (0, 2, 1, 3))
    got = bf16_bits_of(c.kh)
    assert np.array_equal(got[:, :, : w.N], want)
    assert (got[:, :, w.N:] == 0).all()
    vpad = np.zeros((w.B, w.H, w.nb * w.block, w.d), dtype=np.uint16)
    vpad[:, :, : w.N] = np.transpose(c.bits["v16"][:, c.perm], (0, 2, 1, 3))
    kb = absh.vt_keys(w.block)
    want_vt = np.zeros((w.B, w.H, w.nb, w.d, kb), dtype=np.uint16)
    want_vt[..., : w.block] = vpad.reshape(w.B, w.H, w.nb, w.block, w.d).transpose(0, 1, 2, 4, 3)
    assert np.array_equal(bf16_bits_of(c.vt).reshape(want_vt.shape), want_vt)


@pytest.mark.parametrize("index", [0, 1])
def test_unpermute_round_trip(index):
    c = case(index)
    back = absh.unpermute(c.ctx, c.qh)
    assert torch.equal(back.view(torch.int16), c.q.view(torch.int16))


# ---------------------------------------------------------------- pooling and scores

@pytest.mark.parametrize("index", [0, 1, 2])
def test_pool_bit_exact(index):
    c = case(index)
    got = absh.pool(c.ctx, c.kh).cpu().numpy()
    want = O.block_means(c.hk, c.w.block)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("index", [0, 1, 2])
def test_scores_within_one_ulp(index):
    c = case(index)
    qbar, kbar = absh.pool(c.ctx, c.qh), absh.pool(c.ctx, c.kh)
    got = absh.block_scores(c.ctx, qbar, kbar).cpu().numpy()
    want = O.block_scores(O.block_means(c.hq, c.w.block), O.block_means(c.hk, c.w.block))
    ulp = np.abs(got.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1
    assert (ulp > 0).mean() <= 1e-5


# ---------------------------------------------------------------- routing

@pytest.mark.parametrize("index,p", [(0, None), (1, None), (2, None), (3, None), (4, 0.8), (4, 0.9), (4, 0.95)])
def test_route_matches_oracle(index, p):
    c = case(index)
    w = c.w
    p = w.p if p is None else p
    r = absh.route(c.ctx, c.qh, c.kh, p, w.k_floor, schedule="lpt")
    torch.cuda.synchronize()
    counts, kv, queue = check_lists_valid(r, w.nb)
    R = c.oracle_route(p=p)
    excused, failures = compare_routing(R, counts, kv, p)
    print(f"[route] {w.name} p={p}: density {counts.mean() / w.nb:.4f}, excused tiles {excused}")
    assert not failures, failures[:5]
    assert excused <= 0.01 * counts.size
    work = r.work.cpu().numpy()
    L = r.L.cpu().numpy()
    assert np.array_equal(work, counts.sum(-1))
    assert np.array_equal(L, (work.astype(np.float32) / np.float32(w.nb)).astype(np.float32))
    assert (counts >= min(w.k_floor, w.nb)).all()
    # LPT tile queue: exactly the oracle's order for these counts
    assert np.array_equal(queue, O.lpt_queue(counts))
    if w.block < 64:  # single tiles: one run holds the whole queue
        assert r.sched.cpu().numpy().tolist() == [0] + [w.tiles] * 8 + [1]
    if excused == 0:
        wo, Lo = O.workloads(R.counts)
        assert np.array_equal(work, wo) and np.array_equal(L, Lo)


@pytest.mark.parametrize("schedule", ["xcd", "lpt"])
def test_route_fp32_inputs(schedule):
    """The tiny fp32 workload routed from float32 rows (ABSH_ROWS_F32), against the
    oracle on the same float32 values; then attention on the bf16 rounding of those
    rows under the GPU's lists, against the oracle's."""
    w = W.workload(0)
    d = W.generate(w, want_fp32=True)
    ctx = absh.create(w.T, w.Y, w.X, w.block)
    q, k = (torch.from_numpy(d[n]).to(DEV) for n in ("q32", "k32"))
    qh, kh = (absh.permute(ctx, x, layout=absh.ABSH_ROWS_F32) for x in (q, k))
    perm, _ = O.hilbert_perm(w.T, w.Y, w.X)
    hq, hk = (O.to_hilbert(d[n], perm) for n in ("q32", "k32"))
    got_qh = qh.cpu().numpy()
    assert np.array_equal(got_qh[:, :, : w.N], hq) and (got_qh[:, :, w.N:] == 0).all()
    r = absh.route(ctx, qh, kh, w.p, w.k_floor, schedule=schedule)
    counts, kv, _ = check_lists_valid(r, ctx.nb)
    R = O.route(hq, hk, w.block, w.p, w.k_floor)
    excused, failures = compare_routing(R, counts, kv, w.p)
    print(f"[route f32] {w.name} {schedule}: excused tiles {excused}")
    assert not failures, failures[:5]
    assert excused <= 0.01 * counts.size
    qb, kb = absh.permute(ctx, q), absh.permute(ctx, k)
    vt = absh.permute(ctx, torch.from_numpy(d["v32"]).to(DEV), layout=absh.ABSH_VT)
    o = absh.unpermute(ctx, absh.sparse_attn(ctx, qb, kb, vt, r)).float().cpu().numpy()
    bf = [W.bf16_to_f32(W.bf16_bits(d[n])) for n in ("q32", "k32", "v32")]
    ref = O.attention(*bf, perm, w.block, lambda b, h, i: kv[b, h, i, : counts[b, h, i]])
    e = np.abs(o - ref)
    assert e.max() <= ATOL_MAX and e.mean() <= ATOL_MEAN


def test_importance_order_prefix():
    c = case(1)
    w = c.w
    r = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor, order_depth=16)
    got = r.order.cpu().numpy().astype(np.int64)
    R = c.oracle_route()
    want = R.order[..., :16]
    mism = np.argwhere((got != want).any(-1))
    # a differing prefix is allowed only where the oracle's scores tie to the last bits
    for b, h, i in mism:
        k = int(np.argmax(got[b, h, i] != want[b, h, i]))
        s = R.scores[b, h, i].astype(np.float64)
        assert abs(s[got[b, h, i, k]] - s[want[b, h, i, k]]) <= 5e-7 * max(1.0, abs(s[want[b, h, i, k]]))
    assert len(mism) <= 0.01 * got.shape[2] * w.H


def test_order_prefix_past_nb_is_minus_one():
    c = case(0)
    r = absh.route(c.ctx, c.qh, c.kh, 0.9, 2, order_depth=20)
    got = r.order.cpu().numpy().astype(np.int64)
    assert (got[..., 16:] == -1).all()
    assert all(sorted(row[:16].tolist()) == list(range(16)) for row in got.reshape(-1, 20))


def test_slack_fill_matches_oracle():
    c = case(3)
    w = c.w
    base = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor, slack_frac=0.0, schedule="lpt")
    filled = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor, slack_frac=w.slack_frac, schedule="lpt")
    torch.cuda.synchronize()
    c0, _, _ = check_lists_valid(base, w.nb)
    c1, kv1, q1 = check_lists_valid(filled, w.nb)
    want = O.slack_fill(c0, w.slack_frac)
    assert np.array_equal(c1, want)
    R0 = c.oracle_route()
    if np.array_equal(c0, R0.counts):  # no excused tile: the fill of the oracle's own counts
        assert np.array_equal(c1, O.slack_fill(R0.counts, w.slack_frac))
    added = int((c1 - c0).sum())
    E = O.slack_budget(c0, w.slack_frac)
    print(f"[slack] {w.name}: sum before {int(c0.sum())}, E {E}, added {added}")
    assert added == min(E, int((w.nb - c0).sum()))
    # the filled sets are the oracle's importance-order prefixes of the new counts
    R = c.oracle_route()
    R.counts = c1.astype(np.int64)
    excused, failures = compare_routing(R, c1, kv1, w.p)
    assert not failures, failures[:5]
    assert np.array_equal(q1, O.lpt_queue(c1))
    work = filled.work.cpu().numpy()
    assert np.array_equal(work, c1.sum(-1))



@pytest.mark.parametrize("index,p,beta", [(0, 0.9, 0.3), (0, 0.99, 0.99), (1, 0.9, 0.02), (1, 0.9, 0.5),
                                          (1, 0.995, 0.99), (4, 0.8, 0.1)])
def test_slack_fill_sweep(index, p, beta):
    """Slack fill and longest-first queue over one chunk (32 tiles) and many (6,144 and
    18,432 tiles, ragged last chunk), from a sliver of slack to a budget that fills
    most tiles up to nb: counts equal the closed-form water level exactly, the queue
    equals the stable longest-first order of the new counts."""
    c = case(index)
    w = c.w
    base = absh.route(c.ctx, c.qh, c.kh, p, w.k_floor, slack_frac=0.0, schedule="lpt")
    filled = absh.route(c.ctx, c.qh, c.kh, p, w.k_floor, slack_frac=beta, schedule="lpt")
    torch.cuda.synchronize()
    c0, _, _ = check_lists_valid(base, w.nb)
    c1, _, q1 = check_lists_valid(filled, w.nb)
    want = O.slack_fill_level(c0, beta)
    print(f"[slack sweep] {w.name} p={p} beta={beta}: E {O.slack_budget(c0, beta)}, "
          f"tiles at nb {(want == w.nb).mean():.3f}")
    assert np.array_equal(c1, want)
    assert np.array_equal(q1, O.lpt_queue(c1))
    assert np.array_equal(filled.work.cpu().numpy(), c1.sum(-1))



def test_route_underflowed_probabilities():
    """Scores 128 apart (exact in float32 and float64): all but the top six blocks of
    a row have probability 0 in float64, so they tie at 0 and follow by block id.
    The floor (10) and a slack fill (to 15) reach into them, in both the Top-p pass
    and the re-selection: counts, lists and the importance order equal the oracle's."""
    T, Y, X, block, H, d = 4, 16, 16, 16, 2, 64
    N = T * Y * X
    nb = N // block
    perm, _ = O.hilbert_perm(T, Y, X)
    ranks = np.stack([np.arange(nb), (np.arange(nb) * 37) % nb])
    qh = np.zeros((1, H, N, d), np.float32)
    kh = np.zeros((1, H, N, d), np.float32)
    qh[..., 0] = 1.0
    for h in range(H):
        kh[0, h, :, 0] = np.repeat(ranks[h] * 1024.0, block)
    q = np.empty((1, N, H, d), np.float32)
    k = np.empty((1, N, H, d), np.float32)
    q[:, perm] = np.transpose(qh, (0, 2, 1, 3))
    k[:, perm] = np.transpose(kh, (0, 2, 1, 3))
    ctx = absh.create(T, Y, X, block)
    qd = absh.permute(ctx, torch.from_numpy(q).to(DEV).bfloat16())
    kd = absh.permute(ctx, torch.from_numpy(k).to(DEV).bfloat16())
    R = O.route(qh, kh, block, 0.9, 10)
    assert (R.P[..., :] == 0).sum(-1).min() == nb - 6
    for beta in (0.0, 0.5):
        want = O.slack_fill_level(R.counts, beta)
        r = absh.route(ctx, qd, kd, 0.9, 10, slack_frac=beta, schedule="lpt", order_depth=12)
        torch.cuda.synchronize()
        counts, kv, _ = check_lists_valid(r, nb)
        assert np.array_equal(counts, want), (beta, np.unique(counts))
        for h in range(H):
            for i in range(nb):
                c = int(want[0, h, i])
                assert np.array_equal(kv[0, h, i, :c], np.sort(R.order[0, h, i, :c])), (beta, h, i)
        assert np.array_equal(r.order.cpu().numpy().astype(np.int64), R.order[..., :12])



@pytest.mark.parametrize("p", [0.5, 0.9, 1 / 3, 0.25, 0.999])
def test_route_uniform_scores(p):
    """All block scores equal (q = k = 0): every block ties, P = 1/60, and the count
    is where the float64 running sum of 1/60 first reaches p. Its rounding decides
    (30 terms sum to just under 0.5, so p = 0.5 takes 31); counts and the lists
    (the first c block ids) equal the oracle's."""
    T, Y, X, block, H, d = 4, 15, 16, 16, 2, 64
    N = T * Y * X
    nb = N // block
    zero = np.zeros((1, H, N, d), np.float32)
    ctx = absh.create(T, Y, X, block)
    zd = absh.permute(ctx, torch.zeros((1, N, H, d), dtype=torch.bfloat16, device=DEV))
    R = O.route(zero, zero, block, p, 2)
    r = absh.route(ctx, zd, zd, p, 2, schedule="lpt")
    torch.cuda.synchronize()
    counts, kv, _ = check_lists_valid(r, nb)
    assert np.array_equal(counts, R.counts), (p, np.unique(counts), np.unique(R.counts))
    c = int(R.counts.reshape(-1)[0])
    assert (kv[..., :c] == np.arange(c)).all()


@pytest.mark.parametrize("p,k,beta", [(0.9, 4, 0.0), (0.5, 1, 0.0), (0.8, 2, 0.1), (0.3, 8, 0.05)])
def test_route_block_patterns_with_many_ties(p, k, beta):
    """Every token of a Hilbert block carries one of five row patterns (entries in
    -1 .. 1 by halves), so the block means are the patterns themselves and the block
    scores (dot products over d = 64, divided by 8) are exact in float32 and float64
    and take at most 25 values per head: rows are made of large groups of exact ties,
    at the threshold and elsewhere. The threshold searches (which stop once one key
    is left in the interval) must reproduce the oracle's counts and lists exactly,
    ties going to the smaller block id, with and without a slack fill."""
    T, Y, X, block, H, d = 5, 20, 40, 16, 4, 64
    N = T * Y * X
    rng = np.random.default_rng(23)
    ctx = absh.create(T, Y, X, block)
    nb = ctx.nb
    perm, _ = O.hilbert_perm(T, Y, X)
    x = []
    for _ in range(2):
        pat = (rng.integers(-2, 3, size=(H, 5, d)) * 0.5).astype(np.float32)
        which = rng.integers(0, 5, size=(H, nb))
        hx = np.zeros((1, H, N, d), np.float32)
        for h in range(H):
            hx[0, h] = pat[h, which[h, np.arange(N) // block]]
        g = np.zeros((1, N, H, d), np.float32)
        g[0, perm] = hx[0].transpose(1, 0, 2)
        x.append(g)
    qh, kh = (absh.permute(ctx, torch.from_numpy(a).to(DEV), layout=absh.ABSH_ROWS_F32) for a in x)
    hq, hk = (O.to_hilbert(a, perm) for a in x)
    R = O.route(hq, hk, block, p, k)
    assert max(len(np.unique(R.scores[0, h])) for h in range(H)) <= 25
    want = R.counts.copy() if beta == 0 else O.slack_fill(R.counts, beta)
    for schedule in ("xcd", "lpt"):
        r = absh.route(ctx, qh, kh, p, k, slack_frac=beta, schedule=schedule)
        torch.cuda.synchronize()
        counts, kv, _ = check_lists_valid(r, nb)
        assert np.array_equal(counts, want), (schedule, int((counts != want).sum()))
        for h in range(H):
            for i in range(nb):
                expect = np.sort(R.order[0, h, i, : want[0, h, i]])
                assert np.array_equal(kv[0, h, i, : counts[0, h, i]], expect), (schedule, h, i)


def test_route_deterministic():
    c = case(1)
    w = c.w
    a = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor, order_depth=8)
    b = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor, order_depth=8)
    for x, y in ((a.counts, b.counts), (a.kv_idx, b.kv_idx), (a.order, b.order), (a.queue, b.queue)):
        cnt = a.counts.reshape(-1)
        if x is a.kv_idx:
            xs, ys = x.reshape(cnt.numel(), -1), y.reshape(cnt.numel(), -1)
            for t in range(cnt.numel()):
                assert torch.equal(xs[t, : cnt[t]], ys[t, : cnt[t]])
        else:
            assert torch.equal(x, y)



@pytest.mark.parametrize("delta", [1e-7, 2e-6])
def test_route_threshold_next_to_p(delta):
    """p set a hair below or above an exact prefix mass: the count is decided there.

    Channel 0 alone is non-zero (q = 1, k of Hilbert block j = b_j / 2 with a
    per-head order of the b_j), so every block mean and every score b_j / 16 is
    exact in float32 and in float64 alike, and all tiles share one sorted mass
    curve. With p = cdf_m -/+ delta the fewest blocks reaching p are m, resp. m + 1,
    for every tile; delta sits inside the error of a float32 sum of the masses.
    """
    T, Y, X, block, H, d = 4, 8, 8, 16, 2, 64
    N = T * Y * X
    nb = N // block
    perm, _ = O.hilbert_perm(T, Y, X)
    ranks = np.stack([np.arange(nb), (np.arange(nb) * 7) % nb])      # head 1: another order
    qh = np.zeros((1, H, N, d), np.float32)
    kh = np.zeros((1, H, N, d), np.float32)
    qh[..., 0] = 1.0
    for h in range(H):
        kh[0, h, :, 0] = np.repeat(ranks[h] / 2.0, block)
    q = np.empty((1, N, H, d), np.float32)
    k = np.empty((1, N, H, d), np.float32)
    q[:, perm] = np.transpose(qh, (0, 2, 1, 3))
    k[:, perm] = np.transpose(kh, (0, 2, 1, 3))
    ctx = absh.create(T, Y, X, block)
    qd = absh.permute(ctx, torch.from_numpy(q).to(DEV).bfloat16())
    kd = absh.permute(ctx, torch.from_numpy(k).to(DEV).bfloat16())
    cdf = O.route(qh, kh, block, 0.5, 1).cdf[0, 0, 0]
    for m in (2, 5, 9, 14):
        for p, want in ((cdf[m - 1] - delta, m), (cdf[m - 1] + delta, m + 1)):
            R = O.route(qh, kh, block, float(p), 1)
            assert (R.counts == want).all()
            r = absh.route(ctx, qd, kd, float(p), 1, schedule="lpt")
            torch.cuda.synchronize()
            counts, kv, _ = check_lists_valid(r, nb)
            assert (counts == want).all(), (m, p, np.unique(counts))
            for h in range(H):
                top = np.sort(R.order[0, h, 0, :want])
                assert (kv[0, h, :, :want] == top).all()


# ---------------------------------------------------------------- attention

def attention_errors(c, r, tiles):
    """Max / mean abs error of the GPU output rows of `tiles` against the oracle on the GPU's mask."""
    w = c.w
    oh = absh.sparse_attn(c.ctx, c.qh, c.kh, c.vt, r)
    o = absh.unpermute(c.ctx, oh).float().cpu().numpy()
    counts = r.counts.cpu().numpy().reshape(-1)
    kv = r.kv_idx.cpu().numpy().astype(np.int64).reshape(counts.size, -1)
    errs = []
    for t in tiles:
        bh, i = divmod(int(t), w.nb)
        b, h = divmod(bh, w.H)
        blocks = kv[t, : counts[t]]
        ref = O.attention_tile(c.hq[b, h], c.hk[b, h], c.hv[b, h], w.block, i, blocks)
        rows = c.perm[i * w.block: min((i + 1) * w.block, w.N)]
        errs.append(np.abs(o[b, rows, h, :] - ref))
    e = np.concatenate([x.ravel() for x in errs])
    return e.max(), e.mean()


def test_attention_tiny_all_tiles():
    c = case(0)
    w = c.w
    r = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor)
    check_lists_valid(r, w.nb)
    mx, mean = attention_errors(c, r, range(w.tiles))
    print(f"[attn] tiny: max {mx:.3e} mean {mean:.3e}")
    assert mx <= ATOL_MAX and mean <= ATOL_MEAN


def stratified_tiles(counts, rng):
    """Tiles to check: per head one random tile and its last (partial) query block; over
    all tiles the lightest, the heaviest and one random tile per count quintile; and one
    random tile per position within a work unit (query block i mod 4: which member of
    its unit, and so which waves and which half of a split unit, computed it)."""
    B, H, nb = counts.shape
    flat = counts.reshape(-1)
    pick = {int(np.argmax(flat)), int(np.argmin(flat))}
    for bh in range(B * H):
        pick |= {bh * nb + int(rng.integers(nb)), bh * nb + nb - 1}
    order = np.argsort(flat, kind="stable")
    for part in np.array_split(order, 5):
        pick.add(int(rng.choice(part)))
    for m in range(4):
        i = int(rng.choice(np.arange(m, nb, 4)))
        pick.add(int(rng.integers(B * H)) * nb + i)
    return sorted(pick)


@pytest.mark.parametrize("index,schedule", [(1, "xcd"), (2, "xcd"), (3, "xcd"), (4, "xcd"), (2, "lpt"),
                                            (3, "lpt")])
def test_attention_sampled_tiles(index, schedule):
    c = case(index)
    w = c.w
    r = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor, slack_frac=w.slack_frac, schedule=schedule)
    counts, _, _ = check_lists_valid(r, w.nb)
    rng = np.random.default_rng(100 + index)
    pick = stratified_tiles(counts, rng)
    mx, mean = attention_errors(c, r, sorted(pick))
    print(f"[attn] {w.name}: max {mx:.3e} mean {mean:.3e} over {len(pick)} tiles")
    assert mx <= ATOL_MAX and mean <= ATOL_MEAN


@pytest.mark.parametrize("index", [0, 1])
def test_p_one_sparse_equals_dense(index):
    c = case(index)
    w = c.w
    # the dense mode runs group units, like the "order" schedule
    r = absh.route(c.ctx, c.qh, c.kh, 1.0, 0, schedule="order")
    counts, kv, _ = check_lists_valid(r, w.nb)
    assert (counts == w.nb).all()
    sparse = absh.sparse_attn(c.ctx, c.qh, c.kh, c.vt, r)
    dense = absh.sparse_attn(c.ctx, c.qh, c.kh, c.vt, None)
    torch.cuda.synchronize()
    assert torch.equal(sparse.view(torch.int16), dense.view(torch.int16))



@pytest.mark.parametrize("schedule", ["xcd", "lpt"])
def test_attention_rising_logits(schedule):
    """Logits that rise by about 2.5 per key block in the walk order, so a row's
    maximum keeps overtaking the kernel's reference maximum and the lazy rescale
    fires again and again (plus a ragged tail). Dense routing (p = 1); output
    against the oracle's float64 attention with the attention bar."""
    T, Y, X, block, H, d = 3, 17, 19, 64, 2, 128   # N = 969 tokens: 16 blocks, tail of 9
    N = T * Y * X
    rng = np.random.default_rng(5)
    perm, _ = O.hilbert_perm(T, Y, X)
    nb = -(-N // block)
    # in Hilbert order: q = 1 on channel 0; k on channel 0 grows with the block index
    qh = np.zeros((1, H, N, d), np.float32)
    kh = (rng.standard_normal((1, H, N, d)) * 0.25).astype(np.float32)
    qh[..., 0] = 1.0
    blk = np.arange(N) // block
    kh[..., 0] = (2.5 * np.sqrt(d) * blk)[None, None, :] + rng.standard_normal((1, H, N)).astype(np.float32)
    vh = rng.standard_normal((1, H, N, d)).astype(np.float32)
    grid = lambda a: np.ascontiguousarray(np.transpose(a, (0, 2, 1, 3)))  # [B, N(hilbert), H, d]
    q = np.empty((1, N, H, d), np.float32)
    k = np.empty_like(q)
    v = np.empty_like(q)
    q[:, perm], k[:, perm], v[:, perm] = grid(qh), grid(kh), grid(vh)
    bits = [W.bf16_bits(a) for a in (q, k, v)]
    ctx = absh.create(T, Y, X, block)
    qd, kd, vd = (to_dev_bf16(b) for b in bits)
    qhd, khd = absh.permute(ctx, qd), absh.permute(ctx, kd)
    vt = absh.permute(ctx, vd, layout=absh.ABSH_VT)
    r = absh.route(ctx, qhd, khd, 1.0, 0, schedule=schedule)
    counts, _, _ = check_lists_valid(r, nb)
    assert (counts == nb).all()
    o = absh.unpermute(ctx, absh.sparse_attn(ctx, qhd, khd, vt, r)).float().cpu().numpy()
    ref = O.attention(W.bf16_to_f32(bits[0]), W.bf16_to_f32(bits[1]), W.bf16_to_f32(bits[2]), perm, block)
    e = np.abs(o - ref)
    print(f"[rising] {schedule}: max {e.max():.3e} mean {e.mean():.3e}")
    assert e.max() <= ATOL_MAX and e.mean() <= ATOL_MEAN


def test_dense_matches_oracle_tiny():
    c = case(0)
    w = c.w
    o = absh.unpermute(c.ctx, absh.sparse_attn(c.ctx, c.qh, c.kh, c.vt, None)).float().cpu().numpy()
    ref = O.attention(c.host("q"), c.host("k"), c.host("v"), c.perm, w.block, None)
    e = np.abs(o - ref)
    assert e.max() <= ATOL_MAX and e.mean() <= ATOL_MEAN


def expected_groups(counts, kv, nb, M):
    """Union lists of the M query blocks qM .. qM+M-1 with membership flags, from the tile lists."""
    B, H, _ = counts.shape
    per_head = -(-nb // M)
    lists, lens = [], []
    for b in range(B):
        for h in range(H):
            for q in range(per_head):
                sets = [set(kv[b, h, i, : counts[b, h, i]].tolist()) if i < nb else set()
                        for i in range(q * M, q * M + M)]
                allj = sorted(set().union(*sets))
                ent = [j | sum((1 << (28 + m)) for m in range(M) if j in sets[m]) for j in allj]
                lists.append(np.array(ent, dtype=np.int64).astype(np.uint32))
                lens.append(len(ent))
    return lists, np.array(lens)


def expected_xcd_bounds(cost, overhead=1, segments=8):
    """Cut the units where the running cost (cost + overhead) first reaches x/8 of the total."""
    cost = np.asarray(cost, dtype=np.int64) + overhead
    before = np.concatenate([[0], np.cumsum(cost)])[:-1]
    total = int(cost.sum())
    bounds = [0]
    for x in range(1, segments):
        target = -(-total * x // segments)
        bounds.append(int(np.searchsorted(before, target, side="left")))
    return bounds + [cost.size]


def expected_unit_queue(cost, bounds):
    """Inside each XCD run, the units by union length descending, ties by unit index."""
    cost = np.asarray(cost)
    out = []
    for x in range(8):
        run = np.arange(bounds[x], bounds[x + 1])
        out.extend(run[np.lexsort((run, -cost[run]))].tolist())
    return np.array(out, dtype=np.int64)


@pytest.mark.parametrize("index", [0, 1, 3, 4])
def test_schedules_bit_identical(index):
    """Every schedule runs the same units with the same kernel, so the outputs agree bit for bit;
    the schedules differ only in the units' order (and the longest-first queue in its grouping,
    single tiles below blocks of 64)."""
    c = case(index)
    w = c.w
    M = 2 if w.block >= 128 else 4
    union = w.block in (64, 128)  # group units on the union kernel, single tiles on the tile kernel
    units = w.B * w.H * (-(-w.nb // M))
    assert absh.lists_units(c.ctx, w.B, w.H, "xcd") == units
    assert absh.lists_units(c.ctx, w.B, w.H, "ranks") == units
    assert absh.lists_units(c.ctx, w.B, w.H, "lpt") == (units if union else w.tiles)
    outs = {}
    for sched in ("order", "lpt", "xcd"):
        r = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor, slack_frac=w.slack_frac, schedule=sched)
        counts, kv, queue = check_lists_valid(r, w.nb)
        bounds = r.sched.cpu().numpy().tolist()
        if sched == "lpt":
            assert np.array_equal(queue, O.lpt_queue(counts))
        else:
            assert np.array_equal(queue, np.arange(w.tiles))
        if sched == "lpt" and not union:
            assert bounds == [0] + [w.tiles] * 8 + [1]
        else:
            want_lists, want_len = expected_groups(counts, kv, w.nb, M)
            got_len = r.unit_cnt.cpu().numpy()[:units]
            got = r.unit_list.cpu().numpy().view(np.uint32)
            assert np.array_equal(got_len, want_len)
            for u in range(units):
                assert np.array_equal(got[u, : got_len[u]], want_lists[u]), u
            if sched == "order":
                assert bounds == [0] + [units] * 8 + [M]
            else:
                assert bounds == expected_xcd_bounds(got_len) + [M], (bounds, expected_xcd_bounds(got_len))
            if sched == "lpt":
                uq = r.unit_queue.cpu().numpy()[:units]
                assert np.array_equal(uq, expected_unit_queue(got_len, bounds))
        outs[sched] = absh.sparse_attn(c.ctx, c.qh, c.kh, c.vt, r)
        outs[sched + "2"] = absh.sparse_attn(c.ctx, c.qh, c.kh, c.vt, r)
    torch.cuda.synchronize()
    rows = torch.arange(w.N, device=DEV)
    ref = outs["order"][:, :, rows].view(torch.int16)
    for k, v in outs.items():
        assert torch.equal(v[:, :, rows].view(torch.int16), ref), k


# ---------------------------------------------------------------- edge shapes


@pytest.mark.parametrize("grid,block,d,H,p,k", [
    ((16, 128, 128), 128, 64, 1, 0.9, 4),   # nb = 2048, the router's maximum, all blocks full
    ((16, 127, 127), 128, 128, 1, 0.8, 8),  # nb = 2017, ragged tail of 16 tokens
    ((5, 20, 40), 16, 64, 2, 0.9, 2),       # nb = 250
    ((9, 30, 41), 16, 128, 2, 0.95, 3),     # nb = 692, ragged tail of 14
])
@pytest.mark.parametrize("schedule", ["xcd", "lpt"])
def test_block_counts_up_to_the_maximum(grid, block, d, H, p, k, schedule):
    """Routing and attention at block counts that use every row width of the
    selection (up to nb = 2048): lists against the oracle's (the routing rule's
    excuses apply), sampled tiles against its attention."""
    T, Y, X = grid
    N = T * Y * X
    print(f"[max-blocks] grid {grid} block {block} d {d} H {H} schedule {schedule}", flush=True)
    rng = np.random.default_rng(11)
    q32 = rng.standard_normal((1, N, H, d)).astype(np.float32) * 2
    k32 = rng.standard_normal((1, N, H, d)).astype(np.float32) * 2
    v32 = rng.standard_normal((1, N, H, d)).astype(np.float32)
    bits = [W.bf16_bits(a) for a in (q32, k32, v32)]
    ctx = absh.create(T, Y, X, block)
    nb = ctx.nb
    qd, kd, vd = (to_dev_bf16(b) for b in bits)
    qh, kh = absh.permute(ctx, qd), absh.permute(ctx, kd)
    vt = absh.permute(ctx, vd, layout=absh.ABSH_VT)
    r = absh.route(ctx, qh, kh, p, k, schedule=schedule)
    counts, kv, _ = check_lists_valid(r, nb)
    perm, _ = O.hilbert_perm(T, Y, X)
    hq, hk, hv = (O.to_hilbert(W.bf16_to_f32(b), perm) for b in bits)
    R = O.route(hq, hk, block, p, k)
    excused, failures = compare_routing(R, counts, kv, p)
    assert not failures, failures[:5]
    assert excused <= 0.01 * counts.size
    if block >= 64 or schedule != "lpt":  # group units: their union lists, built inside the selection
        M = 2 if block >= 128 else 4
        units = absh.lists_units(ctx, 1, H, schedule)
        want_lists, want_len = expected_groups(counts, kv, nb, M)
        got_len = r.unit_cnt.cpu().numpy()[:units]
        got = r.unit_list.cpu().numpy().view(np.uint32)
        assert np.array_equal(got_len, want_len)
        for u in range(units):
            assert np.array_equal(got[u, : got_len[u]], want_lists[u]), u
    oh = absh.sparse_attn(ctx, qh, kh, vt, r)
    o = absh.unpermute(ctx, oh).float().cpu().numpy()
    flat = counts.reshape(-1)
    pick = sorted({0, nb - 1, int(np.argmax(flat)), int(np.argmin(flat)), flat.size - 1}
                  | set(rng.choice(flat.size, size=4, replace=False).tolist()))
    kvf = kv.reshape(flat.size, nb)
    for t in pick:
        h, i = divmod(t, nb)
        ref = O.attention_tile(hq[0, h], hk[0, h], hv[0, h], block, i, kvf[t, : flat[t]])
        rows = perm[i * block: min((i + 1) * block, N)]
        e = np.abs(o[0, rows, h, :] - ref)
        assert e.max() <= ATOL_MAX and e.mean() <= ATOL_MEAN, (t, e.max(), e.mean())


@pytest.mark.parametrize("grid,block,d,H,B,p,k", [
    ((1, 1, 1), 16, 64, 1, 1, 0.9, 2),      # one token, one partial block
    ((2, 3, 5), 16, 64, 2, 2, 0.5, 0),      # N = 30 < 2 blocks, batch of 2
    ((4, 4, 4), 64, 128, 3, 1, 0.7, 9),     # exactly one full block, floor above nb
    ((5, 6, 7), 64, 128, 2, 1, 0.3, 1),     # ragged tail of 18
    ((3, 9, 10), 128, 128, 2, 1, 0.99, 1),  # ragged tail with block 128
    ((2, 8, 8), 16, 128, 2, 1, 0.05, 3),    # tiny p: the floor decides
])
@pytest.mark.parametrize("schedule", ["xcd", "lpt"])
def test_edge_shapes(grid, block, d, H, B, p, k, schedule):
    T, Y, X = grid
    N = T * Y * X
    rng = np.random.default_rng(7)
    q32 = rng.standard_normal((B, N, H, d)).astype(np.float32) * 2
    k32 = rng.standard_normal((B, N, H, d)).astype(np.float32) * 2
    v32 = rng.standard_normal((B, N, H, d)).astype(np.float32)
    bits = [W.bf16_bits(a) for a in (q32, k32, v32)]
    ctx = absh.create(T, Y, X, block)
    qd, kd, vd = (to_dev_bf16(b) for b in bits)
    qh, kh = absh.permute(ctx, qd), absh.permute(ctx, kd)
    vt = absh.permute(ctx, vd, layout=absh.ABSH_VT)
    r = absh.route(ctx, qh, kh, p, k, slack_frac=0.25, schedule=schedule)
    counts, kv, _ = check_lists_valid(r, ctx.nb)
    perm, _ = O.hilbert_perm(T, Y, X)
    hq, hk, hv = (O.to_hilbert(W.bf16_to_f32(b), perm) for b in bits)
    base = O.route(hq, hk, block, p, k)
    want = O.slack_fill(base.counts, 0.25)
    assert np.array_equal(counts, want)
    o = absh.unpermute(ctx, absh.sparse_attn(ctx, qh, kh, vt, r)).float().cpu().numpy()
    ref = O.attention(W.bf16_to_f32(bits[0]), W.bf16_to_f32(bits[1]), W.bf16_to_f32(bits[2]), perm, block,
                      lambda b, h, i: kv[b, h, i, : counts[b, h, i]])
    e = np.abs(o - ref)
    assert e.max() <= ATOL_MAX and e.mean() <= ATOL_MEAN


# ---------------------------------------------------------------- launch state

def test_attention_on_two_streams_with_own_counters():
    """Each set of lists carries its own work counters, so attention on two sets can run
    concurrently on two streams; every output equals the same call run alone, and the
    counters are zero again afterwards."""
    c = case(1)
    w = c.w
    r1 = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor, schedule="xcd")
    r2 = absh.route(c.ctx, c.qh, c.kh, 0.8, w.k_floor, schedule="lpt")
    ref1 = absh.sparse_attn(c.ctx, c.qh, c.kh, c.vt, r1)
    ref2 = absh.sparse_attn(c.ctx, c.qh, c.kh, c.vt, r2)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        o1, o2 = torch.empty_like(ref1), torch.empty_like(ref2)
        absh.sparse_attn(c.ctx, c.qh, c.kh, c.vt, r1, out=o1, stream=s1)
        absh.sparse_attn(c.ctx, c.qh, c.kh, c.vt, r2, out=o2, stream=s2)
        outs.append((o1, o2))
    torch.cuda.synchronize()
    rows = torch.arange(w.N, device=DEV)
    for o1, o2 in outs:
        assert torch.equal(o1[:, :, rows].view(torch.int16), ref1[:, :, rows].view(torch.int16))
        assert torch.equal(o2[:, :, rows].view(torch.int16), ref2[:, :, rows].view(torch.int16))
    assert (r1.pull == 0).all() and (r2.pull == 0).all()


@pytest.mark.parametrize("index,schedule", [(1, "xcd"), (0, "lpt")])
def test_busy_record(index, schedule):
    """The busy record holds one (start, end) pair per workgroup of the launch, end after
    start, and leaves the rows past the grid untouched."""
    c = case(index)
    w = c.w
    r = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor, schedule=schedule)
    rec = absh.busy_record(c.ctx, r)
    rec.fill_(0)
    absh.sparse_attn(c.ctx, c.qh, c.kh, c.vt, r)
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    host = rec.cpu().numpy()
    ran = host[:, 1] > 0
    n = int(ran.sum())
    assert n >= cus and n % cus == 0 and ran[:n].all() and not ran[n:].any()
    assert (host[:n, 1] > host[:n, 0]).all()
    ticks = absh.busy_ticks(rec)
    print(f"[busy] {w.name} {schedule}: {n} workgroups, rho {ticks.max() / ticks.mean():.3f}")
    if w.tiles > 64 * n:  # enough work for every workgroup: the pulls keep them within 2x of the mean
        assert ticks.max() / ticks.mean() < 2.0
