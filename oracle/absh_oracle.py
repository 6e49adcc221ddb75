"""CPU oracle for the Hilbert-ordered Top-p block router and block-sparse attention.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The GPU library never calls it, and the
two share no code.

What it computes follows the FVAttn pages (the alanhou.org explainer of FVAttn,
sections "Core Mechanism" and "Key Concepts"; the xllm-io review of FVAttn,
sections 三 "技术架构" Stage 1, 核心公式 Eq. 1-2, 3.1 and the SASA steps of 五
"代码实现分析"). Where the pages leave a step open the plainest reading is taken;
each is named where it is used:

  * Hilbert order (review 3.1): tokens of the (T, Y, X) latent grid are sorted by
    their index on a 3-D Hilbert curve over the enclosing 2^m cube (cells outside
    the grid are skipped), using Skilling's transform (J. Skilling, "Programming
    the Hilbert curve", AIP Conf. Proc. 707, 2004) with axes (t, y, x), most
    significant bit first. The sorted sequence is cut into blocks of b tokens;
    the last block may be partial.
  * Block summaries: the arithmetic mean of each block's q (and k) rows.
  * Block scores s_ij = qbar_i . kbar_j / sqrt(d), softmax over key blocks j.
  * Top-p (explainer, "Top-p Routing with Safety Floor"): the fewest blocks, in
    descending probability (ties: smaller block id first), whose cumulative
    probability reaches p (CDF >= p); p >= 1 keeps every block.
  * Top-k floor: count' = max(count, min(k, nb)), taking the next blocks of the
    same importance order.
  * Eq. 1: L_h = mean over query blocks of the retained count.
  * Slack fill (one-GPU reading of SASA): E = floor(beta * sum count') extra
    blocks; repeatedly raise the lightest tile (ties: lowest tile id; full tiles
    skipped) by the next block of its own importance order.
  * LPT queue (one-GPU reading of RLB): tiles sorted by retained count,
    descending, ties by ascending tile id.
  * Structured router (LVSA note): a local window over block ids plus every
    stride-th key block as a global anchor, the anchors' offset rotating with
    the diffusion step.
  * Rank-level RLB and SASA (review Eq. 2, 5-10, 3.2, 3.3) with the eight XCDs
    of one GPU as the ranks: contiguous head placement, the piecewise policy on
    rho, an exact search of the one-send-one-receive migration space over the
    review's pair topologies (ranks matched in pairs; a pair moves one head
    either way or swaps one head each), and per-rank slack budgets spent by
    water-filling the rank's tiles.
  * Attention: exact softmax(Q K_R^T / sqrt(d)) V_R over the tokens of the
    retained key blocks R of each query block.
  * V quantization (review, "Block-Sparse Attention Execution" and 3.4): V is
    stored in the OCP 8-bit E4M3 format with one power-of-two scale per head and
    channel (the smallest that brings the channel's largest magnitude to 448 or
    below); quantized attention is the exact attention above with V replaced by
    its dequantized values.

Precision: routing decisions are integers decided by floating point, so the
oracle takes them in the same precision as the GPU library: block means as the
float64 mean of the rows rounded to float32; scores as a float64 dot product
divided by sqrt(d) and rounded to float32; softmax, cumulative sums and the p
comparison in float64. Attention is computed in float64.

Parity pins: every function here is checked in tests/test_oracle_*.py against
properties the pages or the mathematics fix (closed forms, brute force, library
special cases); see the header of each test file.
"""
from __future__ import annotations

import heapq
import itertools
import math
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

# --------------------------------------------------------------------------
# Hilbert order
# --------------------------------------------------------------------------


def hilbert_bits(*extent: int) -> int:
    """Bits per axis m of the enclosing 2^m cube: m = max(1, ceil(log2(max extent))).

    Follows: xllm-io review, 3.1 (Hilbert block organisation); reading: the enclosing 2^m cube.
    """
    biggest = max(extent)
    m = 1
    while (1 << m) < biggest:
        m += 1
    return m


def hilbert_index(coords: np.ndarray, m: int) -> np.ndarray:
    """Hilbert index of each cell (rows of `coords`, one column per axis) on the 2^m cube.

    Skilling's axes-to-index direction: undo the per-level reflections and axis
    exchanges from the top bit down, Gray-encode across the axes, then read the
    transposed bits out most-significant first, axis 0 first within each level.
    """
    coords = np.asarray(coords, dtype=np.int64)
    n = coords.shape[1]
    x = [coords[:, i].copy() for i in range(n)]
    q = 1 << (m - 1)
    while q > 1:
        low = q - 1
        for i in range(n):
            on = (x[i] & q) != 0
            if i == 0:
                x[0] = np.where(on, x[0] ^ low, x[0])
                continue
            swap = (x[0] ^ x[i]) & low
            new0 = np.where(on, x[0] ^ low, x[0] ^ swap)
            newi = np.where(on, x[i], x[i] ^ swap)
            x[0], x[i] = new0, newi
        q >>= 1
    for i in range(1, n):
        x[i] = x[i] ^ x[i - 1]
    flip = np.zeros_like(x[0])
    q = 1 << (m - 1)
    while q > 1:
        flip = np.where((x[n - 1] & q) != 0, flip ^ (q - 1), flip)
        q >>= 1
    for i in range(n):
        x[i] = x[i] ^ flip
    index = np.zeros_like(x[0])
    for level in range(m - 1, -1, -1):
        for i in range(n):
            index = (index << 1) | ((x[i] >> level) & 1)
    return index


def hilbert_perm(T: int, Y: int, X: int):
    """perm[r] = row-major index (t*Y + y)*X + x of the r-th grid cell in Hilbert order.
    Follows: xllm-io review, 3.1; alanhou.org explainer, "Core Mechanism", layer 1.

    Returns (perm, inv) as int64 arrays, inv = perm^-1.
    """
    m = hilbert_bits(T, Y, X)
    t, y, x = np.meshgrid(np.arange(T), np.arange(Y), np.arange(X), indexing="ij")
    cells = np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1)
    idx = hilbert_index(cells, m)
    perm = np.argsort(idx, kind="stable")
    assert len(np.unique(idx)) == len(idx)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    return perm.astype(np.int64), inv.astype(np.int64)


# --------------------------------------------------------------------------
# Blocks and block summaries
# --------------------------------------------------------------------------


def block_sizes(N: int, b: int) -> np.ndarray:
    """True token count n_j of each of the ceil(N/b) consecutive blocks (last may be partial).

    Follows: xllm-io review, 3.1: consecutive blocks along the curve.
    """
    nb = -(-N // b)
    starts = np.arange(nb) * b
    return np.minimum(b, N - starts).astype(np.int64)


def to_hilbert(x: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """[B, N, H, d] grid order -> [B, H, N, d] in Hilbert token order.

    Follows: xllm-io review, 3.1.
    """
    return np.ascontiguousarray(np.transpose(x[:, perm], (0, 2, 1, 3)))


def block_means(xh: np.ndarray, b: int) -> np.ndarray:
    """Mean of each block's rows: [B, H, N, d] -> float32 [B, H, nb, d].
    Follows: xllm-io review, 三 Stage 1 (block summaries); reading: the arithmetic mean.

    The sum is taken in float64 (exact for bf16 rows), divided by the true
    token count in float64 and rounded once to float32.
    """
    B, H, N, d = xh.shape
    sizes = block_sizes(N, b)
    out = np.empty((B, H, sizes.size, d), dtype=np.float32)
    for j, n in enumerate(sizes):
        seg = xh[:, :, j * b: j * b + n, :].astype(np.float64)
        out[:, :, j, :] = (seg.sum(axis=2) / np.float64(n)).astype(np.float32)
    return out


def block_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """s_ij = qbar_i . kbar_j / sqrt(d) per head, float64 products and sums, rounded to float32.
    Follows: xllm-io review, 三 Stage 1; alanhou.org explainer, "Key Concepts".

    qbar, kbar: [..., nb, d] float32. Returns float32 [..., nb, nb].
    """
    d = qbar.shape[-1]
    q64 = qbar.astype(np.float64)
    k64 = kbar.astype(np.float64)
    s = np.matmul(q64, np.swapaxes(k64, -1, -2)) / math.sqrt(d)
    return s.astype(np.float32)


def block_softmax(s: np.ndarray) -> np.ndarray:
    """Row softmax over key blocks in float64: exp(s - max) / sum.

    Follows: alanhou.org explainer, "Key Concepts" (probabilities over key blocks).
    """
    s64 = s.astype(np.float64)
    e = np.exp(s64 - s64.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


# --------------------------------------------------------------------------
# Top-p with the Top-k floor
# --------------------------------------------------------------------------


@dataclass
class RowRouting:
    order: np.ndarray     # [nb] block ids, probability descending, ties by smaller id
    cdf: np.ndarray       # [nb] float64 running sums of P along `order`
    count_topp: int       # c: fewest blocks reaching p
    count: int            # c' after the floor


def importance_order(P: np.ndarray) -> np.ndarray:
    """Block ids sorted by probability descending, ties broken by the smaller block id.
    Follows: alanhou.org explainer, "Top-p Routing with Safety Floor".

    Works on the last axis of P (any leading shape).
    """
    ids = np.broadcast_to(np.arange(P.shape[-1]), P.shape)
    return np.lexsort((ids, -P), axis=-1)


def topp_count(cdf: np.ndarray, p: float) -> np.ndarray:
    """c = smallest r (1-based) with cdf_r >= p; nb when p >= 1 or when no prefix reaches p.

    Follows: alanhou.org explainer, "Top-p Routing with Safety Floor".
    """
    nb = cdf.shape[-1]
    if p >= 1.0:
        return np.full(cdf.shape[:-1], nb, dtype=np.int64)
    reached = cdf >= p
    first = np.argmax(reached, axis=-1) + 1
    return np.where(reached.any(axis=-1), first, nb).astype(np.int64)


def floor_count(c: np.ndarray, k_floor: int, nb: int) -> np.ndarray:
    """count' = max(c, min(k, nb)).

    Follows: alanhou.org explainer, "Top-p Routing with Safety Floor" (the Top-k floor).
    """
    return np.maximum(c, min(k_floor, nb)).astype(np.int64)


def route_row(s_row: np.ndarray, p: float, k_floor: int) -> RowRouting:
    """Top-p + floor for one query block's score row (plain, one row at a time).

    Follows: xllm-io review, 三 Stage 1; alanhou.org explainer, "Key Concepts".
    """
    P = block_softmax(s_row[None, :])[0]
    order = importance_order(P)
    cdf = np.cumsum(P[order])
    c = int(topp_count(cdf[None, :], p)[0])
    return RowRouting(order, cdf, c, int(floor_count(np.array(c), k_floor, P.size)))


@dataclass
class Routing:
    """Routing of a whole [B, H] problem."""

    nb: int
    sizes: np.ndarray          # [nb] true token count per block
    scores: np.ndarray         # float32 [B, H, nb, nb]
    P: np.ndarray              # float64 [B, H, nb, nb]
    order: np.ndarray          # int64 [B, H, nb, nb] importance order per tile
    cdf: np.ndarray            # float64 [B, H, nb, nb] along `order`
    count_topp: np.ndarray     # int64 [B, H, nb]
    counts: np.ndarray         # int64 [B, H, nb] after floor (and slack fill, if applied)

    def retained(self, b: int, h: int, i: int) -> np.ndarray:
        """Ascending ids of the retained key blocks of tile (b, h, i)."""
        return np.sort(self.order[b, h, i, : self.counts[b, h, i]])


def route(qh: np.ndarray, kh: np.ndarray, block: int, p: float, k_floor: int) -> Routing:
    """Stage-1 routing on Hilbert-ordered q, k of shape [B, H, N, d] (float32 values).

    Follows: xllm-io review, 三 Stage 1; alanhou.org explainer, "Key Concepts".
    """
    B, H, N, d = qh.shape
    sizes = block_sizes(N, block)
    nb = sizes.size
    qbar = block_means(qh, block)
    kbar = block_means(kh, block)
    s = block_scores(qbar, kbar)
    P = block_softmax(s)
    order = importance_order(P)
    cdf = np.cumsum(np.take_along_axis(P, order, axis=-1), axis=-1)
    c = topp_count(cdf, p)
    return Routing(nb, sizes, s, P, order, cdf, c, floor_count(c, k_floor, nb))


# --------------------------------------------------------------------------
# Eq. 1 workloads, Eq. 2 imbalance
# --------------------------------------------------------------------------


def workloads(counts: np.ndarray):
    """work_h = sum_i count'_{h,i} (exact); L_h = work_h / nb (float32 division).

    Follows: xllm-io review, 核心公式 Eq. 1.
    """
    nb = counts.shape[-1]
    work = counts.sum(axis=-1).astype(np.int64)
    L = (work.astype(np.float32) / np.float32(nb)).astype(np.float32)
    return work, L


def imbalance(loads: Sequence[float]) -> float:
    """Eq. 2: rho = max_r L_r / mean_r L_r."""
    loads = np.asarray(loads, dtype=np.float64)
    return float(loads.max() / loads.mean())


# --------------------------------------------------------------------------
# Slack fill (one-GPU reading of SASA)
# --------------------------------------------------------------------------


def slack_budget(counts: np.ndarray, beta: float) -> int:
    """E = floor(beta * sum count'), in float64.

    Follows: xllm-io review, 3.3 and the SASA steps of 五, read for one GPU.
    """
    return int(math.floor(np.float64(beta) * np.float64(int(counts.sum()))))


def slack_fill(counts: np.ndarray, beta: float) -> np.ndarray:
    """Heap loop: E times, raise the tile with the smallest (count, tile id) among tiles below nb.
    Follows: xllm-io review, 3.3 and the SASA steps of 五, read for one GPU.

    counts: any shape whose last axis is the nb query blocks of a head; tile id
    is the flat row-major index. Returns the new counts (same shape). Each raise
    appends the tile's next block in its own importance order, so the retained
    set stays a prefix of that order.
    """
    nb = counts.shape[-1]
    flat = counts.reshape(-1).astype(np.int64).copy()
    E = slack_budget(counts, beta)
    heap = [(int(c), t) for t, c in enumerate(flat) if c < nb]
    heapq.heapify(heap)
    for _ in range(E):
        if not heap:
            break
        c, t = heapq.heappop(heap)
        flat[t] = c + 1
        if c + 1 < nb:
            heapq.heappush(heap, (c + 1, t))
    return flat.reshape(counts.shape)


def slack_fill_level(counts: np.ndarray, beta: float) -> np.ndarray:
    """Closed form of the heap loop: a water level lambda plus a remainder by tile id.

    Follows: xllm-io review, 3.3, read for one GPU.
    """
    nb = counts.shape[-1]
    flat = counts.reshape(-1).astype(np.int64)
    E = slack_budget(counts, beta)

    def need(lam):
        return int(np.maximum(0, np.minimum(lam, nb) - flat).sum())

    lo, hi = 0, nb
    while lo < hi:  # largest lam in [0, nb] with need(lam) <= E
        mid = (lo + hi + 1) // 2
        if need(mid) <= E:
            lo = mid
        else:
            hi = mid - 1
    lam = lo
    out = np.maximum(flat, lam)
    rest = E - need(lam)
    if lam < nb and rest > 0:
        at_level = np.nonzero(out == lam)[0]
        out[at_level[:rest]] += 1
    return out.reshape(counts.shape)


# --------------------------------------------------------------------------
# LPT tile queue and list scheduling
# --------------------------------------------------------------------------


def lpt_queue(counts: np.ndarray) -> np.ndarray:
    """Tile ids (flat row-major) by retained count descending, ties by ascending tile id.

    Follows: xllm-io review, 3.2 and the RLB steps of 五, read for one GPU.
    """
    flat = counts.reshape(-1)
    ids = np.arange(flat.size)
    return np.lexsort((ids, -flat)).astype(np.int64)


def list_schedule(costs: Sequence[float], order: Sequence[int], workers: int):
    """Greedy list scheduling: each next item goes to the earliest-free worker (ties: lowest id).
    Follows: R. L. Graham, "Bounds on multiprocessing timing anomalies", 1969; review Eq. 2 for rho.

    Returns (per-worker loads, makespan).
    """
    heap = [(0.0, w) for w in range(workers)]
    loads = np.zeros(workers)
    for t in order:
        free, w = heapq.heappop(heap)
        loads[w] += costs[t]
        heapq.heappush(heap, (free + costs[t], w))
    return loads, float(loads.max())


# --------------------------------------------------------------------------
# Structured router: local window plus rotating global anchors (LVSA note)
# --------------------------------------------------------------------------


def anchor_offset(stride: int, shift: int, step: int) -> int:
    """Offset of the anchor blocks at diffusion step `step`: (step * shift) mod stride (0 without anchors).

    Follows: LVSA note: global anchors rotating across diffusion steps.
    """
    return (step * shift) % stride if stride > 0 else 0


def window_anchor_list(nb: int, i: int, window: int, stride: int, shift: int, step: int) -> np.ndarray:
    """Key blocks of query block i, ascending: the local window |j - i| <= window plus the anchors.

    Reading of the LVSA note ("a structured local window pattern with rotating
    global anchors"): the window is over block ids, which in Hilbert order are
    neighbours in (t, y, x); the anchors are every stride-th key block, starting
    at anchor_offset(), so they shift with the diffusion step. stride = 0: no
    anchors.
    """
    blocks = set(range(max(0, i - window), min(nb - 1, i + window) + 1))
    if stride > 0:
        blocks |= set(range(anchor_offset(stride, shift, step), nb, stride))
    return np.array(sorted(blocks), dtype=np.int64)


def window_anchor_counts(nb: int, window: int, stride: int, shift: int, step: int) -> np.ndarray:
    """Retained count of every query block (the same for every head).

    Follows: LVSA note.
    """
    return np.array([window_anchor_list(nb, i, window, stride, shift, step).size for i in range(nb)],
                    dtype=np.int64)


# --------------------------------------------------------------------------
# Rank-level runtime stages with the eight XCDs of one GPU as the ranks
# (review 核心公式 Eq. 1-2 and 5-10; 3.2 RLB; 3.3 SASA and its piecewise
# policy; the RLB and SASA steps of 五; parameters of 五)
# --------------------------------------------------------------------------

RANKS = 8                     # XCDs of an MI355X, each with its own L2
RLB_K1, RLB_K2 = 1.05, 1.10   # rho below k1: nothing; below k2: SASA only; else RLB, then SASA
SASA_N1, SASA_N2 = 0.8, 0.07  # augmentation coefficient, trigger threshold


def rank_of_heads(BH: int, R: int = RANKS) -> np.ndarray:
    """Initial placement: rank r holds the contiguous heads floor(r BH / R) .. floor((r+1) BH / R) - 1.

    This is the head split of Ulysses sequence parallelism (review, 三 "技术架构").
    """
    owner = np.empty(BH, dtype=np.int64)
    for r in range(R):
        owner[r * BH // R:(r + 1) * BH // R] = r
    return owner


def rank_loads(work: np.ndarray, owner: np.ndarray, R: int = RANKS) -> np.ndarray:
    """Eq. 1 at rank level, in retained blocks: W_r = sum of work_h over the heads rank r holds (int64).

    L_r of Eq. 1 is W_r / nb; every ratio used below is the same in either unit.
    """
    W = np.zeros(R, dtype=np.int64)
    np.add.at(W, owner, np.asarray(work, dtype=np.int64).reshape(-1))
    return W


def rank_policy(rho: float, k1: float = RLB_K1, k2: float = RLB_K2) -> str:
    """Piecewise enabling (review 3.3): 'none' below k1, 'sasa' below k2, else 'rlb+sasa'."""
    if rho < k1:
        return "none"
    return "sasa" if rho < k2 else "rlb+sasa"


def pair_matchings(R: int = RANKS):
    """The pair topologies of R ranks (R even): every perfect matching, in canonical order.

    Follows: xllm-io review, 3.2 (pair topologies over which the candidate matchings of
    S_20% are enumerated). Canonical order: the lowest unpaired rank is paired with each
    higher unpaired rank in ascending order, recursively; a matching is a list of pairs
    (a, b), a < b, by ascending a.
    """
    if R % 2:
        raise ValueError("pair topologies need an even number of ranks")

    def rec(free):
        if not free:
            yield []
            return
        a = free[0]
        for j in range(1, len(free)):
            rest = free[1:j] + free[j + 1:]
            for m in rec(rest):
                yield [(a, free[j])] + m

    return list(rec(list(range(R))))


def pair_options(owner: np.ndarray, a: int, b: int):
    """The moves pair (a, b) may make: one head each way at most (one send and one receive per rank).

    Follows: xllm-io review, Eq. 5-6 and the RLB steps of 五 (rank r sends h_r to
    sigma(r) and receives from sigma^-1(r), at most one local head per rank). Order:
    no move; a sends one of its heads to b (heads ascending); b sends one to a; a and
    b swap one head each (a's head varying slowest). A move is (head, from, to).
    """
    ha = [int(h) for h in np.nonzero(owner == a)[0]]
    hb = [int(h) for h in np.nonzero(owner == b)[0]]
    opts = [()]
    opts += [((h, a, b),) for h in ha]
    opts += [((h, b, a),) for h in hb]
    opts += [((x, a, b), (y, b, a)) for x in ha for y in hb]
    return opts


def rlb_space(work: np.ndarray, owner: np.ndarray, R: int = RANKS) -> int:
    """Number of candidate plans: the sum over pair topologies of the product of their pairs' option counts.

    Follows: xllm-io review, Eq. 6 (the space S_20% read as pair topologies).
    """
    total = 0
    for m in pair_matchings(R):
        n = 1
        for a, b in m:
            n *= len(pair_options(owner, a, b))
        total += n
    return total


def rlb_plan(work: np.ndarray, owner: np.ndarray, R: int = RANKS):
    """Eq. 5-6: the plan of least (max_r W_r^new, Var_r W_r^new), ties to the first in enumeration order.

    Follows: xllm-io review, Eq. 5-6, 3.2 and the RLB steps of 五. Plans are
    enumerated pair topology by pair topology (canonical order), and within one the
    pairs' options as a product with the first pair varying slowest. Var is compared
    through sum W^2 (migration keeps the total). The pairs of a topology touch
    disjoint ranks, so its best plan is found pair by pair: its least maximum M is the
    largest over its pairs of the pair's least maximum, and each pair then takes,
    among its options whose maximum is at most M, the first of least sum of squares.
    Returns (new owner array, moves (head, from, to) by sending rank).
    """
    work = np.asarray(work, dtype=np.int64).reshape(-1)
    W = rank_loads(work, owner, R)
    best = None
    for m in pair_matchings(R):
        pairs = []
        for a, b in m:
            opts = []
            for moves in pair_options(owner, a, b):
                wa, wb = int(W[a]), int(W[b])
                for h, src, dst in moves:  # Eq. 5: L_r - L_{h_r} + L_{h_{sigma^-1(r)}}
                    d = int(work[h])
                    if src == a:
                        wa, wb = wa - d, wb + d
                    else:
                        wa, wb = wa + d, wb - d
                opts.append((max(wa, wb), wa * wa + wb * wb, moves))
            pairs.append(opts)
        M = max(min(o[0] for o in opts) for opts in pairs)
        chosen, S = [], 0
        for opts in pairs:
            least = min(o[1] for o in opts if o[0] <= M)
            S += least
            chosen.append(next(o[2] for o in opts if o[0] <= M and o[1] == least))
        if best is None or (M, S) < best[0]:
            best = ((M, S), chosen)
    moves = sorted((mv for ch in best[1] for mv in ch), key=lambda mv: mv[1])
    new_owner = owner.copy()
    for h, _, dst in moves:
        new_owner[h] = dst
    return new_owner, moves


def sasa_budgets(W: np.ndarray, n1: float = SASA_N1, n2: float = SASA_N2) -> np.ndarray:
    """Eq. 7-8 with the trigger: E_r = floor(n1 dW_r) if dW_r > n2 W_max, else 0, where dW_r = W_max - W_r.

    In retained blocks (float64 arithmetic); n1 < 1 keeps E_r <= dW_r, so no rank
    passes the current critical path (Eq. 10 with A = 0).
    """
    W = np.asarray(W, dtype=np.int64)
    wmax = int(W.max())
    E = np.zeros(W.size, dtype=np.int64)
    for r in range(W.size):
        dW = wmax - int(W[r])
        if np.float64(dW) > np.float64(n2) * np.float64(wmax):
            E[r] = int(math.floor(np.float64(n1) * np.float64(dW)))
    return E


def water_fill(flat: np.ndarray, nb: int, E: int) -> np.ndarray:
    """Raise the lightest of the given counts E times by one (ties: lowest position; full ones skipped).
    Follows: xllm-io review, the SASA steps of 五 (augmentation inside a rank).

    Closed form of that loop: the highest level lambda whose need sum max(0,
    lambda - c) is at most E, then one more for the first E - need(lambda) counts
    at the level, by position.
    """
    flat = np.asarray(flat, dtype=np.int64)

    def need(lam):
        return int(np.maximum(0, np.minimum(lam, nb) - flat).sum())

    lo, hi = 0, nb
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if need(mid) <= E:
            lo = mid
        else:
            hi = mid - 1
    out = np.maximum(flat, lo)
    rest = E - need(lo)
    if lo < nb and rest > 0:
        out[np.nonzero(out == lo)[0][:rest]] += 1
    return out


def rank_stage(counts: np.ndarray, R: int = RANKS, k1: float = RLB_K1, k2: float = RLB_K2,
               n1: float = SASA_N1, n2: float = SASA_N2, policy: Optional[str] = None) -> dict:
    """RLB then SASA over ranks, enabled by the piecewise policy on rho (or a forced policy:
    Follows: xllm-io review, Eq. 2, 5-10, 3.2 and 3.3.
    'none', 'sasa', 'rlb+sasa', or 'rlb' for migration alone).

    counts: [B, H, nb] retained counts after Top-p and the floor. Returns the
    initial and final head owners, the moves, the budgets E_r, the new counts
    (each tile extended along its own importance order: SASA step 2b), rho before
    migration, after migration and after augmentation, the policy taken, and the
    head order of the per-rank queue segments (ranks ascending, heads ascending
    within a rank) with the number of heads per rank.
    """
    B, H, nb = counts.shape
    BH = B * H
    flat = counts.reshape(BH, nb).astype(np.int64)
    work = flat.sum(axis=1)
    owner0 = rank_of_heads(BH, R)
    W0 = rank_loads(work, owner0, R)
    rho0 = imbalance(W0)
    mode = rank_policy(rho0, k1, k2) if policy is None else policy
    owner, moves = owner0.copy(), []
    if mode in ("rlb+sasa", "rlb"):
        owner, moves = rlb_plan(work, owner0, R)
    W1 = rank_loads(work, owner, R)
    E = sasa_budgets(W1, n1, n2) if mode in ("sasa", "rlb+sasa") else np.zeros(R, dtype=np.int64)
    new = flat.copy()
    for r in range(R):
        heads = np.nonzero(owner == r)[0]
        if E[r] > 0 and heads.size:
            new[heads] = water_fill(flat[heads].reshape(-1), nb, int(E[r])).reshape(heads.size, nb)
    W2 = rank_loads(new.sum(axis=1), owner, R)
    order = np.concatenate([np.nonzero(owner == r)[0] for r in range(R)]).astype(np.int64)
    return dict(owner0=owner0, owner=owner, moves=moves, policy=mode, E=E, counts=new.reshape(B, H, nb),
                W0=W0, W1=W1, W2=W2, rho0=rho0, rho_rlb=imbalance(W1), rho_final=imbalance(W2),
                head_order=order, heads_per_rank=np.bincount(owner, minlength=R).astype(np.int64))


# --------------------------------------------------------------------------
# Block-sparse attention
# --------------------------------------------------------------------------


def attention_tile(qh_bh: np.ndarray, kh_bh: np.ndarray, vh_bh: np.ndarray,
                   block: int, i: int, kv_blocks: Sequence[int]) -> np.ndarray:
    """Output rows of query block i over the tokens of the given key blocks (float64).
    Follows: xllm-io review, 三 "Block-Sparse Attention Execution"; alanhou.org explainer, "Core Mechanism", layer 3.

    qh_bh, kh_bh, vh_bh: [N, d] one head's rows in Hilbert order.
    Returns [n_i, d].
    """
    N, d = qh_bh.shape
    rows = slice(i * block, min((i + 1) * block, N))
    keys = np.concatenate([np.arange(j * block, min((j + 1) * block, N)) for j in kv_blocks])
    q = qh_bh[rows].astype(np.float64)
    k = kh_bh[keys].astype(np.float64)
    v = vh_bh[keys].astype(np.float64)
    s = q @ k.T / math.sqrt(d)
    s -= s.max(axis=1, keepdims=True)
    w = np.exp(s)
    w /= w.sum(axis=1, keepdims=True)
    return w @ v


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, perm: np.ndarray, block: int,
              retained: Optional[callable] = None) -> np.ndarray:
    """Block-sparse attention in grid order: [B, N, H, d] in, float64 [B, N, H, d] out.
    Follows: xllm-io review, 三 "Block-Sparse Attention Execution"; alanhou.org explainer, "Core Mechanism", layer 3.

    retained(b, h, i) gives the key-block ids of tile (b, h, i); None means every block.
    """
    B, N, H, d = q.shape
    qh, kh, vh = to_hilbert(q, perm), to_hilbert(k, perm), to_hilbert(v, perm)
    nb = -(-N // block)
    out = np.zeros((B, N, H, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                blocks = range(nb) if retained is None else retained(b, h, i)
                rows = perm[i * block: min((i + 1) * block, N)]
                out[b, rows, h, :] = attention_tile(qh[b, h], kh[b, h], vh[b, h], block, i, blocks)
    return out


def retained_flops(sizes: np.ndarray, d: int, tiles) -> float:
    """F_ret = sum over tiles and retained blocks of 4 * n_i * n_j * d (true token counts).
    Follows: the attention work measure of the benchmark: 4 n_i n_j d per retained pair.

    tiles: iterable of (i, retained block ids) pairs.
    """
    total = 0
    for i, blocks in tiles:
        total += 4 * int(sizes[i]) * int(sizes[np.asarray(blocks, dtype=np.int64)].sum()) * d
    return float(total)


# --------------------------------------------------------------------------
# V quantization: OCP FP8 E4M3 with a power-of-two scale per head and channel
# --------------------------------------------------------------------------

E4M3_MAX = 448.0        # largest finite E4M3 magnitude: 1.75 * 2^8
E4M3_BIAS = 7
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_QUANTUM = 2.0 ** -9  # spacing of the subnormals (exponent field 0)


def e4m3_encode(x) -> np.ndarray:
    """Codes of the OCP E4M3 format (sign, 4 exponent bits, bias 7, 3 mantissa bits,
    no infinities, S.1111.111 is NaN) for finite x with |x| < 464, rounding to the
    nearest value and ties to an even mantissa. Larger magnitudes raise.

    Normal values (|x| >= 2^-6) are (1 + m/8) 2^E with exponent field E + 7; below
    that the field is 0 and the value is m 2^-9. Rounding the mantissa up to 8
    carries into the exponent field, which the code sum (E + 7) * 8 + m does by
    itself, as does m = 8 in the subnormal range (the smallest normal, code 8).
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.isfinite(x).all():
        raise ValueError("e4m3_encode: non-finite input")
    a = np.abs(x)
    if (a > 464.0).any():
        raise ValueError("e4m3_encode: magnitude beyond the E4M3 range")
    sub = a < E4M3_MIN_NORMAL
    safe = np.where(sub, 1.0, a)
    _, ex = np.frexp(safe)               # safe = f 2^ex with f in [0.5, 1)
    E = ex.astype(np.int64) - 1          # safe = (1 + frac) 2^E
    frac = np.ldexp(safe, -E) - 1.0      # exact: a power-of-two scaling
    m_norm = np.rint(frac * 8.0).astype(np.int64)      # np.rint rounds half to even
    m_sub = np.rint(np.ldexp(a, 9)).astype(np.int64)    # a / 2^-9, exact
    code = np.where(sub, m_sub, (E + E4M3_BIAS) * 8 + m_norm)
    if (code >= 0x7F).any():
        raise ValueError("e4m3_encode: rounds past 448")
    return (code | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def e4m3_decode(code) -> np.ndarray:
    """Values of E4M3 codes as float64 (NaN for 0x7f and 0xff).

    Follows: OCP 8-bit floating point specification, E4M3.
    """
    c = np.asarray(code, dtype=np.int64)
    ef = (c >> 3) & 15
    m = c & 7
    mag = np.where(ef == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m / 8.0, ef - E4M3_BIAS))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def v_scale_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax * 2^-e <= 448 (0 where amax is 0).
    Follows: xllm-io review, "Block-Sparse Attention Execution" and 3.4 (V quantization); reading: power-of-two scales.

    With amax = f 2^E, f in [0.5, 1): amax 2^-e <= 0.875 * 2^9 holds for
    E - e <= 9 when f <= 0.875 and for E - e <= 8 otherwise.
    """
    amax = np.asarray(amax, dtype=np.float64)
    f, E = np.frexp(amax)
    e = np.where(f <= 0.875, E - 9, E - 8).astype(np.int64)
    return np.where(amax > 0, e, 0)


def quantize_v(v: np.ndarray):
    """Per-channel E4M3 quantization of one head's values v [n, d].
    Follows: xllm-io review, "Block-Sparse Attention Execution" and 3.4 (V quantization).

    Returns (codes uint8 [n, d], e int64 [d]): codes = E4M3(v * 2^-e) with e from
    the channel's largest magnitude. The scaling by 2^-e is exact, so the only
    rounding is the encoding.
    """
    v = np.asarray(v, dtype=np.float64)
    amax = np.abs(v).max(axis=0) if v.shape[0] else np.zeros(v.shape[1])
    e = v_scale_exponent(amax)
    return e4m3_encode(np.ldexp(v, -e[None, :])), e


def dequantize_v(codes: np.ndarray, e: np.ndarray) -> np.ndarray:
    """v~ = E4M3 value of the code times 2^e, exactly (float64).

    Follows: xllm-io review, 3.4 (V quantization).
    """
    return np.ldexp(e4m3_decode(codes), np.asarray(e, dtype=np.int64)[None, :])


def quantized_v(v: np.ndarray) -> np.ndarray:
    """Grid-order [B, N, H, d] values replaced by their dequantized E4M3 values, each
    Follows: xllm-io review, "Block-Sparse Attention Execution" and 3.4 (V quantization).
    (batch, head) with its own per-channel scales over all N tokens (float64)."""
    v = np.asarray(v)
    out = np.empty(v.shape, dtype=np.float64)
    for b in range(v.shape[0]):
        for h in range(v.shape[2]):
            codes, e = quantize_v(v[b, :, h, :])
            out[b, :, h, :] = dequantize_v(codes, e)
    return out


def attention_tile_spread(qh_bh: np.ndarray, kh_bh: np.ndarray, vh_bh: np.ndarray,
                          block: int, i: int, kv_blocks: Sequence[int], small: float = 0.0):
    """Output rows of query block i as in attention_tile, with spreads of the values
    Follows: xllm-io review, 三 "Block-Sparse Attention Execution" (the attention); the spreads bound weight rounding.
    around each output under the softmax weights w:
      A1[r, c] = sum_j w_rj |v_jc - O_rc|,
      A2[r, c] = sqrt(sum_j w_rj^2 (v_jc - O_rc)^2),
      As[r, c] = sum over the keys j with w_rj <= small of |v_jc - O_rc|.
    If every unnormalised weight P_j is replaced by P_j (1 + delta_j) with
    |delta_j| <= u and the result renormalised, O moves by at most u / (1 - u) * A1;
    for independent zero-mean delta_j of standard deviation s it moves by about
    s * A2; an extra absolute change of at most a in each normalised weight at or
    below `small` adds at most about a * As. Returns (O, A1, A2, As), each [n_i, d]
    float64.
    """
    N, d = qh_bh.shape
    rows = slice(i * block, min((i + 1) * block, N))
    keys = np.concatenate([np.arange(j * block, min((j + 1) * block, N)) for j in kv_blocks])
    q = qh_bh[rows].astype(np.float64)
    k = kh_bh[keys].astype(np.float64)
    v = vh_bh[keys].astype(np.float64)
    s = q @ k.T / math.sqrt(d)
    s -= s.max(axis=1, keepdims=True)
    w = np.exp(s)
    w /= w.sum(axis=1, keepdims=True)
    O = w @ v
    A1 = np.empty_like(O)
    A2 = np.empty_like(O)
    As = np.empty_like(O)
    for r in range(O.shape[0]):                           # one query row at a time keeps memory small
        dev = np.abs(v - O[r][None, :])                    # [keys, d]
        A1[r] = w[r] @ dev
        A2[r] = np.sqrt((w[r] * w[r]) @ (dev * dev))
        As[r] = (w[r] <= small).astype(np.float64) @ dev
    return O, A1, A2, As
