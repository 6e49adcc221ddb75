"""Python binding of libabsh.so: the Hilbert-ordered Top-p block router and block-sparse attention for MI355X.

This module only marshals arguments: it takes torch tensors (for device memory
and the current stream), checks their shapes and dtypes, and passes raw
pointers to the C ABI declared in include/absh.h. Every step of the path runs in
the library's HIP kernels. If libabsh.so is missing, importing the binding still
works but the first call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libabsh.so")

ABSH_BF16, ABSH_F32 = 0, 1
ABSH_ROWS, ABSH_VT, ABSH_VT8, ABSH_ROWS_F32 = 0, 1, 2, 3
SCHED_ORDER, SCHED_LPT, SCHED_XCD, SCHED_RANKS = 0, 1, 2, 3
SCHEDULES = {"order": SCHED_ORDER, "lpt": SCHED_LPT, "xcd": SCHED_XCD, "ranks": SCHED_RANKS}
RANK_POLICIES = {"auto": -1, "none": 0, "sasa": 1, "rlb+sasa": 2, "rlb": 3}
RANK_INFO = 64  # doubles in Routing.rank_info (layout in include/absh.h)
PULL_WORDS = 16  # int32 work counters in Routing.pull
STATIC_SCRATCH_BYTES = 64 << 20  # route workspace limit of absh_route_static
ROUTERS = {"topp": 0, "window-anchor": 1}
# the review's parameters of the rank-level stages (section 五)
RLB_K1, RLB_K2, SASA_N1, SASA_N2 = 1.05, 1.10, 0.8, 0.07

EXPORTED = (
    "absh_version", "absh_status_string", "absh_last_error", "absh_create", "absh_destroy", "absh_dims",
    "absh_perm", "absh_perm_copy", "absh_permute", "absh_unpermute", "absh_pool", "absh_block_scores",
    "absh_route_workspace_bytes", "absh_route", "absh_sparse_attn", "absh_lists_units", "absh_quantize_v",
    "absh_sparse_attn_v8", "absh_lists_bytes", "absh_lists_carve", "absh_workspace_bytes", "absh_attn_workgroups",
    "absh_route_static", "absh_permute_pool", "absh_route_means", "absh_forward", "absh_forward_workspace_bytes",
    "absh_sparse_attn_grid",
)


class AbshError(RuntimeError):
    """A non-OK status from the library; .status holds the code."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class RouteOpts(ctypes.Structure):
    _fields_ = [("p", ctypes.c_double), ("k_floor", ctypes.c_int32), ("slack_frac", ctypes.c_double),
                ("schedule", ctypes.c_int32), ("order_depth", ctypes.c_int32),
                ("rank_policy", ctypes.c_int32), ("strict_ranks", ctypes.c_int32),
                ("k1", ctypes.c_double), ("k2", ctypes.c_double), ("n1", ctypes.c_double), ("n2", ctypes.c_double),
                ("router", ctypes.c_int32), ("window", ctypes.c_int32), ("anchor_stride", ctypes.c_int32),
                ("anchor_shift", ctypes.c_int32), ("step", ctypes.c_int32)]


class Lists(ctypes.Structure):
    _fields_ = [("counts", ctypes.c_void_p), ("kv_idx", ctypes.c_void_p), ("order", ctypes.c_void_p),
                ("work", ctypes.c_void_p), ("L", ctypes.c_void_p), ("queue", ctypes.c_void_p),
                ("sched", ctypes.c_void_p), ("unit_list", ctypes.c_void_p), ("unit_cnt", ctypes.c_void_p),
                ("schedule", ctypes.c_int32), ("head_order", ctypes.c_void_p), ("rank_info", ctypes.c_void_p),
                ("strict_ranks", ctypes.c_int32), ("unit_queue", ctypes.c_void_p), ("pull", ctypes.c_void_p),
                ("wg_busy", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libabsh.so (built in-tree by build.py); raises if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    sig = {
        "absh_version": ([], i),
        "absh_status_string": ([i], ctypes.c_char_p),
        "absh_last_error": ([], ctypes.c_char_p),
        "absh_create": ([ctypes.POINTER(vp), i, i, i, i, i, vp], i),
        "absh_destroy": ([vp], i),
        "absh_dims": ([vp, ctypes.POINTER(i), ctypes.POINTER(i), ctypes.POINTER(i)], i),
        "absh_perm": ([vp, ctypes.POINTER(vp), ctypes.POINTER(vp)], i),
        "absh_perm_copy": ([vp, vp, vp, vp], i),
        "absh_permute": ([vp, vp, i, vp, i, i, i, i, vp], i),
        "absh_unpermute": ([vp, vp, vp, i, i, i, vp], i),
        "absh_pool": ([vp, vp, vp, i, i, i, vp], i),
        "absh_block_scores": ([vp, vp, vp, vp, i, i, i, vp], i),
        "absh_route_workspace_bytes": ([vp, i, i, i], sz),
        "absh_workspace_bytes": ([vp, i, i, i], sz),
        "absh_attn_workgroups": ([vp], i),
        "absh_lists_units": ([vp, i, i, i], i),
        "absh_route": ([vp, vp, vp, i, i, i, i, ctypes.POINTER(RouteOpts), ctypes.POINTER(Lists), vp, sz, vp], i),
        "absh_route_static": ([vp, vp, vp, i, i, i, i, ctypes.POINTER(RouteOpts), ctypes.POINTER(Lists), vp], i),
        "absh_lists_bytes": ([vp, i, i, i], sz),
        "absh_lists_carve": ([vp, i, i, i, vp, sz, ctypes.POINTER(Lists)], i),
        "absh_sparse_attn": ([vp, vp, vp, vp, i, i, i, ctypes.POINTER(Lists), vp, vp], i),
        "absh_quantize_v": ([vp, vp, i, i, i, vp, vp, vp], i),
        "absh_sparse_attn_v8": ([vp, vp, vp, vp, vp, i, i, i, ctypes.POINTER(Lists), vp, vp], i),
        "absh_permute_pool": ([vp, vp, i, vp, vp, i, i, i, i, vp], i),
        "absh_route_means": ([vp, vp, vp, i, i, i, ctypes.POINTER(RouteOpts), ctypes.POINTER(Lists), vp, sz, vp], i),
        "absh_forward": ([vp, vp, vp, vp, i, vp, i, i, i, ctypes.POINTER(RouteOpts), ctypes.POINTER(Lists), vp, sz,
                          vp], i),
        "absh_forward_workspace_bytes": ([vp, i, i, i], sz),
        "absh_sparse_attn_grid": ([vp, vp, vp, vp, vp, i, i, i, ctypes.POINTER(Lists), vp, vp], i),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        L = lib()
        raise AbshError(status, f"{L.absh_status_string(status).decode()}: {L.absh_last_error().decode()}")


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


class Context:
    """One (T, Y, X) grid and block size on one device; owns the Hilbert permutation."""

    def __init__(self, T: int, Y: int, X: int, block: int, device: int = 0, stream=None):
        self._h = ctypes.c_void_p()
        s = _stream(stream) if stream is not None else ctypes.c_void_p(0)
        _check(lib().absh_create(ctypes.byref(self._h), T, Y, X, block, device, s))
        self.T, self.Y, self.X, self.block, self.device = T, Y, X, block, device
        N, nb, n_pad = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        _check(lib().absh_dims(self._h, ctypes.byref(N), ctypes.byref(nb), ctypes.byref(n_pad)))
        self.N, self.nb, self.n_pad = N.value, nb.value, n_pad.value

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._h

    def close(self) -> None:
        if self._h:
            _check(lib().absh_destroy(self._h))
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            if self._h and _lib is not None:
                _lib.absh_destroy(self._h)
        except Exception:
            pass


def create(T: int, Y: int, X: int, block: int, device: int = 0, stream=None) -> Context:
    return Context(T, Y, X, block, device, stream)


def _dev(ctx: Context):
    import torch
    return torch.device("cuda", ctx.device)


def perm_copy(ctx: Context, stream=None):
    """(perm, inv) as int32 device tensors (copies of the context's arrays)."""
    import torch
    perm = torch.empty(ctx.N, dtype=torch.int32, device=_dev(ctx))
    inv = torch.empty(ctx.N, dtype=torch.int32, device=_dev(ctx))
    _check(lib().absh_perm_copy(ctx.handle, _ptr(perm), _ptr(inv), _stream(stream)))
    return perm, inv


def permute(ctx: Context, x, layout: int = ABSH_ROWS, out=None, stream=None):
    """x [B, N, H, d] (bf16 or f32, grid order) -> Hilbert-order tensor in `layout` (bf16, or
    float32 rows for ABSH_ROWS_F32)."""
    import torch
    B, N, H, d = x.shape
    assert N == ctx.N and x.is_contiguous() and x.dtype in (torch.bfloat16, torch.float32)
    xt = ABSH_F32 if x.dtype == torch.float32 else ABSH_BF16
    rows = layout in (ABSH_ROWS, ABSH_ROWS_F32)
    shape = (B, H, ctx.n_pad, d) if rows else (B, H, ctx.nb, d, vt_keys(ctx.block))
    dtype = torch.float32 if layout == ABSH_ROWS_F32 else torch.bfloat16
    if out is None:
        out = torch.empty(shape, dtype=dtype, device=x.device)
    assert tuple(out.shape) == shape and out.dtype == dtype and out.is_contiguous(), "out does not fit the layout"
    _check(lib().absh_permute(ctx.handle, _ptr(x), xt, _ptr(out), B, H, d, layout, _stream(stream)))
    return out


def permute_pool(ctx: Context, x, layout: int = ABSH_ROWS, out=None, means=None, stream=None):
    """permute() in a rows layout and the block means of the rows it writes, in one pass
    over x -> (xh, xbar float32 [B, H, nb, d])."""
    import torch
    B, N, H, d = x.shape
    assert N == ctx.N and x.is_contiguous() and x.dtype in (torch.bfloat16, torch.float32)
    if layout not in (ABSH_ROWS, ABSH_ROWS_F32):
        raise ValueError("permute_pool writes rows: layout ABSH_ROWS or ABSH_ROWS_F32")
    xt = ABSH_F32 if x.dtype == torch.float32 else ABSH_BF16
    shape = (B, H, ctx.n_pad, d)
    dtype = torch.float32 if layout == ABSH_ROWS_F32 else torch.bfloat16
    if out is None:
        out = torch.empty(shape, dtype=dtype, device=x.device)
    if means is None:
        means = torch.empty((B, H, ctx.nb, d), dtype=torch.float32, device=x.device)
    assert tuple(out.shape) == shape and out.dtype == dtype and out.is_contiguous(), "out does not fit the layout"
    assert tuple(means.shape) == (B, H, ctx.nb, d) and means.dtype == torch.float32 and means.is_contiguous()
    _check(lib().absh_permute_pool(ctx.handle, _ptr(x), xt, _ptr(out), _ptr(means), B, H, d, layout,
                                   _stream(stream)))
    return out, means


def vt_keys(block: int) -> int:
    """Keys per block in the ABSH_VT layout (blocks shorter than 32 keys are zero-padded)."""
    return max(block, 32)


def unpermute(ctx: Context, oh, out=None, stream=None):
    """oh [B, H, n_pad, d] bf16 (Hilbert order) -> o [B, N, H, d] bf16 (grid order)."""
    import torch
    B, H, n_pad, d = oh.shape
    assert n_pad == ctx.n_pad and oh.dtype == torch.bfloat16 and oh.is_contiguous()
    if out is None:
        out = torch.empty((B, ctx.N, H, d), dtype=torch.bfloat16, device=oh.device)
    _check(lib().absh_unpermute(ctx.handle, _ptr(oh), _ptr(out), B, H, d, _stream(stream)))
    return out


def pool(ctx: Context, xh, out=None, stream=None):
    """Block means of a Hilbert-order tensor [B, H, n_pad, d] -> float32 [B, H, nb, d]."""
    import torch
    B, H, n_pad, d = xh.shape
    if out is None:
        out = torch.empty((B, H, ctx.nb, d), dtype=torch.float32, device=xh.device)
    _check(lib().absh_pool(ctx.handle, _ptr(xh), _ptr(out), B, H, d, _stream(stream)))
    return out


def block_scores(ctx: Context, qbar, kbar, out=None, stream=None):
    """float32 block scores [B, H, nb, nb] from block means."""
    import torch
    B, H, nb, d = qbar.shape
    if out is None:
        out = torch.empty((B, H, nb, nb), dtype=torch.float32, device=qbar.device)
    _check(lib().absh_block_scores(ctx.handle, _ptr(qbar), _ptr(kbar), _ptr(out), B, H, d, _stream(stream)))
    return out


@dataclass
class Routing:
    counts: object   # int32 [B, H, nb]
    kv_idx: object   # int16 [B, H, nb, nb]
    order: Optional[object]  # int16 [B, H, nb, depth] or None
    work: object     # int32 [B, H]
    L: object        # float32 [B, H]
    queue: object    # int32 [B*H*nb]
    sched: object    # int32 [10] bounds of the per-XCD runs of the work queue + query blocks per unit
    unit_list: object  # int32 [units, nb] flagged union lists of query-block groups
    unit_cnt: object   # int32 [units]
    head_order: object  # int32 [B*H] heads by rank (schedule "ranks")
    rank_info: object   # float64 [RANK_INFO] rank-stage report (schedule "ranks")
    unit_queue: object = None  # int32 [units] units longest first within each run (schedule "lpt")
    pull: object = None        # int32 [PULL_WORDS] the attention launches' work counters
    wg_busy: object = None     # optional uint64 [attn_workgroups, 2]: per-workgroup start / end ticks
    schedule: int = -1  # the schedule absh_route made these lists for
    strict_ranks: int = 0

    def lists(self) -> Lists:
        opt = lambda t: t.data_ptr() if t is not None else 0
        return Lists(self.counts.data_ptr(), self.kv_idx.data_ptr(), opt(self.order),
                     self.work.data_ptr(), self.L.data_ptr(), self.queue.data_ptr(), self.sched.data_ptr(),
                     self.unit_list.data_ptr(), self.unit_cnt.data_ptr(), self.schedule,
                     self.head_order.data_ptr(), self.rank_info.data_ptr(), self.strict_ranks,
                     opt(self.unit_queue), opt(self.pull), opt(self.wg_busy))

    def check(self, ctx: "Context", B: int, H: int, order_depth: int) -> None:
        """Raise unless every buffer has the shape and dtype absh_route writes for (ctx, B, H,
        order_depth): the library cannot see buffer sizes, so this is where a mismatch is caught."""
        import torch
        nb = ctx.nb
        units = max_units(ctx, B, H)
        want = {"counts": ((B, H, nb), torch.int32), "kv_idx": ((B, H, nb, nb), torch.int16),
                "work": ((B, H), torch.int32), "L": ((B, H), torch.float32),
                "queue": ((B * H * nb,), torch.int32), "sched": ((10,), torch.int32),
                "unit_list": ((units, nb), torch.int32), "unit_cnt": ((units,), torch.int32),
                "head_order": ((B * H,), torch.int32), "rank_info": ((RANK_INFO,), torch.float64),
                "unit_queue": ((units,), torch.int32), "pull": ((PULL_WORDS,), torch.int32)}
        if order_depth > 0:
            want["order"] = ((B, H, nb, order_depth), torch.int16)
        elif self.order is not None and self.order.dim() != 4:
            raise ValueError("order must be [B, H, nb, depth]")
        for name, (shape, dtype) in want.items():
            t = getattr(self, name)
            if t is None or tuple(t.shape) != shape or t.dtype != dtype or not t.is_contiguous():
                got = None if t is None else (tuple(t.shape), t.dtype)
                raise ValueError(f"Routing.{name} is {got}, expected {shape} {dtype}")
        for name in want:
            t = getattr(self, name)
            if t.device != torch.device("cuda", ctx.device):
                raise ValueError(f"Routing.{name} is on {t.device}, not cuda:{ctx.device}")


def route_workspace_bytes(ctx: Context, B: int, H: int, d: int) -> int:
    return int(lib().absh_route_workspace_bytes(ctx.handle, B, H, d))


def lists_units(ctx: Context, B: int, H: int, schedule) -> int:
    """Attention work units for this schedule (rows of Routing.unit_list)."""
    sched = SCHEDULES[schedule] if isinstance(schedule, str) else int(schedule)
    return int(lib().absh_lists_units(ctx.handle, B, H, sched))


def max_units(ctx: Context, B: int, H: int) -> int:
    """The most work units any schedule makes for this shape (rows of the unit buffers)."""
    return max(max(lists_units(ctx, B, H, s) for s in SCHEDULES), 1)


def attn_workgroups(ctx: Context) -> int:
    """Rows of a per-workgroup busy record (Routing.wg_busy) for attention on this context."""
    return int(lib().absh_attn_workgroups(ctx.handle))


def busy_record(ctx: Context, routing: Routing):
    """Attach a zeroed per-workgroup busy record to `routing`; attention launches on it fill it."""
    import torch
    routing.wg_busy = torch.zeros((attn_workgroups(ctx), 2), dtype=torch.int64, device=_dev(ctx))
    return routing.wg_busy


def busy_ticks(wg_busy):
    """Busy time of each workgroup that ran (end - start, in 100 MHz ticks) from a busy record."""
    rec = wg_busy.cpu()
    ran = rec[:, 1] > 0
    return (rec[ran, 1] - rec[ran, 0]).numpy()


def lists_bytes(ctx: Context, B: int, H: int, order_depth: int = 0) -> int:
    """Device bytes of all routing buffers in one arena (absh_lists_bytes)."""
    return int(lib().absh_lists_bytes(ctx.handle, B, H, order_depth))


def alloc_routing(ctx: Context, B: int, H: int, order_depth: int = 0) -> Routing:
    """Routing buffers sized for every schedule."""
    import torch
    dev = _dev(ctx)
    nb = ctx.nb
    units = max_units(ctx, B, H)
    return Routing(
        counts=torch.empty((B, H, nb), dtype=torch.int32, device=dev),
        kv_idx=torch.empty((B, H, nb, nb), dtype=torch.int16, device=dev),
        order=torch.empty((B, H, nb, order_depth), dtype=torch.int16, device=dev) if order_depth else None,
        work=torch.empty((B, H), dtype=torch.int32, device=dev),
        L=torch.empty((B, H), dtype=torch.float32, device=dev),
        queue=torch.empty((B * H * nb,), dtype=torch.int32, device=dev),
        sched=torch.empty((10,), dtype=torch.int32, device=dev),
        unit_list=torch.empty((units, nb), dtype=torch.int32, device=dev),
        unit_cnt=torch.empty((units,), dtype=torch.int32, device=dev),
        head_order=torch.empty((B * H,), dtype=torch.int32, device=dev),
        rank_info=torch.zeros((RANK_INFO,), dtype=torch.float64, device=dev),
        unit_queue=torch.empty((units,), dtype=torch.int32, device=dev),
        pull=torch.zeros((PULL_WORDS,), dtype=torch.int32, device=dev),
    )


def route(ctx: Context, qh, kh, p: float, k_floor: int, slack_frac: float = 0.0, schedule="lpt",
          order_depth: int = 0, out: Optional[Routing] = None, workspace=None, stream=None,
          rank_policy="auto", strict_ranks: bool = False, k1: float = RLB_K1, k2: float = RLB_K2,
          n1: float = SASA_N1, n2: float = SASA_N2, router="topp", window: int = 0, anchor_stride: int = 0,
          anchor_shift: int = 0, step: int = 0, qbar=None, kbar=None) -> Routing:
    """Stage-1 routing of Hilbert-order qh, kh [B, H, n_pad, d] (bf16 rows, or float32 rows from
    permute(..., ABSH_ROWS_F32)) -> Routing (device tensors).

    schedule: "order", "lpt", "xcd" or "ranks" (or the SCHED_* integer). The
    rank_* and k/n arguments apply to "ranks" only: rank_policy "auto" (by rho),
    "none", "sasa", "rlb+sasa" or "rlb"; strict_ranks keeps each XCD on its own rank.
    router "window-anchor" builds the structured lists (window, anchor_stride,
    anchor_shift, step; see include/absh.h) instead of Top-p; qh and kh then only
    give the shape. qbar, kbar: block means already computed (permute_pool); then
    qh and kh are not used (pass None) and the routing starts at the scores.
    """
    import torch
    if qbar is not None:
        B, H, nb, d = qbar.shape
        if kbar is None or tuple(kbar.shape) != tuple(qbar.shape) or nb != ctx.nb:
            raise ValueError(f"qbar, kbar must be float32 [B, H, {ctx.nb}, d]")
        if qbar.dtype != torch.float32 or kbar.dtype != torch.float32 or not (qbar.is_contiguous() and kbar.is_contiguous()):
            raise ValueError("qbar and kbar must be contiguous float32")
        device = qbar.device
    else:
        B, H, n_pad, d = qh.shape
        if qh.dtype != kh.dtype or qh.dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("qh and kh must both be bf16 or both float32")
        if tuple(kh.shape) != tuple(qh.shape) or n_pad != ctx.n_pad or not (qh.is_contiguous() and kh.is_contiguous()):
            raise ValueError(f"qh, kh must be contiguous [B, H, {ctx.n_pad}, d] (got {tuple(qh.shape)}, {tuple(kh.shape)})")
        qk_type = ABSH_F32 if qh.dtype == torch.float32 else ABSH_BF16
        device = qh.device
    if out is None:
        out = alloc_routing(ctx, B, H, order_depth)
    else:
        out.check(ctx, B, H, order_depth)
    need = route_workspace_bytes(ctx, B, H, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    sched = SCHEDULES[schedule] if isinstance(schedule, str) else int(schedule)
    policy = RANK_POLICIES[rank_policy] if isinstance(rank_policy, str) else int(rank_policy)
    opts = RouteOpts(float(p), int(k_floor), float(slack_frac), sched, int(order_depth), policy,
                     int(bool(strict_ranks)), float(k1), float(k2), float(n1), float(n2),
                     ROUTERS[router] if isinstance(router, str) else int(router), int(window), int(anchor_stride),
                     int(anchor_shift), int(step))
    lists = out.lists()
    if qbar is not None:
        _check(lib().absh_route_means(ctx.handle, _ptr(qbar), _ptr(kbar), B, H, d, ctypes.byref(opts),
                                      ctypes.byref(lists), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                                      _stream(stream)))
    else:
        _check(lib().absh_route(ctx.handle, _ptr(qh), _ptr(kh), qk_type, B, H, d, ctypes.byref(opts),
                                ctypes.byref(lists), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                                _stream(stream)))
    out.schedule = lists.schedule
    out.strict_ranks = lists.strict_ranks
    return out


def forward_workspace_bytes(ctx: Context, B: int, H: int, d: int) -> int:
    return int(lib().absh_forward_workspace_bytes(ctx.handle, B, H, d))


def forward(ctx: Context, q, k, v, p: float, k_floor: int, slack_frac: float = 0.0, schedule="xcd",
            order_depth: int = 0, routing: Optional[Routing] = None, out=None, workspace=None, stream=None):
    """The whole path in one library call: grid-order q, k, v [B, N, H, d] (bf16 or float32)
    -> (o [B, N, H, d] bf16, Routing)."""
    import torch
    B, N, H, d = q.shape
    if N != ctx.N or tuple(k.shape) != tuple(q.shape) or tuple(v.shape) != tuple(q.shape):
        raise ValueError(f"q, k, v must be [B, {ctx.N}, H, d] of one shape")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must all be bf16 or all float32")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    xt = ABSH_F32 if q.dtype == torch.float32 else ABSH_BF16
    if routing is None:
        routing = alloc_routing(ctx, B, H, order_depth)
    else:
        routing.check(ctx, B, H, order_depth)
    if out is None:
        out = torch.empty((B, N, H, d), dtype=torch.bfloat16, device=q.device)
    assert tuple(out.shape) == (B, N, H, d) and out.dtype == torch.bfloat16 and out.is_contiguous()
    need = forward_workspace_bytes(ctx, B, H, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    sched = SCHEDULES[schedule] if isinstance(schedule, str) else int(schedule)
    opts = RouteOpts(float(p), int(k_floor), float(slack_frac), sched, int(order_depth), RANK_POLICIES["auto"], 0,
                     RLB_K1, RLB_K2, SASA_N1, SASA_N2, ROUTERS["topp"], 0, 0, 0, 0)
    lists = routing.lists()
    _check(lib().absh_forward(ctx.handle, _ptr(q), _ptr(k), _ptr(v), xt, _ptr(out), B, H, d, ctypes.byref(opts),
                              ctypes.byref(lists), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                              _stream(stream)))
    routing.schedule = lists.schedule
    routing.strict_ranks = lists.strict_ranks
    return out, routing


def sparse_attn(ctx: Context, qh, kh, vt, routing: Optional[Routing] = None, out=None, stream=None):
    """Block-sparse attention (routing=None: dense) -> oh [B, H, n_pad, d] bf16 in Hilbert order."""
    import torch
    B, H, n_pad, d = qh.shape
    if out is None:
        out = torch.empty_like(qh)
    lists = routing.lists() if routing is not None else None
    _check(lib().absh_sparse_attn(ctx.handle, _ptr(qh), _ptr(kh), _ptr(vt), B, H, d,
                                  ctypes.byref(lists) if lists is not None else None, _ptr(out), _stream(stream)))
    return out


def sparse_attn_grid(ctx: Context, qh, kh, vt, routing: Optional[Routing] = None, vscale=None, out=None,
                     stream=None):
    """sparse_attn (vscale=None; vt from permute ABSH_VT) or sparse_attn_v8 (vt8 and vscale
    from quantize_v) writing o [B, N, H, d] bf16 in grid order directly, as unpermute of
    their Hilbert-order output would (routing=None: dense)."""
    import torch
    B, H, n_pad, d = qh.shape
    assert n_pad == ctx.n_pad and qh.dtype == torch.bfloat16
    if out is None:
        out = torch.empty((B, ctx.N, H, d), dtype=torch.bfloat16, device=qh.device)
    assert tuple(out.shape) == (B, ctx.N, H, d) and out.dtype == torch.bfloat16 and out.is_contiguous()
    lists = routing.lists() if routing is not None else None
    _check(lib().absh_sparse_attn_grid(ctx.handle, _ptr(qh), _ptr(kh), _ptr(vt),
                                       _ptr(vscale) if vscale is not None else None, B, H, d,
                                       ctypes.byref(lists) if lists is not None else None, _ptr(out),
                                       _stream(stream)))
    return out


def quantize_v(ctx: Context, vh, out=None, scale=None, stream=None):
    """vh [B, H, n_pad, d] bf16 (Hilbert order) -> (vt8, vscale): E4M3 codes in the
    ABSH_VT8 layout, uint8 [B, H, n_pad / 64, 64 * d], and the per-channel
    power-of-two scales, float32 [B, H, d]."""
    import torch
    B, H, n_pad, d = vh.shape
    assert n_pad == ctx.n_pad and vh.dtype == torch.bfloat16 and vh.is_contiguous()
    if out is None:
        out = torch.empty((B, H, n_pad // 64, 64 * d), dtype=torch.uint8, device=vh.device)
    if scale is None:
        scale = torch.empty((B, H, d), dtype=torch.float32, device=vh.device)
    _check(lib().absh_quantize_v(ctx.handle, _ptr(vh), B, H, d, _ptr(out), _ptr(scale), _stream(stream)))
    return out, scale


def sparse_attn_v8(ctx: Context, qh, kh, vt8, vscale, routing: Optional[Routing] = None, out=None, stream=None):
    """sparse_attn with 8-bit values from quantize_v (routing=None: dense) -> oh [B, H, n_pad, d] bf16."""
    import torch
    B, H, n_pad, d = qh.shape
    if out is None:
        out = torch.empty_like(qh)
    lists = routing.lists() if routing is not None else None
    _check(lib().absh_sparse_attn_v8(ctx.handle, _ptr(qh), _ptr(kh), _ptr(vt8), _ptr(vscale), B, H, d,
                                     ctypes.byref(lists) if lists is not None else None, _ptr(out),
                                     _stream(stream)))
    return out
