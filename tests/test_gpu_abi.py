"""C ABI validation on a real context: every bad argument is rejected with its status
before anything is launched (outputs keep their sentinel values)."""
import ctypes

import pytest
import torch

import adaptive_block_sparse_hilbert_amd as absh

pytestmark = pytest.mark.gpu

EINVAL, EUNSUPPORTED, EWORKSPACE = -1, -2, -3
DEV = torch.device("cuda", 0)


@pytest.fixture(scope="module")
def env():
    ctx = absh.create(3, 8, 8, 16)            # N = 192, nb = 12
    B, H, d = 1, 2, 64
    qh = torch.zeros((B, H, ctx.n_pad, d), dtype=torch.bfloat16, device=DEV)
    r = absh.alloc_routing(ctx, B, H, order_depth=4)
    ws = torch.empty(absh.route_workspace_bytes(ctx, B, H, d), dtype=torch.uint8, device=DEV)
    return ctx, qh, r, ws


def call_route(ctx, qh, r, ws, p=0.9, k=2, slack=0.0, sched=1, depth=0, nbytes=None, ws_ptr=None, d=64,
               lists=None, qk_type=0):
    opts = absh.RouteOpts(p, k, slack, sched, depth)
    lists = r.lists() if lists is None else lists
    ptr = ws.data_ptr() if ws_ptr is None else ws_ptr
    n = ws.numel() if nbytes is None else nbytes
    return absh.lib().absh_route(ctx.handle, ctypes.c_void_p(qh.data_ptr()), ctypes.c_void_p(qh.data_ptr()),
                                 qk_type, 1, 2, d, ctypes.byref(opts), ctypes.byref(lists), ctypes.c_void_p(ptr),
                                 ctypes.c_size_t(n), None)


@pytest.mark.parametrize("kw,status", [
    (dict(p=0.0), EINVAL), (dict(p=-0.5), EINVAL), (dict(p=1.5), EINVAL), (dict(p=float("nan")), EINVAL),
    (dict(k=-1), EINVAL), (dict(slack=1.0), EINVAL), (dict(slack=-0.1), EINVAL),
    (dict(depth=65), EINVAL), (dict(depth=-1), EINVAL), (dict(sched=3), EINVAL), (dict(sched=-1), EINVAL),
    (dict(d=96), EUNSUPPORTED), (dict(nbytes=1024), EWORKSPACE), (dict(ws_ptr=0), EWORKSPACE),
    (dict(qk_type=2), EINVAL), (dict(qk_type=-1), EINVAL),
])
def test_route_rejects(env, kw, status):
    ctx, qh, r, ws = env
    r.counts.fill_(-7)
    torch.cuda.synchronize()
    assert call_route(ctx, qh, r, ws, **kw) == status
    torch.cuda.synchronize()
    assert (r.counts == -7).all(), "a rejected call launched work"
    assert absh.lib().absh_last_error()


def test_route_needs_outputs(env):
    ctx, qh, r, ws = env
    lists = r.lists()
    lists.counts = None
    assert call_route(ctx, qh, r, ws, lists=lists) == EINVAL
    lists = r.lists()
    lists.unit_list = None
    assert call_route(ctx, qh, r, ws, sched=2, lists=lists) == EINVAL
    assert call_route(ctx, qh, r, ws, sched=1, lists=lists) == 0     # LPT does not use unit lists
    lists = r.lists()
    lists.order = None
    assert call_route(ctx, qh, r, ws, depth=4, lists=lists) == EINVAL


def test_route_rejects_misaligned_workspace(env):
    ctx, qh, r, ws = env
    big = torch.empty(ws.numel() + 256, dtype=torch.uint8, device=DEV)
    assert call_route(ctx, qh, r, big, ws_ptr=big.data_ptr() + 4, nbytes=big.numel() - 4) == EINVAL
    assert b"aligned" in absh.lib().absh_last_error()


def test_router_block_count_limit():
    ctx = absh.create(64, 64, 64, 16)          # nb = 16384 > 2048
    qh = torch.zeros((1, 1, ctx.n_pad, 64), dtype=torch.bfloat16, device=DEV)
    opts = absh.RouteOpts(0.9, 2, 0.0, 1, 0)
    lists = absh.Lists(*([ctypes.c_void_p(qh.data_ptr()).value] * 9 + [1]))
    st = absh.lib().absh_route(ctx.handle, ctypes.c_void_p(qh.data_ptr()), ctypes.c_void_p(qh.data_ptr()), 0, 1, 1,
                               64, ctypes.byref(opts), ctypes.byref(lists), ctypes.c_void_p(qh.data_ptr()),
                               ctypes.c_size_t(1 << 40), None)
    assert st == EUNSUPPORTED and b"nb" in absh.lib().absh_last_error()


def test_sparse_attn_rejects(env):
    ctx, qh, r, ws = env
    vt = torch.zeros((1, 2, ctx.nb, 64, absh.vt_keys(16)), dtype=torch.bfloat16, device=DEV)
    oh = torch.full_like(qh, 3.0)
    L = absh.lib()
    lists = r.lists()
    lists.schedule = 9
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    assert L.absh_sparse_attn(ctx.handle, p(qh), p(qh), p(vt), 1, 2, 64, ctypes.byref(lists), p(oh), None) == EINVAL
    lists = r.lists()
    lists.schedule = 2
    lists.unit_list = None
    assert L.absh_sparse_attn(ctx.handle, p(qh), p(qh), p(vt), 1, 2, 64, ctypes.byref(lists), p(oh), None) == EINVAL
    assert L.absh_sparse_attn(ctx.handle, p(qh), p(qh), p(vt), 1, 2, 96, None, p(oh), None) == EUNSUPPORTED
    assert L.absh_sparse_attn(ctx.handle, ctypes.c_void_p(qh.data_ptr() + 2), p(qh), p(vt), 1, 2, 64, None, p(oh),
                              None) == EINVAL
    torch.cuda.synchronize()
    assert (oh == 3.0).all()


def test_permute_rejects(env):
    ctx, qh, r, ws = env
    x = torch.zeros((1, ctx.N, 2, 64), dtype=torch.bfloat16, device=DEV)
    L = absh.lib()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    assert L.absh_permute(ctx.handle, p(x), 5, p(qh), 1, 2, 64, 0, None) == EINVAL
    assert L.absh_permute(ctx.handle, p(x), 0, p(qh), 1, 2, 64, 7, None) == EINVAL
    assert L.absh_permute(ctx.handle, p(x), 0, p(qh), 0, 2, 64, 0, None) == EINVAL
    assert L.absh_permute(ctx.handle, None, 0, p(qh), 1, 2, 64, 0, None) == EINVAL
    assert L.absh_unpermute(ctx.handle, p(qh), None, 1, 2, 64, None) == EINVAL


def test_dims_and_units(env):
    ctx, qh, r, ws = env
    assert (ctx.N, ctx.nb, ctx.n_pad) == (192, 12, 192)
    assert absh.lists_units(ctx, 1, 2, "lpt") == 24
    assert absh.lists_units(ctx, 1, 2, "xcd") == 2 * 3      # groups of 4 query blocks


def test_lpt_group_units_need_the_unit_queue():
    """Blocks of 64: the longest-first schedule runs group units, so it needs unit lists
    and the unit queue; a carved arena supplies every buffer."""
    ctx = absh.create(2, 8, 16, 64)           # N = 256, nb = 4
    B, H, d = 1, 3, 64
    qh = torch.zeros((B, H, ctx.n_pad, d), dtype=torch.bfloat16, device=DEV)
    r = absh.alloc_routing(ctx, B, H)
    ws = torch.empty(absh.route_workspace_bytes(ctx, B, H, d), dtype=torch.uint8, device=DEV)
    assert absh.lists_units(ctx, B, H, "lpt") == H * 1
    opts = absh.RouteOpts(0.9, 2, 0.0, absh.SCHEDULES["lpt"], 0)
    L = absh.lib()
    p = lambda t: ctypes.c_void_p(t.data_ptr())

    def call(lists):
        return L.absh_route(ctx.handle, p(qh), p(qh), 0, B, H, d, ctypes.byref(opts), ctypes.byref(lists), p(ws),
                            ctypes.c_size_t(ws.numel()), None)
    lists = r.lists()
    lists.unit_queue = None
    assert call(lists) == EINVAL and b"unit_queue" in L.absh_last_error()
    lists = r.lists()
    lists.unit_list = None
    assert call(lists) == EINVAL
    assert call(r.lists()) == 0
    nbytes = absh.lists_bytes(ctx, B, H)
    arena = torch.empty(nbytes + 256, dtype=torch.uint8, device=DEV)
    carved = absh.Lists()
    assert L.absh_lists_carve(ctx.handle, B, H, 0, ctypes.c_void_p(arena.data_ptr() + 1), ctypes.c_size_t(nbytes),
                              ctypes.byref(carved)) == EINVAL
    assert L.absh_lists_carve(ctx.handle, B, H, 0, p(arena), ctypes.c_size_t(nbytes - 1),
                              ctypes.byref(carved)) == EWORKSPACE
    assert L.absh_lists_carve(ctx.handle, B, H, 0, p(arena), ctypes.c_size_t(nbytes), ctypes.byref(carved)) == 0
    assert carved.order is None and carved.unit_queue is not None
    assert call(carved) == 0
    torch.cuda.synchronize()
    assert torch.equal(arena[carved.counts - arena.data_ptr():][: B * H * ctx.nb * 4].view(torch.int32),
                       r.counts.view(-1))
