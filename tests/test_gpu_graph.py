"""The whole path (absh_forward) captured in a HIP graph and replayed.

Inside absh_forward the library allocates nothing and does not synchronise with the
host. It clears its counters and scratch with kernels of its own, not memset nodes,
and the attention leaves its pull counters at zero. So each replay of the captured
graph must reproduce the eager call's lists and output bit for bit. The test runs
eager work and a host synchronisation between the replays, and checks every replay
against the eager call."""
import numpy as np
import pytest
import torch

import adaptive_block_sparse_hilbert_amd as absh
import workloads as W

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def routing_tensors(r, units, schedule):
    """The routing outputs the call writes for this schedule (units: its work units)."""
    t = dict(counts=r.counts, kv_idx=r.kv_idx, work=r.work, L=r.L, queue=r.queue, sched=r.sched,
             unit_list=r.unit_list[:units], unit_cnt=r.unit_cnt[:units])
    if schedule == "lpt":
        t["unit_queue"] = r.unit_queue[:units]
    if schedule == "ranks":
        t["head_order"] = r.head_order
    return t


def written(name, t, r, units):
    """The part of a routing tensor the call writes: lists are row-padded, and only the
    first counts[tile] (kv_idx) or unit_cnt[unit] (unit_list) entries of a row are set."""
    nb = t.shape[-1]
    if name == "kv_idx":
        return t[torch.arange(nb, device=t.device) < r.counts[..., None]]
    if name == "unit_list":
        return t[torch.arange(nb, device=t.device) < r.unit_cnt[:units, None]]
    return t


@pytest.mark.parametrize("index,schedule", [(1, "xcd"), (3, "lpt"), (2, "ranks"), (4, "xcd")])
def test_forward_graph_replays_equal_the_eager_call(index, schedule):
    w = W.workload(index)
    print(f"[graph] {w.name} {schedule}", flush=True)
    d = W.generate(w)
    q, k, v = (bf16_dev(d[n]) for n in ("q16", "k16", "v16"))
    ctx = absh.create(w.T, w.Y, w.X, w.block)
    B, _, H, hd = q.shape
    args = dict(slack_frac=w.slack_frac, schedule=schedule)

    # the eager reference (its own routing, output and workspace)
    o_ref, r_ref = absh.forward(ctx, q, k, v, w.p, w.k_floor, **args)
    torch.cuda.synchronize()
    units = absh.lists_units(ctx, B, H, schedule)
    assert units > 0
    want = {n: written(n, t, r_ref, units).clone() for n, t in routing_tensors(r_ref, units, schedule).items()}

    # everything the captured call touches is allocated before the capture
    ws = torch.empty(absh.forward_workspace_bytes(ctx, B, H, hd), dtype=torch.uint8, device=DEV)
    routing = absh.alloc_routing(ctx, B, H)
    out = torch.empty_like(o_ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one call on a side stream before capturing
        absh.forward(ctx, q, k, v, w.p, w.k_floor, routing=routing, out=out, workspace=ws, **args)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        absh.forward(ctx, q, k, v, w.p, w.k_floor, routing=routing, out=out, workspace=ws, **args)
    torch.cuda.synchronize()

    for rep in range(3):
        # eager work between the replays: clear every output of the captured call
        out.zero_()
        for t in routing_tensors(routing, units, schedule).values():
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), o_ref.view(torch.int16)), f"output, replay {rep}"
        for n, t in routing_tensors(routing, units, schedule).items():
            assert torch.equal(written(n, t, routing, units), want[n]), f"{n}, replay {rep}"
        print(f"[graph] replay {rep} identical", flush=True)
    del graph
    ctx.close()


def test_separate_calls_graph_replays_equal_the_eager_calls():
    """The same with the calls made one by one (permute with pooling of q and k, permute
    of v, routing from the block means, attention writing grid order), 480p, xcd."""
    w = W.workload(1)
    schedule = "xcd"
    print(f"[graph] {w.name} separate calls", flush=True)
    d = W.generate(w)
    q, k, v = (bf16_dev(d[n]) for n in ("q16", "k16", "v16"))
    ctx = absh.create(w.T, w.Y, w.X, w.block)
    B, _, H, hd = q.shape
    units = absh.lists_units(ctx, B, H, schedule)

    def path(bufs=None):
        b = bufs or {}
        qh, qbar = absh.permute_pool(ctx, q, out=b.get("qh"), means=b.get("qbar"))
        kh, kbar = absh.permute_pool(ctx, k, out=b.get("kh"), means=b.get("kbar"))
        vt = absh.permute(ctx, v, layout=absh.ABSH_VT, out=b.get("vt"))
        r = absh.route(ctx, None, None, w.p, w.k_floor, schedule=schedule, qbar=qbar, kbar=kbar,
                       out=b.get("routing"), workspace=b.get("ws"))
        o = absh.sparse_attn_grid(ctx, qh, kh, vt, r, out=b.get("o"))
        return dict(qh=qh, qbar=qbar, kh=kh, kbar=kbar, vt=vt, routing=r, o=o)

    ref = path()
    torch.cuda.synchronize()
    want = {n: written(n, t, ref["routing"], units).clone()
            for n, t in routing_tensors(ref["routing"], units, schedule).items()}
    # every buffer of the captured calls, allocated before the capture
    bufs = {n: torch.empty_like(t) for n, t in ref.items() if n != "routing"}
    bufs["routing"] = absh.alloc_routing(ctx, B, H)
    bufs["ws"] = torch.empty(absh.route_workspace_bytes(ctx, B, H, hd), dtype=torch.uint8, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        path(bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path(bufs)
    torch.cuda.synchronize()

    for rep in range(3):
        for n in ("qh", "qbar", "kh", "kbar", "vt", "o"):
            bufs[n].zero_()
        for t in routing_tensors(bufs["routing"], units, schedule).values():
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in ("qh", "kh", "vt", "o"):
            assert torch.equal(bufs[n].view(torch.int16), ref[n].view(torch.int16)), f"{n}, replay {rep}"
        for n in ("qbar", "kbar"):
            assert torch.equal(bufs[n].view(torch.int32), ref[n].view(torch.int32)), f"{n}, replay {rep}"
        for n, t in routing_tensors(bufs["routing"], units, schedule).items():
            assert torch.equal(written(n, t, bufs["routing"], units), want[n]), f"{n}, replay {rep}"
        print(f"[graph] separate calls: replay {rep} identical", flush=True)
    del graph
    ctx.close()
