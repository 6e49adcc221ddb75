"""Sharding by head (the multi-GPU plan): one rank's share of the heads, run on its own, gives the
same routing and the same attention output, bit for bit, as those heads inside the full run.

Routing and attention never mix heads, and every query row is computed the same way whatever
the schedule (same blocks, same ascending order), so a head's results cannot depend on which
other heads share the launch. Checked at 720p with 40 heads: heads 10..14 (rank 2 of 8 under
the contiguous Ulysses split) against the full run, with bf16 and with 8-bit values.
"""
import numpy as np
import pytest
import torch

import adaptive_block_sparse_hilbert_amd as absh
from test_gpu_parity import case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("schedule", ["xcd", "order"])
def test_one_rank_share_equals_full_run(schedule):
    c = case(2)
    w = c.w
    h0, h1 = 10, 15
    full = absh.route(c.ctx, c.qh, c.kh, w.p, w.k_floor, schedule=schedule)
    o_full = absh.sparse_attn(c.ctx, c.qh, c.kh, c.vt, full)
    vh = absh.permute(c.ctx, c.v)
    vt8, vs = absh.quantize_v(c.ctx, vh)
    o8_full = absh.sparse_attn_v8(c.ctx, c.qh, c.kh, vt8, vs, full)

    q, k, v = (x[:, :, h0:h1, :].contiguous() for x in (c.q, c.k, c.v))
    qh, kh = absh.permute(c.ctx, q), absh.permute(c.ctx, k)
    vt = absh.permute(c.ctx, v, layout=absh.ABSH_VT)
    part = absh.route(c.ctx, qh, kh, w.p, w.k_floor, schedule=schedule)
    o_part = absh.sparse_attn(c.ctx, qh, kh, vt, part)
    vt8p, vsp = absh.quantize_v(c.ctx, absh.permute(c.ctx, v))
    o8_part = absh.sparse_attn_v8(c.ctx, qh, kh, vt8p, vsp, part)
    torch.cuda.synchronize()

    assert torch.equal(part.counts, full.counts[:, h0:h1])
    n = full.counts[:, h0:h1].cpu().numpy()
    kv_f = full.kv_idx[:, h0:h1].cpu().numpy().astype(np.int64)
    kv_p = part.kv_idx.cpu().numpy().astype(np.int64)
    for i in range(w.nb):
        for hh in range(h1 - h0):
            assert np.array_equal(kv_p[0, hh, i, : n[0, hh, i]], kv_f[0, hh, i, : n[0, hh, i]])
    assert torch.equal(part.work, full.work[:, h0:h1]) and torch.equal(part.L, full.L[:, h0:h1])
    rows = torch.arange(w.N, device=o_full.device)
    assert torch.equal(o_part[:, :, rows].view(torch.int16), o_full[:, h0:h1][:, :, rows].view(torch.int16))
    assert torch.equal(vsp, vs[:, h0:h1])
    assert torch.equal(o8_part[:, :, rows].view(torch.int16), o8_full[:, h0:h1][:, :, rows].view(torch.int16))
