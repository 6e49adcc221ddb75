"""Throughput of the Hilbert-ordered Top-p router + block-sparse attention on one MI355X.

One step is one pass of the whole path over one batch of synthetic input that is
already resident in HBM:
    permute q, k (rows, with their block means) and v (block-transposed) into
    Hilbert order
    -> route (block scores, Top-p + floor [+ slack fill], Eq. 1, tile queue)
    -> block-sparse attention over the retained blocks, whose output stores put
       each row back at its grid position (no separate unpermute).
The default workload is 720p video at 40 heads (grid 21 x 45 x 80 = 75,600 tokens,
d = 128, block 64, p = 0.9, k = 4, the "xcd" schedule). --all-configs runs the
five synthetic workloads one after another (the 6x horizon at p = 0.8, 0.9 and
0.95), one JSON line each; the head-skew workload runs on the longest-first
schedule its configuration names, the tiny one routes from float32 q and k.

value = retained FLOPs / step time, where retained FLOPs = sum over tiles and
retained blocks of 4 * n_i * n_j * d with true token counts. Each stage is timed
with HIP events on the stream its kernels run on; the attention kernel's own
average duration gives the roofline figure against the bf16 MFMA peak.

--values fp8 runs the review's V quantization instead: v is permuted as rows and
quantized to E4M3 with per-channel scales (its own stage), and the attention's
value product runs on fp8 MFMAs. Half the retained FLOPs (Q K^T) stay bf16 and
half (P V) are fp8, so the roofline peak is then 1 / (0.5 / 2.5 + 0.5 / 5.0)
PFLOP/s = 3.33 PFLOP/s.

Besides the throughput, each line reports the balance of the attention launch:
rho_wg = max / mean busy time over its workgroups, from the per-workgroup busy
record the attention kernel writes (Eq. 2 of the review read over workgroups),
and rho_sim, the same ratio for a list schedule of the launch's work units over
as many workers, each worker pulling from its XCD's run first as the kernel does,
with unit cost = union length + 1. The cpu_baseline leg also checks head 0's
lists (before slack fill) against the oracle's routing of that head and reports
how many tiles differ and how many of those the routing tolerance excuses.

Prints one JSON line per workload. Inputs are synthetic (see workloads/), data = "synthetic".
"""
from __future__ import annotations

import argparse
import glob
import json
import os
import re
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
# half the attention's FLOPs on each: the time-weighted peak of bf16 Q K^T + fp8 P V
PEAK_MIXED_TFLOPS = 1.0 / (0.5 / PEAK_BF16_TFLOPS + 0.5 / PEAK_FP8_TFLOPS)
PEAK_HBM_GBS = 8000.0
PEAK_CLOCK_MHZ = 2400.0      # MI355X peak engine clock, at which the MFMA peaks are quoted


class ClockSampler(threading.Thread):
    """Reads the current graphics-clock level from sysfs every `period` seconds until stopped.

    pp_dpm_sclk lists the clock levels and marks the current one with '*'. Host-side
    reads only: the GPU's work is untouched.
    """

    def __init__(self, path, period=0.02):
        super().__init__(daemon=True)
        self.path, self.period, self.samples = path, period, []
        self.halt = threading.Event()

    def run(self):
        while not self.halt.wait(self.period):
            try:
                text = open(self.path).read()
            except OSError:
                return
            for line in text.splitlines():
                m = re.search(r"(\d+)\s*mhz\s*\*\s*$", line, re.IGNORECASE)
                if m:
                    self.samples.append(int(m.group(1)))

    def report(self):
        if not self.samples:
            return None
        v = sorted(self.samples)
        return {"median_mhz": v[len(v) // 2], "min_mhz": v[0], "max_mhz": v[-1], "samples": len(v)}


def gpu_sysfs():
    """(sclk file, power cap in W) of the first GPU card in sysfs; None where the host hides them."""
    files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if not files:
        return None, None
    cap = None
    for f in sorted(glob.glob(os.path.join(os.path.dirname(files[0]), "hwmon", "hwmon*", "power1_cap"))):
        try:
            cap = int(open(f).read().strip()) / 1e6
            break
        except (OSError, ValueError):
            pass
    return files[0], cap


def gpu_env(dev, clock, cap):
    import torch

    props = torch.cuda.get_device_properties(dev)
    try:
        rocm = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        rocm = None
    return {"device": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "hip_runtime": torch.version.hip, "rocm": rocm,
            "power_cap_w": cap, "sclk_during_timed_steps": clock}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="720p-40h")
    ap.add_argument("--all-configs", action="store_true",
                    help="run every synthetic workload (one JSON line each) instead of --workload")
    ap.add_argument("--route-f32", action="store_true",
                    help="route from float32 q and k rows (an extra float32 permute of q and k)")
    ap.add_argument("--p", type=float, default=None, help="override the workload's Top-p")
    ap.add_argument("--schedule", default="xcd", choices=("order", "lpt", "xcd", "ranks"),
                    help="tile schedule of the attention kernel")
    ap.add_argument("--rank-policy", default="auto", choices=("auto", "none", "sasa", "rlb+sasa", "rlb"),
                    help="schedule 'ranks': RLB / SASA policy (auto: the piecewise policy on rho)")
    ap.add_argument("--strict-ranks", action="store_true",
                    help="schedule 'ranks': each XCD runs only its own rank's work (as separate GPUs would)")
    ap.add_argument("--router", default="topp", choices=("topp", "window-anchor"),
                    help="Top-p routing, or the structured local window + rotating anchors pattern")
    ap.add_argument("--window", type=int, default=24, help="window-anchor router: blocks on each side")
    ap.add_argument("--anchor-stride", type=int, default=32, help="window-anchor router: anchor spacing")
    ap.add_argument("--anchor-shift", type=int, default=5, help="window-anchor router: offset advance per step")
    ap.add_argument("--step", type=int, default=0, help="window-anchor router: diffusion step")
    ap.add_argument("--pool", default="fused", choices=("fused", "separate"),
                    help="block means of q and k: in the permute's pass (absh_permute_pool, then "
                         "absh_route_means), or pooled inside absh_route")
    ap.add_argument("--overlap-v", action=argparse.BooleanOptionalAction, default=False,
                    help="permute (and quantize) v on a second stream (default priority) while the "
                         "router runs, which reads no rows (off by default: the attention after it then "
                         "runs at a lower clock, and the step takes longer)")
    ap.add_argument("--values", default="bf16", choices=("bf16", "fp8"),
                    help="fp8: quantize V to E4M3 and run the value product on fp8 MFMAs")
    ap.add_argument("--dense-reps", type=int, default=3)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--out-order", choices=("grid", "hilbert"), default="grid",
                    help="grid: the attention writes o in grid order itself (absh_sparse_attn_grid); "
                         "hilbert: Hilbert-order output, then absh_unpermute as a stage of its own")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity-all", action="store_true",
                    help="in the cpu_baseline leg, route and compare head 0 only (not every head)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="host time budget of the oracle's attention sample")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the steps, run one plain device copy of this size (for counter scaling)")
    ap.add_argument("--traffic-profile", default=None,
                    help="counter summary giving the attention kernel's HBM bytes per launch "
                         "(default: profiles/attn_<workload>_hbm.md)")
    return ap.parse_args()


ALL_RUNS = ((0, None), (1, None), (2, None), (3, None), (4, 0.8), (4, 0.9), (4, 0.95))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the path would shard by head across GPUs).", file=sys.stderr)
        sys.exit(2)
    import workloads as W

    if not args.all_configs:
        print(json.dumps(measure(args, W.workload(args.workload), args.p, args.schedule, args.route_f32)))
        return
    for index, p in ALL_RUNS:
        w = W.workload(index)
        if args.values == "fp8" and w.block not in (64, 128):
            print(f"[bench] {w.name}: 8-bit values need blocks of 64 or 128 (block {w.block}); skipped",
                  file=sys.stderr, flush=True)
            continue
        schedule = "lpt" if w.lpt else args.schedule
        print(json.dumps(measure(args, w, p, schedule, args.route_f32 or w.dtype == "fp32")), flush=True)


def measure(args, w, p, schedule, route_f32):
    """One workload: warm-up, timed steps, dense reference, balance, cpu baseline -> the JSON record."""
    import numpy as np
    import torch

    import adaptive_block_sparse_hilbert_amd as absh
    import workloads as W

    p = w.p if p is None else p
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    t0 = time.time()
    data = W.generate(w, want_fp32=route_f32)
    to_dev = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = to_dev(data["q16"]), to_dev(data["k16"]), to_dev(data["v16"])
    gen_s = time.time() - t0
    print(f"[bench] {w.name}: inputs ready in {gen_s:.1f}s", file=sys.stderr, flush=True)

    ctx = absh.create(w.T, w.Y, w.X, w.block, device=0)
    B, H, d = w.B, w.H, w.d
    stream = torch.cuda.current_stream()
    # every buffer of the step, allocated once
    qh = torch.empty((B, H, ctx.n_pad, d), dtype=torch.bfloat16, device=dev)
    kh = torch.empty_like(qh)
    fp8 = args.values == "fp8"
    if fp8:
        vh = torch.empty_like(qh)
        vt8 = torch.empty((B, H, ctx.n_pad // 64, 64 * d), dtype=torch.uint8, device=dev)
        vscale = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    else:
        vt = torch.empty((B, H, ctx.nb, d, absh.vt_keys(w.block)), dtype=torch.bfloat16, device=dev)
    grid_out = args.out_order == "grid"
    oh = None if grid_out else torch.empty_like(qh)
    o = torch.empty_like(q)
    routing = absh.alloc_routing(ctx, B, H)
    wg_busy = absh.busy_record(ctx, routing)
    ws = torch.empty(absh.route_workspace_bytes(ctx, B, H, d), dtype=torch.uint8, device=dev)
    if route_f32:  # float32 rows of q and k for the router
        q32 = torch.from_numpy(data["q32"]).to(dev)
        k32 = torch.from_numpy(data["k32"]).to(dev)
        qr = torch.empty((B, H, ctx.n_pad, d), dtype=torch.float32, device=dev)
        kr = torch.empty_like(qr)
    # block means of q and k from the permute's own pass (Top-p router), else pooled by the router
    fused_pool = args.pool == "fused" and args.router == "topp"
    qbar = torch.empty((B, H, ctx.nb, d), dtype=torch.float32, device=dev)
    kbar = torch.empty_like(qbar)

    stages = ("permute", "quantize", "route", "attn", "unpermute")
    overlap_v = args.overlap_v
    side = torch.cuda.Stream(device=dev) if overlap_v else None  # default priority

    def attention(lists):
        if grid_out:
            absh.sparse_attn_grid(ctx, qh, kh, vt8 if fp8 else vt, lists, vscale=vscale if fp8 else None, out=o)
        elif fp8:
            absh.sparse_attn_v8(ctx, qh, kh, vt8, vscale, lists, out=oh)
        else:
            absh.sparse_attn(ctx, qh, kh, vt, lists, out=oh)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if fused_pool and not route_f32:
            absh.permute_pool(ctx, q, out=qh, means=qbar)
            absh.permute_pool(ctx, k, out=kh, means=kbar)
        else:
            absh.permute(ctx, q, out=qh)
            absh.permute(ctx, k, out=kh)
        if route_f32 and fused_pool:
            absh.permute_pool(ctx, q32, layout=absh.ABSH_ROWS_F32, out=qr, means=qbar)
            absh.permute_pool(ctx, k32, layout=absh.ABSH_ROWS_F32, out=kr, means=kbar)
        elif route_f32:
            absh.permute(ctx, q32, layout=absh.ABSH_ROWS_F32, out=qr)
            absh.permute(ctx, k32, layout=absh.ABSH_ROWS_F32, out=kr)
        def v_work(st):
            if fp8:
                absh.permute(ctx, v, out=vh, stream=st)
                absh.quantize_v(ctx, vh, out=vt8, scale=vscale, stream=st)
            else:
                absh.permute(ctx, v, layout=absh.ABSH_VT, out=vt, stream=st)
        if overlap_v:
            # v's permute (and quantization) on a second stream, beside the routing,
            # which reads no rows; the attention waits for both
            side.wait_stream(stream)
            v_work(side)
        elif fp8:
            absh.permute(ctx, v, out=vh)
        else:
            absh.permute(ctx, v, layout=absh.ABSH_VT, out=vt)
        if ev is not None:
            ev[1].record(stream)
        if fp8 and not overlap_v:
            absh.quantize_v(ctx, vh, out=vt8, scale=vscale)
        if ev is not None:
            ev[2].record(stream)
        absh.route(ctx, qr if route_f32 else qh, kr if route_f32 else kh, p, w.k_floor,
                   slack_frac=w.slack_frac if args.router == "topp" else 0.0, schedule=schedule, out=routing,
                   rank_policy=args.rank_policy, strict_ranks=args.strict_ranks, router=args.router,
                   window=args.window, anchor_stride=args.anchor_stride, anchor_shift=args.anchor_shift,
                   step=args.step,
                   workspace=ws, qbar=qbar if fused_pool else None, kbar=kbar if fused_pool else None)
        if ev is not None:
            ev[3].record(stream)
        if overlap_v:
            stream.wait_stream(side)
        attention(routing)
        if ev is not None:
            ev[4].record(stream)
        if not grid_out:
            absh.unpermute(ctx, oh, out=o)
        if ev is not None:
            ev[5].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    sclk_file, power_cap = gpu_sysfs()
    sampler = ClockSampler(sclk_file) if sclk_file else None
    torch.cuda.synchronize()
    if sampler:
        sampler.start()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    if sampler:
        sampler.halt.set()
        sampler.join()
    ms_per_step = wall * 1e3 / args.steps
    stage_ms = {s: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in events])) for i, s in enumerate(stages)}
    stage_min = {s: float(np.min([e[i].elapsed_time(e[i + 1]) for e in events])) for i, s in enumerate(stages)}
    stage_med = {s: float(np.median([e[i].elapsed_time(e[i + 1]) for e in events])) for i, s in enumerate(stages)}
    if not fp8:  # no quantization stage with bf16 values
        del stage_ms["quantize"], stage_min["quantize"], stage_med["quantize"]
    if grid_out:  # the attention writes o itself
        del stage_ms["unpermute"], stage_min["unpermute"], stage_med["unpermute"]

    # retained work of this routing (identical every step: the path is deterministic)
    counts = routing.counts.cpu().numpy().reshape(-1)
    kv = routing.kv_idx.cpu().numpy().astype(np.int64).reshape(counts.size, ctx.nb)
    sizes = np.minimum(w.block, w.N - np.arange(ctx.nb) * w.block).astype(np.int64)
    # sum of n_j over each retained list: only the last block can be partial, and an
    # ascending list holds it in its last slot
    has_last = kv[np.arange(counts.size), counts - 1] == ctx.nb - 1
    kv_tokens = counts.astype(np.int64) * w.block - has_last * (w.block - sizes[-1])
    qi = np.tile(sizes, B * H)
    f_ret = float(4.0 * d * np.sum(qi * kv_tokens))
    density = float(counts.mean() / ctx.nb)
    L_h = routing.L.cpu().numpy().reshape(-1).astype(np.float64)
    work = {"sum_counts": int(counts.astype(np.int64).sum()),
            "L_h": {"min": round(float(L_h.min()), 3), "mean": round(float(L_h.mean()), 3),
                    "max": round(float(L_h.max()), 3)},
            "density_h": {"min": round(float(L_h.min()) / ctx.nb, 5), "max": round(float(L_h.max()) / ctx.nb, 5)}}

    balance = launch_balance(absh, routing, schedule, wg_busy, w.block)

    value = f_ret / (ms_per_step * 1e-3) / 1e12
    attn_tflops = f_ret / (stage_ms["attn"] * 1e-3) / 1e12

    dense_ms = None
    if not args.no_dense:
        attention(None)
        torch.cuda.synchronize()
        de = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        times = []
        for _ in range(args.dense_reps):
            de[0].record(stream)
            attention(None)
            de[1].record(stream)
            torch.cuda.synchronize()
            times.append(de[0].elapsed_time(de[1]))
        dense_ms = float(np.mean(times))
    n_all = float(4.0 * d * B * H * float(w.N) ** 2)

    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    traffic = measured_traffic(args.traffic_profile or os.path.join(
        ROOT, "profiles", "attn_" + w.name.replace("-", "") + ("_fp8" if fp8 else "") + "_hbm.md"),
        w.name, schedule, args.values)

    peak = PEAK_MIXED_TFLOPS if fp8 else PEAK_BF16_TFLOPS
    clock = sampler.report() if sampler else None
    # the published peak assumes the 2.4 GHz peak engine clock; the same peak at the
    # clock sampled over the timed steps, for reference
    peak_clk = None if clock is None else peak * clock["median_mhz"] / PEAK_CLOCK_MHZ
    roof = {
        "bound": "mfma",
        "kernel": attention_kernel_name(d, w.block, unit_members(w.block, schedule), fp8),
        "achieved": round(attn_tflops, 2),
        "peak": round(peak, 1),
        "unit": "TFLOP/s",
        "frac": round(attn_tflops / peak, 4),
        "traffic": traffic,
        # HBM bytes the launch must move at least: q, k, v read once (v in 8 bits with --values fp8), o written once
        "traffic_minimum": float(B * H * w.N * d * (2 + 2 + (1 if fp8 else 2) + 2)),
        "traffic_over_minimum": None if traffic is None else round(
            traffic / float(B * H * w.N * d * (2 + 2 + (1 if fp8 else 2) + 2)), 2),
        "peak_at_measured_clock": None if peak_clk is None else round(peak_clk, 1),
        "frac_at_measured_clock": None if peak_clk is None else round(attn_tflops / peak_clk, 4),
    }

    cpu = None
    if not args.no_cpu_baseline:
        # head 0's lists before any slack fill, for the parity sample of the baseline leg
        base = routing
        if w.slack_frac > 0 and args.router == "topp":
            base = absh.route(ctx, qr if route_f32 else qh, kr if route_f32 else kh, p, w.k_floor, schedule=schedule)
        head0 = (base.counts[:, :1].cpu().numpy(), base.kv_idx[:, :1].cpu().numpy().astype(np.int64))
        lists_all = None
        if args.router == "topp" and not args.no_parity_all:
            lists_all = (base.counts.cpu().numpy(), base.kv_idx.cpu().numpy().astype(np.int64))
        cpu = cpu_baseline(w, p, data, args.cpu_seconds, head0 if args.router == "topp" else None, lists_all)

    out = {
        "metric": "effective bf16 TFLOP/s on retained blocks + speedup vs dense, 720p 40-head",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+fp8" if fp8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": B, "heads": H, "head_dim": d, "grid_t_y_x": [w.T, w.Y, w.X],
            "tokens": w.N, "block": w.block, "blocks": ctx.nb, "p": p, "k_floor": w.k_floor,
            "slack_frac": w.slack_frac, "schedule": schedule, "router": args.router, "values": args.values,
            "route_inputs": "f32" if route_f32 else "bf16",
            "pooling": "in the permute pass" if fused_pool else "in the router",
            "v_permute": "beside the routing, second stream" if overlap_v else "in order",
            "output": "grid order, written by the attention" if grid_out else "Hilbert order, then unpermute",
            **({"window": args.window, "anchor_stride": args.anchor_stride, "anchor_shift": args.anchor_shift,
                "step": args.step} if args.router == "window-anchor" else {}),
        },
        "ranks": rank_report(routing, args) if schedule == "ranks" else None,
        "balance": balance,
        "density": round(density, 5),
        "work": work,
        "retained_tflop": round(f_ret / 1e12, 4),
        "dense_tflop": round(n_all / 1e12, 4),
        "stage_ms": {s: round(x, 4) for s, x in stage_ms.items()},
        "stage_ms_min": {s: round(x, 4) for s, x in stage_min.items()},
        "stage_ms_median": {s: round(x, 4) for s, x in stage_med.items()},
        "attn_effective_tflops": round(attn_tflops, 2),
        "route_share_of_attn": round(stage_ms["route"] / stage_ms["attn"], 4),
        "dense_attn_ms": None if dense_ms is None else round(dense_ms, 3),
        "dense_tflops": None if dense_ms is None else round(n_all / (dense_ms * 1e-3) / 1e12, 2),
        "speedup_vs_dense": None if dense_ms is None else round(dense_ms / stage_ms["attn"], 3),
        "speedup_vs_dense_incl_route": None if dense_ms is None else
        round(dense_ms / (stage_ms["attn"] + stage_ms["route"]), 3),
        "roofline": roof,
        "cpu_baseline": cpu,
        "env": gpu_env(dev, clock, power_cap),
    }
    return out


def rank_report(routing, args):
    """The rank stage's report (rho before / after migration / after augmentation, moves, budgets)."""
    info = routing.rank_info.cpu().numpy()
    return {
        "policy_asked": args.rank_policy, "strict": bool(args.strict_ranks),
        "policy_taken": ["none", "sasa", "rlb+sasa", "rlb"][int(info[3])],
        "rho_before": round(float(info[0]), 4), "rho_after_rlb": round(float(info[1]), 4),
        "rho_after_sasa": round(float(info[2]), 4),
        "moves": [[int(x) for x in info[37 + 3 * i: 40 + 3 * i]] for i in range(int(info[4]))],
        "rank_blocks_before": [int(x) for x in info[5:13]], "rank_blocks_after": [int(x) for x in info[21:29]],
        "sasa_budgets": [int(x) for x in info[29:37]],
    }


def unit_members(block, schedule):
    """Query blocks per attention work unit: four 64-row or two 128-row blocks on every
    schedule, single tiles for blocks of 16 under the longest-first schedule."""
    if schedule == "lpt" and block < 64:
        return 1
    return 2 if block >= 128 else 4


def attention_kernel_name(d, block, members, fp8=False):
    """Name of the kernel that runs the attention launch (as the profiler lists it).

    Units of four 64-row or two 128-row query blocks at head dim 64 or 128 run on
    the union kernel (its last template argument: 8-bit values); any other shape
    runs on the general one.
    """
    if d in (64, 128) and (block, members) in ((64, 4), (128, 2)):
        return f"union_attn_kernel<{d}, {block}, {'true' if fp8 else 'false'}>"
    return f"attn_kernel<{d}, {block}>"


def measured_traffic(path, workload, schedule, values="bf16"):
    """HBM bytes per attention launch from a committed counter summary, or None.

    The summary holds FETCH_SIZE + WRITE_SIZE of the attention kernel, scaled by a
    plain-copy calibration, together with the sha256 of the attention sources it
    was taken on (attn.hip followed by attn_union.hip). A figure taken on another
    source, workload or schedule is stale and gives None.
    """
    import hashlib

    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            m = line.strip().split(": ", 1)
            if len(m) == 2:
                fields[m[0]] = m[1]
    h = hashlib.sha256()
    for name in ("attn.hip", "attn_union.hip"):
        with open(os.path.join(ROOT, "adaptive_block_sparse_hilbert_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    if (fields.get("attn_src_sha256") != h.hexdigest() or fields.get("workload") != workload
            or fields.get("schedule") != schedule or fields.get("values", "bf16") != values
            or "hbm_bytes_per_launch" not in fields):
        return None
    return int(fields["hbm_bytes_per_launch"])


def launch_balance(absh, routing, schedule, wg_busy, block):
    """rho over the workgroups of the last attention launch (from its busy record), and
    rho_sim of a list schedule of the same work units over as many workers."""
    import heapq

    import numpy as np

    busy = absh.busy_ticks(wg_busy).astype(np.float64)
    if busy.size == 0:
        return None
    bounds = routing.sched.cpu().numpy().tolist()
    members = bounds[9]
    if members == 1:  # single tiles in queue order
        cost = routing.counts.cpu().numpy().reshape(-1)[routing.queue.cpu().numpy()]
    else:
        ucnt = routing.unit_cnt.cpu().numpy()
        n = bounds[8]
        if schedule == "lpt":
            units = routing.unit_queue.cpu().numpy()[:n]
        elif schedule == "ranks":
            per_head = -(-routing.counts.shape[2] // members)
            pos = np.arange(n)
            units = routing.head_order.cpu().numpy()[pos // per_head] * per_head + pos % per_head
        else:
            units = np.arange(n)
        cost = ucnt[units]
    cost = cost.astype(np.float64) + 1.0
    workers = busy.size
    nxt, hi = list(bounds[:8]), bounds[1:9]
    load = np.zeros(workers)
    heap = [(0.0, x) for x in range(workers)]
    while heap:
        t, x = heapq.heappop(heap)
        for k in range(8):
            seg = (x + k) & 7
            if nxt[seg] < hi[seg]:
                c = cost[nxt[seg]]
                nxt[seg] += 1
                load[x] += c
                heapq.heappush(heap, (t + c, x))
                break
    return {"workgroups": int(workers), "rho_wg": round(float(busy.max() / busy.mean()), 4),
            "min_over_mean_wg": round(float(busy.min() / busy.mean()), 4),
            "rho_sim": round(float(load.max() / load.mean()), 4), "block": block}


def cpu_baseline(w, p, data, budget_s, head0=None, lists_all=None):
    """The oracle on a bounded sample of the same workload, timed on the host cores.

    Sample: head 0 of the workload. The oracle computes the Hilbert order, gathers
    head 0's q, k, v, routes all of head 0's query blocks (block means, scores,
    softmax, Top-p + floor), then runs attention for query blocks of head 0 taken
    in a fixed spread-out order until budget_s seconds of attention have run.
    Routing time is prorated to the tiles done (n / nb of it), so the figure is the
    retained FLOPs of the sample tiles divided by their share of the oracle's time.
    With lists_all (the GPU's counts and lists of every head, before any slack fill)
    the oracle also routes every head, timed, and every tile is compared.
    """
    import numpy as np
    import threadpoolctl

    import workloads as W
    from oracle import absh_oracle as O

    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    t0 = time.perf_counter()
    perm, _ = O.hilbert_perm(w.T, w.Y, w.X)
    head = lambda name: W.bf16_to_f32(data[name + "16"][:, :, :1, :])
    qh, kh, vh = (O.to_hilbert(head(n), perm) for n in ("q", "k", "v"))
    if "q32" in data:  # routing from the float32 rows
        qr, kr = (O.to_hilbert(np.ascontiguousarray(data[n][:, :, :1, :]), perm) for n in ("q32", "k32"))
    else:
        qr, kr = qh, kh
    R = O.route(qr, kr, w.block, p, w.k_floor)
    t_route = time.perf_counter() - t0
    parity = None
    if head0 is not None:  # head 0's GPU lists against the oracle's, under the routing tolerance
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from routing_compare import compare_routing

        counts_g, kv_g = head0
        same = sum(int(np.array_equal(kv_g[0, 0, i, : counts_g[0, 0, i]], R.retained(0, 0, i)))
                   for i in range(R.nb))
        excused, failures = compare_routing(R, counts_g, kv_g, p)
        parity = {"tiles": int(R.nb), "identical": same, "excused": int(excused), "failures": len(failures)}
    all_heads = None
    if lists_all is not None:  # every head: the oracle's routing time and the GPU's lists against it
        full = lambda name: O.to_hilbert(np.ascontiguousarray(
            data[name + "32"] if name + "32" in data else W.bf16_to_f32(data[name + "16"])), perm)
        qa, ka = full("q"), full("k")
        t2 = time.perf_counter()
        RA = O.route(qa, ka, w.block, p, w.k_floor)
        t_all = time.perf_counter() - t2
        del qa, ka
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from routing_compare import compare_routing

        counts_a, kv_a = lists_all
        excused, failures = compare_routing(RA, counts_a, kv_a, p)
        all_heads = {"heads": int(counts_a.shape[0] * counts_a.shape[1]), "tiles": int(counts_a.size),
                     "identical": int(counts_a.size) - int(excused) - len(failures), "excused": int(excused),
                     "failures": len(failures), "oracle_route_s": round(t_all, 3)}
        del RA
    nb = R.nb
    order = np.argsort((np.arange(nb) * 0.6180339887) % 1.0, kind="stable")  # spread over the head
    t1 = time.perf_counter()
    flops, done = 0.0, 0
    for i in order:
        blocks = R.retained(0, 0, i)
        O.attention_tile(qh[0, 0], kh[0, 0], vh[0, 0], w.block, i, blocks)
        flops += 4.0 * w.d * R.sizes[i] * R.sizes[blocks].sum()
        done += 1
        if time.perf_counter() - t1 > budget_s:
            break
    t_attn = time.perf_counter() - t1
    t = t_attn + t_route * done / nb
    return {
        "value": round(flops / t / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"head 0 of {w.name}: Hilbert order + full routing of its {nb} query blocks "
                   f"({t_route:.2f} s, prorated to the sample), attention for {done} query blocks "
                   f"spread over the head ({t_attn:.2f} s); float64 NumPy"),
        "route_parity_head0": parity,
        "route_parity_all_heads": all_heads,
        "oracle_route_s_head0": round(t_route, 3),
        "oracle_attn_s": round(t_attn, 3),
        "oracle_attn_tiles": done,
    }


if __name__ == "__main__":
    main()
