"""The C ABI without a GPU: the library loads, exports every function include/absh.h
declares, and rejects bad arguments on the host before any HIP call (a machine
without a device reports ABSH_ENODEV instead of crashing)."""
import ctypes
import os
import re

import pytest

import adaptive_block_sparse_hilbert_amd as absh

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "absh.h")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, ENODEV, EHIP = 0, -1, -2, -3, -4, -5


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(absh_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(absh.LIB_PATH):
        pytest.skip("libabsh.so not built")
    return absh.lib()


def test_every_declared_function_is_exported(L):
    names = declared_functions()
    assert len(names) >= 15
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(absh.EXPORTED)


# The calls of the boundary as the hot-path scope lays it out (context, sizes,
# permute, route, sparse attention, errors); the library may export more.
BOUNDARY = ("absh_create", "absh_destroy", "absh_dims", "absh_perm", "absh_lists_bytes", "absh_workspace_bytes",
            "absh_permute", "absh_unpermute", "absh_route", "absh_sparse_attn", "absh_status_string",
            "absh_last_error")


def test_boundary_calls_are_declared_and_exported(L):
    names = set(declared_functions())
    for name in BOUNDARY:
        assert name in names and hasattr(L, name), name


def test_routing_buffers_are_checked_before_the_call():
    """The binding rejects a caller-supplied Routing whose buffers do not fit the shape:
    the library cannot see buffer sizes, so an undersized buffer would be written past its end."""
    import types
    import torch
    if not os.path.exists(absh.LIB_PATH):
        pytest.skip("libabsh.so not built")
    ctx = types.SimpleNamespace(nb=4, n_pad=64, device=0, handle=ctypes.c_void_p())
    good = dict(counts=((1, 2, 4), torch.int32), kv_idx=((1, 2, 4, 4), torch.int16), work=((1, 2), torch.int32),
                L=((1, 2), torch.float32), queue=((8,), torch.int32), sched=((10,), torch.int32),
                unit_list=((1, 4), torch.int32), unit_cnt=((1,), torch.int32), head_order=((2,), torch.int32),
                rank_info=((absh.RANK_INFO,), torch.float64), unit_queue=((1,), torch.int32),
                pull=((absh.PULL_WORDS,), torch.int32))
    for bad, shape in (("kv_idx", (1, 2, 4, 3)), ("counts", (1, 2, 3)), ("unit_list", (0, 4)),
                       ("unit_queue", (0,)), ("rank_info", (8,)), ("pull", (8,))):
        fields = {k: torch.empty(sh, dtype=dt) for k, (sh, dt) in good.items()}
        fields[bad] = torch.empty(shape, dtype=good[bad][1])
        r = absh.Routing(order=None, **fields)
        with pytest.raises(ValueError, match=bad):
            r.check(ctx, 1, 2, 0)
    fields = {k: torch.empty(sh, dtype=dt) for k, (sh, dt) in good.items()}
    with pytest.raises(ValueError, match="order"):  # order_depth 2 needs an order buffer
        absh.Routing(order=None, **fields).check(ctx, 1, 2, 2)
    with pytest.raises(ValueError, match="cuda:0"):  # right shapes, host memory
        absh.Routing(order=None, **fields).check(ctx, 1, 2, 0)
    with pytest.raises(ValueError, match="counts"):  # wrong dtype
        fields["counts"] = torch.empty((1, 2, 4), dtype=torch.int64)
        absh.Routing(order=None, **fields).check(ctx, 1, 2, 0)


def test_version_and_status_strings(L):
    assert L.absh_version() >= 100
    for code, name in [(OK, b"ABSH_OK"), (EINVAL, b"ABSH_EINVAL"), (EUNSUPPORTED, b"ABSH_EUNSUPPORTED"),
                       (EWORKSPACE, b"ABSH_EWORKSPACE"), (ENODEV, b"ABSH_ENODEV"), (EHIP, b"ABSH_EHIP")]:
        assert L.absh_status_string(code) == name
    assert L.absh_status_string(7) == b"ABSH_UNKNOWN"


def create(L, *args):
    h = ctypes.c_void_p()
    st = L.absh_create(ctypes.byref(h), *args)
    return st, h


@pytest.mark.parametrize("args,status,msg", [
    ((0, 8, 8, 16, 0, None), EINVAL, b"grid extents"),
    ((4, -1, 8, 16, 0, None), EINVAL, b"grid extents"),
    ((4, 8, 8, 32, 0, None), EUNSUPPORTED, b"block size"),
    ((4, 8, 8, 0, 0, None), EUNSUPPORTED, b"block size"),
    ((2048, 2048, 2048, 64, 0, None), EINVAL, b"grid too large"),
    ((4, 8, 2000, 64, 0, None), EINVAL, b"above 1024"),
    ((4, 8, 8, 16, -1, None), EINVAL, b"device index"),
])
def test_create_rejects_bad_arguments_before_hip(L, args, status, msg):
    st, h = create(L, *args)
    assert st == status
    assert msg in L.absh_last_error()
    assert not h.value


def test_create_null_out_pointer(L):
    assert L.absh_create(None, 4, 8, 8, 16, 0, None) == EINVAL


def test_create_without_device_is_enodev():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    L = absh.lib()
    st, h = create(L, 4, 8, 8, 16, 0, None)
    assert st == ENODEV and not h.value
    assert b"no HIP device" in L.absh_last_error()


def test_null_context_everywhere(L):
    vp = ctypes.c_void_p
    N, nb, npad = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    assert L.absh_dims(None, ctypes.byref(N), ctypes.byref(nb), ctypes.byref(npad)) == EINVAL
    assert L.absh_perm(None, None, None) == EINVAL
    assert L.absh_perm_copy(None, None, None, None) == EINVAL
    assert L.absh_permute(None, vp(16), 0, vp(16), 1, 1, 64, 0, None) == EINVAL
    assert L.absh_unpermute(None, vp(16), vp(16), 1, 1, 64, None) == EINVAL
    assert L.absh_pool(None, vp(16), vp(16), 1, 1, 64, None) == EINVAL
    assert L.absh_block_scores(None, vp(16), vp(16), vp(16), 1, 1, 64, None) == EINVAL
    opts = absh.RouteOpts(0.9, 4, 0.0, 1, 0)
    lists = absh.Lists()
    assert L.absh_route(None, vp(16), vp(16), 0, 1, 1, 64, ctypes.byref(opts), ctypes.byref(lists), vp(256),
                        ctypes.c_size_t(1 << 20), None) == EINVAL
    assert L.absh_route_static(None, vp(16), vp(16), 0, 1, 1, 64, ctypes.byref(opts), ctypes.byref(lists),
                               None) == EINVAL
    assert L.absh_route_means(None, vp(16), vp(16), 1, 1, 64, ctypes.byref(opts), ctypes.byref(lists), vp(256),
                              ctypes.c_size_t(1 << 20), None) == EINVAL
    assert b"ctx is NULL" in L.absh_last_error()
    assert L.absh_route_means(None, None, vp(16), 1, 1, 64, ctypes.byref(opts), ctypes.byref(lists), vp(256),
                              ctypes.c_size_t(1 << 20), None) == EINVAL
    assert b"qbar is NULL" in L.absh_last_error()
    assert L.absh_permute_pool(None, vp(16), 0, vp(16), vp(16), 1, 1, 64, 0, None) == EINVAL
    assert L.absh_forward(None, vp(16), vp(16), vp(16), 0, vp(16), 1, 1, 64, ctypes.byref(opts), ctypes.byref(lists),
                          vp(256), ctypes.c_size_t(1 << 20), None) == EINVAL
    assert L.absh_forward_workspace_bytes(None, 1, 1, 64) == 0
    assert L.absh_sparse_attn(None, vp(16), vp(16), vp(16), 1, 1, 64, None, vp(16), None) == EINVAL
    assert b"ctx is NULL" in L.absh_last_error()
    assert L.absh_quantize_v(None, vp(16), 1, 1, 64, vp(16), vp(16), None) == EINVAL
    assert L.absh_sparse_attn_v8(None, vp(16), vp(16), vp(16), vp(16), 1, 1, 64, None, vp(16), None) == EINVAL
    assert b"ctx is NULL" in L.absh_last_error()
    assert L.absh_sparse_attn_grid(None, vp(16), vp(16), vp(16), None, 1, 1, 64, None, vp(16), None) == EINVAL
    assert L.absh_sparse_attn_grid(None, vp(16), vp(16), vp(16), vp(16), 1, 1, 64, None, vp(16), None) == EINVAL
    assert b"ctx is NULL" in L.absh_last_error()
    assert L.absh_route_workspace_bytes(None, 1, 1, 64) == 0
    assert L.absh_lists_units(None, 1, 1, 0) == 0
    assert L.absh_lists_bytes(None, 1, 1, 0) == 0
    assert L.absh_workspace_bytes(None, 1, 1, 64) == 0
    assert L.absh_attn_workgroups(None) == 0
    assert L.absh_lists_carve(None, 1, 1, 0, vp(256), ctypes.c_size_t(1 << 20), ctypes.byref(lists)) == EINVAL
    assert L.absh_destroy(None) == OK


def test_last_error_is_thread_local(L):
    import threading
    assert L.absh_create(None, 4, 8, 8, 16, 0, None) == EINVAL
    seen = []

    def other():
        seen.append(L.absh_last_error())
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen == [b""]
    assert b"NULL" in L.absh_last_error()


def test_python_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(absh, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(absh, "_lib", None)
    with pytest.raises(ImportError):
        absh.lib()


def test_struct_layout_matches_header(tmp_path):
    """The binding's ctypes structs have the C header's sizes and field offsets (compiled with gcc)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    src = tmp_path / "layout.c"
    fields = {"absh_route_opts": [f for f, _ in absh.RouteOpts._fields_],
              "absh_lists": [f for f, _ in absh.Lists._fields_]}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "absh.h"', "int main(void) {"]
    for struct, names in fields.items():
        lines.append(f'  printf("{struct} %zu\\n", sizeof({struct}));')
        for n in names:
            lines.append(f'  printf("{struct}.{n} %zu\\n", offsetof({struct}, {n}));')
    lines += ["  return 0;", "}"]
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(root, "include"), str(src), "-o", str(exe)], check=True)
    out = dict(line.rsplit(" ", 1) for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                              check=True).stdout.split("\n") if line)
    for struct, cls in (("absh_route_opts", absh.RouteOpts), ("absh_lists", absh.Lists)):
        assert int(out[struct]) == ctypes.sizeof(cls), struct
        for n, _ in cls._fields_:
            assert int(out[f"{struct}.{n}"]) == getattr(cls, n).offset, (struct, n)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: asking for more exits with a message before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_bench_clock_sampler_reads_the_current_level(tmp_path):
    """The bench's clock sampler takes the level pp_dpm_sclk marks with '*', and reports
    median / min / max over its samples; a missing file gives no report."""
    import importlib.util
    import time
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 2031Mhz *\n2: 2400Mhz\n")
    s = bench.ClockSampler(str(f), period=0.005)
    s.start()
    time.sleep(0.05)
    f.write_text("0: 500Mhz\n1: 1987Mhz *\n2: 2400Mhz\n")
    time.sleep(0.05)
    s.halt.set()
    s.join()
    rep = s.report()
    assert rep["samples"] >= 2 and rep["min_mhz"] == 1987 and rep["max_mhz"] == 2031
    assert rep["median_mhz"] in (1987, 2031)
    gone = bench.ClockSampler(str(tmp_path / "absent"), period=0.005)
    gone.start()
    time.sleep(0.02)
    gone.halt.set()
    gone.join()
    assert gone.report() is None


def test_bench_balance_from_busy_record():
    """The bench's rho over workgroups comes from the busy record (end - start of the
    workgroups that ran) and rho_sim from a list schedule that pulls the XCD's own run
    first: four units of union length 3, 1, 1, 1 (cost + 1) on two workers give loads
    6 and 4, so rho_sim = 1.2."""
    import importlib.util
    import types
    import torch
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    routing = types.SimpleNamespace(
        sched=torch.tensor([0, 1, 2, 3, 4, 4, 4, 4, 4, 4], dtype=torch.int32),
        unit_cnt=torch.tensor([3, 1, 1, 1], dtype=torch.int32),
        counts=torch.ones((1, 1, 16), dtype=torch.int32))
    busy = torch.tensor([[100, 700], [100, 500], [0, 0]], dtype=torch.int64)  # the third never ran
    rep = bench.launch_balance(absh, routing, "xcd", busy, 64)
    assert rep["workgroups"] == 2
    assert rep["rho_wg"] == round(600 / 500, 4) and rep["min_over_mean_wg"] == round(400 / 500, 4)
    assert rep["rho_sim"] == 1.2



def test_cpu_baseline_compares_every_head():
    """The bench's CPU leg with every head's lists: lists equal to the oracle's own come
    out identical on every tile, and one changed list is reported as a failure."""
    import importlib.util
    import numpy as np
    import workloads as W
    from oracle import absh_oracle as O
    spec = importlib.util.spec_from_file_location("bench_under_test_cpu", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    w = W.workload(0)
    data = W.generate(w, want_fp32=True)
    perm, _ = O.hilbert_perm(w.T, w.Y, w.X)
    R = O.route(O.to_hilbert(data["q32"], perm), O.to_hilbert(data["k32"], perm), w.block, w.p, w.k_floor)
    counts = R.counts.astype(np.int32)
    kv = np.full(counts.shape + (R.nb,), -1, dtype=np.int64)
    for b in range(counts.shape[0]):
        for h in range(counts.shape[1]):
            for i in range(R.nb):
                kv[b, h, i, : counts[b, h, i]] = R.retained(b, h, i)
    out = bench.cpu_baseline(w, w.p, data, 0.05, (counts[:, :1], kv[:, :1]), (counts, kv))
    a = out["route_parity_all_heads"]
    assert a["tiles"] == counts.size and a["identical"] == counts.size and a["failures"] == 0
    # a list that drops its last block is not excusable
    t = np.unravel_index(int(np.argmax(counts)), counts.shape)
    counts2 = counts.copy()
    counts2[t] -= 1
    out = bench.cpu_baseline(w, w.p, data, 0.05, None, (counts2, kv))
    assert out["route_parity_all_heads"]["failures"] + out["route_parity_all_heads"]["excused"] == 1
