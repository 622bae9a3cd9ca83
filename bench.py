#!/usr/bin/env python3
"""Benchmark of the fused residual-add + RMSNorm row kernels on one MI355X.

One step = one call of the fused add+RMSNorm entry point over the prefill
workload 16384 rows x 8192 (bf16 x, f32 residual stream in and out, bf16
weight, bf16 out), inputs resident in HBM.  The JSON line's ``value`` is the
achieved HBM bandwidth in GB/s over the algorithmic bytes of one step (every
input read once, every output written once, the weight once), from HIP events
on the stream the kernel runs on.

The same line carries:
  * ``roofline``: the kernel against MI355X's 8 TB/s HBM peak, plus the HBM
    bytes measured by rocprofv3 counters when profiles/ holds a counter
    summary taken on this very library build (same sha256), else null;
  * ``cpu_baseline``: the CPU oracle (numpy, float64) timed on a bounded
    sample of the same workload, one process per host core (``cores``), and
    ``cpu_baseline_1core`` the same in one process;
  * ``decode``: the metric's second half, us/call of the decode workloads
    (8 x 1024 and 256 x 4096, and an 8-partial 64-token call) against an
    empty kernel launched the same way: in a HIP graph, eagerly from a native
    loop through the C ABI, and eagerly from Python through the package's
    prepared call;
  * ``secondary``: the streaming lines in compact form -- per-head QK-norm
    (and the same heads through the rows kernel), one GPU's 2048-row share of
    the headline, the fp8-output prefill with per-row scales, the same
    prefill with block-scaled outputs (fp8 per-128 scales, MXFP8, MXFP4,
    NVFP4), the exact sum of 8 partial inputs in front of the add (one GPU's
    share of a tensor-parallel reduce-scatter; bf16 and MXFP4 out), and the
    SiLU-and-mul activation (bf16, MXFP8, MXFP4, NVFP4 out): us/call, GB/s,
    fraction of peak, the same-size copy and the counter traffic ratio, with
    rotating buffer sets larger than the 256 MB Infinity Cache so that every
    call streams from HBM.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused add+RMSNorm achieved HBM GB/s (% of peak) prefill; decode us/call"
PEAK_HBM_GBS = 8000.0  # MI355X published HBM3E bandwidth, 8 TB/s
MAIN = "prefill_16384x8192"
PROFILE_DIR = os.path.join(ROOT, "profiles")


_T0 = time.monotonic()


def log(msg: str) -> None:
    print(f"[bench +{time.monotonic() - _T0:6.1f}s] {msg}", file=sys.stderr, flush=True)


def library_digest() -> str:
    """sha256 of the built library (what the counter summaries were measured on).

    The build is byte-for-byte reproducible, so this changes exactly when the
    compiled code does (kernels, selector or ABI), not on comment-only edits."""
    from residual_add_rmsnorm_rows_amd import _lib as L

    h = hashlib.sha256()
    with open(L.LIB_PATH, "rb") as f:
        h.update(f.read())
    return h.hexdigest()


def read_traffic(workload: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the library as built now; else None."""
    path = os.path.join(PROFILE_DIR, f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("library_sha256") != library_digest():
        return None
    try:
        return int(float(fields["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def attach_traffic(name: str, entry: dict) -> None:
    """Add the counter-measured HBM bytes per launch of a secondary workload
    (null where no summary of the current sources exists)."""
    t = read_traffic(name)
    entry["traffic_bytes"] = t
    entry["traffic_over_algorithmic"] = None if t is None else round(t / entry["algorithmic_bytes"], 4)


SCALE_BYTES = {"row": lambda h: 4, "group128": lambda h: 4 * (h // 128), "mx32": lambda h: h // 32,
               "nv16": lambda h: h // 16}
SCHEME_TEXT = {"row": "a float32 scale amax/448 per row", "group128": "a float32 scale per 128 elements",
               "mx32": "an E8M0 scale per 32 elements (MX)",
               "nv16": "an E4M3FN scale per 16 elements and a float32 tensor scale (NVFP4)"}
# NVFP4 tensor scales: fixed values near amax / (6 * 448) of each workload's
# outputs (any positive value is a valid input; the traffic does not depend on it).
POWER_WARMUP = 200  # launches before the SwiGLU and partial-input lines are timed (15-20 ms of load)
NV_TENSOR_SCALE = {"prefill_fp8_8192x7168": 2.0 ** -5, "silu_mul_8192x14336": 2.0 ** -7}
QUANT_TEXT = {"fp8_e4m3fn": "fp8 e4m3fn", "fp4_e2m1": "fp4 e2m1"}


def rownorm_bytes(wl, rows=None, scale_scheme: str = "row") -> int:
    """Algorithmic bytes: x, residual read once; out, residual_out written once; weight once; scales."""
    r = wl.rows if rows is None else rows
    size = {"bf16": 2, "f32": 4, "fp8_e4m3fn": 1, "fp4_e2m1": 0.5}
    per_row = wl.hidden * (size[wl.x_dtype] + size[wl.out_dtype])
    if wl.res_dtype is not None:
        per_row += 2 * wl.hidden * size[wl.res_dtype]
    if wl.out_dtype in ("fp8_e4m3fn", "fp4_e2m1"):
        per_row += SCALE_BYTES[scale_scheme](wl.hidden)
    return int(r * per_row + wl.hidden * size[wl.w_dtype])


def qknorm_bytes(wl) -> int:
    size = {"bf16": 2, "f32": 4}
    n = wl.tokens * (wl.num_q_heads + wl.num_k_heads) * wl.head_dim
    return 2 * n * size[wl.dtype] + wl.head_dim * size[wl.w_dtype] * (2 if wl.num_k_heads else 1)


class RowCall:
    """Device buffers of one fused add+RMSNorm workload and a raw C-ABI call over them."""

    def __init__(self, wl, inputs, sets: int = 1, scale_scheme: str = "row", config=None):
        import torch
        from residual_add_rmsnorm_rows_amd import _lib as L
        from workloads.device import TORCH_DTYPES, to_dev

        self.wl = wl
        quant = wl.out_dtype in ("fp8_e4m3fn", "fp4_e2m1")
        out_cols = wl.hidden // 2 if wl.out_dtype == "fp4_e2m1" else wl.hidden
        scale_bytes = SCALE_BYTES[scale_scheme](wl.hidden)
        self.L = L.lib()
        x = to_dev(inputs["x"], wl.x_dtype)
        res = None if inputs["residual"] is None else to_dev(inputs["residual"], wl.res_dtype)
        self.w = to_dev(inputs["weight"], wl.w_dtype)
        self.sets = []
        for i in range(sets):
            xs = x if i == 0 else x.clone()
            rs = None if res is None else (res if i == 0 else res.clone())
            out = torch.empty((wl.rows, out_cols), dtype=TORCH_DTYPES[wl.out_dtype], device="cuda")
            ro = None if rs is None else torch.empty_like(rs)
            sc = torch.empty((wl.rows, scale_bytes), dtype=torch.uint8, device="cuda") if quant else None
            self.sets.append((xs, rs, out, ro, sc))
        self.flags = L.make_flags(wl.x_dtype, wl.res_dtype, wl.w_dtype, wl.out_dtype, wl.weight_plus_one,
                                  scale_scheme)
        self.ts = (torch.tensor([NV_TENSOR_SCALE[wl.name]], dtype=torch.float32, device="cuda")
                   if scale_scheme == "nv16" else None)
        self.config = config  # an explicit rn_launch_config, or None for the selector's
        self.i = 0

    def __call__(self, stream: int) -> None:
        xs, rs, out, ro, sc = self.sets[self.i]
        self.i = (self.i + 1) % len(self.sets)
        if self.config is not None:
            st = self.L.rmsnorm_fwd_config(xs.data_ptr(), None if rs is None else rs.data_ptr(), self.w.data_ptr(),
                                           out.data_ptr(), None if ro is None else ro.data_ptr(),
                                           None if sc is None else sc.data_ptr(), None,
                                           None if self.ts is None else self.ts.data_ptr(), self.wl.rows,
                                           self.wl.hidden, self.wl.eps, self.flags, ctypes.byref(self.config), stream)
            if st != 0:
                from residual_add_rmsnorm_rows_amd._lib import check
                check(st)
            return
        st = self.L.rmsnorm_fwd_ex(xs.data_ptr(), None if rs is None else rs.data_ptr(), self.w.data_ptr(),
                                   out.data_ptr(), None if ro is None else ro.data_ptr(),
                                   None if sc is None else sc.data_ptr(), None,
                                   None if self.ts is None else self.ts.data_ptr(), self.wl.rows, self.wl.hidden,
                                   self.wl.eps, self.flags, stream)
        if st != 0:
            from residual_add_rmsnorm_rows_amd._lib import check
            check(st)


def time_stream_loop(fn, steps: int, warmup: int) -> float:
    """Average milliseconds per call of fn(stream) over `steps` back-to-back calls (HIP events)."""
    import torch

    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(warmup):
        fn(stream)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn(stream)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_prepared_loop(call, steps: int, warmup: int) -> float:
    """time_stream_loop for a prepared call (its stream is bound when it is
    prepared): the loop calls it the way a caller does, call()."""
    import torch

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        call()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def launch_percentiles(fn, launches: int = 50) -> dict:
    """p10 / p50 / p90 of single-launch durations (each launch between its own
    pair of events on the launch stream), in microseconds."""
    import torch

    stream = torch.cuda.current_stream().cuda_stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    for a, b in evs:
        a.record()
        fn(stream)
        b.record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) * 1000.0 for a, b in evs)
    pick = lambda q: round(per[min(len(per) - 1, int(q * len(per)))], 2)  # noqa: E731
    return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9), "launches": len(per)}


def time_graph_loop(fn, calls: int = 200, replays: int = 10) -> float:
    """Average microseconds per call with `calls` calls captured in one HIP graph."""
    import torch

    fn(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=s):
        cs = torch.cuda.current_stream().cuda_stream
        for _ in range(calls):
            fn(cs)
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1000.0 / (replays * calls)


def copy_ceiling(nbytes: int, sets: int, steps: int, warmup: int) -> dict:
    """The library's streaming copy moving `nbytes` per call (half read, half
    written) over `sets` rotating buffer pairs, timed like the kernels."""
    import torch

    from residual_add_rmsnorm_rows_amd import _lib as L

    half = (nbytes // 2) // 16 * 16
    pairs = [(torch.empty(half, dtype=torch.uint8, device="cuda"), torch.empty(half, dtype=torch.uint8, device="cuda"))
             for _ in range(sets)]
    lib = L.lib()
    state = {"i": 0}

    def copy(stream):
        src, dst = pairs[state["i"]]
        state["i"] = (state["i"] + 1) % sets
        st = lib.rn_launch_copy(src.data_ptr(), dst.data_ptr(), half, stream)
        if st != 0:
            L.check(st)

    ms = time_stream_loop(copy, steps, warmup)
    gbs = 2 * half / (ms * 1e-3) / 1e9
    del pairs
    torch.cuda.empty_cache()
    return {"bytes_per_launch": 2 * half, "buffer_sets": sets, "us_per_call": round(ms * 1000, 3),
            "GBps": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}


def native_decode_latency(name: str, calls: int = 2000) -> dict:
    """Eager decode latency through the C ABI from native code (the library's
    rn_decode_latency driver, a child process): rmsnorm_fwd against
    rn_launch_empty, back to back on one stream, no Python in the loop."""
    import subprocess

    import workloads as WL
    from residual_add_rmsnorm_rows_amd import build as B

    wl = WL.WORKLOADS[name]
    if not os.path.exists(B.DECODE_LATENCY_PATH):
        return {"error": "rn_decode_latency is not built"}
    try:
        p = subprocess.run([B.DECODE_LATENCY_PATH, str(wl.rows), str(wl.hidden), str(int(wl.weight_plus_one)),
                            str(calls)], capture_output=True, text=True, timeout=120)
    except subprocess.TimeoutExpired:
        return {"error": "timed out"}
    if p.returncode != 0:
        return {"error": (p.stderr or p.stdout).strip()[-300:]}
    r = json.loads(p.stdout.strip().splitlines()[-1])
    return {k: r[k] for k in ("us_per_call", "empty_us_per_call", "ratio", "calls", "host_enqueue_us",
                              "empty_host_enqueue_us", "select_and_check_ns")}


def decode_metrics(name: str) -> dict:
    import workloads as WL
    import residual_add_rmsnorm_rows_amd as R
    from residual_add_rmsnorm_rows_amd import _lib as L

    wl = WL.WORKLOADS[name]
    call = RowCall(wl, WL.generate_rownorm(wl, seed=0))
    lib = L.lib()

    def empty(stream):
        lib.rn_launch_empty(stream)

    eager = time_stream_loop(call, 2000, 100) * 1000.0
    eager_empty = time_stream_loop(empty, 2000, 100) * 1000.0
    graph = time_graph_loop(call)
    graph_empty = time_graph_loop(empty)
    # the package's prepared call (arguments marshalled once), eager from Python
    from workloads.device import to_dev

    inp = WL.generate_rownorm(wl, seed=0)
    prepared = R.prepare_fused_add_rmsnorm(to_dev(inp["x"], wl.x_dtype), to_dev(inp["residual"], wl.res_dtype),
                                           to_dev(inp["weight"], wl.w_dtype), wl.eps,
                                           weight_plus_one=wl.weight_plus_one)
    py_eager = time_prepared_loop(prepared, 2000, 100) * 1000.0
    # the one-wave-per-row decode shape (the whole row in one wave64's
    # registers, no LDS, no barrier), timed the same way for comparison
    vec = 8 if wl.x_dtype == "bf16" else 4
    cfg = L.LaunchConfig()
    cfg.kernel, cfg.waves_per_row, cfg.grid = L.RN_KERNEL_ROWS, 1, wl.rows
    cfg.vecs_per_lane = next(nv for nv in (1, 2, 4, 8) if 64 * nv * vec >= wl.hidden)
    one = RowCall(wl, WL.generate_rownorm(wl, seed=0), config=cfg)
    graph_one = time_graph_loop(one)
    sel = R.query_config(wl.rows, wl.hidden, x_dtype=wl.x_dtype, res_dtype=wl.res_dtype, w_dtype=wl.w_dtype,
                         out_dtype=wl.out_dtype, weight_plus_one=wl.weight_plus_one, num_cus=0)
    return {
        "workload": wl.description, "rows": wl.rows, "hidden": wl.hidden,
        "launch": {"waves_per_row": sel["waves_per_row"], "vecs_per_lane": sel["vecs_per_lane"]},
        "us_per_call_eager": round(eager, 3), "empty_us_per_call_eager": round(eager_empty, 3),
        "ratio_eager": round(eager / eager_empty, 3),
        "us_per_call_graph": round(graph, 3), "empty_us_per_call_graph": round(graph_empty, 3),
        "ratio_graph": round(graph / graph_empty, 3),
        "us_per_call_python_prepared": round(py_eager, 3), "ratio_python_prepared": round(py_eager / eager_empty, 3),
        "one_wave_per_row": {"vecs_per_lane": cfg.vecs_per_lane, "us_per_call_graph": round(graph_one, 3),
                             "ratio_graph": round(graph_one / graph_empty, 3)},
        "algorithmic_bytes": rownorm_bytes(wl),
    }


def stream_metrics(name: str, steps: int, warmup: int, sets: int, out_dtype=None,
                   scale_scheme: str = "row", rows=None) -> dict:
    from dataclasses import replace

    import workloads as WL

    wl = WL.WORKLOADS[name]
    if out_dtype is not None:
        wl = replace(wl, out_dtype=out_dtype)
    if rows is not None:
        wl = wl.with_rows(rows)
    call = RowCall(wl, WL.generate_rownorm(wl, seed=0), sets=sets, scale_scheme=scale_scheme)
    ms = time_stream_loop(call, steps, warmup)
    spread = launch_percentiles(call)
    b = rownorm_bytes(wl, scale_scheme=scale_scheme)
    desc = wl.description
    if wl.out_dtype in QUANT_TEXT:
        desc = (f"prefill fused add+RMSNorm, {wl.rows} x {wl.hidden} {wl.x_dtype} x and residual "
                f"(1% outliers x20), {QUANT_TEXT[wl.out_dtype]} out with {SCHEME_TEXT[scale_scheme]}")
    if rows is not None:
        desc = f"{desc}; {rows} of its rows, one GPU's share when the rows are split over GPUs"
    return {"workload": desc, "out": wl.out_dtype, "scale_scheme": scale_scheme,
            "us_per_call": round(ms * 1000, 3), "algorithmic_bytes": b,
            "GBps": round(b / (ms * 1e-3) / 1e9, 1), "frac_of_peak": round(b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "buffer_sets": sets, "launch_us": spread}


def qknorm_metrics(steps: int, warmup: int, sets: int = 8) -> dict:
    import torch

    import workloads as WL
    from residual_add_rmsnorm_rows_amd import _lib as L
    from workloads.device import to_dev

    wl = WL.WORKLOADS["qknorm_4096x32x128"]
    inp = WL.generate_qknorm(wl, seed=0)
    q0 = to_dev(inp["q"].reshape(wl.tokens, -1), wl.dtype)
    w = to_dev(inp["q_weight"], wl.w_dtype)
    bufs = [(q0 if i == 0 else q0.clone(), torch.empty_like(q0)) for i in range(sets)]
    lib = L.lib()
    flags = L.DTYPE_CODES[wl.dtype] | (L.DTYPE_CODES[wl.w_dtype] << L.RN_FLAGS_W_SHIFT)
    state = {"i": 0}

    def call(stream):
        q, o = bufs[state["i"]]
        state["i"] = (state["i"] + 1) % sets
        st = lib.qknorm_fwd(q.data_ptr(), None, w.data_ptr(), None, o.data_ptr(), None, wl.tokens,
                            wl.num_q_heads, 0, wl.head_dim, 0, 0, wl.eps, flags, stream)
        if st != 0:
            L.check(st)

    ms = time_stream_loop(call, steps, warmup)
    spread = launch_percentiles(call)
    b = qknorm_bytes(wl)
    return {"workload": wl.description, "us_per_call": round(ms * 1000, 3), "algorithmic_bytes": b,
            "GBps": round(b / (ms * 1e-3) / 1e9, 1), "frac_of_peak": round(b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "buffer_sets": sets, "launch_us": spread}


def partials_bytes(wl, scale_scheme: str = "row") -> int:
    """Algorithmic bytes: every partial and the residual read once; out (and its scales) and residual_out
    written once; weight once."""
    size = {"bf16": 2, "f32": 4, "fp8_e4m3fn": 1, "fp4_e2m1": 0.5}
    per_row = wl.hidden * (wl.num_partials * size[wl.x_dtype] + size[wl.out_dtype])
    if wl.res_dtype is not None:
        per_row += 2 * wl.hidden * size[wl.res_dtype]
    if wl.out_dtype in ("fp8_e4m3fn", "fp4_e2m1"):
        per_row += SCALE_BYTES[scale_scheme](wl.hidden)
    return int(wl.rows * per_row + wl.hidden * size[wl.w_dtype])


class PartialsCall:
    """Device buffers of one partial-input workload and a raw C-ABI call over them."""

    def __init__(self, wl, sets: int = 1, scale_scheme: str = "row", tensor_scale=None):
        import torch

        import workloads as WL
        from residual_add_rmsnorm_rows_amd import _lib as L
        from workloads.device import TORCH_DTYPES, to_dev

        self.wl = wl
        inp = WL.generate_partials(wl, seed=0)
        parts0 = [to_dev(p, wl.x_dtype) for p in inp["partials"]]
        res0 = to_dev(inp["residual"], wl.res_dtype)
        self.w = to_dev(inp["weight"], wl.w_dtype)
        quant = wl.out_dtype in ("fp8_e4m3fn", "fp4_e2m1")
        out_cols = wl.hidden // 2 if wl.out_dtype == "fp4_e2m1" else wl.hidden
        self.sets = []
        for i in range(sets):
            parts = parts0 if i == 0 else [p.clone() for p in parts0]
            res = res0 if i == 0 else res0.clone()
            ptrs = (ctypes.c_void_p * len(parts))(*[p.data_ptr() for p in parts])
            out = torch.empty(wl.rows, out_cols, dtype=TORCH_DTYPES[wl.out_dtype], device="cuda")
            sc = (torch.empty(wl.rows, SCALE_BYTES[scale_scheme](wl.hidden), dtype=torch.uint8, device="cuda")
                  if quant else None)
            self.sets.append((parts, ptrs, res, torch.empty_like(res), out, sc))
        self.ts = (torch.tensor([tensor_scale], dtype=torch.float32, device="cuda")
                   if scale_scheme == "nv16" else None)
        self.L = L.lib()
        self.flags = L.make_flags(wl.x_dtype, wl.res_dtype, wl.w_dtype, wl.out_dtype, wl.weight_plus_one,
                                  scale_scheme)
        self.i = 0

    def __call__(self, stream: int) -> None:
        _, ptrs, res, ro, out, sc = self.sets[self.i]
        self.i = (self.i + 1) % len(self.sets)
        wl = self.wl
        st = self.L.rmsnorm_fwd_partials(ptrs, wl.num_partials, res.data_ptr(), self.w.data_ptr(), out.data_ptr(),
                                         ro.data_ptr(), None if sc is None else sc.data_ptr(), None,
                                         None if self.ts is None else self.ts.data_ptr(), wl.rows, wl.hidden, wl.eps,
                                         self.flags, stream)
        if st != 0:
            from residual_add_rmsnorm_rows_amd._lib import check
            check(st)


def partials_metrics(name: str, steps: int, warmup: int, sets: int = 2, out_dtype=None,
                     scale_scheme: str = "row") -> dict:
    from dataclasses import replace

    import workloads as WL

    wl = WL.WORKLOADS[name]
    desc = wl.description
    if out_dtype is not None:
        wl = replace(wl, out_dtype=out_dtype)
        desc = desc.replace("bf16 out", f"{QUANT_TEXT[out_dtype]} out with {SCHEME_TEXT[scale_scheme]}")
    call = PartialsCall(wl, sets, scale_scheme)
    ms = time_stream_loop(call, steps, warmup)
    spread = launch_percentiles(call)
    b = partials_bytes(wl, scale_scheme)
    return {"workload": desc, "out": wl.out_dtype, "scale_scheme": scale_scheme, "us_per_call": round(ms * 1000, 3),
            "algorithmic_bytes": b, "GBps": round(b / (ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "buffer_sets": sets, "warmup": warmup,
            "launch_us": spread}


def partials_decode_metrics(name: str) -> dict:
    """Latency of a decode-sized partial-input call against an empty launch (graph and eager)."""
    import workloads as WL
    import residual_add_rmsnorm_rows_amd as R
    from residual_add_rmsnorm_rows_amd import _lib as L

    wl = WL.WORKLOADS[name]
    call = PartialsCall(wl)
    lib = L.lib()

    def empty(stream):
        lib.rn_launch_empty(stream)

    eager = time_stream_loop(call, 2000, 100) * 1000.0
    eager_empty = time_stream_loop(empty, 2000, 100) * 1000.0
    graph = time_graph_loop(call)
    graph_empty = time_graph_loop(empty)
    sel = R.query_partials_config(wl.rows, wl.hidden, wl.num_partials, x_dtype=wl.x_dtype, res_dtype=wl.res_dtype,
                                  w_dtype=wl.w_dtype, out_dtype=wl.out_dtype, num_cus=0)
    return {
        "workload": wl.description, "rows": wl.rows, "hidden": wl.hidden, "num_partials": wl.num_partials,
        "launch": {"waves_per_row": sel["waves_per_row"], "vecs_per_lane": sel["vecs_per_lane"]},
        "us_per_call_eager": round(eager, 3), "empty_us_per_call_eager": round(eager_empty, 3),
        "ratio_eager": round(eager / eager_empty, 3),
        "us_per_call_graph": round(graph, 3), "empty_us_per_call_graph": round(graph_empty, 3),
        "ratio_graph": round(graph / graph_empty, 3),
        "algorithmic_bytes": partials_bytes(wl),
    }


def act_metrics(steps: int, warmup: int, out_dtype: str = "bf16", scale_scheme: str = "row", sets: int = 2) -> dict:
    """SiLU-and-mul on the 8192 x 14336 workload (bytes: x read once, out and scales written once)."""
    import torch

    import workloads as WL
    from residual_add_rmsnorm_rows_amd import _lib as L
    from workloads.device import TORCH_DTYPES, to_dev

    wl = WL.WORKLOADS["silu_mul_8192x14336"]
    x0 = to_dev(WL.generate_act(wl, seed=0), wl.x_dtype)
    quant = out_dtype in ("fp8_e4m3fn", "fp4_e2m1")
    out_cols = wl.d // 2 if out_dtype == "fp4_e2m1" else wl.d
    sb = SCALE_BYTES[scale_scheme](wl.d) if quant else 0
    bufs = []
    for i in range(sets):
        x = x0 if i == 0 else x0.clone()
        o = torch.empty((wl.rows, out_cols), dtype=TORCH_DTYPES[out_dtype], device="cuda")
        sc = torch.empty((wl.rows, sb), dtype=torch.uint8, device="cuda") if quant else None
        bufs.append((x, o, sc))
    lib = L.lib()
    flags = (L.DTYPE_CODES[wl.x_dtype] << L.RN_FLAGS_X_SHIFT) | (L.DTYPE_CODES[out_dtype] << L.RN_FLAGS_OUT_SHIFT)
    flags |= L.SCALE_SCHEMES[scale_scheme] << L.RN_FLAGS_SCALE_SHIFT
    ts_t = (torch.tensor([NV_TENSOR_SCALE[wl.name]], dtype=torch.float32, device="cuda")
            if scale_scheme == "nv16" else None)
    ts = None if ts_t is None else ts_t.data_ptr()
    state = {"i": 0}

    def call(stream):
        x, o, sc = bufs[state["i"]]
        state["i"] = (state["i"] + 1) % sets
        st = lib.silu_mul_fwd(x.data_ptr(), o.data_ptr(), None if sc is None else sc.data_ptr(), None, ts,
                              wl.rows, wl.d, flags, stream)
        if st != 0:
            L.check(st)

    ms = time_stream_loop(call, steps, warmup)
    spread = launch_percentiles(call)
    size = {"bf16": 2, "f32": 4, "fp8_e4m3fn": 1, "fp4_e2m1": 0.5}
    b = int(wl.rows * (2 * wl.d * size[wl.x_dtype] + wl.d * size[out_dtype] + sb))
    desc = wl.description
    if quant:
        desc = (f"SwiGLU silu(gate) * up, {wl.rows} tokens, merged gate/up projection 2 x {wl.d} {wl.x_dtype} "
                f"~ N(0,1), {QUANT_TEXT[out_dtype]} out with {SCHEME_TEXT[scale_scheme]}")
    return {"workload": desc, "out": out_dtype, "scale_scheme": scale_scheme,
            "us_per_call": round(ms * 1000, 3), "algorithmic_bytes": b,
            "GBps": round(b / (ms * 1e-3) / 1e9, 1), "frac_of_peak": round(b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "buffer_sets": sets, "warmup": warmup, "launch_us": spread}


def qknorm_vs_rows_metrics(steps: int, warmup: int, sets: int = 8) -> dict:
    """The per-head QK-norm kernel against the rows kernel on the same data:
    4096 tokens x 32 heads x 128 as qknorm_fwd, and as rmsnorm_fwd over its
    [131072, 128] row view (no residual, bf16 in and out), timed interleaved.
    The two write the same bits (a GPU parity test checks this)."""
    import torch

    import workloads as WL
    import residual_add_rmsnorm_rows_amd as R
    from residual_add_rmsnorm_rows_amd import _lib as L
    from workloads.device import to_dev

    wl = WL.WORKLOADS["qknorm_4096x32x128"]
    inp = WL.generate_qknorm(wl, seed=0)
    q0 = to_dev(inp["q"].reshape(wl.tokens, -1), wl.dtype)
    w = to_dev(inp["q_weight"], wl.w_dtype)
    bufs = [(q0 if i == 0 else q0.clone(), torch.empty_like(q0)) for i in range(sets)]
    lib = L.lib()
    qflags = L.DTYPE_CODES[wl.dtype] | (L.DTYPE_CODES[wl.w_dtype] << L.RN_FLAGS_W_SHIFT)
    rflags = L.make_flags(wl.dtype, None, wl.w_dtype, wl.dtype, False)
    rows = wl.tokens * wl.num_q_heads
    state = {"i": 0}

    def nxt():
        b = bufs[state["i"]]
        state["i"] = (state["i"] + 1) % sets
        return b

    def qk(stream):
        q, o = nxt()
        st = lib.qknorm_fwd(q.data_ptr(), None, w.data_ptr(), None, o.data_ptr(), None, wl.tokens, wl.num_q_heads,
                            0, wl.head_dim, 0, 0, wl.eps, qflags, stream)
        if st != 0:
            L.check(st)

    def rows_call(stream):
        q, o = nxt()
        st = lib.rmsnorm_fwd(q.data_ptr(), None, w.data_ptr(), o.data_ptr(), None, None, rows, wl.head_dim, wl.eps,
                             rflags, stream)
        if st != 0:
            L.check(st)

    t_qk, t_rows = [], []
    for _ in range(3):
        t_qk.append(time_stream_loop(qk, steps, warmup) * 1000.0)
        t_rows.append(time_stream_loop(rows_call, steps, warmup) * 1000.0)
    b = qknorm_bytes(wl)
    uq, ur = min(t_qk), min(t_rows)
    sel = R.query_config(rows, wl.head_dim, x_dtype=wl.dtype, res_dtype=None, w_dtype=wl.w_dtype,
                         out_dtype=wl.dtype, num_cus=0)
    return {"qknorm_us": round(uq, 3), "qknorm_GBps": round(b / uq / 1e3, 1),
            "rows_kernel_us": round(ur, 3), "rows_kernel_GBps": round(b / ur / 1e3, 1),
            "rows_kernel_launch": f"{sel['waves_per_row']}x{sel['vecs_per_lane']}",
            "rows_over_qknorm_time": round(ur / uq, 3),
            "pages_figure": "2-3x for the specialized QK-norm over a regular RMS-norm kernel (NVIDIA fleet; "
                            "context only)"}


def compact_stream(e: dict) -> dict:
    """The figures of a streaming line kept in the JSON line."""
    out = {"us": e["us_per_call"], "bytes": e["algorithmic_bytes"], "GBps": e["GBps"], "frac": e["frac_of_peak"]}
    if "launch_us" in e:
        out["launch_us_p50"] = e["launch_us"]["p50"]
    if "copy_ceiling" in e:
        out["copy_GBps"] = e["copy_ceiling"]["GBps"]
        out["vs_copy"] = e["copy_ceiling"]["value_over_ceiling"]
    if e.get("traffic_over_algorithmic") is not None:
        out["traffic_ratio"] = e["traffic_over_algorithmic"]
    return out


def compact_decode(e: dict) -> dict:
    """Decode us/call against an empty launch: graph, C-ABI eager (native loop)
    and the package's prepared call (Python loop)."""
    out = {"launch": f"{e['launch']['waves_per_row']}x{e['launch']['vecs_per_lane']}",
           "graph_us": e["us_per_call_graph"], "empty_graph_us": e["empty_us_per_call_graph"],
           "graph_ratio": e["ratio_graph"]}
    c = e.get("c_abi_eager")
    if c and "us_per_call" in c:
        out.update({"c_abi_eager_us": c["us_per_call"], "empty_eager_us": c["empty_us_per_call"],
                    "c_abi_eager_ratio": c["ratio"]})
    if "us_per_call_python_prepared" in e:
        out.update({"python_prepared_us": e["us_per_call_python_prepared"],
                    "python_prepared_ratio": e["ratio_python_prepared"]})
    if "one_wave_per_row" in e:
        out["one_wave_per_row_graph_ratio"] = e["one_wave_per_row"]["ratio_graph"]
    return out


def host_cpu() -> dict:
    """The host's CPU model (from /proc/cpuinfo) and its logical CPU count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "logical_cpus": os.cpu_count()}


def cpu_baseline(wl, budget_s: float = 12.0) -> dict:
    """The oracle as it stands, timed on a bounded sample of the workload's rows."""
    import numpy as np

    import workloads as WL
    from oracle import rownorm as O

    chunk = 64
    inputs = WL.generate_rownorm(wl, seed=0, row_range=(0, chunk))
    X = inputs["x"]
    RES = inputs["residual"]
    W = inputs["weight"]
    done_rows = 0
    t0 = time.perf_counter()
    while True:
        x = O.decode(X, wl.x_dtype)
        res = None if RES is None else O.decode(RES, wl.res_dtype)
        w = O.decode(W, wl.w_dtype)
        ref = O.rmsnorm_rows(x, w, wl.eps, 1.0 if wl.weight_plus_one else 0.0, residual=res,
                             res_dtype=wl.res_dtype)
        if res is not None:
            O.encode(ref["h"], wl.res_dtype)
        O.encode(ref["y"], wl.out_dtype)
        done_rows += chunk
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    b = rownorm_bytes(wl, rows=done_rows)
    return {"value": round(b / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle", "host": host_cpu(),
            "sample": f"{done_rows} rows x {wl.hidden} of the {wl.rows}-row workload "
                      f"({chunk}-row batches, decode + residual add + norm + output rounding, float64 numpy, "
                      f"one thread), {dt:.1f} s"}


def _oracle_worker(args):
    """One process of the parallel CPU baseline: the oracle on its own 64-row
    batch of the workload, repeated for `budget_s` seconds."""
    name, first_row, budget_s = args
    import workloads as WL
    from oracle import rownorm as O

    wl = WL.WORKLOADS[name]
    chunk = 64
    inputs = WL.generate_rownorm(wl, seed=0, row_range=(first_row, first_row + chunk))
    done = 0
    t0 = time.perf_counter()
    while True:
        x = O.decode(inputs["x"], wl.x_dtype)
        res = None if inputs["residual"] is None else O.decode(inputs["residual"], wl.res_dtype)
        ref = O.rmsnorm_rows(x, O.decode(inputs["weight"], wl.w_dtype), wl.eps, 1.0 if wl.weight_plus_one else 0.0,
                             residual=res, res_dtype=wl.res_dtype)
        if res is not None:
            O.encode(ref["h"], wl.res_dtype)
        O.encode(ref["y"], wl.out_dtype)
        done += chunk
        if time.perf_counter() - t0 >= budget_s:
            break
    return done, time.perf_counter() - t0


def host_cores(cap: int = 16) -> int:
    """The host cores this process may run on (its CPU affinity), at most `cap`:
    the GPU machines give one GPU's job a share of 16 CPUs whatever the machine has."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def cpu_baseline_parallel(wl, budget_s: float = 8.0, procs: int = 0) -> dict:
    """The same oracle in one process per host core (`procs`, default every core
    this process may use, up to 16), each on its own rows; the rate is the sum
    of the processes' rates."""
    from concurrent.futures import ProcessPoolExecutor
    import multiprocessing as mp

    n = procs or host_cores()
    with ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn")) as ex:
        parts = list(ex.map(_oracle_worker, [(wl.name, 64 * i, budget_s) for i in range(n)]))
    rate = sum(rownorm_bytes(wl, rows=r) / t for r, t in parts)
    rows = sum(r for r, _ in parts)
    return {"value": round(rate / 1e9, 4), "unit": "GB/s", "cores": n, "kind": "oracle", "host": host_cpu(),
            "sample": f"{rows} rows x {wl.hidden} in {n} processes (each its own 64-row batch, float64 numpy, "
                      f"one thread each), {budget_s:.0f} s"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode latency lines (thousands of tiny launches; for counter runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of 1 GiB (torch copy_), the reference for scaling "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this benchmark runs on one GPU only (--gpus 1); multi-GPU runs are not part "
              "of it.", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("bench.py: --steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import workloads as WL

    # The parallel CPU baseline starts its worker processes before this process
    # touches the GPU (no process is started from one that has initialised it).
    cpu_parallel = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline (oracle), one process per host core ({host_cores()})")
        cpu_parallel = cpu_baseline_parallel(WL.WORKLOADS[MAIN])
    # likewise the native decode-latency driver (its own GPU process, run to completion first)
    native = {}
    if not args.no_secondary and not args.no_decode:
        for name in ("decode_8x1024", "decode_256x4096"):
            log(f"native decode latency {name}")
            native[name] = native_decode_latency(name)

    import torch

    from residual_add_rmsnorm_rows_amd import _lib as L
    import residual_add_rmsnorm_rows_amd as R

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    L.lib()  # fails loudly if the HIP library is not built
    torch.cuda.set_device(0)

    wl = WL.WORKLOADS[MAIN]
    log(f"generating {MAIN}")
    call = RowCall(wl, WL.generate_rownorm(wl, seed=0))
    cfg = R.query_config(wl.rows, wl.hidden, x_dtype=wl.x_dtype, res_dtype=wl.res_dtype, w_dtype=wl.w_dtype,
                         out_dtype=wl.out_dtype, weight_plus_one=wl.weight_plus_one, num_cus=0)
    log(f"timing {MAIN}: warmup {args.warmup}, steps {args.steps}, config {cfg}")
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(args.warmup):
        call(stream)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        call(stream)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    # per-launch spread: each launch bracketed by its own events (after the timed region)
    spread = launch_percentiles(call, args.steps)
    nbytes = rownorm_bytes(wl)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"{MAIN}: {ms * 1000:.1f} us/step, {gbs:.1f} GB/s")
    traffic = read_traffic(MAIN)
    result = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{MAIN}: {wl.description}", "rows": wl.rows, "hidden": wl.hidden,
                   "x": wl.x_dtype, "residual": wl.res_dtype, "weight": wl.w_dtype, "out": wl.out_dtype,
                   "eps": wl.eps, "launch": cfg, "algorithmic_bytes_per_step": nbytes,
                   "library_sha256": library_digest()},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic},
        "launch_us": spread,
    }
    del call
    torch.cuda.empty_cache()
    # practical ceiling in the same run: the library's plain streaming copy
    # moving the same bytes (half read, half written), timed the same way
    half = (nbytes // 2) // 16 * 16
    src = torch.empty(half, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    lib = L.lib()

    def copy(stream):
        st = lib.rn_launch_copy(src.data_ptr(), dst.data_ptr(), half, stream)
        if st != 0:
            L.check(st)

    cms = time_stream_loop(copy, args.steps, args.warmup)
    cgbs = 2 * half / (cms * 1e-3) / 1e9
    log(f"copy ceiling: {cms * 1000:.1f} us, {cgbs:.1f} GB/s")
    result["ceiling"] = {"kernel": "rn_launch_copy: nontemporal 16-byte loads and stores, 8 KiB per workgroup",
                         "bytes_per_launch": 2 * half, "GBps": round(cgbs, 1),
                         "frac_of_peak": round(cgbs / PEAK_HBM_GBS, 4), "value_over_ceiling": round(gbs / cgbs, 4)}
    del src, dst
    torch.cuda.empty_cache()
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration"] = {"bytes_read": n, "bytes_written": n, "launches": 3}
        del src, dst
        torch.cuda.empty_cache()
    if not args.no_secondary:
        sec = {}
        decode = {}
        for name in () if args.no_decode else ("decode_8x1024", "decode_256x4096"):
            log(f"decode {name}")
            d = decode_metrics(name)
            if name in native:
                d["c_abi_eager"] = native[name]
            decode[name] = d
        log("qknorm_4096x32x128")
        sec["qknorm_4096x32x128"] = qknorm_metrics(args.steps * 4, args.warmup)
        log("qknorm_fwd against rmsnorm_fwd on the same 4096 x 32 x 128 heads")
        qk_vs_rows = qknorm_vs_rows_metrics(args.steps * 4, args.warmup)
        log("one GPU's share of the headline step over 8 GPUs (2048 x 8192)")
        sec["prefill_16384x8192_share_of_8"] = stream_metrics(MAIN, args.steps * 4, args.warmup, sets=3, rows=2048)
        log("prefill_fp8_8192x7168")
        sec["prefill_fp8_8192x7168"] = stream_metrics("prefill_fp8_8192x7168", args.steps, args.warmup, sets=3)
        log("block-scaled outputs on the 8192 x 7168 prefill")
        sec["prefill_8192x7168_fp8_group128"] = stream_metrics("prefill_fp8_8192x7168", args.steps, args.warmup,
                                                               sets=3, scale_scheme="group128")
        sec["prefill_8192x7168_mxfp8"] = stream_metrics("prefill_fp8_8192x7168", args.steps, args.warmup, sets=3,
                                                        scale_scheme="mx32")
        sec["prefill_8192x7168_mxfp4"] = stream_metrics("prefill_fp8_8192x7168", args.steps, args.warmup, sets=3,
                                                        out_dtype="fp4_e2m1", scale_scheme="mx32")
        sec["prefill_8192x7168_nvfp4"] = stream_metrics("prefill_fp8_8192x7168", args.steps, args.warmup, sets=3,
                                                        out_dtype="fp4_e2m1", scale_scheme="nv16")
        # the kernels of the next two groups do more arithmetic per byte (exact
        # sums; silu and block scales): the GPU's power management lowers clocks
        # for a few ms once such a load starts, so these lines are timed after a
        # warm-up long enough to reach steady state
        aw = max(args.warmup, POWER_WARMUP)
        log("partials_8x2048x8192")
        sec["partials_8x2048x8192"] = partials_metrics("partials_8x2048x8192", args.steps * 2, aw)
        sec["partials_8x2048x8192_mxfp4"] = partials_metrics("partials_8x2048x8192", args.steps * 2, aw,
                                                             out_dtype="fp4_e2m1", scale_scheme="mx32")
        if not args.no_decode:
            log("partials_decode_8x64x8192")
            decode["partials_decode_8x64x8192"] = partials_decode_metrics("partials_decode_8x64x8192")
        log("silu_mul_8192x14336")
        sec["silu_mul_8192x14336"] = act_metrics(args.steps, aw)
        sec["silu_mul_8192x14336_mxfp8"] = act_metrics(args.steps, aw, "fp8_e4m3fn", "mx32")
        sec["silu_mul_8192x14336_mxfp4"] = act_metrics(args.steps, aw, "fp4_e2m1", "mx32")
        sec["silu_mul_8192x14336_nvfp4"] = act_metrics(args.steps, aw, "fp4_e2m1", "nv16")
        log("copy ceilings at the secondary workloads' sizes")
        for name, sets, steps in (("qknorm_4096x32x128", 8, args.steps * 4), ("prefill_fp8_8192x7168", 3, args.steps),
                                  ("partials_8x2048x8192", 2, args.steps * 2), ("silu_mul_8192x14336", 2, args.steps)):
            c = copy_ceiling(sec[name]["algorithmic_bytes"], sets, steps, args.warmup)
            sec[name]["copy_ceiling"] = {**c, "value_over_ceiling": round(sec[name]["GBps"] / c["GBps"], 4)}
        for name, entry in sec.items():
            if "GBps" in entry:
                attach_traffic(name, entry)
        # decode us/call (the metric's second half) right after the headline
        # figures; the streaming lines in compact form
        if decode:
            result["decode"] = {k: compact_decode(v) for k, v in decode.items()}
        result["secondary"] = {k: compact_stream(v) for k, v in sec.items()}
        result["secondary"]["qknorm_vs_rows_4096x32x128"] = qk_vs_rows
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle), one process")
        one = cpu_baseline(wl)
        if cpu_parallel is not None:
            result["cpu_baseline"] = cpu_parallel
            result["cpu_baseline_1core"] = {k: one[k] for k in ("value", "unit", "cores", "sample")}
        else:
            result["cpu_baseline"] = one
    # a closing summary on stderr (the end of a run's log): headline and decode ratios
    log(f"headline {MAIN}: {result['value']} GB/s = {result['roofline']['frac']:.4f} of 8 TB/s, "
        f"{result['ceiling']['value_over_ceiling']:.3f} of the same-run copy")
    for k, v in result.get("decode", {}).items():
        parts = [f"graph {v['graph_us']} us = {v['graph_ratio']}x empty"]
        if v.get("c_abi_eager_us") is not None:
            parts.append(f"C-ABI eager {v['c_abi_eager_us']} us = {v['c_abi_eager_ratio']}x")
        if v.get("python_prepared_us") is not None:
            parts.append(f"Python prepared {v['python_prepared_us']} us = {v['python_prepared_ratio']}x")
        log(f"decode {k} ({v['launch']}): " + "; ".join(parts))
    order = ["metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
             "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "decode", "ceiling"]
    result = {**{k: result[k] for k in order if k in result}, **{k: v for k, v in result.items() if k not in order}}
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
