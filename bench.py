#!/usr/bin/env python3
"""Benchmark of the low-rank draft LM head on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one draft-head call (the whole hot path: z = Q.h, the
vocabulary-wide score pass with its fused top-k, the merge of the slice
lists, and the exact rescoring of the k candidates with W) on the batch-1
bf16 drafter head: B=1, d=5120, V=151936, r=128, k=32. Inputs are seeded
synthetic tensors already resident in HBM.

Timing: the calls are captured in a HIP graph and replayed (as a serving
loop would run them), bracketed by device synchronisation. The headline is
cache-cold: the calls rotate over enough distinct (Q, P, h) sets that their
bytes exceed twice the 256 MB Infinity Cache, so P streams from HBM. A
single-set ("hot") figure is reported beside it. The dominant kernel (the
score/selection pass) is timed with HIP events recorded around it on its
stream. The full-head baseline (W . h over all V, then top-k) is timed the
same way. The CPU oracle is timed on the host cores on a bounded sample.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "draft-head µs/call & rows/s at V=151936,d=5120,r=128; % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}   # MI355X dense matrix peaks
MALL_BYTES = 256 << 20
BENCH_CONFIG = 2
_CSRC = "rank_lm_head_amd/csrc/"
# The sources each measured kernel is built from: its committed HBM counters
# stay valid while these are unchanged.
KERNEL_SOURCES = {
    name: [_CSRC + f for f in srcs + ("topk.h", "device.h", "launch.h")]
    for name, srcs in (("select_short_kernel", ("kernels_small.hip", "stream.h")),
                       ("select_rows_kernel", ("kernels_small.hip", "stream.h")),
                       ("select_mfma_kernel", ("kernels_mfma.hip",)),
                       ("gemm_sel_kernel", ("kernels_gemm.hip",)), ("strip_sel_kernel", ("kernels_gemm.hip",)),
                       ("draft1_kernel", ("kernels_b1.hip", "merge.h", "stream.h")))
}
B1_MAX_BLOCKS, B1_MAX_ROWS_PER_BLOCK, N_CU = 512, 16 * 64, 256


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2800)
    ap.add_argument("--warmup", type=int, default=280)
    ap.add_argument("--baseline-steps", type=int, default=120)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--config", type=int, default=BENCH_CONFIG,
                    help="workload id (the headline is the batch-1 bf16 drafter head)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, copy a buffer of this many MiB with a plain device copy, so "
                         "that hardware byte counters can be scaled against a known size")
    ap.add_argument("--table", action="store_true",
                    help="instead of the headline: a latency table of the draft-head call over "
                         "B x r x k (and of the full-head baseline over B x k), one JSON object")
    ap.add_argument("--factor", action="store_true",
                    help="instead of the headline: time building P and Q from W (r = 128/256/512, one "
                         "subspace iteration) at V=151936, d=5120, one JSON object")
    ap.add_argument("--peak", action="store_true",
                    help="instead of the headline: the achievable-peak probes (HBM read bandwidth of a "
                         "plain streaming read at P's size and at 1 GiB, bf16 GEMM rate of the vendor "
                         "library), one JSON object")
    ap.add_argument("--draft-only", action="store_true",
                    help="time only the draft-head call (no full-head baseline, vendor GEMM or CPU "
                         "oracle): the run to put under rocprofv3 for the counters of the draft path")
    ap.add_argument("--summarise-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="instead of the headline: turn two rocprofv3 counter_collection.csv files "
                         "(FETCH_SIZE, WRITE_SIZE) of a --draft-only run with --copy-calibration-mib "
                         "into profiles/counters.json entries for --config (keyed by the full kernel "
                         "name) and print a markdown table")
    ap.add_argument("--recall", action="store_true",
                    help="instead of the headline: recall of the full head's top-b inside the "
                         "low-rank top-k for r in 128/256/512, one JSON object")
    return ap.parse_args()


class Hip:
    """The few HIP runtime calls the bench needs beyond torch (events)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        ev = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(ev)) == 0
        return ev

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return float(ms.value)

    def destroy(self, ev) -> None:
        self.lib.hipEventDestroy(ev)


def kernel_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes (read + written) per launch of `kernel` from the committed
    rocprofv3 counter summary (FETCH_SIZE / WRITE_SIZE of a --draft-only run,
    scaled by a copy of known size; written by --summarise-counters), if it
    was taken on the current kernel sources; else None. Entries are keyed by
    the full kernel name: of the instantiations of `kernel` in that run, the
    one that moves the most bytes per launch (the main pass where a kernel
    also runs as a sampling pass)."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path) or kernel not in KERNEL_SOURCES:
        return None
    try:
        recs = json.load(open(path))[workload]
    except Exception:
        return None
    mine = [r for name, r in recs.items() if isinstance(r, dict) and f"lrh::{kernel}<" in name]
    if not mine:
        return None
    rec = max(mine, key=lambda r: r["bytes_per_launch"])
    if rec.get("kernel_hash") != kernel_hash(kernel):
        return None
    return float(rec["bytes_per_launch"])


def summarise_counters(fetch_csv: str, write_csv: str, workload: str, calib_mib: int) -> str:
    """counters.json entries for `workload` from a FETCH_SIZE and a WRITE_SIZE
    rocprofv3 run (counter_collection.csv), scaled so that the calibration
    copy of calib_mib MiB (__amd_rocclr_copyBuffer) reads and writes exactly
    its size; returns a markdown table of the figures."""
    import csv

    def per_kernel(path):
        acc, per_dispatch = {}, {}
        for row in csv.DictReader(open(path)):
            name = row["Kernel_Name"]
            key = (name, row.get("Dispatch_Id") or row.get("Correlation_Id"))
            per_dispatch[key] = per_dispatch.get(key, 0.0) + float(row["Counter_Value"])
        for (name, _), v in per_dispatch.items():
            a = acc.setdefault(name, [0, 0.0, 0.0])
            a[0] += 1
            a[1] += v
            a[2] = max(a[2], v)
        return acc

    fetch, write = per_kernel(fetch_csv), per_kernel(write_csv)
    cal = calib_mib * 1024.0
    # the calibration copy is the largest device copy of the run (the others
    # are the inputs' uploads)
    cf = [v[2] for n, v in fetch.items() if "copyBuffer" in n]
    cw = [v[2] for n, v in write.items() if "copyBuffer" in n]
    f_scale = cal / cf[0] if cf and cf[0] > 0 else 1.0
    w_scale = cal / cw[0] if cw and cw[0] > 0 else 1.0
    path = os.path.join(ROOT, "profiles", "counters.json")
    allrec = json.load(open(path)) if os.path.exists(path) else {}
    recs = {}
    lines = [f"Calibration: a {calib_mib} MiB device copy; FETCH_SIZE x {f_scale:.3f}, WRITE_SIZE x {w_scale:.3f}.",
             "", "| Kernel | Dispatches | read MB / launch | written MB / launch |", "|---|---|---|---|"]
    for name, (nd, kib, _) in fetch.items():
        if "copyBuffer" in name:
            continue
        wk = write.get(name, (nd, 0.0, 0.0))[1]
        rd = kib / nd * 1024 * f_scale
        wr = wk / nd * 1024 * w_scale
        rec = {"dispatches": nd, "read_bytes": rd, "written_bytes": wr, "bytes_per_launch": rd + wr}
        for base in KERNEL_SOURCES:
            if f"lrh::{base}<" in name:
                rec["kernel_hash"] = kernel_hash(base)
        recs[name] = rec
        lines.append(f"| `{name[:110]}` | {nd} | {rd / 1e6:.3f} | {wr / 1e6:.3f} |")
    allrec[workload] = recs
    with open(path, "w") as f:
        json.dump(allrec, f, indent=1, sort_keys=True)
    return "\n".join(lines)


def timed_graph_replays(torch, graph, n_replays: int) -> float:
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_replays):
        graph.replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def capture(torch, fn, n: int):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(n):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


def event_timed(torch, hip, heads, fn, n: int) -> float:
    """Mean duration (s) of the score-pass kernel over n eager calls, timed by
    HIP events attached to its dispatch (start and end of that kernel, on its
    stream). A device-side delay is queued first so the host runs ahead."""
    evs = [(hip.event(), hip.event()) for _ in range(n)]
    torch.cuda.synchronize()
    torch.cuda._sleep(400_000_000)
    for i in range(n):
        heads[i % len(heads)].set_stage_events(evs[i][0], evs[i][1])
        fn(i)
    for h in heads:
        h.set_stage_events(None, None)
    torch.cuda.synchronize()
    ms = [hip.elapsed_ms(a, b) for a, b in evs]
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)
    ms.sort()
    return sum(ms) / len(ms) * 1e-3


def host_model() -> str:
    """The host CPU as lscpu names it (model, sockets x cores x threads)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        f = dict(ln.split(":", 1) for ln in out.splitlines() if ":" in ln)
        g = lambda k: f.get(k, "?").strip()
        return (f"{g('Model name')}, {g('Socket(s)')} socket(s) x {g('Core(s) per socket')} cores x "
                f"{g('Thread(s) per core')} threads, {g('CPU(s)')} logical CPUs")
    except Exception:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    return "unknown"


def cpu_baseline(inp: dict, seconds: float, max_rows: int = 64) -> dict:
    """The float64 oracle (steps O1-O4 of the method) on the host cores: with
    all the BLAS threads NumPy uses, and with one thread. Batches above
    max_rows rows are sampled (their first max_rows rows, whose cost per row
    is that of the whole batch: every row is scored, selected and rescored
    on its own), so that each leg stays within its time budget."""
    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
        threads = 1
    cfg = inp["cfg"]
    model = host_model()
    rows = min(cfg.B, max_rows)
    H = inp["H"][:rows]
    what = (f"full draft-head calls of the benchmark workload (B={cfg.B})" if rows == cfg.B else
            f"draft-head calls on the first {rows} of the benchmark workload's {cfg.B} rows")

    def rate(limit_s):
        n, t0 = 0, time.perf_counter()
        while True:
            oracle.lowrank_head(inp["Q"], inp["P"], inp["W"], H, cfg.k, cfg.dtype)
            n += 1
            el = time.perf_counter() - t0
            if el >= limit_s:
                return n, el

    n, el = rate(seconds)
    one = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            n1, el1 = rate(seconds / 2)
        one = {"value": n1 * rows / el1, "unit": "rows/s", "cores": 1,
               "sample": f"{n1} calls in {el1:.1f} s, BLAS limited to one thread"}
    return {"value": n * rows / el, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} {what} in {el:.1f} s (float64 NumPy, BLAS threads {threads}, host: {model})",
            "one_thread": one, "host": model, "us_per_call": el / n * 1e6 * cfg.B / rows}


# ------------------------------------------------ achievable peaks
def probe_hbm_read(torch, dev, nbytes: int, rotate: int, reps: int) -> float:
    """Achievable HBM read bandwidth (GB/s) of a plain streaming read
    (csrc/probe_read.hip) over `rotate` distinct buffers of nbytes each, read
    in turn (cache-cold when rotate * nbytes is well past the 256 MB
    Infinity Cache), timed by HIP events around each launch."""
    import ctypes as C
    lib = C.CDLL(os.path.join(ROOT, "rank_lm_head_amd", "libprobe.so"))
    lib.probe_read.argtypes = [C.c_void_p, C.c_size_t, C.c_uint32, C.c_void_p, C.c_int, C.c_void_p]
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(i + 1) for i in range(rotate)]
    sink = torch.zeros(4, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    best = 0.0
    for blocks in (N_CU * 2, N_CU * 4, N_CU * 8):
        for i in range(rotate):   # warm-up
            assert lib.probe_read(bufs[i].data_ptr(), nbytes, 0x9E3779B9, sink.data_ptr(), blocks, stream) == 0
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for j in range(reps):
            evs[j][0].record()
            lib.probe_read(bufs[j % rotate].data_ptr(), nbytes, 0x9E3779B9, sink.data_ptr(), blocks, stream)
            evs[j][1].record()
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in evs)
        best = max(best, nbytes / (ms[len(ms) // 2] * 1e-3) / 1e9)
    del bufs
    torch.cuda.empty_cache()
    return best


def probe_mfma_bf16(torch, dev, n: int = 8192, reps: int = 20) -> float:
    """Achievable dense bf16 matrix rate (TFLOP/s): the vendor library's
    (hipBLASLt, through torch.matmul) n x n x n product."""
    a = torch.randn(n, n, device=dev).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev).to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    return 2.0 * n ** 3 / (e0.elapsed_time(e1) / reps * 1e-3) / 1e12


def peak_probes(torch, dev) -> dict:
    p_bytes = 151936 * 128 * 2 // 16 * 16
    rot = math.ceil(2 * MALL_BYTES / p_bytes)
    return {"hbm_read_gbs": {f"{p_bytes} B x {rot} rotating buffers (P of the headline head, cold)":
                             probe_hbm_read(torch, dev, p_bytes, rot, 140),
                             "1 GiB": probe_hbm_read(torch, dev, 1 << 30, 1, 12)},
            "mfma_bf16_tflops": {"8192^3 torch.matmul (hipBLASLt)": probe_mfma_bf16(torch, dev)},
            "spec": {"hbm_gbs": HBM_PEAK_GBS, "mfma_tflops": MFMA_PEAK_TFLOPS}}


# ------------------------------------------------ latency table and recall
# Synthetic heads for the sweeps, generated on the device with torch's
# seeded generator in the recipe of the workloads: Q, P and E with standard
# deviation 1/sqrt(d), W = P.Q + 0.1 E rounded once to bf16, hidden rows
# RMS-normalised. (The headline and the parity tests use the numpy
# generator of gen/; the sweeps need many shapes quickly.)
TABLE_V, TABLE_D = 151936, 5120
TABLE_B = (1, 4, 8, 16, 64, 256, 2048)
TABLE_R = (128, 256, 512)
TABLE_K = (8, 32, 64)


def synthetic_head(torch, dev, V, d, r, seed, with_w=True):
    g = torch.Generator(device=dev).manual_seed(seed)
    sd = 1.0 / math.sqrt(d)
    Q = (torch.randn(r, d, generator=g, device=dev) * sd).to(torch.bfloat16)
    P = (torch.randn(V, r, generator=g, device=dev) * sd).to(torch.bfloat16)
    if not with_w:
        return Q, P, None
    W = torch.empty(V, d, dtype=torch.bfloat16, device=dev)
    Qf = Q.float()
    for c0 in range(0, V, 16384):
        c1 = min(V, c0 + 16384)
        E = torch.randn(c1 - c0, d, generator=g, device=dev) * sd
        W[c0:c1] = (P[c0:c1].float() @ Qf + 0.1 * E).to(torch.bfloat16)
    return Q, P, W


def synthetic_rows(torch, dev, B, d, seed):
    g = torch.Generator(device=dev).manual_seed(seed)
    h = torch.randn(B, d, generator=g, device=dev)
    return (h / h.pow(2).mean(dim=1, keepdim=True).sqrt()).to(torch.bfloat16)


def latency_table(torch, lr, dev, steps: int) -> dict:
    """Draft-head call latency (cache-cold graph replay, as the headline) for
    every (B, r, k) of the grid, and the full-head baseline for every (B, k)."""
    rows, full = [], []
    for r in TABLE_R:
        Q0, P0, W = synthetic_head(torch, dev, TABLE_V, TABLE_D, r, seed=7000 + r)
        R = max(1, math.ceil(2 * MALL_BYTES / ((r * TABLE_D + TABLE_V * r) * 2)))
        sets = [(Q0, P0)] + [synthetic_head(torch, dev, TABLE_V, TABLE_D, r, 7000 + r + 97 * i, False)[:2]
                             for i in range(1, R)]
        for B in TABLE_B:
            Hs = [synthetic_rows(torch, dev, B, TABLE_D, 9000 + 31 * i + B) for i in range(R)]
            for k in TABLE_K:
                ws = torch.empty(lr.load().lrhead_workspace_bytes(lr.BF16, TABLE_V, TABLE_D, r, B, k),
                                 dtype=torch.uint8, device=dev)
                heads = [lr.Head(Q, P, W, B_max=B, k_max=k, workspace=ws) for Q, P in sets]
                out = (torch.empty((B, k), dtype=torch.int32, device=dev),
                       torch.empty((B, k), dtype=torch.float32, device=dev),
                       torch.empty((B, k), dtype=torch.float32, device=dev))
                g = capture(torch, lambda i: heads[i % R].draft(Hs[i % R], k, out=out), R)
                n = max(1, min(steps, int(4e5 // (B * 2 + 20))) // R)
                g.replay()
                us = timed_graph_replays(torch, g, n) / (n * R) * 1e6
                rows.append({"B": B, "r": r, "k": k, "us_per_call": round(us, 2),
                             "rows_per_s": round(B / (us * 1e-6), 1)})
                if r == TABLE_R[0]:
                    fo = (out[0], out[2])
                    gf = capture(torch, lambda i: heads[0].full_topk(Hs[0], k, out=fo), 2)
                    gf.replay()
                    nf = max(1, min(60, int(2e4 // (B + 10))))
                    usf = timed_graph_replays(torch, gf, nf) / (nf * 2) * 1e6
                    full.append({"B": B, "k": k, "us_per_call": round(usf, 2)})
                for h in heads:
                    h.close()
                del heads, ws, g
            print(f"[table] r={r} B={B}: {[x['us_per_call'] for x in rows[-len(TABLE_K):]]}", file=sys.stderr,
                  flush=True)
        del sets, W
        torch.cuda.empty_cache()
    return {"table": "draft-head call latency, cache-cold graph replay", "V": TABLE_V, "d": TABLE_D,
            "dtype": "bf16", "data": "synthetic (torch generator, workload recipe)",
            "draft_head": rows, "full_head_baseline": full}


def recall_sweep(torch, lr, dev, rows: int = 256) -> dict:
    """Recall of the full head's top-b inside the low-rank top-k, on the heads
    of gen/ (the workload recipe: r = 128 and r = 512 are the batch-1
    configurations, r = 256 the same recipe, each with `rows` i.i.d. rows):
    the share of each row's b best full-head tokens (fullhead_topk, exact
    logits over all V) among its k low-rank candidates (lrhead_candidates),
    averaged over rows. The GPU tests check this table against the oracle's
    own lists, at small heads and at these shapes."""
    import numpy as np
    import gen

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    out = []
    for r in TABLE_R:
        if r == 128:
            inp = gen.make(2, B=rows)
        elif r == 512:
            inp = gen.make(3, B=rows)
        else:
            inp = gen.make_custom(TABLE_V, TABLE_D, r, rows, "bf16", seed=r)
        Q, P, W, H = (to_dev(inp[x]) for x in ("Q", "P", "W", "H"))
        head = lr.Head(Q, P, W, B_max=rows, k_max=64)
        cidx, _ = head.candidates(H, 64)
        fidx, _ = head.full_topk(H, 8)
        c = cidx.cpu().numpy()
        f = fidx.cpu().numpy()
        for b in (1, 4, 8):
            for k in (8, 16, 32, 64):
                hit = sum(len(set(f[i, :b].tolist()) & set(c[i, :k].tolist())) for i in range(rows))
                out.append({"r": r, "b": b, "k": k, "recall": round(hit / (b * rows), 4)})
        head.close()
        del head, Q, P, W, H, inp
        torch.cuda.empty_cache()
    return {"recall": "share of the full head's top-b found in the low-rank top-k", "V": TABLE_V,
            "d": TABLE_D, "rows": rows, "heads": "gen/: W = round(P.Q + 0.1 E), i.i.d. RMS-normalised rows",
            "data": "synthetic", "results": out}


def factor_timing(torch, lr, dev, reps: int = 3) -> dict:
    """Wall time of lrhead_factor (one subspace iteration) per r, with the
    work of its four W-sized products (W.Omega, W^T.Y, W.Z, W^T.Y: 2*V*d*r
    flops each) over the whole build as the rate, against the bf16 matrix-core
    peak the products run on (each with the fp32 panel as two bf16 halves,
    so twice those flops), and the relative error of P.Q on every 97th row."""
    out = []
    for r in TABLE_R:
        _, _, W = synthetic_head(torch, dev, TABLE_V, TABLE_D, r, seed=7000 + r)
        omega = torch.randn(TABLE_D, r, generator=torch.Generator(device=dev).manual_seed(r), device=dev)
        P, Q = lr.factor(W, r, omega, 1)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            P, Q = lr.factor(W, r, omega, 1)
        torch.cuda.synchronize()
        s_per = (time.perf_counter() - t0) / reps
        big = 4 * 2.0 * TABLE_V * TABLE_D * r
        rows = torch.arange(0, TABLE_V, 97, device=dev)
        Wf = W[rows].float()
        rel = float(torch.linalg.norm(Wf - P[rows].float() @ Q.float()) / torch.linalg.norm(Wf))
        out.append({"r": r, "q": 1, "ms": round(s_per * 1e3, 2),
                    "w_products_tflops": round(big / s_per / 1e12, 2),
                    "mfma_frac": round(big / s_per / (MFMA_PEAK_TFLOPS["bf16"] * 1e12), 4),
                    "rel_error": round(rel, 5)})
        del W, P, Q
        torch.cuda.empty_cache()
    return {"factor": "P, Q from W by a randomized range finder, one subspace iteration", "V": TABLE_V,
            "d": TABLE_D, "peak": "bf16 matrix cores 2500 TFLOP/s (W products on the whole build's time)",
            "data": "synthetic", "results": out}


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py measures one GPU: the low-rank head path here is built and "
                                   "timed on a single MI355X, with no collectives; the multi-GPU sharding "
                                   "is a design note only. Run with --gpus 1."}), flush=True)
        return 2
    if args.summarise_counters:
        print(summarise_counters(*args.summarise_counters, f"c{args.config}", args.copy_calibration_mib or 256))
        return 0
    if args.table or args.recall or args.factor or args.peak:
        import torch
        import rank_lm_head_amd as lr
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        if args.table:
            res = latency_table(torch, lr, dev, args.steps)
        elif args.recall:
            res = recall_sweep(torch, lr, dev)
        elif args.peak:
            res = peak_probes(torch, dev)
        else:
            res = factor_timing(torch, lr, dev)
        print(json.dumps(res), flush=True)
        return 0

    import numpy as np
    import torch

    import gen
    import rank_lm_head_amd as lr

    cid = args.config
    cfg = gen.CONFIGS[cid]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    s = 2 if cfg.dtype == "bf16" else 4

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    base = gen.make(cid)
    lowrank_bytes = (cfg.r * cfg.d + cfg.V * cfg.r) * s
    R = max(1, math.ceil(2 * MALL_BYTES / lowrank_bytes))
    sets = [base] + [gen.make_lowrank_set(cid, i) for i in range(1, R)]
    W = to_dev(base["W"])
    dsets = [{x: to_dev(st[x]) for x in ("Q", "P", "H")} for st in sets]
    ws_bytes = lr.load().lrhead_workspace_bytes(lr.BF16 if cfg.dtype == "bf16" else lr.FP32,
                                                cfg.V, cfg.d, cfg.r, cfg.B, cfg.k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    heads = [lr.Head(d["Q"], d["P"], W, B_max=cfg.B, k_max=cfg.k, workspace=ws) for d in dsets]
    out = (torch.empty((cfg.B, cfg.k), dtype=torch.int32, device=dev),
           torch.empty((cfg.B, cfg.k), dtype=torch.float32, device=dev),
           torch.empty((cfg.B, cfg.k), dtype=torch.float32, device=dev))
    fout = (torch.empty((cfg.B, cfg.k), dtype=torch.int32, device=dev),
            torch.empty((cfg.B, cfg.k), dtype=torch.float32, device=dev))

    def cold(i):
        heads[i % R].draft(dsets[i % R]["H"], cfg.k, out=out)

    def hot(i):
        heads[0].draft(dsets[0]["H"], cfg.k, out=out)

    def full(i):
        heads[0].full_topk(dsets[0]["H"], cfg.k, out=fout)

    hip = Hip()
    K = max(R, (args.steps + R - 1) // R * R)
    Wm = (args.warmup + R - 1) // R * R

    g_cold = capture(torch, cold, R)
    g_hot = capture(torch, hot, R)
    for _ in range(Wm // R):
        g_cold.replay()
    t_cold = timed_graph_replays(torch, g_cold, K // R)
    for _ in range(Wm // R):
        g_hot.replay()
    t_hot = timed_graph_replays(torch, g_hot, K // R)
    us_cold = t_cold / K * 1e6
    us_hot = t_hot / K * 1e6
    # spread of the cold figure: 7 more trials of about K/7 calls each,
    # outside the timed region above
    n_tr = max(1, (K // 7) // R)
    trials = sorted(timed_graph_replays(torch, g_cold, n_tr) / (n_tr * R) * 1e6 for _ in range(7))
    sel_s = event_timed(torch, hip, heads, cold, min(K, 1400))

    # distinct W rows gathered by the last call of the cold loop
    idx_last = out[0].cpu().numpy()
    U = int(np.unique(idx_last).size)

    # full-head baseline (and the vendor GEMM's rate beside it)
    us_full = full_sel_s = None
    vendor = None
    if not args.draft_only:
        KB = max(1, args.baseline_steps)
        g_full = capture(torch, full, 4)
        for _ in range(2):
            g_full.replay()
        t_full = timed_graph_replays(torch, g_full, (KB + 3) // 4)
        us_full = t_full / ((KB + 3) // 4 * 4) * 1e6
        full_sel_s = event_timed(torch, hip, heads[:1], full, min(KB, 200))

        # vendor context: the library GEMM (hipBLASLt through torch) for all V
        # logits of the full head on the same rows, without any selection
        vendor = None
        if cfg.dtype == "bf16":
            Hb = dsets[0]["H"]
            lin = torch.nn.functional.linear
            for _ in range(2):
                lin(Hb, W)
            torch.cuda.synchronize()
            reps = max(2, min(50, int(2e5 // max(1.0, us_full))))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                lin(Hb, W)
            e1.record()
            torch.cuda.synchronize()
            v_us = e0.elapsed_time(e1) / reps * 1e3
            vendor = {"op": "torch.nn.functional.linear(H, W): all V logits of the full head, bf16 out, no selection",
                      "us_per_call": v_us, "tflops": 2.0 * cfg.B * cfg.V * cfg.d / v_us / 1e6,
                      "hbm_frac": (cfg.V * cfg.d * s + cfg.B * cfg.d * s + cfg.B * cfg.V * s) / (v_us * 1e-6)
                                  / (HBM_PEAK_GBS * 1e9)}

    # roofline of the dominant kernel. Algorithmic work per launch of the
    # vocabulary score pass: every P row once (V units of r*s bytes) plus the
    # B rows of z, and 2*B*r flops per vocabulary row. One row of bf16 runs
    # the whole call after the down-projection in one kernel (draft1_kernel:
    # scores, selection, merge and rescoring), whose bytes add the k rows of
    # W it gathers (U distinct) and h. Other small batches stream P once
    # (HBM-bound); row batches run the matrix-core GEMM, bound by
    # whichever of HBM and MFMA its arithmetic intensity points to.
    sel_bytes = cfg.V * cfg.r * s + cfg.B * cfg.r * s
    sel_flops = 2.0 * cfg.B * cfg.V * cfg.r
    pow2_r = cfg.r in (8, 16, 32, 64, 128, 256, 512)
    small = cfg.dtype == "bf16" and cfg.B <= 8 and pow2_r
    n_b1 = max(1, min((cfg.V + 63) // 64, N_CU, B1_MAX_BLOCKS))
    one_row = cfg.dtype == "bf16" and cfg.B == 1 and pow2_r and (cfg.V + n_b1 - 1) // n_b1 <= B1_MAX_ROWS_PER_BLOCK
    rows = cfg.dtype == "bf16" and 5 <= cfg.B <= 64 and cfg.r in (32, 64, 128, 256, 512) and cfg.V <= 512 * 512
    batch = cfg.dtype == "bf16" and cfg.B > 4 and not small and not rows
    if batch and cfg.r <= 256 and cfg.B > 128:
        sel_kernel, what = "strip_sel_kernel", "main pass: scores of all rows, flagged above the sampled bound"
    elif batch:
        sel_kernel, what = "gemm_sel_kernel", "main GEMM pass: scores of all rows, flagged above the sampled bound"
    elif one_row:
        sel_kernel, what = "draft1_kernel", "score stream + per-slice top-k + merge + rescoring of the winners"
        sel_bytes += (U + 1) * cfg.d * s + cfg.k * 12
        sel_flops += 2.0 * cfg.k * cfg.d
    elif rows:
        sel_kernel, what = "select_rows_kernel", "matrix-core score pass + per-slice best 4 kept in registers"
    elif small:
        sel_kernel, what = "select_short_kernel", "score pass + per-slice top-k"
    else:
        sel_kernel, what = "select_mfma_kernel", "score pass + per-slice top-k"
    peak_flops = MFMA_PEAK_TFLOPS[cfg.dtype] * 1e12
    mfma_bound = sel_flops / sel_bytes > peak_flops / (HBM_PEAK_GBS * 1e9)
    traffic = traffic_from_profiles(sel_kernel, f"c{cid}")
    if mfma_bound:
        ach = probe_mfma_bf16(torch, dev) if cfg.dtype == "bf16" else None
        roof = {"bound": "mfma", "kernel": f"{sel_kernel} ({what})",
                "achieved": sel_flops / sel_s / 1e12, "peak": peak_flops / 1e12, "unit": "TFLOP/s",
                "frac": sel_flops / sel_s / peak_flops, "traffic": traffic,
                "us_per_launch": sel_s * 1e6, "flops_per_launch": sel_flops, "bytes_per_launch": sel_bytes}
        if ach:
            roof["achievable"] = {"peak": ach, "frac": sel_flops / sel_s / 1e12 / ach,
                                  "probe": "8192^3 bf16 torch.matmul (hipBLASLt)"}
    else:
        ach = probe_hbm_read(torch, dev, (sel_bytes // 16) * 16, max(1, math.ceil(2 * MALL_BYTES / sel_bytes)), 140)
        roof = {"bound": "hbm", "kernel": f"{sel_kernel} ({what})",
                "achieved": sel_bytes / sel_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": sel_bytes / sel_s / (HBM_PEAK_GBS * 1e9), "traffic": traffic,
                "us_per_launch": sel_s * 1e6, "bytes_per_launch": sel_bytes,
                "achievable": {"peak": ach, "frac": sel_bytes / sel_s / 1e9 / ach,
                               "probe": "plain streaming read of the same bytes, cold (csrc/probe_read.hip)"}}
    call_bytes = (cfg.r * cfg.d + cfg.V * cfg.r + cfg.B * cfg.d + U * cfg.d) * s + cfg.B * cfg.k * 12
    call_flops = 2.0 * cfg.B * (cfg.r * cfg.d + cfg.V * cfg.r + cfg.k * cfg.d)
    full_bytes = cfg.V * cfg.d * s + cfg.B * cfg.d * s
    line = {
        "metric": METRIC,
        "value": cfg.B / (us_cold * 1e-6),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": us_cold / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: B={cfg.B}, d={cfg.d}, V={cfg.V}, r={cfg.r}, k={cfg.k}, {cfg.dtype}",
                   "B": cfg.B, "d": cfg.d, "V": cfg.V, "r": cfg.r, "k": cfg.k,
                   "cache": f"cold: {R} rotating (Q, P, h) sets, {R * lowrank_bytes / 2**20:.0f} MiB",
                   "launch": "HIP graph replay"},
        "us_per_call": us_cold,
        "us_per_call_trials": {"n": 7, "calls_each": n_tr * R, "median": trials[3], "min": trials[0],
                               "max": trials[-1]},
        "us_per_call_hot": us_hot,
        "call_hbm_frac": call_bytes / (us_cold * 1e-6) / (HBM_PEAK_GBS * 1e9),
        "call_bytes": call_bytes,
        "call_flops": call_flops,
        "distinct_W_rows": U,
        "roofline": roof,
    }
    if us_full is not None:
        line["full_head"] = {"us_per_call": us_full, "speedup_of_draft_head": us_full / us_cold,
                             "select_us_per_launch": full_sel_s * 1e6,
                             "hbm_frac": full_bytes / (full_sel_s) / (HBM_PEAK_GBS * 1e9),
                             "mfma_frac": 2.0 * cfg.B * cfg.V * cfg.d / full_sel_s / peak_flops,
                             "vendor_gemm_context": vendor}
        if vendor:
            line["full_head"]["speedup_of_draft_head_vs_vendor_gemm"] = vendor["us_per_call"] / us_cold
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = n
        del src, dst
    if not args.no_cpu_baseline and not args.draft_only:
        line["cpu_baseline"] = cpu_baseline(base, args.cpu_seconds)
    for h in heads:
        h.close()
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
