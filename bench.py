"""Benchmark of the MosaicQuant path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole path over one batch of synthetic input, every
step on the GPU: the diagonal-Hessian estimate of the batch, Delta-score top-K
block selection, packing of the 4-bit base and residual, per-token activation
quantization and the fused W4A4 + sparse-residual GEMM. Inputs are resident in
HBM before the timed region; consecutive steps read different copies of them
(more than 600 MB in total) so the 256 MB Infinity Cache cannot serve them.

Printed on stdout: one JSON line. `value` is the step's algorithmic HBM bytes
per second, the step timed as one replay of a HIP graph of `steps` steps;
`roofline` is the call that takes most of the step, timed alone in its own graph
with HIP events on the launch stream; `gemm` is the fused kernel alone (the metric's
TOPS and GB/s), timed over rotated packed-weight copies, beside the dense-only
kernel and the separate-kernel alternative; `cpu_baseline` is the CPU oracle on
the host, one core, on the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "fused W4A4+10% residual GEMM: TOPS & HBM GB/s (% roofline); overhead vs dense"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0         # MI355X dense int8 MFMA
ROTATE_BYTES = 640 << 20        # > 2 x (256 MB Infinity Cache + 8 x 4 MB L2)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------- algorithmic work
def gemm_bytes(cfg, nnz, residual=True, y_bytes=2):
    M, N, K, G = cfg.M, cfg.N, cfg.K, cfg.K // cfg.group
    b = N * K // 2 + N * G * 2 + M * K // 2 + M * 4 + M * N * y_bytes
    if residual:
        b += nnz * cfg.bn * cfg.bk // 2 + nnz * 4 + (N // cfg.bn + 1) * 4
    return b


def gemm_ops(cfg, nnz, residual=True):
    return 2 * cfg.M * (cfg.N * cfg.K + (nnz * cfg.bn * cfg.bk if residual else 0))


def step_bytes(cfg, nnz, x_bytes):
    """Bytes each call of the step must move at minimum (read inputs once, write outputs once)."""
    M, N, K, G = cfg.M, cfg.N, cfg.K, cfg.K // cfg.group
    nb = (N // cfg.bn) * (K // cfg.bk)
    csr = (N // cfg.bn + 1) * 4 + nnz * 4
    return {
        "hessian_diag": M * K * x_bytes + K * 4,
        "select_blocks": N * K * 4 + K * 4 + nb * 8 + csr,
        "pack_weights": N * K * 4 + csr + N * K // 2 + N * G * 2 + nnz * cfg.bn * cfg.bk // 2,
        "quantize_act": M * K * x_bytes + M * K // 2 + M * 4,
        "gemm_w4a4_residual": gemm_bytes(cfg, nnz),
    }


# --------------------------------------------------------------------------- GPU legs
def _graph_time_us(torch, fn, n_calls, reps=5):
    """Median per-call time of `n_calls` back-to-back calls of fn(i) captured in one
    HIP graph (HIP events around each replay, on the capturing stream)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n_calls):
            fn(i)
    times = []
    for _ in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / n_calls)
    del graph
    return float(np.median(times[1:]))


def bench_step(mq, torch, cfg, inp, k_blocks, steps, warmup):
    """The whole path, step after step, over rotating input copies. The timed
    region is one replay of a HIP graph holding exactly `steps` steps (launch
    overhead of the Python binding excluded); each call is also timed alone."""
    dev = torch.device("cuda:0")
    x_bytes = 2 if inp.X_bits is not None else 4
    per_copy = cfg.N * cfg.K * 4 + cfg.M * cfg.K * x_bytes
    copies = max(2, min(64, -(-ROTATE_BYTES // per_copy)))
    if inp.X_bits is not None:
        x0 = torch.from_numpy(inp.X_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        x0 = torch.from_numpy(inp.X).to(dev)
    w0 = torch.from_numpy(inp.W).to(dev)
    xs = [x0.clone() for _ in range(copies)]
    ws = [w0.clone() for _ in range(copies)]
    del x0, w0
    N, K, M, bn = cfg.N, cfg.K, cfg.M, cfg.bn
    G = K // 128
    nb = (N // bn) * (K // cfg.bk)
    h = torch.empty(K, dtype=torch.float32, device=dev)
    sel_out = (torch.empty(N // bn + 1, dtype=torch.int32, device=dev),
               torch.empty(max(k_blocks, 1), dtype=torch.int32, device=dev),
               torch.empty(nb, dtype=torch.float64, device=dev))
    sel_ws = mq.select_workspace(N, K, bn=bn, device=dev)
    pack_out = (torch.empty((N // 16, G, 1024), dtype=torch.uint8, device=dev),
                torch.empty((N // 16, (G + 3) // 4, 16, 4), dtype=torch.int16, device=dev),
                torch.empty((max(k_blocks, 1), bn, 32), dtype=torch.uint8, device=dev))
    xq = torch.empty((G, M, 64), dtype=torch.uint8, device=dev)
    sx = torch.empty(M, dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    gemm_ws = mq.workspace(M, N, K, device=dev)
    log(f"[bench] step workload {cfg.name}: M={M} K={K} N={N} bn={bn} k_blocks={k_blocks}, "
        f"{copies} input copies ({copies * per_copy / 2**20:.0f} MiB)")

    def hess(i):
        mq.hessian_diag(xs[i % copies], out=h)

    def select(i):
        return mq.select_blocks(ws[i % copies], h, k_blocks, bn=bn, out=sel_out, workspace=sel_ws)

    def pack(i):
        rp, ci = sel_out[0], sel_out[1][:k_blocks]
        return mq.pack_weights(ws[i % copies], rp, ci, bn=bn, out=pack_out)

    def quant(i):
        mq.quantize_act(xs[i % copies], xq=xq, sx=sx)

    def gemm(i):
        wq, sw, rq = pack_out[0], pack_out[1], pack_out[2][:k_blocks]
        mq.gemm_w4a4_residual(xq, sx, wq, sw, sel_out[0], sel_out[1][:k_blocks], rq, K, bn=bn, y=y,
                              workspace=gemm_ws)

    def one_step(i):
        hess(i)
        select(i)
        pack(i)
        quant(i)
        gemm(i)

    for i in range(warmup):
        one_step(i)
    torch.cuda.synchronize()
    # eager steps (Python launch path included), for reference
    t0 = time.perf_counter()
    for i in range(steps):
        one_step(i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / steps

    # the timed region: one replay of a graph of exactly `steps` steps
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one_step(0)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            one_step(i)
    graph.replay()                       # untimed replay (first-replay setup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    gpu_ms = e0.elapsed_time(e1) / steps
    del graph

    # each call alone, back to back over the copies, in its own graph
    calls = 2 * copies
    us = {"hessian_diag": _graph_time_us(torch, hess, calls),
          "select_blocks": _graph_time_us(torch, select, calls),
          "pack_weights": _graph_time_us(torch, pack, calls),
          "quantize_act": _graph_time_us(torch, quant, calls),
          "gemm_w4a4_residual": _graph_time_us(torch, gemm, calls)}
    for n, v in us.items():
        log(f"[bench] {n}: {v:.3f} us per call")
    log(f"[bench] step: {gpu_ms * 1e3:.2f} us (graph), {eager_ms * 1e3:.2f} us (eager Python launches)")
    return dict(gpu_ms=gpu_ms, wall_ms=wall_ms, eager_ms=eager_ms, us=us, copies=copies)


def bench_gemm(mq, torch, cfg, inp, k_blocks, calls):
    """Fused, dense-only and separate-kernel GEMM over rotated packed-weight copies,
    each in its own HIP graph of `calls` back-to-back calls; every variant's graph
    output is checked against its eager call."""
    dev = torch.device("cuda:0")
    if inp.X_bits is not None:
        x = torch.from_numpy(inp.X_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        x = torch.from_numpy(inp.X).to(dev)
    w = torch.from_numpy(inp.W).to(dev)
    g = mq.forward_layer(x, w, k_blocks, bn=cfg.bn)
    del w
    packed = gemm_bytes(cfg, k_blocks) - cfg.M * (cfg.K // 2 + 4 + cfg.N * 2)
    copies = max(2, min(256, -(-ROTATE_BYTES // packed)))
    sets = [(g["wq"].clone(), g["sw"].clone(), g["rq"].clone(), g["row_ptr"].clone(),
             g["col_idx"].clone()) for _ in range(copies)]
    xq, sx, K, bn = g["xq"], g["sx"], cfg.K, cfg.bn
    y = torch.empty((cfg.M, cfg.N), dtype=torch.bfloat16, device=dev)
    wsb = torch.empty((cfg.M, cfg.N), dtype=torch.float32, device=dev)
    gws = mq.workspace(cfg.M, cfg.N, K, device=dev)
    log(f"[bench] gemm legs: {copies} packed-weight copies ({copies * packed / 2**20:.0f} MiB), "
        f"{calls} calls each")

    def fused(i):
        wq, sw, rq, rp, ci = sets[i % copies]
        mq.gemm_w4a4_residual(xq, sx, wq, sw, rp, ci, rq, K, bn=bn, y=y, workspace=gws)

    def dense(i):
        wq, sw, *_ = sets[i % copies]
        mq.gemm_w4a4_dense(xq, sx, wq, sw, K, y=y, workspace=gws)

    def separate(i):
        wq, sw, rq, rp, ci = sets[i % copies]
        mq.gemm_residual_separate(xq, sx, wq, sw, rp, ci, rq, K, bn=bn, y=y, ws=wsb, workspace=gws)

    out = {}
    for name, fn in (("dense", dense), ("fused", fused), ("separate", separate)):
        # eager result of the last call, to check the graph replays against
        fn(calls - 1)
        torch.cuda.synchronize()
        y_eager = y.clone()
        out[name] = _graph_time_us(torch, fn, calls)
        if not torch.equal(y.view(torch.int16), y_eager.view(torch.int16)):
            raise RuntimeError(f"graph replay of the {name} GEMM differs from the eager call")
        log(f"[bench] gemm {name}: {out[name]:.3f} us/call")
    return out


# --------------------------------------------------------------------------- calibration
def calibrate(torch, sizes_mb=(9.65, 64.0, 512.0), calls=50):
    """Achievable HBM rate of a plain device copy (torch's copy kernel) at the sizes
    this path moves, over rotating slices of a 1 GiB source so the Infinity Cache
    cannot serve the reads; and the duration of a one-element fill (launch floor)."""
    dev = torch.device("cuda:0")
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    src.fill_(1)
    out = {}
    for mb in sizes_mb:
        n = int(mb * 1e6) // 256 * 256
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        slices = max(1, (1 << 30) // n)
        for i in range(5):
            dst.copy_(src[(i % slices) * n:(i % slices) * n + n])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(calls):
            j = i % slices
            dst.copy_(src[j * n:j * n + n])
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / calls
        out[f"copy_{mb:g}MB"] = {"us": round(us, 3), "GB/s(read+write)": round(2 * n / us / 1e3, 1)}
        log(f"[bench] calib copy {mb:g} MB: {us:.2f} us/call, {2 * n / us / 1e3:.0f} GB/s read+write")
        del dst
    tiny = torch.empty(1, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(200):
        tiny.fill_(1.0)
    e1.record()
    torch.cuda.synchronize()
    out["fill_1_element_us"] = round(e0.elapsed_time(e1) * 1e3 / 200, 3)
    del src
    torch.cuda.empty_cache()
    return out


# --------------------------------------------------------------------------- CPU oracle leg
def cpu_baseline(cfg, inp, k_blocks, seconds, step_total_bytes):
    import oracle
    orc = oracle.Oracle()
    runs, t0 = 0, time.perf_counter()
    while True:
        orc.forward(inp.x_raw(), inp.W, k_blocks, cfg.group, cfg.bn, cfg.bk)
        runs += 1
        el = time.perf_counter() - t0
        if el >= seconds or runs >= 50:
            break
    per = el / runs
    return {"value": step_total_bytes / per / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{runs} full passes of the whole path on this workload (all steps, all "
                      f"{cfg.M} tokens), single-threaded C, {per * 1e3:.0f} ms per pass",
            "s_per_step": per}


# --------------------------------------------------------------------------- profiles
CALIB_COPY_BYTES = 256 << 20     # the copy of known size the HBM counters are scaled by


def pmc_pass(mq, torch, cfg, inp, k_blocks):
    """What `rocprofv3 --pmc` runs: a few whole steps, then CALIB_COPY_BYTES copied
    device to device five times (a plain copy of known size, to scale the counters)."""
    bench_step(mq, torch, cfg, inp, k_blocks, steps=3, warmup=1)
    src = torch.ones(CALIB_COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)                       # the runtime's blit copy
    fsrc, fdst = src.view(torch.float32), dst.view(torch.float32)
    for _ in range(5):
        torch.mul(fsrc, 1.0, out=fdst)       # an elementwise kernel with 16-byte lane accesses
    torch.cuda.synchronize()


def _db(path):
    import glob
    import sqlite3
    dbs = [path] if path.endswith(".db") else sorted(glob.glob(os.path.join(path, "**", "*.db"), recursive=True))
    if not dbs:
        raise SystemExit(f"no rocprofv3 results database under {path}")
    return sqlite3.connect(dbs[0])


def profile_summary(db_path, title, command):
    """Kernel-trace statistics of a rocprofv3 results database, as text."""
    con = _db(db_path)
    rows = list(con.execute("select name, total_calls, total_duration, average, percentage from top_kernels"))
    out = [f"# {title}", "", f"command: {command}", "",
           "rocprofv3 --kernel-trace --stats, kernel durations (us):", "",
           f"{'calls':>6} {'avg_us':>10} {'total_us':>11} {'pct':>6}  kernel"]
    for name, calls, tot, avg, pct in rows:
        out.append(f"{calls:>6} {avg:>10.3f} {tot:>11.1f} {pct:>6.2f}  {name[:110]}")
    return "\n".join(out)


def _counter_means(db_path, counter):
    """Mean of one counter per kernel name, and per-dispatch values of the two copy
    kernels (runtime blit, elementwise multiply by one)."""
    con = _db(db_path)
    per, blit, elem = {}, [], []
    for k, c, v, grid in con.execute(
            "select kernel_name, counter_name, value, grid_size from counters_collection"):
        if c != counter:
            continue
        per.setdefault(k, []).append(v)
        if "copyBuffer" in k:
            blit.append((grid, v))
        if "elementwise" in k and "Mul" in k:
            elem.append((grid, v))
    return {k: sum(v) / len(v) for k, v in per.items()}, blit, elem


def pmc_summary(fetch_db, write_db, title, commands):
    """HBM traffic per dispatch from FETCH_SIZE and WRITE_SIZE passes, each scaled by
    what the same counter reads for the largest copy (CALIB_COPY_BYTES each way)."""
    fetch, fblit, felem = _counter_means(fetch_db, "FETCH_SIZE")
    write, wblit, welem = _counter_means(write_db, "WRITE_SIZE")
    kib = CALIB_COPY_BYTES / 1024

    def largest(pairs):
        big = max(g for g, _ in pairs)
        return float(np.mean([v for g, v in pairs if g == big]))
    bf, bw = largest(fblit), largest(wblit)
    cf, cw = largest(felem), largest(welem)
    ff, fw = kib / cf, kib / cw
    import hashlib
    digest = hashlib.sha256(open(os.path.join(ROOT, "dense_sparse_bit_amd", "csrc", "prep.hip"), "rb")
                            .read()).hexdigest()[:16]
    out = [f"# {title}", "", "commands:"] + [f"  {c}" for c in commands] + [
        "", f"kernel source (dense_sparse_bit_amd/csrc/prep.hip) source sha256: {digest}"] + [
        "", f"calibration: {CALIB_COPY_BYTES >> 20} MiB read and written by an elementwise kernel "
        f"(y = x * 1, 16-byte lane accesses like this library's): FETCH_SIZE {cf:.0f} KiB, WRITE_SIZE "
        f"{cw:.0f} KiB per dispatch -> scale factors {ff:.4f} (fetch), {fw:.4f} (write), used below",
        f"(the runtime blit copy of the same size reads FETCH_SIZE {bf:.0f} KiB, WRITE_SIZE {bw:.0f} KiB: "
        f"factors {kib / bf:.4f}, {kib / bw:.4f}; its request sizes differ)", "",
        f"{'fetch_KiB':>12} {'write_KiB':>12} {'scaled_MB':>10}  kernel"]
    for k in sorted(set(fetch) | set(write), key=lambda n: -fetch.get(n, 0)):
        if "mq::" not in k:
            continue
        f, w = fetch.get(k, 0.0), write.get(k, 0.0)
        out.append(f"{f:>12.1f} {w:>12.1f} {(f * ff + w * fw) * 1024 / 1e6:>10.3f}  {k[:100]}")
    return "\n".join(out)


def traffic_from_profile(kernels, source):
    """HBM bytes per call of the given kernels from the committed counter summary,
    or None when the summary is missing or was taken from different kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "select_blocks_llama3_8b_qo_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    digest = hashlib.sha256(open(os.path.join(ROOT, source), "rb").read()).hexdigest()[:16]
    if f"source sha256: {digest}" not in text:
        return None
    total = 0.0
    for k in kernels:
        line = [l for l in text.splitlines() if l.rstrip().endswith(k) or f" {k}(" in l]
        if not line:
            return None
        total += float(line[0].split()[2]) * 1e6
    return total


# --------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=synth.BENCH_CONFIG, choices=sorted(synth.CONFIGS))
    ap.add_argument("--budget", type=int, default=None, help="residual budget in percent")
    ap.add_argument("--gemm-calls", type=int, default=200)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--no-calib", action="store_true")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="run a few steps and a copy of known size (for rocprofv3 --pmc), print nothing")
    ap.add_argument("--profile-summary", metavar="DB", help="print a rocprofv3 kernel-trace summary")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="print HBM traffic per kernel from FETCH_SIZE and WRITE_SIZE passes")
    ap.add_argument("--title", default="")
    ap.add_argument("--command", action="append", default=[])
    args = ap.parse_args()
    if args.profile_summary:
        print(profile_summary(args.profile_summary, args.title, " ; ".join(args.command)))
        return
    if args.pmc_summary:
        print(pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.title, args.command))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU leg in this build)", file=sys.stderr)
        sys.exit(2)

    import torch
    import dense_sparse_bit_amd as mq
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    cfg = synth.CONFIGS[args.workload]
    pct = cfg.default_budget if args.budget is None else args.budget
    k_blocks = cfg.k_blocks(pct)
    inp = synth.make_inputs(cfg)
    if args.pmc_pass:
        pmc_pass(mq, torch, cfg, inp, k_blocks)
        return
    x_bytes = 2 if inp.X_bits is not None else 4
    sb = step_bytes(cfg, k_blocks, x_bytes)
    total_bytes = sum(sb.values())

    st = bench_step(mq, torch, cfg, inp, k_blocks, args.steps, args.warmup)
    kernels = {}
    for n, us in st["us"].items():
        gbs = sb[n] / us / 1e3
        kernels[n] = {"us": round(us, 3), "bytes": sb[n], "GB/s": round(gbs, 1),
                      "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    dom = max(st["us"], key=st["us"].get)
    value = total_bytes / (st["gpu_ms"] * 1e-3) / 1e9

    gemm = None
    if not args.no_gemm:
        t = bench_gemm(mq, torch, cfg, inp, k_blocks, args.gemm_calls)
        fb, db = gemm_bytes(cfg, k_blocks), gemm_bytes(cfg, k_blocks, residual=False)
        fo, do = gemm_ops(cfg, k_blocks), gemm_ops(cfg, k_blocks, residual=False)
        leg = lambda us, b, o: {"us": round(us, 3), "GB/s": round(b / us / 1e3, 1),
                                "hbm_frac": round(b / us / 1e3 / HBM_PEAK_GBS, 4),
                                "TOPS": round(o / us / 1e6, 3),
                                "int8_frac": round(o / us / 1e6 / INT8_PEAK_TOPS, 5), "bytes": b,
                                "ops": o}
        gemm = {"fused": leg(t["fused"], fb, fo), "dense": leg(t["dense"], db, do),
                "separate": leg(t["separate"], fb, fo),
                "overhead_vs_dense": round(t["fused"] / t["dense"] - 1, 4),
                "separate_overhead_vs_dense": round(t["separate"] / t["dense"] - 1, 4),
                "residual_bytes_vs_base": round((fb - db) / (cfg.N * cfg.K // 2 + cfg.N * cfg.K // 64), 4),
                "timing": "median of 5 replays of a HIP graph of %d back-to-back calls over rotated "
                          "packed-weight copies, HIP events around each replay" % args.gemm_calls}

    calib = None if args.no_calib else calibrate(torch)

    cpu = None
    if not args.no_cpu:
        log(f"[bench] CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(cfg, inp, k_blocks, args.cpu_seconds, total_bytes)

    dom_b = sb[dom]
    traffic = None
    if dom == "select_blocks":
        t = traffic_from_profile(["mq::k_delta", "mq::k_rank", "mq::k_csr"],
                                 os.path.join("dense_sparse_bit_amd", "csrc", "prep.hip"))
        traffic = None if t is None else int(t)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(st["gpu_ms"], 5),
        "wall_ms_per_step": round(st["wall_ms"], 5),
        "eager_ms_per_step": round(st["eager_ms"], 5),
        "timing": "one replay of a HIP graph holding exactly `steps` steps (after `warmup` eager "
                  "steps), HIP events on the launch stream, inputs rotated over %d HBM-resident "
                  "copies; per-call figures: each call alone in its own graph" % st["copies"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic, seeded (synth.py): random weights and activations with the shapes and "
                "outlier structure of the workload",
        "config": {"workload": f"{cfg.name}: M={cfg.M} K={cfg.K} N={cfg.N}, residual budget {pct}% "
                               f"of {cfg.bn}x{cfg.bk} blocks ({k_blocks}/{(cfg.N // cfg.bn) * (cfg.K // cfg.bk)}), "
                               f"int4 weights group 128, per-token int4 activations",
                   "M": cfg.M, "K": cfg.K, "N": cfg.N, "bn": cfg.bn, "bk": cfg.bk,
                   "budget_pct": pct, "k_blocks": k_blocks,
                   "step": "hessian_diag -> select_blocks -> pack_weights -> quantize_act -> "
                           "gemm_w4a4_residual"},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(dom_b / st["us"][dom] / 1e3, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_b / st["us"][dom] / 1e3 / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "bytes_per_launch": dom_b, "us_per_launch": round(st["us"][dom], 3),
                     "traffic_source": "profiles/select_blocks_llama3_8b_qo_hbm_traffic.txt (rocprofv3 "
                                       "FETCH_SIZE and WRITE_SIZE passes, scaled by a copy of known size; "
                                       "null when the kernel source changed since)"},
        "cpu_baseline": None if cpu is None else {k: (round(v, 4) if isinstance(v, float) else v)
                                                  for k, v in cpu.items() if k != "s_per_step"},
        "step_kernels": kernels,
        "gemm": gemm,
        "calib": calib,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
