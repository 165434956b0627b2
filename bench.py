"""Benchmark of the MosaicQuant ZipperEngine path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--budget PCT]
    python bench.py --sweep           # batch sweep and a LLaMA3-8B-shaped linear stack

A step is one pass of the per-call path over one batch of synthetic input, on
the GPU: per-token int4 activation quantization (mq_quantize_act), then the fused
W4A4 + sparse-residual GEMM (mq_gemm_w4a4_residual). The layer's weights are
prepared once beforehand (Hessian diagonal, Delta-score top-K, packing: the
offline steps) and copied so that consecutive steps read different weight and
activation copies (more than 600 MB in total): neither the 256 MB Infinity
Cache nor L2 can serve them. Inputs are resident in HBM before the timed region.

Printed on stdout: one JSON line.
  value      algorithmic ops of the step (2*M*(N*K + nnz*bn*bk)) / step time, in TOPS;
             the K steps are one replay of a HIP graph, HIP events around it
  roofline   the fused GEMM kernel alone (the step's dominant kernel): its
             algorithmic ops (MFMA-bound, M > 32) or bytes (HBM-bound, M <= 32)
             per launch over its average launch duration (back-to-back launches
             in a HIP graph, HIP events on the launch stream), against the
             published MI355X peak
  gemm       the fused kernel beside the dense-only kernel and the separate-kernel
             alternative on the same workload (fusion overhead)
  legs       the same three variants, plus a bf16 torch.matmul of the same layer,
             on every other workload (decode shapes, budget sweeps)
  cpu_baseline  the CPU oracle's per-call path (quantize, exact group sums,
             output) on a bounded sample of the workload's tokens
"""
from __future__ import annotations

import argparse
import hashlib
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
F8_PEAK_TOPS = 5000.0           # MI355X dense fp8 (and int8) MFMA
ROTATE_BYTES = 640 << 20        # > 2 x (256 MB Infinity Cache + 8 x 4 MB L2)
GEMM_SRC = os.path.join("dense_sparse_bit_amd", "csrc", "gemm.hip")
# rocprofv3 FETCH_SIZE / WRITE_SIZE summaries per workload, all taken at the 10% budget
TRAFFIC_SUMMARIES = {w: os.path.join("profiles", f"gemm_{p}_counters.txt") for w, p in (
    ("qwen3_14b_prefill", "prefill_qwen3_14b"), ("llama3_8b_qo", "decode_llama3_8b_qo"),
    ("llama3_8b_up_m4", "decode_llama3_8b_up_m4"), ("llama3_8b_down_m4", "decode_llama3_8b_down_m4"))}
TRAFFIC_BUDGET_PCT = 10

# workloads measured beside the headline in one default run: (config, budgets in %)
LEGS = [("llama3_8b_qo", (10,)),
        ("llama3_8b_up_m4", (0, 5, 10, 20)), ("llama3_8b_up_m32", (0, 5, 10, 20)),
        ("llama3_8b_down_m4", (0, 5, 10, 20)), ("llama3_8b_down_m32", (0, 5, 10, 20)),
        ("qwen3_32b_up", (10,)), ("qwen3_32b_down", (10,))]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------- algorithmic work
def gemm_bytes(cfg, nnz, residual=True, y_bytes=2):
    """Bytes the GEMM must move at minimum: base nibbles, fp16 group scales, activation
    nibbles and scales, the output; plus residual nibbles and the CSR lists."""
    M, N, K, G = cfg.M, cfg.N, cfg.K, cfg.K // cfg.group
    b = N * K // 2 + N * G * 2 + M * K // 2 + M * 4 + M * N * y_bytes
    if residual:
        b += nnz * cfg.bn * cfg.bk // 2 + nnz * 4 + (N // cfg.bn + 1) * 4
    return b


def gemm_ops(cfg, nnz, residual=True):
    return 2 * cfg.M * (cfg.N * cfg.K + (nnz * cfg.bn * cfg.bk if residual else 0))


def roofline_kind(cfg):
    return "mfma" if cfg.M > 32 else "hbm"


# --------------------------------------------------------------------------- GPU helpers
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


def _x_device(torch, inp, dev):
    if inp.X_bits is not None:
        return torch.from_numpy(inp.X_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(inp.X).to(dev)


class Layer:
    """One synthetic layer on the device: W, X, and the packed operands for a budget."""

    def __init__(self, mq, torch, cfg, inp=None):
        self.mq, self.torch, self.cfg = mq, torch, cfg
        self.inp = synth.make_inputs(cfg) if inp is None else inp
        dev = torch.device("cuda:0")
        self.x = _x_device(torch, self.inp, dev)
        self.w = torch.from_numpy(self.inp.W).to(dev)
        self.h = mq.hessian_diag(self.x)
        self.xq, self.sx = mq.quantize_act(self.x)

    def pack(self, k_blocks):
        mq, cfg = self.mq, self.cfg
        rp, ci, _ = mq.select_blocks(self.w, self.h, k_blocks, bn=cfg.bn, return_delta=False)
        wq, sw, rq = mq.pack_weights(self.w, rp, ci, bn=cfg.bn)
        rmap = mq.block_map(rp, ci, cfg.N, cfg.K, bn=cfg.bn)
        return dict(wq=wq, sw=sw, rq=rq, row_ptr=rp, col_idx=ci, rmap=rmap)

    def copies(self, packed, nbytes):
        n = max(2, min(256, -(-ROTATE_BYTES // max(nbytes, 1))))
        return [{k: v.clone() for k, v in packed.items()} for _ in range(n)]


def bench_variants(mq, torch, layer, k_blocks, calls, bf16=True):
    """Fused, dense-only and separate-kernel GEMM (and a bf16 torch.matmul of the same
    layer) over rotated weight copies, each in its own HIP graph of `calls`
    back-to-back calls; every graph's output is checked against its eager call."""
    cfg = layer.cfg
    packed = layer.pack(k_blocks)
    pbytes = gemm_bytes(cfg, k_blocks) - cfg.M * (cfg.K // 2 + 4 + cfg.N * 2)
    sets = layer.copies(packed, pbytes)
    n = len(sets)
    xq, sx, K, bn = layer.xq, layer.sx, cfg.K, cfg.bn
    y = torch.empty((cfg.M, cfg.N), dtype=torch.bfloat16, device="cuda")
    wsb = torch.empty((cfg.M, cfg.N), dtype=torch.float32, device="cuda")

    def fused(i):
        s = sets[i % n]
        mq.gemm_w4a4_residual(xq, sx, s["wq"], s["sw"], s["row_ptr"], s["col_idx"], s["rq"], K, bn=bn, y=y,
                              rmap=s["rmap"])

    def fused_csr(i):
        s = sets[i % n]
        mq.gemm_w4a4_residual(xq, sx, s["wq"], s["sw"], s["row_ptr"], s["col_idx"], s["rq"], K, bn=bn, y=y)

    def dense(i):
        s = sets[i % n]
        mq.gemm_w4a4_dense(xq, sx, s["wq"], s["sw"], K, y=y)

    def separate(i):
        s = sets[i % n]
        mq.gemm_residual_separate(xq, sx, s["wq"], s["sw"], s["row_ptr"], s["col_idx"], s["rq"], K,
                                  bn=bn, y=y, ws=wsb)

    # the per-call path from unquantized activations: quantize_act then the fused
    # GEMM (two launches), against the GEMM that quantizes its own activations
    xq2, sx2 = torch.empty_like(xq), torch.empty_like(sx)
    sync = mq.sync_words()

    def quant_then_fused(i):
        s = sets[i % n]
        mq.quantize_act(layer.x, xq=xq2, sx=sx2)
        mq.gemm_w4a4_residual(xq2, sx2, s["wq"], s["sw"], s["row_ptr"], s["col_idx"], s["rq"], K, bn=bn, y=y,
                              rmap=s["rmap"])

    def fused_act(i, launch="auto"):
        s = sets[i % n]
        mq.gemm_w4a4_residual_act(layer.x, s["wq"], s["sw"], s["rmap"], s["rq"], K, bn=bn, y=y, xq=xq2, sx=sx2,
                                  sync=sync, launch=launch)

    legs = [("dense", dense), ("fused", fused), ("fused_csr", fused_csr), ("separate", separate),
            ("quant_then_fused", quant_then_fused), ("fused_act", fused_act)]
    if cfg.M <= 32:
        legs.append(("fused_act_one", lambda i: fused_act(i, "one")))
    out = {}
    for name, fn in legs:
        fn(calls - 1)
        torch.cuda.synchronize()
        y_eager = y.clone()
        out[name] = _graph_time_us(torch, fn, calls)
        if not torch.equal(y.view(torch.int16), y_eager.view(torch.int16)):
            raise RuntimeError(f"graph replay of the {name} GEMM differs from the eager call")
    # dense and fused again, after the other legs: the first graph a process times can
    # run while the clocks ramp, so each of the two reports the better of its passes
    for name, fn in legs[:2]:
        out[name] = min(out[name], _graph_time_us(torch, fn, calls))
    out["act_auto_one"] = 1.0 if mq.act_one_launch(cfg.M, cfg.N, cfg.K) else 0.0
    del sets
    if bf16:
        # the W16A16 context: the same layer as a bf16 matmul (hipBLASLt), weights rotated too
        wb = layer.w.to(torch.bfloat16)
        xb = layer.x.to(torch.bfloat16)
        nw = max(2, min(64, -(-ROTATE_BYTES // (wb.numel() * 2))))
        ws_ = [wb.clone() for _ in range(nw)]
        yb = torch.empty((cfg.M, cfg.N), dtype=torch.bfloat16, device="cuda")

        def mm(i):
            torch.matmul(xb, ws_[i % nw].t(), out=yb)
        out["bf16_matmul"] = _graph_time_us(torch, mm, max(20, calls // 4))
        del ws_, wb
    torch.cuda.empty_cache()
    return out


def leg_record(cfg, pct, k_blocks, t):
    fb, db = gemm_bytes(cfg, k_blocks), gemm_bytes(cfg, k_blocks, residual=False)
    fo, do = gemm_ops(cfg, k_blocks), gemm_ops(cfg, k_blocks, residual=False)

    def one(us, b, o):
        return {"us": round(us, 3), "GB/s": round(b / us / 1e3, 1),
                "hbm_frac": round(b / us / 1e3 / HBM_PEAK_GBS, 4),
                "TOPS": round(o / us / 1e6, 2), "mfma_frac": round(o / us / 1e6 / F8_PEAK_TOPS, 4)}
    rec = {"workload": cfg.name, "M": cfg.M, "K": cfg.K, "N": cfg.N, "bn": cfg.bn, "budget_pct": pct,
           "k_blocks": k_blocks, "bound": roofline_kind(cfg), "bytes": fb, "ops": fo,
           "fused": one(t["fused"], fb, fo), "dense": one(t["dense"], db, do),
           "fused_csr": one(t["fused_csr"], fb, fo),
           "separate": one(t["separate"], fb, fo),
           "overhead_vs_dense": round(t["fused"] / t["dense"] - 1, 4),
           "overhead_csr_vs_dense": round(t["fused_csr"] / t["dense"] - 1, 4),
           "separate_overhead_vs_dense": round(t["separate"] / t["dense"] - 1, 4)}
    if "fused_act" in t:
        # from unquantized activations: quantize_act + the GEMM (two launches), the
        # self-quantizing call as its "auto" rule runs it, and forced to one launch
        rec["quant_then_fused_us"] = round(t["quant_then_fused"], 3)
        rec["act_auto_us"] = round(t["fused_act"], 3)
        rec["act_auto_form"] = "one" if t["act_auto_one"] else "two"
        if "fused_act_one" in t:
            rec["act_one_launch_us"] = round(t["fused_act_one"], 3)
            rec["act_one_launch_saving"] = round(1 - t["fused_act_one"] / t["quant_then_fused"], 4)
    if "bf16_matmul" in t:
        rec["bf16_matmul_us"] = round(t["bf16_matmul"], 3)
        rec["speedup_fused_vs_bf16"] = round(t["bf16_matmul"] / t["fused"], 3)
    if "read_ceiling_us" in t:
        rec["read_ceiling_us"] = round(t["read_ceiling_us"], 3)
        rec["fused_vs_read_ceiling"] = round(t["read_ceiling_us"] / t["fused"], 4)
    return rec


def read_ceiling_us(mq, torch, nbytes, calls=100):
    """Time of a plain streaming read of `nbytes` (the library's read probe: 16-byte
    loads, four in flight per lane) over rotating slices of a 1 GiB buffer, as a
    graph of back-to-back launches: the read rate a kernel reaches at this size."""
    n = max(16, (int(nbytes) + 15) // 16 * 16)
    src = torch.ones((1 << 30) // 4, dtype=torch.int32, device="cuda")
    slices = max(1, (1 << 30) // n)
    out = torch.empty(mq.READ_PROBE_WORDS, dtype=torch.int32, device="cuda")
    views = [src.view(torch.uint8)[j * n:(j + 1) * n] for j in range(slices)]

    def rd(i):
        mq.read_probe(views[i % slices], n, out=out)
    us = _graph_time_us(torch, rd, calls)
    del src, views
    torch.cuda.empty_cache()
    return us


# --------------------------------------------------------------------------- the headline step
def bench_step(mq, torch, layer, k_blocks, steps, warmup):
    """The per-call path (quantize activations, fused GEMM), step after step over
    rotated weight and activation copies; K steps captured in one HIP graph and
    timed as one replay. The fused GEMM is also timed alone (its launches back to
    back in a graph, same copies): the roofline kernel's average launch time."""
    cfg = layer.cfg
    packed = layer.pack(k_blocks)
    pbytes = gemm_bytes(cfg, k_blocks) - cfg.M * (cfg.K // 2 + 4 + cfg.N * 2)
    sets = layer.copies(packed, pbytes)
    n = len(sets)
    nx = max(2, min(16, -(-(64 << 20) // (layer.x.numel() * layer.x.element_size()))))
    xs = [layer.x.clone() for _ in range(nx)]
    xq = torch.empty_like(layer.xq)
    sx = torch.empty_like(layer.sx)
    y = torch.empty((cfg.M, cfg.N), dtype=torch.bfloat16, device="cuda")
    K, bn = cfg.K, cfg.bn
    log(f"[bench] step workload {cfg.name}: M={cfg.M} K={K} N={cfg.N} bn={bn} k_blocks={k_blocks}, "
        f"{n} weight copies ({n * pbytes / 2**20:.0f} MiB), {nx} activation copies")

    def gemm(i):
        s = sets[i % n]
        mq.gemm_w4a4_residual(xq, sx, s["wq"], s["sw"], s["row_ptr"], s["col_idx"], s["rq"], K, bn=bn, y=y,
                              rmap=s["rmap"])

    def quant(i):
        mq.quantize_act(xs[i % nx], xq=xq, sx=sx)

    def one_step(i):
        quant(i)
        gemm(i)

    for i in range(warmup):
        one_step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        one_step(i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / steps

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
    # the last step's output against its eager call (same inputs, same kernels)
    y_graph = y.clone()
    one_step(steps - 1)
    torch.cuda.synchronize()
    if not torch.equal(y.view(torch.int16), y_graph.view(torch.int16)):
        raise RuntimeError("graph replay of the step differs from the eager step")

    gemm_us = _graph_time_us(torch, gemm, max(steps, 2 * n))
    quant_us = _graph_time_us(torch, quant, max(steps, 2 * nx))
    log(f"[bench] step {gpu_ms * 1e3:.2f} us (graph), eager {eager_ms * 1e3:.2f} us; "
        f"fused GEMM alone {gemm_us:.3f} us, quantize_act alone {quant_us:.3f} us")
    del sets, xs
    torch.cuda.empty_cache()
    return dict(gpu_ms=gpu_ms, wall_ms=wall_ms, eager_ms=eager_ms, gemm_us=gemm_us, quant_us=quant_us,
                copies=n)


# --------------------------------------------------------------------------- CPU oracle leg
def cpu_baseline(cfg, inp, k_blocks, rows):
    """The oracle's per-call path (O1 activation quantization, O8 exact group sums,
    O9 output) on the first `rows` tokens and every output; its weight preparation
    (selection, packing) is done beforehand and not timed. Single-threaded C, as
    the oracle stands. Beside it, the same O8 + O9 calls over slices of whole block
    rows of W, run in as many host threads as this process may use (each call is
    the same single-threaded C; ctypes releases the interpreter lock), and the
    single-threaded O8 + O9 time alone (the oracle's GEMM)."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    orc = oracle.Oracle()
    xr = inp.x_raw()[:rows]
    h = orc.hessian_diag(inp.x_raw())
    rp, ci, _, _ = orc.select_blocks(inp.W, h, k_blocks, cfg.group, cfg.bn, cfg.bk)
    wq, sw, rq = orc.pack_weights(inp.W, rp, ci, cfg.group, cfg.bn, cfg.bk)
    t0 = time.perf_counter()
    xq, sx = orc.quantize_act(xr)
    t1 = time.perf_counter()
    P, Pr = orc.accumulators(xq, wq, rp, ci, rq, cfg.K, cfg.group, cfg.bn, cfg.bk)
    y1 = orc.output(sx, sw, P, Pr)
    t2 = time.perf_counter()
    el, el_gemm = t2 - t0, t2 - t1
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    nbr = cfg.N // cfg.bn
    cuts = [round(i * nbr / avail) for i in range(avail + 1)]

    def part(i):
        b0, b1 = cuts[i], cuts[i + 1]
        if b0 == b1:
            return None
        n0, n1, p0, p1 = b0 * cfg.bn, b1 * cfg.bn, int(rp[b0]), int(rp[b1])
        Ps, Prs = orc.accumulators(xq, wq[n0:n1], rp[b0:b1 + 1] - p0, ci[p0:p1], rq[p0:p1], cfg.K,
                                   cfg.group, cfg.bn, cfg.bk)
        return n0, n1, orc.output(sx, sw[n0:n1], Ps, Prs)
    t3 = time.perf_counter()
    with ThreadPoolExecutor(avail) as ex:
        parts = [r for r in ex.map(part, range(avail)) if r is not None]
    el_par = time.perf_counter() - t3
    yp = np.empty_like(y1)
    for n0, n1, ys in parts:
        yp[:, n0:n1] = ys
    if not np.array_equal(yp, y1):
        raise RuntimeError("the sliced oracle run differs from the whole-layer run")
    ops = 2 * rows * (cfg.N * cfg.K + k_blocks * cfg.bn * cfg.bk)
    return {"value": round(ops / el / 1e12, 6), "unit": "TOPS", "cores": 1, "kind": "oracle",
            "sample": f"tokens 0-{rows - 1} of {cfg.M} x all {cfg.N} outputs x K={cfg.K} "
                      f"(O1 quantize + O8 exact group sums + O9 fp64 output, single-threaded C), "
                      f"{el:.1f} s", "seconds": round(el, 2),
            "gemm_only": {"value": round(ops / el_gemm / 1e12, 6), "unit": "TOPS", "cores": 1,
                          "seconds": round(el_gemm, 2), "steps": "O8 + O9"},
            "all_cores": {"value": round(ops / el_par / 1e12, 6), "unit": "TOPS", "cores": avail,
                          "seconds": round(el_par, 2),
                          "steps": "O8 + O9 over slices of whole block rows, one host thread each"},
            "host_cores_available": avail, "host_nproc": os.cpu_count()}


# --------------------------------------------------------------------------- profiles
CALIB_COPY_BYTES = 256 << 20     # the copy of known size the HBM counters are scaled by


def pmc_pass(mq, torch, cfg, k_blocks, calls=5):
    """What `rocprofv3 --pmc` runs: a few fused GEMM calls and a few dense-only calls
    of the workload, then CALIB_COPY_BYTES read and written by an elementwise kernel
    (a copy of known size, to scale the counters)."""
    layer = Layer(mq, torch, cfg)
    p = layer.pack(k_blocks)
    y = torch.empty((cfg.M, cfg.N), dtype=torch.bfloat16, device="cuda")
    for _ in range(calls):
        mq.gemm_w4a4_residual(layer.xq, layer.sx, p["wq"], p["sw"], p["row_ptr"], p["col_idx"], p["rq"],
                              cfg.K, bn=cfg.bn, y=y, rmap=p["rmap"])
    for _ in range(calls):
        mq.gemm_w4a4_dense(layer.xq, layer.sx, p["wq"], p["sw"], cfg.K, y=y)
    src = torch.ones(CALIB_COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()


def trace_pass(mq, torch, cfg, k_blocks, calls=100):
    """What a per-shape `rocprofv3 --kernel-trace` runs: `calls` fused GEMM calls (block
    map), then `calls` dense-only calls of the workload, eagerly, over rotated weight
    copies (as the GEMM legs), so each kernel's average is that of cold weights."""
    layer = Layer(mq, torch, cfg)
    p = layer.pack(k_blocks)
    sets = layer.copies(p, gemm_bytes(cfg, k_blocks))
    n = len(sets)
    y = torch.empty((cfg.M, cfg.N), dtype=torch.bfloat16, device="cuda")
    for i in range(calls):
        s = sets[i % n]
        mq.gemm_w4a4_residual(layer.xq, layer.sx, s["wq"], s["sw"], s["row_ptr"], s["col_idx"], s["rq"],
                              cfg.K, bn=cfg.bn, y=y, rmap=s["rmap"])
    for i in range(calls):
        s = sets[i % n]
        mq.gemm_w4a4_dense(layer.xq, layer.sx, s["wq"], s["sw"], cfg.K, y=y)
    torch.cuda.synchronize()


def _db(path):
    import glob
    import sqlite3
    dbs = [path] if path.endswith(".db") else sorted(glob.glob(os.path.join(path, "**", "*.db"), recursive=True))
    if not dbs:
        raise SystemExit(f"no rocprofv3 results database under {path}")
    return sqlite3.connect(dbs[0])


def _src_digest():
    return hashlib.sha256(open(os.path.join(ROOT, GEMM_SRC), "rb").read()).hexdigest()[:16]


def profile_summary(db_path, title, command):
    """Kernel-trace statistics of a rocprofv3 results database, as text."""
    con = _db(db_path)
    rows = list(con.execute("select name, total_calls, total_duration, average, percentage from top_kernels"))
    out = [f"# {title}", "", f"command: {command}", "",
           f"kernel source ({GEMM_SRC}) sha256: {_src_digest()}", "",
           "rocprofv3 --kernel-trace --stats, kernel durations (us):", "",
           f"{'calls':>6} {'avg_us':>10} {'total_us':>11} {'pct':>6}  kernel"]
    for name, calls, tot, avg, pct in rows:
        out.append(f"{calls:>6} {avg:>10.3f} {tot:>11.1f} {pct:>6.2f}  {name[:110]}")
    return "\n".join(out)


def _counter_means(db_path, counter):
    con = _db(db_path)
    per, calib = {}, []
    for k, c, v, grid in con.execute(
            "select kernel_name, counter_name, value, grid_size from counters_collection"):
        if c != counter:
            continue
        per.setdefault(k, []).append(v)
        if "elementwise" in k and "Mul" in k:
            calib.append((grid, v))
    return {k: sum(v) / len(v) for k, v in per.items()}, calib


def counters_summary(db_paths, title, commands, only="k_gemm"):
    """Mean per dispatch of every counter in the given rocprofv3 --pmc databases, for
    the library's kernels; FETCH_SIZE and WRITE_SIZE are also scaled to bytes by what
    they read for the calibration copy (CALIB_COPY_BYTES read and written)."""
    kib = CALIB_COPY_BYTES / 1024
    table, scale = {}, {}
    for path in db_paths:
        con = _db(path)
        names = sorted({c for (c,) in con.execute("select distinct counter_name from counters_collection")})
        for c in names:
            per, calib = _counter_means(path, c)
            for k, v in per.items():
                if "mq::" in k and only in k:
                    table.setdefault(k, {})[c] = v
            if c in ("FETCH_SIZE", "WRITE_SIZE") and calib:
                big = max(g for g, _ in calib)
                scale[c] = kib / float(np.mean([v for g, v in calib if g == big]))
    out = [f"# {title}", "", "commands:"] + [f"  {c}" for c in commands] + [
        "", f"kernel source ({GEMM_SRC}) sha256: {_src_digest()}", ""]
    if scale:
        out.append("calibration: an elementwise kernel reading and writing "
                   f"{CALIB_COPY_BYTES >> 20} MiB; bytes per KiB of counter: " +
                   ", ".join(f"{c} x{v * 1024:.1f}" for c, v in sorted(scale.items())))
        out.append("")
    for k in sorted(table):
        out.append(f"kernel {k[:120]}")
        for c, v in sorted(table[k].items()):
            extra = ""
            if c in scale:
                extra = f"   -> {v * scale[c] * 1024 / 1e6:.3f} MB per dispatch"
            out.append(f"  {c:<28} {v:>16.1f}{extra}")
        out.append("")
    return "\n".join(out)


def fused_kernel_match(cfg):
    """(prefix, suffix) that pick the fused GEMM's kernel (residual on, no accumulator
    dump, output mode 0) out of a kernel list: k_gemm_wide when M > 32, else
    k_gemm_decode; its tile template arguments sit between the two."""
    if cfg.M > 32:
        return "k_gemm_wide<", ", true, false, 0>"
    return "k_gemm_decode<", ", true, false, 0, false>"


def traffic_from_profile(cfg, pct):
    """(kernel name, HBM bytes per launch) of the fused GEMM's kernel in the committed
    counter summary of this workload and budget; None for either when there is no such
    summary, bytes None when it was taken from different kernel source."""
    path = TRAFFIC_SUMMARIES.get(cfg.name)
    if path is None or pct != TRAFFIC_BUDGET_PCT:
        return None, None
    path = os.path.join(ROOT, path)
    if not os.path.exists(path):
        return None, None
    text = open(path).read()
    if f"sha256: {_src_digest()}" not in text:
        return None, None
    lines = text.splitlines()
    pre, suf = fused_kernel_match(cfg)
    total, found = 0.0, 0
    for i, l in enumerate(lines):
        if l.startswith("kernel ") and pre in l and suf in l:
            name = l[len("kernel "):].split("(")[0].removeprefix("void ").removeprefix("mq::")
            for l2 in lines[i + 1:]:
                if l2.startswith("kernel "):
                    break
                if ("FETCH_SIZE" in l2 or "WRITE_SIZE" in l2) and "MB per dispatch" in l2:
                    total += float(l2.split("->")[1].split()[0]) * 1e6
                    found += 1
            return name, (int(total) if found == 2 else None)
    return None, None


# --------------------------------------------------------------------------- sweep (batch sizes, layer stack)
def sweep(mq, torch, calls):
    """Fused, dense-only, separate and bf16 matmul at M = 1..256 on the LLaMA3-8B-shaped
    MLP up layer (10%), and a LLaMA3-8B-shaped linear stack (q, k, v, o, gate, up,
    down; per-layer activation quantization + fused GEMM, or the self-quantizing GEMM,
    vs bf16 matmuls) end to end."""
    res = {"batch": [], "stack": []}
    for M in (1, 2, 4, 8, 16, 24, 32, 64, 128, 256):
        cfg = synth.custom_config(f"llama3_8b_up_m{M}", M=M, K=4096, N=14336, bn=64)
        layer = Layer(mq, torch, cfg)
        kb = cfg.k_blocks(10)
        t = bench_variants(mq, torch, layer, kb, calls)
        rec = leg_record(cfg, 10, kb, t)
        res["batch"].append(rec)
        log(f"[sweep] M={M}: fused {t['fused']:.2f} dense {t['dense']:.2f} sep {t['separate']:.2f} "
            f"bf16 {t['bf16_matmul']:.2f} us")
        del layer
    shapes = [("q", 4096, 4096), ("k", 4096, 1024), ("v", 4096, 1024), ("o", 4096, 4096),
              ("gate", 4096, 14336), ("up", 4096, 14336), ("down", 14336, 4096)]
    for M in (1, 4, 16, 32):
        layers = []
        for nm, K, N in shapes:
            cfg = synth.custom_config(f"llama3_8b_{nm}", M=M, K=K, N=N, bn=64)
            lay = Layer(mq, torch, cfg)
            p = lay.pack(cfg.k_blocks(10))
            layers.append((lay, p, torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
                           lay.w.to(torch.bfloat16), lay.x.to(torch.bfloat16)))
            del lay.w

        def ours(i):
            for lay, p, y, _, _ in layers:
                mq.quantize_act(lay.x, xq=lay.xq, sx=lay.sx)
                mq.gemm_w4a4_residual(lay.xq, lay.sx, p["wq"], p["sw"], p["row_ptr"], p["col_idx"], p["rq"],
                                      lay.cfg.K, bn=64, y=y, rmap=p["rmap"])

        sync = mq.sync_words()

        def ours_act(i):
            # the same stack through the self-quantizing call (its launch rule picks one
            # launch or two per layer); the layers run in stream order, so they share one
            # counter array
            for lay, p, y, _, _ in layers:
                mq.gemm_w4a4_residual_act(lay.x, p["wq"], p["sw"], p["rmap"], p["rq"], lay.cfg.K, bn=64, y=y,
                                          xq=lay.xq, sx=lay.sx, sync=sync)

        def dense_only(i):
            for lay, p, y, _, _ in layers:
                mq.quantize_act(lay.x, xq=lay.xq, sx=lay.sx)
                mq.gemm_w4a4_dense(lay.xq, lay.sx, p["wq"], p["sw"], lay.cfg.K, y=y)

        def bf16(i):
            for lay, p, y, wb, xb in layers:
                torch.matmul(xb, wb.t(), out=y)
        t_ours = _graph_time_us(torch, ours, 20)
        t_act = _graph_time_us(torch, ours_act, 20)
        t_dense = _graph_time_us(torch, dense_only, 20)
        t_bf16 = _graph_time_us(torch, bf16, 20)
        res["stack"].append({"M": M, "fused_us": round(t_ours, 2), "fused_act_us": round(t_act, 2),
                             "dense_us": round(t_dense, 2),
                             "bf16_us": round(t_bf16, 2), "speedup_vs_bf16": round(t_bf16 / t_ours, 3),
                             "overhead_vs_dense": round(t_ours / t_dense - 1, 4),
                             "note": "weights of each layer read once per pass (7 layers, 218 MB of "
                                     "bf16 weights; the Infinity Cache can hold part of the packed ones)"})
        log(f"[sweep] stack M={M}: fused {t_ours:.1f} act {t_act:.1f} dense {t_dense:.1f} bf16 {t_bf16:.1f} us")
        del layers
        torch.cuda.empty_cache()
    return res


# --------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=synth.BENCH_CONFIG, choices=sorted(synth.CONFIGS))
    ap.add_argument("--budget", type=int, default=None, help="residual budget in percent")
    ap.add_argument("--gemm-calls", type=int, default=200, help="calls per graph for the decode legs")
    ap.add_argument("--cpu-rows", type=int, default=None, help="tokens in the CPU oracle sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-legs", action="store_true")
    ap.add_argument("--sweep", action="store_true", help="batch sweep + layer stack, one JSON line")
    ap.add_argument("--trace-pass", action="store_true",
                    help="eager fused then dense calls of --workload over rotated copies (for a kernel trace)")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="a few GEMM calls and a copy of known size (for rocprofv3 --pmc), print nothing")
    ap.add_argument("--profile-summary", metavar="DB", help="print a rocprofv3 kernel-trace summary")
    ap.add_argument("--counters-summary", nargs="+", metavar="DB",
                    help="print per-kernel counter means from rocprofv3 --pmc databases")
    ap.add_argument("--kernels", default="k_gemm", help="counters summary: kernels whose name holds this")
    ap.add_argument("--title", default="")
    ap.add_argument("--command", action="append", default=[])
    args = ap.parse_args()
    if args.profile_summary:
        print(profile_summary(args.profile_summary, args.title, " ; ".join(args.command)))
        return
    if args.counters_summary:
        print(counters_summary(args.counters_summary, args.title, args.command, args.kernels))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the path has "
              "no multi-GPU leg (each GPU would run the same kernel on its shard)", file=sys.stderr)
        sys.exit(2)

    import torch
    import dense_sparse_bit_amd as mq
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.sweep:
        print(json.dumps(sweep(mq, torch, args.gemm_calls)), flush=True)
        return

    cfg = synth.CONFIGS[args.workload]
    pct = cfg.default_budget if args.budget is None else args.budget
    k_blocks = cfg.k_blocks(pct)
    if args.trace_pass:
        trace_pass(mq, torch, cfg, k_blocks)
        return
    if args.pmc_pass:
        pmc_pass(mq, torch, cfg, k_blocks)
        return

    layer = Layer(mq, torch, cfg)
    st = bench_step(mq, torch, layer, k_blocks, args.steps, args.warmup)
    ops = gemm_ops(cfg, k_blocks)
    value = ops / (st["gpu_ms"] * 1e-3) / 1e12
    t = bench_variants(mq, torch, layer, k_blocks, max(10, min(args.gemm_calls, 30 if cfg.M > 32 else 200)))
    gemm = leg_record(cfg, pct, k_blocks, t)
    inp = layer.inp
    del layer
    torch.cuda.empty_cache()

    legs = []
    if not args.no_legs:
        for name, budgets in LEGS:
            c = synth.CONFIGS[name]
            if c.name == cfg.name:
                continue
            lay = Layer(mq, torch, c)
            rc = read_ceiling_us(mq, torch, gemm_bytes(c, c.k_blocks(10)))
            for b in budgets:
                tb = bench_variants(mq, torch, lay, c.k_blocks(b), args.gemm_calls, bf16=(b == 10))
                tb["read_ceiling_us"] = rc
                rec = leg_record(c, b, c.k_blocks(b), tb)
                legs.append(rec)
                log(f"[bench] leg {c.name} {b}%: fused {tb['fused']:.2f} dense {tb['dense']:.2f} "
                    f"separate {tb['separate']:.2f} us, overhead {rec['overhead_vs_dense']:.3f}, "
                    f"{rec['fused']['hbm_frac']:.3f} of 8 TB/s; quantize+fused {tb['quant_then_fused']:.2f}, "
                    f"self-quantizing one launch {tb.get('fused_act_one', float('nan')):.2f}, "
                    f"auto ({rec['act_auto_form']}) {tb['fused_act']:.2f} us")
            del lay
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        rows = args.cpu_rows or min(cfg.M, 256)
        log(f"[bench] CPU oracle baseline on {rows} tokens")
        cpu = cpu_baseline(cfg, inp, k_blocks, rows)

    kind = roofline_kind(cfg)
    if kind == "mfma":
        achieved, peak, unit = ops / st["gemm_us"] / 1e6, F8_PEAK_TOPS, "TOPS"
    else:
        achieved, peak, unit = gemm_bytes(cfg, k_blocks) / st["gemm_us"] / 1e3, HBM_PEAK_GBS, "GB/s"
    kname, traffic = traffic_from_profile(cfg, pct)
    if kname is None:
        kname = fused_kernel_match(cfg)[0] + "...>"
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(st["gpu_ms"], 5),
        "wall_ms_per_step": round(st["wall_ms"], 5),
        "eager_ms_per_step": round(st["eager_ms"], 5),
        "timing": "one replay of a HIP graph holding exactly `steps` steps (after `warmup` eager steps), "
                  "HIP events on the launch stream; weights rotated over %d HBM-resident packed copies "
                  "(> 600 MB)" % st["copies"],
        "higher_is_better": True,
        "vs_baseline": None,
        "dtype": "int4 codes as fp8-e4m3 MFMA operands, fp32 accumulate (exact per-group integer sums)",
        "data": "synthetic, seeded (synth.py): random weights and activations with the shapes and "
                "outlier structure of the workload; no trained weights",
        "config": {"workload": f"{cfg.name}: M={cfg.M} K={cfg.K} N={cfg.N}, residual budget {pct}% of "
                               f"{cfg.bn}x{cfg.bk} blocks ({k_blocks}/{cfg.nb}), int4 weights group 128, "
                               f"per-token int4 activations",
                   "M": cfg.M, "K": cfg.K, "N": cfg.N, "bn": cfg.bn, "bk": cfg.bk, "budget_pct": pct,
                   "k_blocks": k_blocks, "step": "quantize_act -> gemm_w4a4_residual"},
        "roofline": {"kernel": kname, "bound": kind, "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": traffic,
                     "per_launch": {"ops": ops, "bytes": gemm_bytes(cfg, k_blocks), "us": round(st["gemm_us"], 3)},
                     "hbm_GBs": round(gemm_bytes(cfg, k_blocks) / st["gemm_us"] / 1e3, 1),
                     "traffic_source": TRAFFIC_SUMMARIES.get(cfg.name, "none for this workload") + " (rocprofv3 FETCH_SIZE and WRITE_SIZE passes, scaled "
                                       "by a copy of known size; null when the kernel source changed since)"},
        "step_kernels_us": {"quantize_act": round(st["quant_us"], 3), "gemm_w4a4_residual": round(st["gemm_us"], 3)},
        "gemm": gemm,
        "legs": legs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
