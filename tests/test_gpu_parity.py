"""GPU parity: every step of the HIP path against the CPU oracle, through the C ABI.

Bit-exact: h, delta, row_ptr/col_idx, wq/sw/rq, xq/sx and the int32 group
accumulators T = 14*P + Pr. Within tolerance: y (max relative error, floor
0.1*rms of the row: fp32 output <= 1e-3, bf16 output <= 1e-2). The dense-only
kernel must equal the fused kernel with an empty residual bit for bit.

Inputs are the seeded synthetic workloads of synth.py at their full sizes; for
the 2048-token prefill the oracle's integer sums and outputs are compared on a
sample of 80 token rows (rows 0-63, which hold the BOS-like row, plus 16 drawn
rows), every other quantity in full.
"""
import sys

import numpy as np
import pytest

import synth
from tests.nibbles import rel_err, rq_to_twos, sw_to_rowmajor, wq_to_rowmajor, xq_to_rowmajor

pytestmark = pytest.mark.gpu

Y_TOL = {"f32": 1e-3, "bf16": 1e-2}
_ORACLE = {}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mq():
    import torch
    assert torch.cuda.is_available(), "GPU parity tests need a visible MI355X"
    import dense_sparse_bit_amd
    return dense_sparse_bit_amd


def _inputs(cfg_or_name):
    key = cfg_or_name if isinstance(cfg_or_name, str) else cfg_or_name
    if ("inp", key) not in _ORACLE:
        _ORACLE[("inp", key)] = synth.make_inputs(cfg_or_name)
    return _ORACLE[("inp", key)]


def _oracle_prep(orc, inp):
    """Oracle steps that do not depend on the budget."""
    key = ("prep", inp.cfg)
    if key not in _ORACLE:
        cfg = inp.cfg
        h = orc.hessian_diag(inp.x_raw())
        delta = orc.delta_scores(inp.W, h, cfg.group, cfg.bn, cfg.bk)
        xq, sx = orc.quantize_act(inp.x_raw())
        _ORACLE[key] = dict(h=h, delta=delta, xq=xq, sx=sx)
    return _ORACLE[key]


def _oracle_budget(orc, inp, k_blocks, rows=None):
    key = ("budget", inp.cfg, k_blocks, None if rows is None else tuple(rows))
    if key not in _ORACLE:
        cfg = inp.cfg
        pre = _oracle_prep(orc, inp)
        rp, ci, sel = orc.select_topk(pre["delta"], cfg.N // cfg.bn, cfg.K // cfg.bk, k_blocks)
        wq, sw, rq = orc.pack_weights(inp.W, rp, ci, cfg.group, cfg.bn, cfg.bk)
        xq, sx = pre["xq"], pre["sx"]
        if rows is not None:
            xq, sx = xq[rows], sx[rows]
        P, Pr = orc.accumulators(xq, wq, rp, ci, rq, cfg.K, cfg.group, cfg.bn, cfg.bk)
        y = orc.output(sx, sw, P, Pr)
        T = 14 * P.astype(np.int64) + Pr
        _ORACLE[key] = dict(row_ptr=rp, col_idx=ci, wq=wq, sw=sw, rq=rq, T=T, P=P, y=y)
    return _ORACLE[key]


def _to_dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def _x_dev(inp):
    import torch
    if inp.X_bits is not None:
        return _to_dev(inp.X_bits.view(np.int16), torch.bfloat16)
    return _to_dev(inp.X)


def _np(t):
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.float().numpy()
    return t.numpy()


def _run_gpu(mq, inp, k_blocks, out_dtype):
    import torch
    cfg = inp.cfg
    x = _x_dev(inp)
    w = _to_dev(inp.W)
    h = mq.hessian_diag(x)
    rp, ci, delta = mq.select_blocks(w, h, k_blocks, bn=cfg.bn)
    # the same selection with no score output (the scores stay in the library's scratch)
    rp2, ci2, none = mq.select_blocks(w, h, k_blocks, bn=cfg.bn, return_delta=False)
    assert none is None
    wq, sw, rq = mq.pack_weights(w, rp, ci, bn=cfg.bn)
    xq, sx = mq.quantize_act(x)
    dump = torch.empty((cfg.M, cfg.N, cfg.K // 128), dtype=torch.int32, device="cuda")
    y = mq.gemm_w4a4_residual(xq, sx, wq, sw, rp, ci, rq, cfg.K, bn=cfg.bn, out_dtype=out_dtype,
                              acc_dump=dump)
    torch.cuda.synchronize()
    assert torch.equal(rp2, rp) and torch.equal(ci2, ci), "selection without score output differs"
    return dict(h=h, row_ptr=rp, col_idx=ci, delta=delta, wq=wq, sw=sw, rq=rq, xq=xq, sx=sx, y=y,
                dump=dump, w=w, x=x)


def _check(mq, orc, inp, k_blocks, out_dtype_name="bf16", rows=None, check_variants=True):
    import torch
    cfg = inp.cfg
    out_dtype = torch.bfloat16 if out_dtype_name == "bf16" else torch.float32
    say(f"[parity] {cfg.name} M={cfg.M} K={cfg.K} N={cfg.N} bn={cfg.bn} k_blocks={k_blocks} "
        f"y={out_dtype_name} W={synth.sha256(inp.W)} X={synth.sha256(inp.X)}")
    pre = _oracle_prep(orc, inp)
    ref = _oracle_budget(orc, inp, k_blocks, rows)
    g = _run_gpu(mq, inp, k_blocks, out_dtype)
    np.testing.assert_array_equal(_np(g["h"]), pre["h"])
    np.testing.assert_array_equal(_np(g["delta"]), pre["delta"])
    np.testing.assert_array_equal(_np(g["row_ptr"]), ref["row_ptr"])
    np.testing.assert_array_equal(_np(g["col_idx"]), ref["col_idx"])
    np.testing.assert_array_equal(wq_to_rowmajor(_np(g["wq"]), cfg.N, cfg.K), ref["wq"])
    sw, pad = sw_to_rowmajor(_np(g["sw"]), cfg.N, cfg.K)
    np.testing.assert_array_equal(sw, ref["sw"])
    assert not pad.any(), "padding slots of sw must be zero"
    np.testing.assert_array_equal(rq_to_twos(_np(g["rq"])), ref["rq"])
    np.testing.assert_array_equal(xq_to_rowmajor(_np(g["xq"]), cfg.M, cfg.K), pre["xq"])
    np.testing.assert_array_equal(_np(g["sx"]), pre["sx"])
    sel = slice(None) if rows is None else rows
    dump = g["dump"][sel] if rows is None else g["dump"][torch.as_tensor(rows, device="cuda")]
    np.testing.assert_array_equal(_np(dump).astype(np.int64), ref["T"])
    y = _np(g["y"])[sel]
    err = rel_err(y, ref["y"])
    say(f"[parity] {cfg.name} y max rel err {err:.3e} (debug build)")
    assert err <= Y_TOL[out_dtype_name]
    # the production build (no dump), the kernel the benchmark times: the same
    # bits as the debug build, hence the same error against the oracle
    bits = (lambda t: t.view(torch.int16)) if out_dtype == torch.bfloat16 else (lambda t: t.view(torch.int32))
    yp = mq.gemm_w4a4_residual(g["xq"], g["sx"], g["wq"], g["sw"], g["row_ptr"], g["col_idx"], g["rq"],
                               cfg.K, bn=cfg.bn, out_dtype=out_dtype)
    torch.cuda.synchronize()
    err_p = rel_err(_np(yp)[sel], ref["y"])
    say(f"[parity] {cfg.name} y max rel err {err_p:.3e} (production build)")
    assert err_p <= Y_TOL[out_dtype_name]
    assert torch.equal(bits(yp), bits(g["y"])), "production and debug builds differ"
    # the block map of the selection, and the same GEMM finding its blocks through it:
    # the map is the oracle's CSR scattered into a dense table; y and the group sums
    # are the list-walking call's bits
    rmap = mq.block_map(g["row_ptr"], g["col_idx"], cfg.N, cfg.K, bn=cfg.bn)
    exp = np.full((cfg.N // cfg.bn, cfg.K // cfg.bk), -1, dtype=np.int32)
    for b in range(cfg.N // cfg.bn):
        for p in range(ref["row_ptr"][b], ref["row_ptr"][b + 1]):
            exp[b, ref["col_idx"][p]] = p
    np.testing.assert_array_equal(_np(rmap), exp)
    ym = mq.gemm_w4a4_residual(g["xq"], g["sx"], g["wq"], g["sw"], g["row_ptr"], g["col_idx"], g["rq"],
                               cfg.K, bn=cfg.bn, out_dtype=out_dtype, rmap=rmap)
    mdump = torch.empty_like(g["dump"])
    ymd = mq.gemm_w4a4_residual(g["xq"], g["sx"], g["wq"], g["sw"], g["row_ptr"], g["col_idx"], g["rq"],
                                cfg.K, bn=cfg.bn, out_dtype=out_dtype, rmap=rmap, acc_dump=mdump)
    torch.cuda.synchronize()
    assert torch.equal(bits(ym), bits(yp)), "the mapped call differs from the list-walking call"
    assert torch.equal(bits(ymd), bits(yp))
    md = mdump[sel] if rows is None else mdump[torch.as_tensor(rows, device="cuda")]
    np.testing.assert_array_equal(_np(md).astype(np.int64), ref["T"])
    # the GEMM that quantizes its own activations, in both forms (one launch up to 32
    # tokens, and two launches): the same codes and scales as the quantization call,
    # the mapped call's y bits, and the counters back at zero; twice each, so the
    # second one-launch call runs on the reset counters
    sync = mq.sync_words()
    for launch in (("one", "two", "auto") if cfg.M <= 32 else ("two", "auto")):
        for _ in range(2):
            ya, xqa, sxa = mq.gemm_w4a4_residual_act(g["x"], g["wq"], g["sw"], rmap, g["rq"], cfg.K, bn=cfg.bn,
                                                     out_dtype=out_dtype, sync=sync, launch=launch)
            torch.cuda.synchronize()
            assert torch.equal(xqa, g["xq"]) and torch.equal(sxa, g["sx"]), f"quantization differs ({launch})"
            assert torch.equal(bits(ya), bits(ym)), f"the self-quantizing call ({launch}) differs from quantize + GEMM"
            assert not sync.any(), f"counters not reset: {sync.tolist()}"
    if check_variants:
        # dense-only kernel: T = 14 P, and y equals the fused kernel with no residual
        ddump = torch.empty_like(g["dump"])
        yd = mq.gemm_w4a4_dense(g["xq"], g["sx"], g["wq"], g["sw"], cfg.K, out_dtype=out_dtype,
                                acc_dump=ddump)
        ydp = mq.gemm_w4a4_dense(g["xq"], g["sx"], g["wq"], g["sw"], cfg.K, out_dtype=out_dtype)
        empty = torch.zeros(cfg.N // cfg.bn + 1, dtype=torch.int32, device="cuda")
        none = torch.empty(0, dtype=torch.int32, device="cuda")
        y0 = mq.gemm_w4a4_residual(g["xq"], g["sx"], g["wq"], g["sw"], empty, none, none, cfg.K,
                                   bn=cfg.bn, out_dtype=out_dtype)
        y0d = mq.gemm_w4a4_residual(g["xq"], g["sx"], g["wq"], g["sw"], empty, none, none, cfg.K,
                                    bn=cfg.bn, out_dtype=out_dtype, acc_dump=torch.empty_like(g["dump"]))
        torch.cuda.synchronize()
        assert torch.equal(bits(yd), bits(y0))
        assert torch.equal(bits(ydp), bits(yd)), "dense production and debug builds differ"
        assert torch.equal(bits(y0d), bits(y0))
        dd = ddump if rows is None else ddump[torch.as_tensor(rows, device="cuda")]
        np.testing.assert_array_equal(_np(dd).astype(np.int64), 14 * ref["P"].astype(np.int64))
        if k_blocks == 0:
            assert torch.equal(bits(yp), bits(ydp)), "an empty residual must give the dense kernel's bits"
        # the separate-kernel alternative computes the same y within tolerance
        ys = mq.gemm_residual_separate(g["xq"], g["sx"], g["wq"], g["sw"], g["row_ptr"], g["col_idx"],
                                       g["rq"], cfg.K, bn=cfg.bn, out_dtype=out_dtype)
        torch.cuda.synchronize()
        err_s = rel_err(_np(ys)[sel], ref["y"])
        say(f"[parity] {cfg.name} separate-kernel y max rel err {err_s:.3e}")
        assert err_s <= Y_TOL[out_dtype_name]
    del g
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------- the workloads
@pytest.mark.parametrize("name", ["tiny", "llama3_8b_qo", "llama3_8b_up_m4", "llama3_8b_up_m32",
                                  "llama3_8b_down_m4", "llama3_8b_down_m32", "qwen3_32b_up",
                                  "qwen3_32b_down"])
def test_decode_workload(mq, orc, name):
    inp = _inputs(name)
    cfg = inp.cfg
    out = "f32" if name == "tiny" else "bf16"
    _check(mq, orc, inp, cfg.k_blocks(cfg.default_budget), out)


@pytest.mark.parametrize("name", ["llama3_8b_up_m32", "llama3_8b_down_m4"])
@pytest.mark.parametrize("pct", [0, 5, 20])
def test_budget_sweep(mq, orc, name, pct):
    inp = _inputs(name)
    _check(mq, orc, inp, inp.cfg.k_blocks(pct), "bf16", check_variants=(pct == 0))


@pytest.mark.parametrize("pct", [10, 0])
def test_prefill_workload_sampled_rows(mq, orc, pct):
    inp = _inputs("qwen3_14b_prefill")
    rng = np.random.default_rng(123)
    rows = np.concatenate([np.arange(64), np.sort(rng.choice(np.arange(64, inp.cfg.M), 16, replace=False))])
    _check(mq, orc, inp, inp.cfg.k_blocks(pct), "bf16", rows=rows, check_variants=(pct == 10))


# --------------------------------------------------------------------------- edge cases
EDGE = [
    # several tiles of the tiled kernel with ragged M and N tails, 64-row blocks
    synth.custom_config("tiled_ragged", M=300, K=1024, N=320, bn=64),
    synth.custom_config("tiled_bn128", M=100, K=768, N=384, bn=128, x_bos_scale=100.0),
    # skinny kernel edges: one token, 17 and 31 tokens, 128-row blocks
    synth.custom_config("one_token", M=1, K=512, N=256, bn=64, x_bf16=False),
    synth.custom_config("m17", M=17, K=640, N=192, bn=64),
    synth.custom_config("m31_bn128", M=31, K=1280, N=256, bn=128),
    synth.custom_config("m33_tiled_small", M=33, K=256, N=128, bn=64, x_dist="t3"),
    # long K: one wavefront per 4 groups up to 16, plus uneven splits
    synth.custom_config("long_k", M=8, K=128 * 75, N=128, bn=64),
    # residual walks after the K loop over tables of more than 64 column blocks
    # (several ballot chunks): the one-row-tile (mid-size) and three-row-tile kernels
    synth.custom_config("mid_long_k", M=64, K=128 * 72, N=256, bn=64),
    synth.custom_config("wide_long_k", M=400, K=128 * 70, N=256, bn=128),
]


@pytest.mark.parametrize("cfg", EDGE, ids=[c.name for c in EDGE])
@pytest.mark.parametrize("pct", [0, 10, 100])
def test_edge_shapes(mq, orc, cfg, pct):
    inp = _inputs(cfg)
    _check(mq, orc, inp, cfg.k_blocks(pct), "f32" if pct == 10 else "bf16",
           check_variants=(pct != 100))


def test_degenerate_rows_and_groups(mq, orc):
    """All-zero token (sx = 0), all-zero weight groups (s = 0), a group whose fp16
    scale is subnormal, a one-hot group, and every block chosen."""
    cfg = synth.custom_config("degenerate", M=20, K=512, N=128, bn=64)
    inp = synth.make_inputs(cfg)
    inp.X[5] = 0.0
    inp.X_bits[5] = 0
    inp.W[3, 0:128] = 0.0
    inp.W[7, 256:384] = np.float32(2.0 ** -20) * np.float32([7, -3, 1, 0.5] * 32)
    inp.W[9, 128:256] = 0.0
    inp.W[9, 200] = -0.75
    inp.W[70:128, 384:512] = 0.0     # whole zero blocks
    _check(mq, orc, inp, cfg.k_blocks(100), "f32")
    _check(mq, orc, inp, 7, "bf16")


@pytest.mark.parametrize("launch,M", [("one", 4), ("two", 4), ("two", 100), ("two", 400)])
def test_self_quantizing_gemm_in_a_graph(mq, launch, M):
    """The self-quantizing GEMM captured in a HIP graph and replayed several times,
    with eager work and synchronizations between replays: every replay gives the
    eager call's y, codes and scales bit for bit, and (one launch) leaves its
    counters zero, so replays need no clearing. M = 4 runs the decode kernel, 100
    the prefill kernel's mid-size tile and 400 its large tile (two launches)."""
    import torch
    cfg = synth.custom_config("graph_act", M=M, K=2048, N=512, bn=64)
    say(f"[graph] self-quantizing GEMM, launch={launch}, M={cfg.M} K={cfg.K} N={cfg.N}")
    inp = _inputs(cfg)
    x = torch.from_numpy(inp.X).cuda()
    w = torch.from_numpy(inp.W).cuda()
    g = mq.forward_layer(x, w, cfg.k_blocks(10), bn=cfg.bn)
    rmap = mq.block_map(g["row_ptr"], g["col_idx"], cfg.N, cfg.K, bn=cfg.bn)
    sync = mq.sync_words()
    call = lambda **kw: mq.gemm_w4a4_residual_act(x, g["wq"], g["sw"], rmap, g["rq"], cfg.K, bn=cfg.bn,
                                                  sync=sync, launch=launch, **kw)
    ye, xqe, sxe = call()
    torch.cuda.synchronize()
    assert torch.equal(xqe, g["xq"]) and torch.equal(sxe, g["sx"])
    y, xq, sx = torch.empty_like(ye), torch.empty_like(xqe), torch.empty_like(sxe)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(y=y, xq=xq, sx=sx)           # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call(y=y, xq=xq, sx=sx)
    noise = torch.randn(1 << 20, device="cuda")
    for r in range(4):
        y.zero_(); xq.zero_(); sx.zero_()
        noise.mul_(1.0001)                # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ye.view(torch.int16)), f"replay {r}: y differs"
        assert torch.equal(xq, xqe) and torch.equal(sx, sxe), f"replay {r}: codes or scales differ"
        assert not sync.any(), f"replay {r}: counters not reset: {sync.nonzero().flatten().tolist()}"


def test_zero_tokens_no_op(mq):
    import torch
    xq = torch.empty((4, 0, 64), dtype=torch.uint8, device="cuda")
    sx = torch.empty(0, dtype=torch.float32, device="cuda")
    wq = torch.zeros((8, 4, 1024), dtype=torch.uint8, device="cuda")
    sw = torch.zeros((8, 1, 16, 4), dtype=torch.int16, device="cuda")
    rp = torch.zeros(3, dtype=torch.int32, device="cuda")
    none = torch.empty(0, dtype=torch.int32, device="cuda")
    y = mq.gemm_w4a4_residual(xq, sx, wq, sw, rp, none, none, 512, bn=64)
    torch.cuda.synchronize()
    assert y.shape == (0, 128)


def test_quantizer_near_ties(mq, orc):
    """Quotients on and next to half-integers, where a division-free quotient
    would round the other way: base codes (w / s), residual codes (E / s_r) and
    activation codes (x / s_x) must still equal the oracle's correctly rounded
    divisions, bit for bit, through the whole path."""
    import torch
    rng = np.random.default_rng(77)
    N, K, M = 128, 512, 8
    cfg = synth.custom_config("near_ties", M=M, K=K, N=N, bn=64, x_bf16=False)
    s = np.float32(2.0) ** rng.integers(-12, 0, size=(N, K // 128)).astype(np.float32)
    sr = (s / np.float32(14)).astype(np.float32)
    k = rng.integers(-7, 7, size=(N, K)).astype(np.float32)
    j = rng.integers(-7, 7, size=(N, K)).astype(np.float32)
    S = np.repeat(s, 128, axis=1)
    SR = np.repeat(sr, 128, axis=1)
    kind = rng.integers(0, 4, size=(N, K))
    w = np.where(kind == 0, S * (k + np.float32(0.5)),                       # exact base ties
        np.where(kind == 1, np.nextafter(S * (k + np.float32(0.5)), np.float32(np.inf)),
        np.where(kind == 2, S * k + SR * (j + np.float32(0.5)),                # residual near-ties
                 np.nextafter(S * k + SR * (j + np.float32(0.5)), np.float32(-np.inf))))).astype(np.float32)
    w[:, ::128] = np.float32(7.0) * S[:, ::128]                               # absmax 7s -> scale s
    x = (rng.integers(-7, 7, size=(M, K)).astype(np.float32) + np.float32(0.5))
    x[:, 1::3] = np.nextafter(x[:, 1::3], np.float32(0))
    x[:, 0] = 7.0                                                             # s_x = 1
    inp = synth.Inputs(cfg, w, x, None)
    _check(mq, orc, inp, cfg.k_blocks(100), "f32")
    _check(mq, orc, inp, cfg.k_blocks(10), "bf16")


# --------------------------------------------------------------------------- outlier migration
MIGRATION = ["tiny", "llama3_8b_qo",
             synth.custom_config("migrated_tiled", M=300, K=1024, N=320, bn=64, x_channel_scale=80.0)]


@pytest.mark.parametrize("which", MIGRATION, ids=lambda c: c if isinstance(c, str) else c.name)
def test_migrated_layer(mq, orc, which):
    """The migration step on the GPU (factors, W^ = W diag(s), the Hessian and the
    activation quantizer applied to x * r on the fly) and the whole path on the
    migrated layer, against the oracle run on its own migrated X^ and W^: bit-exact
    on s, r, W^, h, Delta, CSR, codes, scales and group sums; y within tolerance."""
    import torch
    inp = _inputs(which)
    cfg = inp.cfg
    kb = cfg.k_blocks(cfg.default_budget)
    say(f"[parity] migrated {cfg.name} M={cfg.M} K={cfg.K} N={cfg.N} k_blocks={kb}")
    xh, wh, s_ref, r_ref = orc.migrate(inp.x_raw(), inp.W)
    ref = orc.forward(xh, wh, kb, cfg.group, cfg.bn, cfg.bk)
    x = _x_dev(inp)
    w = _to_dev(inp.W)
    g = mq.forward_layer(x, w, kb, bn=cfg.bn, out_dtype=torch.float32, migrate=True)
    dump = torch.empty((cfg.M, cfg.N, cfg.K // 128), dtype=torch.int32, device="cuda")
    mq.gemm_w4a4_residual(g["xq"], g["sx"], g["wq"], g["sw"], g["row_ptr"], g["col_idx"], g["rq"], cfg.K,
                          bn=cfg.bn, out_dtype=torch.float32, acc_dump=dump)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(g["s"]), s_ref)
    np.testing.assert_array_equal(_np(g["r"]), r_ref)
    np.testing.assert_array_equal(_np(g["w_hat"]), wh)
    for k in ("h", "delta", "row_ptr", "col_idx", "sx"):
        np.testing.assert_array_equal(_np(g[k]), ref[k], err_msg=k)
    np.testing.assert_array_equal(xq_to_rowmajor(_np(g["xq"]), cfg.M, cfg.K), ref["xq"])
    np.testing.assert_array_equal(wq_to_rowmajor(_np(g["wq"]), cfg.N, cfg.K), ref["wq"])
    sw, pad = sw_to_rowmajor(_np(g["sw"]), cfg.N, cfg.K)
    np.testing.assert_array_equal(sw, ref["sw"])
    np.testing.assert_array_equal(rq_to_twos(_np(g["rq"])), ref["rq"])
    np.testing.assert_array_equal(_np(dump).astype(np.int64), 14 * ref["P"].astype(np.int64) + ref["Pr"])
    err = rel_err(_np(g["y"]), ref["y"])
    say(f"[parity] migrated {cfg.name} y max rel err {err:.3e}")
    assert err <= Y_TOL["f32"]
