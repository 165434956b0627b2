"""Host-only checks of the C ABI: the library loads, exports every symbol that
include/mq.h declares, and rejects bad arguments before any launch (so these
run without a GPU)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mq.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mq_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def mq():
    lib = os.path.join(ROOT, "dense_sparse_bit_amd", "libmq.so")
    if not os.path.exists(lib):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_mq_build", os.path.join(ROOT, "dense_sparse_bit_amd", "_build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    import dense_sparse_bit_amd
    return dense_sparse_bit_amd


def test_header_declares_the_boundary():
    names = _declared()
    for fn in ["mq_quantize_act", "mq_pack_weights", "mq_select_blocks", "mq_gemm_w4a4_residual",
               "mq_select_workspace_bytes", "mq_block_map", "mq_gemm_w4a4_residual_mapped",
               "mq_gemm_w4a4_residual_act", "mq_read_probe",
               "mq_hessian_diag", "mq_gemm_w4a4_dense", "mq_gemm_residual_separate",
               "mq_status_string", "mq_version"]:
        assert fn in names


def test_library_exports_every_declared_symbol(mq):
    lib = C.CDLL(mq.LIB_PATH)
    for fn in _declared():
        assert hasattr(lib, fn), fn
    assert set(_declared()) == set(mq.EXPORTS)
    assert mq.version() == 10100
    for s in (0, -1, -2, -3, -4):
        assert mq.status_string(s)


FAKE = 0x10000   # never dereferenced: every call below fails its checks first


@pytest.fixture(scope="module")
def lib_nogpu(mq):
    """The raw library, only where no GPU is visible: a fake-pointer call that
    slipped past a check would launch, which must never happen on a real GPU."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only argument checks run where no GPU is visible")
    return mq.lib()


def _gemm(lib, **kw):
    a = dict(xq=FAKE, sx=FAKE, wq=FAKE, sw=FAKE, row_ptr=FAKE, col_idx=FAKE, rq=FAKE, nnz=10, M=4,
             N=512, K=512, group=128, bn=64, bk=64, y=FAKE, y_dtype=1, dump=None, stream=None)
    a.update(kw)
    return lib.mq_gemm_w4a4_residual(a["xq"], a["sx"], a["wq"], a["sw"], a["row_ptr"], a["col_idx"],
                                     a["rq"], a["nnz"], a["M"], a["N"], a["K"], a["group"], a["bn"],
                                     a["bk"], a["y"], a["y_dtype"], a["dump"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(K=500), -2), (dict(K=192), -2), (dict(N=500), -2), (dict(group=64), -2),
    (dict(bk=32), -2), (dict(bn=32), -2), (dict(bn=128, N=64 * 3), -2), (dict(N=0), -1),
    (dict(M=-1), -1), (dict(y_dtype=7), -1), (dict(xq=None), -1), (dict(wq=None), -1),
    (dict(sw=None), -1), (dict(row_ptr=None), -1), (dict(col_idx=None), -1), (dict(rq=None), -1),
    (dict(xq=FAKE + 8), -1), (dict(rq=FAKE + 4), -1), (dict(nnz=-1), -1), (dict(nnz=65), -1),
    (dict(sw=FAKE + 2), -1), (dict(K=65536 + 128), -2),
])
def test_gemm_rejects_bad_arguments(lib_nogpu, kw, status):
    assert _gemm(lib_nogpu, **kw) == status


def test_zero_tokens_is_a_no_op(lib_nogpu):
    # M == 0 returns before any launch, even with no activation buffers
    assert _gemm(lib_nogpu, M=0, xq=None, sx=None, y=None) == 0


def test_preparation_calls_reject_bad_arguments(lib_nogpu):
    lib = lib_nogpu
    assert lib.mq_quantize_act(FAKE, 1, 4, 511, FAKE, FAKE, None) == -1
    assert lib.mq_quantize_act(FAKE, 3, 4, 512, FAKE, FAKE, None) == -1
    assert lib.mq_quantize_act(None, 1, 0, 512, None, None, None) == 0
    assert lib.mq_hessian_diag(FAKE, 1, 0, 512, FAKE, None) == -1
    assert lib.mq_hessian_diag(None, 1, 4, 512, FAKE, None) == -1
    nb = (512 // 64) * (512 // 64)
    assert lib.mq_select_blocks(FAKE, FAKE, 512, 512, 128, 64, 64, nb + 1, FAKE, FAKE, FAKE, None, 0, None) == -1
    assert lib.mq_select_blocks(FAKE, FAKE, 512, 512, 128, 64, 64, -1, FAKE, FAKE, FAKE, None, 0, None) == -1
    assert lib.mq_select_blocks(FAKE, FAKE, 512, 500, 128, 64, 64, 3, FAKE, FAKE, FAKE, None, 0, None) == -2
    # a workspace smaller than the scratch the call needs, or misaligned, is rejected before
    # any launch: 4 * NB bytes of ranks, plus 8 * NB of scores when delta is NULL
    assert lib.mq_select_workspace_bytes(512, 512, 64, 64) == 12 * nb
    assert lib.mq_select_blocks(FAKE, FAKE, 512, 512, 128, 64, 64, 3, FAKE, FAKE, FAKE, FAKE,
                                4 * nb - 1, None) == -1
    assert lib.mq_select_blocks(FAKE, FAKE, 512, 512, 128, 64, 64, 3, FAKE, FAKE, None, FAKE,
                                12 * nb - 1, None) == -1
    assert lib.mq_select_blocks(FAKE, FAKE, 512, 512, 128, 64, 64, 3, FAKE, FAKE, FAKE, FAKE + 4,
                                4 * nb, None) == -1
    assert lib.mq_select_blocks(FAKE, FAKE, 512, 512, 128, 64, 64, 3, None, FAKE, FAKE, None, 0, None) == -1
    assert lib.mq_pack_weights(FAKE, 512, 512, 128, 64, 64, None, FAKE, 3, FAKE, FAKE, FAKE, None) == -1
    assert lib.mq_pack_weights(FAKE + 4, 512, 512, 128, 64, 64, FAKE, FAKE, 3, FAKE, FAKE, FAKE, None) == -1
    assert lib.mq_gemm_w4a4_dense(FAKE, FAKE, FAKE, FAKE, 4, 512, 320, 128, FAKE, 0, None, None) == -2
    assert lib.mq_gemm_residual_separate(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 3, 4, 512, 512,
                                         128, 64, 64, FAKE, 0, None, None) == -1
    # the no-allocation selection refuses a shape whose ranks (and scores, with no
    # delta output) exceed its static scratch, before touching the device
    assert lib.mq_select_blocks_noalloc(FAKE, FAKE, 65536, 65536, 128, 64, 64, 5, FAKE, FAKE, None,
                                        None) == -4
    assert lib.mq_select_blocks_noalloc(FAKE, FAKE, 65536 + 64, 65536, 128, 64, 64, 5, FAKE, FAKE,
                                        FAKE, None) == -4
    assert lib.mq_select_blocks_noalloc(FAKE, FAKE, 512, 512, 128, 64, 64, nb + 1, FAKE, FAKE, FAKE,
                                        None) == -1
    # the packed activation layout is group-major, so K must be a multiple of 128
    assert lib.mq_quantize_act(FAKE, 1, 4, 130, FAKE, FAKE, None) == -2
    # block map: outputs and lists are checked, shapes as for the other calls
    assert lib.mq_block_map(FAKE, FAKE, 3, 512, 512, 64, 64, None, None) == -1
    assert lib.mq_block_map(None, FAKE, 3, 512, 512, 64, 64, FAKE, None) == -1
    assert lib.mq_block_map(FAKE, None, 3, 512, 512, 64, 64, FAKE, None) == -1
    assert lib.mq_block_map(FAKE, FAKE, nb + 1, 512, 512, 64, 64, FAKE, None) == -1
    assert lib.mq_block_map(FAKE, FAKE, 3, 512, 500, 64, 64, FAKE, None) == -2
    # the mapped GEMM needs a map, a 16-byte aligned payload, and 32-bit payload offsets
    mapped = lambda **kw: lib.mq_gemm_w4a4_residual_mapped(
        FAKE, FAKE, FAKE, FAKE, kw.get("rmap", FAKE), kw.get("rq", FAKE), kw.get("nnz", 3), 4,
        kw.get("N", 512), kw.get("K", 512), 128, kw.get("bn", 64), 64, FAKE, 1, None, None)
    assert mapped(rmap=None) == -1
    assert mapped(rq=None) == -1
    assert mapped(rq=FAKE + 4) == -1
    assert mapped(nnz=nb + 1) == -1
    assert mapped(K=320) == -2
    assert mapped(N=1 << 17, K=65536, bn=128, nnz=(1 << 31) // (128 * 32) + 1) == -2
    # the self-quantizing GEMM: activations, map and (for one launch) the counters are required
    act = lambda **kw: lib.mq_gemm_w4a4_residual_act(
        kw.get("x", FAKE), kw.get("xd", 1), FAKE, FAKE, kw.get("rmap", FAKE), FAKE, 3, kw.get("M", 4),
        kw.get("N", 512), kw.get("K", 512), 128, 64, 64, FAKE, FAKE, kw.get("sync", FAKE), kw.get("launch", 1),
        FAKE, 1, None)
    assert act(x=None) == -1
    assert act(x=FAKE + 8) == -1
    assert act(xd=5) == -1
    assert act(rmap=None) == -1
    assert act(sync=None) == -1
    assert act(sync=FAKE + 2) == -1
    assert act(launch=3) == -1 and act(launch=-1) == -1
    assert act(M=33) == -1, "one launch takes at most 32 tokens"
    # "auto" takes one launch for one token of 8192 inputs over 4096 columns (16-wave
    # producers): then the counters are required
    assert lib.mq_act_one_launch(1, 4096, 8192) == 1
    assert act(launch=0, M=1, N=4096, K=8192, sync=None) == -1
    assert act(M=0, x=None, sync=None) == 0


def test_read_probe_rejections(lib_nogpu):
    probe = lambda p=FAKE, n=4096, out=FAKE: lib_nogpu.mq_read_probe(p, n, out, None)
    assert probe(n=4004) == -1                  # not a multiple of 16
    assert probe(p=FAKE + 8) == -1               # unaligned
    assert probe(p=None) == -1 and probe(out=None) == -1
    assert probe(n=-16) == -1
    assert probe(n=0, p=None) == 0


def test_act_launch_rule(mq):
    """The library's "auto" rule for the self-quantizing GEMM (mq_act_one_launch, a
    host function), on shapes where it was measured, and the header's constants as
    the binding uses them."""
    txt = open(HEADER).read()
    defs = dict(re.findall(r"#define (MQ_[A-Z_]+) (\d+)", txt))
    assert int(defs["MQ_SYNC_WORDS"]) == mq.SYNC_WORDS
    assert [int(defs[k]) for k in ("MQ_ACT_AUTO", "MQ_ACT_ONE_LAUNCH", "MQ_ACT_TWO_LAUNCHES")] == \
        [mq._ACT_LAUNCH[k] for k in ("auto", "one", "two")]
    rule = mq.act_one_launch   # (M, N, K)
    # one token over 4096 to 8192 columns: one launch (its producers are as wide as
    # the stand-alone quantizer)
    assert rule(1, 4096, 4096) and rule(1, 5120, 5120) and rule(1, 4096, 14336) and rule(1, 8192, 8192)
    # narrow layers, and more than one token: two launches
    assert not rule(1, 1024, 4096) and not rule(1, 1024, 8192)
    assert not rule(4, 4096, 14336) and not rule(16, 4096, 14336) and not rule(32, 4096, 14336)
    assert not rule(4, 4096, 4096) and not rule(8, 5120, 5120) and not rule(16, 1024, 4096)
    # producers narrower than the stand-alone quantizer: two launches at any M
    assert not rule(1, 5120, 25600) and not rule(1, 8192, 28672) and not rule(1, 14336, 4096)
    assert not rule(1, 12288, 12288) and not rule(1, 28672, 8192)
    assert not rule(33, 16, 1 << 16) and not rule(0, 4096, 4096), "one launch takes 1..32 tokens"
    assert not rule(1, 1 << 40, 4096) and not rule(1, 4096, 1 << 40), "no plan outside the GEMM's shapes"
    assert rule(64, 1, 1, "one") and not rule(1, 1024, 4096, "two")


def test_binding_fails_loudly_without_library(tmp_path):
    """The package has no fallback: with the library absent, import raises."""
    import subprocess
    import sys
    pkg = os.path.join(ROOT, "dense_sparse_bit_amd")
    dst = tmp_path / "dense_sparse_bit_amd"
    dst.mkdir()
    (dst / "__init__.py").write_text(open(os.path.join(pkg, "__init__.py")).read())
    # and the build script still runs there (it does not import the package)
    import shutil
    shutil.copy(os.path.join(pkg, "_build.py"), dst / "_build.py")
    r = subprocess.run([sys.executable, "-c", "import dense_sparse_bit_amd"], cwd=str(tmp_path),
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "libmq.so is missing" in r.stderr


# --------------------------------------------------------------------------- binding checks
def test_binding_rejects_bad_buffers(mq):
    """The Python binding checks every caller-supplied tensor (type, dtype, size,
    contiguity, device) before a pointer reaches the library. Run on host tensors:
    each call must fail in the binding, never launch."""
    import torch
    M, N, K = 4, 64, 256
    xq = torch.zeros((K // 128, M, 64), dtype=torch.uint8)
    sx = torch.zeros(M, dtype=torch.float32)
    wq = torch.zeros((N // 16, K // 128, 1024), dtype=torch.uint8)
    sw = torch.zeros((N // 16, 1, 16, 4), dtype=torch.int16)
    rp = torch.zeros(N // 64 + 1, dtype=torch.int32)
    ci = torch.zeros(2, dtype=torch.int32)
    rq = torch.zeros((2, 64, 32), dtype=torch.uint8)
    none = torch.zeros(0, dtype=torch.int32)
    # too-small outputs and dumps
    with pytest.raises(ValueError, match="y holds"):
        mq.gemm_w4a4_residual(xq, sx, wq, sw, rp, none, none, K, y=torch.zeros((M, N - 1)))
    with pytest.raises(ValueError, match="acc_dump holds"):
        mq.gemm_w4a4_dense(xq, sx, wq, sw, K, y=torch.zeros((M, N)),
                           acc_dump=torch.zeros((M, N, 1), dtype=torch.int32))
    with pytest.raises(ValueError, match="ws holds"):
        mq.gemm_residual_separate(xq, sx, wq, sw, rp, none, none, K, ws=torch.zeros((M, N - 1)))
    # too-small packed inputs, wrong dtypes
    with pytest.raises(ValueError, match="xq holds"):
        mq.gemm_w4a4_dense(xq[:, :2], sx, wq, sw, K)
    with pytest.raises(ValueError, match="sw holds"):
        mq.gemm_w4a4_dense(xq, sx, wq, sw[:2], K)
    with pytest.raises(ValueError, match="rq holds"):
        mq.gemm_w4a4_residual(xq, sx, wq, sw, rp, ci, rq[:1], K)
    with pytest.raises(ValueError, match="row_ptr holds"):
        mq.gemm_w4a4_residual(xq, sx, wq, sw, rp[:1], ci, rq, K)
    with pytest.raises(TypeError, match="sx must have dtype"):
        mq.gemm_w4a4_dense(xq, sx.double(), wq, sw, K)
    with pytest.raises(TypeError, match="y must have dtype"):
        mq.gemm_w4a4_dense(xq, sx, wq, sw, K, y=torch.zeros((M, N), dtype=torch.float64))
    with pytest.raises(ValueError, match="multiple of 128"):
        mq.gemm_w4a4_dense(xq, sx, wq, sw, 200)
    # a strided (non-contiguous) output of the right size
    with pytest.raises(ValueError, match="contiguous"):
        mq.gemm_w4a4_dense(xq, sx, wq, sw, K, y=torch.zeros((N, M)).t())
    # host tensors of the right size never reach the library
    with pytest.raises(ValueError, match="device tensor"):
        mq.gemm_w4a4_dense(xq, sx, wq, sw, K, y=torch.zeros((M, N)))
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="xq holds"):
        mq.quantize_act(x, xq=torch.zeros(M * K // 2 - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="sx holds"):
        mq.quantize_act(x, sx=torch.zeros(M - 1))
    w = torch.zeros((N, K), dtype=torch.float32)
    h = torch.zeros(K, dtype=torch.float32)
    with pytest.raises(ValueError, match="k_blocks"):
        mq.select_blocks(w, h, (N // 64) * (K // 64) + 1)
    with pytest.raises(ValueError, match="col_idx holds"):
        mq.select_blocks(w, h, 3, out=(rp, ci, torch.zeros(4, dtype=torch.float64)))
    with pytest.raises(ValueError, match="wq holds"):
        mq.pack_weights(w, rp, ci, out=(wq[:1], sw, rq))
