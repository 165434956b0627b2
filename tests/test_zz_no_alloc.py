"""The no-allocation selection entry point (mq_select_blocks_noalloc) against the
allocating one (mq_select_blocks), through the raw C ABI: identical CSR lists and
scores, bit for bit, on two calls in a row (the second on a smaller layer, so the
static scratch holds the first call's larger contents), with and without a score
output; a shape beyond the static scratch is refused before any launch."""
import ctypes as C

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _select_both(mq, torch, cfg, pct, with_delta):
    inp = synth.make_inputs(cfg)
    lib = mq.lib()
    x = torch.from_numpy(inp.X).cuda()
    w = torch.from_numpy(inp.W).cuda()
    h = mq.hessian_diag(x)
    N, K, bn = cfg.N, cfg.K, cfg.bn
    nb = (N // bn) * (K // 64)
    kb = cfg.k_blocks(pct)
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = []
    for fn in ("mq_select_blocks", "mq_select_blocks_noalloc"):
        rp = torch.full((N // bn + 1,), -7, dtype=torch.int32, device="cuda")
        ci = torch.full((max(kb, 1),), -7, dtype=torch.int32, device="cuda")
        d = torch.full((nb,), -1.0, dtype=torch.float64, device="cuda") if with_delta else None
        if fn == "mq_select_blocks":
            rc = lib.mq_select_blocks(_p(w), _p(h), N, K, 128, bn, 64, kb, _p(rp), _p(ci), _p(d), None, 0, st)
        else:
            rc = lib.mq_select_blocks_noalloc(_p(w), _p(h), N, K, 128, bn, 64, kb, _p(rp), _p(ci), _p(d), st)
        assert rc == 0, (fn, rc, mq.status_string(rc))
        torch.cuda.synchronize()
        out.append((rp.cpu().numpy(), ci[:kb].cpu().numpy(), None if d is None else d.cpu().numpy()))
    return out


@pytest.mark.parametrize("with_delta", [True, False])
def test_noalloc_select_matches_allocating_call(with_delta):
    import torch
    assert torch.cuda.is_available()
    import dense_sparse_bit_amd as mq
    big = synth.custom_config("noalloc_big", M=32, K=4096, N=2048, bn=64, x_bf16=False)
    small = synth.custom_config("noalloc_small", M=8, K=512, N=256, bn=128, x_bf16=False)
    for cfg, pct in ((big, 10), (small, 20)):
        print(f"[noalloc] {cfg.name} N={cfg.N} K={cfg.K} bn={cfg.bn} pct={pct} delta={with_delta}", flush=True)
        (rp_a, ci_a, d_a), (rp_b, ci_b, d_b) = _select_both(mq, torch, cfg, pct, with_delta)
        np.testing.assert_array_equal(rp_b, rp_a)
        np.testing.assert_array_equal(ci_b, ci_a)
        assert len(ci_a) == cfg.k_blocks(pct)
        if with_delta:
            np.testing.assert_array_equal(d_b.view(np.uint64), d_a.view(np.uint64))


def test_noalloc_select_refuses_shapes_beyond_the_scratch():
    import torch
    assert torch.cuda.is_available()
    import dense_sparse_bit_amd as mq
    lib = mq.lib()
    # a 65536 x 65536 layer in 64 x 64 blocks has NB = 2^20: 12 MiB of ranks and scores
    N, K = 65536, 65536
    fake = C.c_void_p(0x10000)     # never dereferenced: the call fails its size check first
    rc = lib.mq_select_blocks_noalloc(fake, fake, N, K, 128, 64, 64, 5, fake, fake, None, None)
    assert rc == -4 and "static" in mq.status_string(rc)
    # with a score output only the ranks (4 MiB for 2^20 blocks) must fit; one more
    # block row does not
    N2 = 65536 + 64
    rc = lib.mq_select_blocks_noalloc(fake, fake, N2, K, 128, 64, 64, 5, fake, fake, fake, None)
    assert rc == -4
