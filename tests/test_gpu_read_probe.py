"""The streaming-read probe the decode GEMM is measured against reads every byte
it is given: the XOR of its per-workgroup words equals the XOR of the buffer's
32-bit words (computed on the host), at a small size, a ragged size that leaves
some workgroups a partial stride, and a size that caps the grid."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mq():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import dense_sparse_bit_amd
    return dense_sparse_bit_amd


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 9_654_192, (1 << 27) + 16 * 1000])
def test_read_probe_reads_every_word(mq, nbytes):
    import torch
    print(f"[probe] {nbytes} bytes", flush=True)
    sys.stdout.flush()
    rng = np.random.default_rng(nbytes)
    host = rng.integers(-2**31, 2**31, size=nbytes // 4 + 8, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(host).to("cuda")
    out = torch.zeros(mq.READ_PROBE_WORDS, dtype=torch.int32, device="cuda")
    mq.read_probe(buf, nbytes, out=out)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host[: nbytes // 4].view(np.uint32))
    assert got == want
