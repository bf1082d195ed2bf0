"""The two measurement helpers behind the bench's on-device references (no arithmetic of the
method): bin1_stream_read folds every 32-bit word of the buffer into per-wave XOR digests, so the
XOR of all digests equals the XOR of the buffer's words; bin1_mfma_rate's per-wave digest is
12 * iters * (A B)[0, 0], exact for small integer operands, computed here from the same lane
fragments laid out as the 32 x 32 x 16 fp16 product reads them."""
import numpy as np
import pytest
import torch

import bit_packed_sign_amd as b1

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.mark.parametrize("nbytes,grid,unroll", [(16, 1, 4), (1 << 20, 64, 8), ((1 << 20) + 48, 37, 16),
                                                 (64 << 20, 2048, 8)])
def test_stream_read_reads_every_word(dev, nbytes, grid, unroll):
    g = torch.Generator().manual_seed(nbytes + grid)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    buf = host.to(dev)
    sink = torch.full((4 * grid,), 0x5A5A5A5A, dtype=torch.int32, device=dev)
    b1.stream_read(buf, sink, grid, unroll)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want


def _fragments(seed):
    """Small-integer A (32 x 16) and B (16 x 32) and their lane fragments: lane l holds A[l % 32, 8 (l // 32)
    .. + 7] and B[8 (l // 32) .. + 7, l % 32]."""
    g = np.random.default_rng(seed)
    A = g.integers(-8, 9, (32, 16)).astype(np.float64)
    B = g.integers(-8, 9, (16, 32)).astype(np.float64)
    frag = np.zeros((2, 64, 8), np.float16)
    for l in range(64):
        r, h = l % 32, l // 32
        frag[0, l] = A[r, 8 * h:8 * h + 8]
        frag[1, l] = B[8 * h:8 * h + 8, r]
    return A, B, frag


@pytest.mark.parametrize("grid,waves,iters,seed", [(1, 4, 1, 1), (256, 4, 100, 2), (512, 8, 1000, 3)])
def test_mfma_rate_digest(dev, grid, waves, iters, seed):
    A, B, frag = _fragments(seed)
    d00 = (A @ B)[0, 0]
    assert abs(d00) * 12 * iters < 2 ** 24                       # every partial sum exact in fp32
    sink = torch.full((grid * waves,), float("nan"), dtype=torch.float32, device=dev)
    b1.mfma_rate(torch.from_numpy(frag).to(dev), sink, grid, waves, iters)
    assert torch.all(sink.cpu() == float(12 * iters * d00))
