"""GPU parity of bin1_gemm_prefill (matrix-core path) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import bit_packed_sign_amd as b1
from bit_packed_sign_amd import synth
from parity import TOL, dev_tensors, norm_err, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _case(t, M, K, N):
    r = synth.rng_for(0, synth.WL_TEST, t)
    return synth.activations(r, M, K), synth.sign_words(r, N, K), synth.group_scales(r, N, K)


@pytest.mark.parametrize("M,K,N", [(1, 128, 1), (16, 128, 7), (17, 256, 129), (255, 512, 200),
                                   (256, 4096, 256), (300, 1024, 333), (512, 4096, 384),
                                   (130, 12288, 140), (64, 17408, 64)])
def test_prefill_matches_oracle(orc, dev, M, K, N):
    x, W, S = _case(5000 + M + K + N, M, K, N)
    ref, nrm = orc.gemv(x, W, S)
    y = b1.gemm_prefill(*dev_tensors(dev, x, W, S))
    assert norm_err(y, ref, nrm) <= TOL


def test_prefill_full_size_sampled(orc, dev):
    """M=2048, K=4096, N=12288: every output on the GPU, sampled weight rows checked for all tokens."""
    M, K, N = synth.PREFILL_M, synth.PREFILL_K, synth.PREFILL_N
    x, W, S = _case(5100, M, K, N)
    y = b1.gemm_prefill(*dev_tensors(dev, x, W, S)).float().cpu().numpy()
    rows = sample_rows(synth.rng_for(0, synth.WL_TEST, 5101), N, k=64, edge=16)
    ref, nrm = orc.gemv_rows(x, W, S, rows)
    assert norm_err(y[:, rows], ref, nrm) <= TOL
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("M,K,N", [(512, 4096, 12288), (2100, 256, 12300), (1030, 640, 6000)])
def test_prefill_wide_and_ragged_sampled(orc, dev, M, K, N):
    """A 512-token prompt at full width, ragged M and N over many tiles (2100 x 12300: 1071
    tiles of 128 x 192, the last row and column tiles partial), and an odd step count (K = 640,
    five 128-wide steps); sampled weight rows checked for every token."""
    x, W, S = _case(5300 + M + K + N, M, K, N)
    y = b1.gemm_prefill(*dev_tensors(dev, x, W, S)).float().cpu().numpy()
    rows = sample_rows(synth.rng_for(0, synth.WL_TEST, 5301 + M), N, k=48, edge=16)
    ref, nrm = orc.gemv_rows(x, W, S, rows)
    assert norm_err(y[:, rows], ref, nrm) <= TOL
    assert np.all(np.isfinite(y))


def test_gemv_routes_large_m_to_prefill(orc, dev):
    M, K, N = 40, 256, 50
    x, W, S = _case(5200, M, K, N)
    ref, nrm = orc.gemv(x, W, S)
    assert norm_err(b1.gemv(*dev_tensors(dev, x, W, S)), ref, nrm) <= TOL


def test_prefill_scale_edge_cases(orc, dev):
    """Negative scales (folded into the sign bits), zero, -0 and subnormal scales, an all-zero
    token row, on the prefill kernel: one 128 x 192 tile, ragged, with every lane group's k-slots
    of a step carrying a different scale sign."""
    M, K, N = 100, 1024, 150
    x, W, S = _case(5400, M, K, N)
    S = S.copy()
    S[::3] = -S[::3]
    S[1, ::2] = -S[1, ::2]
    S[2] = 0
    S[4, 1] = np.float16(-0.0)
    S[5] = np.float16(2.0 ** -24)
    S[6, 3:] = np.float16(-3.0e-6)
    x = x.copy()
    x[7] = 0
    ref, nrm = orc.gemv(x, W, S)
    y = b1.gemm_prefill(*dev_tensors(dev, x, W, S))
    assert norm_err(y, ref, nrm) <= TOL
    yn = y.float().cpu().numpy()
    assert np.all(yn[:, 2] == 0) and np.all(yn[7] == 0)
