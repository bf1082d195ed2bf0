"""GPU parity of the ternary g128 products (2-bit slots) against the fp64 oracle: the batch-1
block-scaled kernel (every K variant, ragged N, odd group counts), other batch sizes and the
prefill kernel, zero and never-written codes, negative and zero scales, full-size sampled rows.
The normaliser is sum_k |s t x|, the terms the product actually adds."""
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
    x = synth.activations(r, M, K)
    T = synth.ternary_words(r, N, K)
    S = synth.group_scales(r, N, K)
    S[::7] = -S[::7]                                   # negative scales fold into the signs
    S[3::11, 0] = np.float16(0.0)
    return x, T, S


# K values cover every kernel variant (pairs per wave 1..5), odd group counts (K/128 odd) and a
# last 1024-wide pair that is partly filled
DECODE = [(128, 1), (384, 1000), (640, 33), (1024, 4096), (4096, 4096), (4096, 6144), (5120, 5120),
          (9216, 300), (12288, 4096), (13312, 77), (17408, 5120), (20480, 64)]


@pytest.mark.parametrize("K,N", DECODE)
def test_ternary_decode_matches_oracle(orc, dev, K, N):
    x, T, S = _case(11000 + K + N, 1, K, N)
    xd, Td, Sd = dev_tensors(dev, x, T, S)
    y = b1.gemv_t2(xd, Td, Sd)
    rows = sample_rows(synth.rng_for(0, synth.WL_TEST, 11001 + N), N, k=384) if N > 2048 else np.arange(N)
    ref, nrm = orc.gemv_t2_rows(x, T, S, rows)
    assert norm_err(y.float().cpu().numpy()[:, rows], ref, nrm) <= TOL


@pytest.mark.parametrize("M,K,N", [(2, 512, 300), (5, 4096, 1024), (16, 12288, 130), (300, 640, 200),
                                   (1, 24576, 96)])
def test_ternary_other_batches_match_oracle(orc, dev, M, K, N):
    """M > 1 (and K past the batch-1 kernel's range) run on the prefill kernel."""
    x, T, S = _case(12000 + M + K + N, M, K, N)
    xd, Td, Sd = dev_tensors(dev, x, T, S)
    ref, nrm = orc.gemv_t2(x, T, S)
    assert norm_err(b1.gemv_t2(xd, Td, Sd), ref, nrm) <= TOL


@pytest.mark.parametrize("M,K,N", [(256, 4096, 192), (513, 1024, 777), (2048, 4096, 12288), (2100, 256, 12300)])
def test_ternary_prefill_matches_oracle(orc, dev, M, K, N):
    x, T, S = _case(13000 + M + N, M, K, N)
    xd, Td, Sd = dev_tensors(dev, x, T, S)
    y = b1.gemm_prefill_t2(xd, Td, Sd)
    r = synth.rng_for(0, synth.WL_TEST, 13001 + N)
    rows = sample_rows(r, N, k=96) if N > 1024 else np.arange(N)
    ms = sample_rows(r, M, k=96) if M > 600 else np.arange(M)
    ref, nrm = orc.gemv_t2_rows(x[ms], T, S, rows)
    assert norm_err(y.float().cpu().numpy()[np.ix_(ms, rows)], ref, nrm) <= TOL


@pytest.mark.parametrize("M", [1, 3, 256])
def test_ternary_zero_and_unwritten_codes(orc, dev, M):
    """Rows of only 00 or only 10 codes give exactly 0; 10 codes mixed into a row read as 0."""
    K, N = 1024, 64
    x, T, S = _case(14000 + M, M, K, N)
    T[0] = 0
    T[1] = np.uint32(0xAAAAAAAA)                       # every slot 10
    T[2] = T[2] | (np.uint32(0xAAAAAAAA) & ~(T[2] << np.uint32(1)))   # 00 -> 10, 01 and 11 kept
    xd, Td, Sd = dev_tensors(dev, x, T, S)
    y = b1.gemv_t2(xd, Td, Sd) if M < 256 else b1.gemm_prefill_t2(xd, Td, Sd)
    ref, nrm = orc.gemv_t2(x, T, S)
    yh = y.float().cpu().numpy()
    assert np.all(yh[:, :2] == 0.0)
    assert norm_err(yh, ref, nrm) <= TOL


def test_ternary_decode_full_27b_mlp_sampled(orc, dev):
    """27B MLP shapes at full size in one process: gate 5120x17408 and down 17408x5120."""
    for K, N in [(5120, 17408), (17408, 5120)]:
        x, T, S = _case(15000 + K, 1, K, N)
        xd, Td, Sd = dev_tensors(dev, x, T, S)
        y = b1.gemv_t2(xd, Td, Sd)
        rows = sample_rows(synth.rng_for(0, synth.WL_TEST, 15001 + K), N, k=256)
        ref, nrm = orc.gemv_t2_rows(x, T, S, rows)
        assert norm_err(y.float().cpu().numpy()[:, rows], ref, nrm) <= TOL


def test_ternary_repeated_calls_are_deterministic(dev):
    x, T, S = _case(16000, 1, 4096, 12288)
    xd, Td, Sd = dev_tensors(dev, x, T, S)
    y0 = b1.gemv_t2(xd, Td, Sd)
    for _ in range(3):
        assert torch.equal(b1.gemv_t2(xd, Td, Sd), y0)


@pytest.mark.parametrize("M,K,Ns", [(1, 4096, (4096, 1024, 1024)), (1, 5120, (17408, 17408)), (1, 384, (7, 33, 100, 16)),
                                    (3, 1024, (300, 65))])
def test_ternary_group_matches_oracle_and_separate_calls(orc, dev, M, K, Ns):
    r = synth.rng_for(0, synth.WL_TEST, 17000 + K + sum(Ns) + M)
    x = synth.activations(r, M, K)
    Ts = [synth.ternary_words(r, n, K) for n in Ns]
    Ss = [synth.group_scales(r, n, K) for n in Ns]
    xd = dev_tensors(dev, x)[0]
    Td = [dev_tensors(dev, W=T)[0] for T in Ts]
    Sd = [dev_tensors(dev, S=S)[0] for S in Ss]
    outs = b1.gemv_group_t2(xd, Td, Sd)
    for T, S, Tdev, Sdev, y in zip(Ts, Ss, Td, Sd, outs):
        N = T.shape[0]
        rows = sample_rows(r, N, k=128) if N > 2048 else np.arange(N)
        ref, nrm = orc.gemv_t2_rows(x, T, S, rows)
        assert norm_err(y.float().cpu().numpy()[:, rows], ref, nrm) <= TOL
        assert torch.equal(b1.gemv_t2(xd, Tdev, Sdev), y)


@pytest.mark.parametrize("K,Ns", [(4096, (4096, 1024, 1024)), (5120, (17408, 17408)), (384, (8, 40, 104, 17))])
def test_ternary_group_back_to_back(orc, dev, K, Ns):
    """Ternary matrices stored back to back (slots, scales and outputs) run as one taller matrix
    at M == 1; outputs match the oracle and the one-call-per-matrix results bit for bit."""
    r = synth.rng_for(0, synth.WL_TEST, 17500 + K + sum(Ns))
    x = synth.activations(r, 1, K)
    Ts = [synth.ternary_words(r, n, K) for n in Ns]
    Ss = [synth.group_scales(r, n, K) for n in Ns]
    xd = dev_tensors(dev, x)[0]
    T_all = dev_tensors(dev, W=np.concatenate(Ts))[0]
    S_all = dev_tensors(dev, S=np.concatenate(Ss))[0]
    y_all = torch.full((1, sum(Ns)), float("nan"), dtype=torch.float16, device=dev)
    offs = np.concatenate([[0], np.cumsum(Ns)])
    Tv = [T_all[a:b] for a, b in zip(offs[:-1], offs[1:])]
    Sv = [S_all[a:b] for a, b in zip(offs[:-1], offs[1:])]
    yv = [y_all[:, a:b] for a, b in zip(offs[:-1], offs[1:])]
    outs = b1.gemv_group_t2(xd, Tv, Sv, outs=yv)
    for T, S, Tdev, Sdev, y in zip(Ts, Ss, Tv, Sv, outs):
        N = T.shape[0]
        rows = sample_rows(r, N, k=128) if N > 2048 else np.arange(N)
        ref, nrm = orc.gemv_t2_rows(x, T, S, rows)
        assert norm_err(y.float().cpu().numpy()[:, rows], ref, nrm) <= TOL
        assert torch.equal(b1.gemv_t2(xd, Tdev, Sdev), y)
