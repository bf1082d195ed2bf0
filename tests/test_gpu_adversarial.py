"""Adversarial activations through every product path (batch 1 on the block-scaled kernel, whose
activations are split into fp8 limbs; 2 <= M <= 16 on the small-batch kernel; the prefill kernel;
ternary batch 1 and prefill): every fp16 binade, subnormals, +-65504, blocks whose maximum is
2^10 .. 2^24 times the other elements, +0 / -0 blocks and all -0 rows, all-subnormal rows.  Checked
against the fp64 oracle at the 2e-3 bar, and bit for bit where the exact result fits fp16."""
import numpy as np
import pytest
import torch

import bit_packed_sign_amd as b1
from adversarial import KINDS, adversarial_x, onehot_exact
from bit_packed_sign_amd import synth
from parity import TOL, dev_tensors, norm_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


# (path, M, K): M = 1 with an even and an odd number of scale groups, small batches, prefill
PATHS = [("gemv", 1, 4096), ("gemv", 1, 3968), ("gemv", 1, 12288), ("gemv", 4, 4096), ("gemv", 7, 2048),
         ("gemv", 16, 4224),
         ("prefill", 300, 1024), ("gemv_t2", 1, 4096), ("gemv_t2", 1, 3968), ("prefill_t2", 300, 1024)]


def _run(path, xd, Wd, Sd):
    f = {"gemv": b1.gemv, "prefill": b1.gemm_prefill, "gemv_t2": b1.gemv_t2, "prefill_t2": b1.gemm_prefill_t2}[path]
    return f(xd, Wd, Sd)


def _weights(r, path, N, K):
    return synth.ternary_words(r, N, K) if path.endswith("t2") else synth.sign_words(r, N, K)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("path,M,K", PATHS)
def test_adversarial_activations_match_oracle(orc, dev, path, M, K, kind):
    N = 256
    r = synth.rng_for(0, synth.WL_TEST, 60000 + 17 * M + K + 1000 * KINDS.index(kind))
    x = adversarial_x(r, M, K, kind)
    W = _weights(r, path, N, K)
    # small scales keep |y| inside fp16 for the largest activations; unit scales for the
    # all-subnormal rows keep their products above the fp16 output's own spacing
    S = synth.group_scales(r, N, K)
    S = (S.astype(np.float64) * (50.0 if kind == "subnormal" else 1.0 / 64)).astype(np.float16)
    S[7::11] = -S[7::11]
    xd, Wd, Sd = dev_tensors(dev, x, W, S)
    y = _run(path, xd, Wd, Sd)
    ref, nrm = (orc.gemv_t2 if path.endswith("t2") else orc.gemv)(x, W, S)
    assert np.all(np.abs(ref) < 60000)
    assert norm_err(y, ref, nrm) <= TOL


@pytest.mark.parametrize("path,M,K", PATHS)
def test_power_of_two_onehot_is_bit_exact(orc, dev, path, M, K):
    """One +-2^e per 128-group and +-2^f scales: the exact product fits fp16, so every path must
    return it exactly (and the oracle's fp64 value is that exact product)."""
    if K // 128 > 64:
        K = 8192
    N = 300
    r = synth.rng_for(0, synth.WL_TEST, 61000 + M + K)
    x, S = onehot_exact(r, M, K, N)
    W = _weights(r, path, N, K)
    xd, Wd, Sd = dev_tensors(dev, x, W, S)
    y = _run(path, xd, Wd, Sd).cpu().numpy()
    ref, _ = (orc.gemv_t2 if path.endswith("t2") else orc.gemv)(x, W, S)
    want = ref.astype(np.float16)
    assert np.array_equal(want.astype(np.float64), ref), "the exact product does not fit fp16"
    # equal as numbers: every bit of every nonzero output (a zero may carry either sign)
    assert np.array_equal(y.astype(np.float64), want.astype(np.float64))


@pytest.mark.parametrize("path,K", [("gemv", 4096), ("gemv", 3968), ("gemv", 12288), ("gemv_t2", 4096),
                                    ("gemv_t2", 3968)])
def test_limb_conversion_paths_agree(dev, path, K):
    """Batch-1 activations are split into fp8 limbs in packed fp16 when a block's largest magnitude
    lies in [2^-4, 2^8), and in fp32 otherwise.  The split is invariant under power-of-two scaling,
    so activations whose every 32-block maximum is in [2, 4) (packed path) and the same activations
    times 2^7 (maxima in [256, 512): fp32 path) must give outputs exactly 2^7 apart."""
    N = 6144
    r = synth.rng_for(0, synth.WL_TEST, 9300 + K + (7 if path == "gemv_t2" else 0))
    x = r.standard_normal((1, K))
    blk = x.reshape(1, K // 32, 32)
    blk *= (2.0 + 1.999 * r.random((1, K // 32, 1))) / np.abs(blk).max(axis=2, keepdims=True)
    x = blk.reshape(1, K).astype(np.float16)
    mx = np.abs(x.astype(np.float64)).reshape(K // 32, 32).max(axis=1)
    assert mx.min() >= 2.0 and mx.max() < 4.0
    W = synth.ternary_words_fast(r, N, K) if path == "gemv_t2" else synth.sign_words(r, N, K)
    S = synth.group_scales(r, N, K)
    xd, Wd, Sd = dev_tensors(dev, x, W, S)
    xs = torch.from_numpy((x.astype(np.float64) * 128.0).astype(np.float16)).to(dev)
    fn = b1.gemv_t2 if path == "gemv_t2" else b1.gemv
    y = fn(xd, Wd, Sd).float().cpu().numpy().astype(np.float64)
    ys = fn(xs, Wd, Sd).float().cpu().numpy().astype(np.float64)
    # fp16 rounding commutes with the 2^7 scaling wherever y is zero or normal and 2^7 y does not
    # overflow; an fp16-subnormal y (a rare near-cancellation) is left out of the comparison
    assert np.all(np.abs(y) < 500)
    normal = (y == 0) | (np.abs(y) >= 2.0 ** -14)
    assert normal.mean() > 0.99
    assert np.array_equal(ys[normal], y[normal] * 128.0)
