"""Every branch of the product dispatch, run on the GPU and checked against the fp64 oracle at every
output.  The shapes come from tests/variants.py; before each run the variant query (the same
dispatch code, nothing launched) must name the branch the shape was chosen for, so each case
proves which kernel variant produced the outputs it checks.  Group calls get outputs that are not
back to back, so they run as separate matrices (three or four of them: the kernel's argument-table
path)."""
import numpy as np
import pytest
import torch

import bit_packed_sign_amd as b1
from bit_packed_sign_amd import synth
from parity import TOL, dev_tensors, norm_err
from variants import ALL_CASES, case_id

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _inputs(seed, M, K, Ns, t2):
    r = synth.rng_for(0, synth.WL_TEST, seed)
    x = synth.activations(r, M, K)
    mats = []
    for N in Ns:
        W = synth.ternary_words_fast(r, N, K) if t2 else synth.sign_words(r, N, K)
        S = synth.group_scales(r, N, K)
        S[5::13] = -S[5::13]                       # negative scales fold into the signs
        mats.append((W, S))
    return x, mats


@pytest.mark.parametrize("case", ALL_CASES, ids=case_id)
def test_dispatch_branch_matches_oracle(orc, dev, case):
    op, M, K, Ns, expect, _ = case
    t2 = op.endswith("t2")
    assert b1.kernel_variant(op, M, K, Ns).split(" ")[0] == expect
    seed = 50000 + (K * 7 + M * 131 + sum(Ns)) % 100000
    x, mats = _inputs(seed, M, K, Ns, t2)
    xd, = dev_tensors(dev, x)
    Wd = [dev_tensors(dev, W=W)[0] for W, _ in mats]
    Sd = [dev_tensors(dev, S=S)[0] for _, S in mats]
    # outputs carved from one buffer with gaps (16-byte aligned starts), so no two are back to back
    gap = 64
    starts, off = [], 0
    for N in Ns:
        starts.append(off)
        off = (off + M * N + 7) // 8 * 8 + gap
    ybuf = torch.full((off,), float("nan"), dtype=torch.float16, device=dev)
    outs = [ybuf[a:a + M * N].view(M, N) for a, N in zip(starts, Ns)]
    if op.startswith("prefill"):
        (b1.gemm_prefill_t2 if t2 else b1.gemm_prefill)(xd, Wd[0], Sd[0], out=outs[0])
    elif op == "gemv_ws":
        need = b1.gemv_workspace_bytes(M, K, Ns[0])
        ws = torch.full((need + 512,), 0xFF, dtype=torch.uint8, device=dev)   # stale bytes: fully overwritten
        b1.gemv_ws(xd, Wd[0], Sd[0], workspace=ws[256:256 + need] if need else None, out=outs[0])
        if need:                                # the bytes around the workspace are untouched
            assert bool((ws[:256] == 0xFF).all()) and bool((ws[256 + need:] == 0xFF).all())
    elif len(Ns) == 1:
        (b1.gemv_t2 if t2 else b1.gemv)(xd, Wd[0], Sd[0], out=outs[0])
    else:
        (b1.gemv_group_t2 if t2 else b1.gemv_group)(xd, Wd, Sd, outs=outs)
    torch.cuda.synchronize()
    ends = [a + M * N for a, N in zip(starts, Ns)]
    gaps = torch.cat([ybuf[e:n] for e, n in zip(ends, starts[1:] + [off])])
    assert bool(torch.isnan(gaps).all()), "a kernel wrote outside its output"
    for i, (W, S) in enumerate(mats):
        ref, nrm = (orc.gemv_t2 if t2 else orc.gemv)(x, W, S)
        e = norm_err(outs[i], ref, nrm)
        assert e <= TOL, f"matrix {i}: {e}"
