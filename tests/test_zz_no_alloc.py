"""bin1_gemv_noalloc, called through the C ABI: the product of bin1_gemv_ws with the library's own
static scratch array instead of a caller's workspace, for callers that cannot allocate.  Two calls
in a row on one GPU (the second with a smaller shape, so the scratch holds the first call's
partial sums when the second starts) each equal bin1_gemv_ws bit for bit and meet the oracle bar;
shapes needing more than the array's 4 MiB are rejected before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import bit_packed_sign_amd as b1
from bit_packed_sign_amd import binding, synth
from parity import TOL, dev_tensors, norm_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def noalloc():
    f = ctypes.CDLL(binding.LIB_PATH).bin1_gemv_noalloc
    p, i = ctypes.c_void_p, ctypes.c_int
    f.argtypes = [p, p, p, p, i, i, i, p]
    f.restype = i
    return f


def test_noalloc_equals_workspace_call_twice(orc, dev, noalloc):
    for t, (M, K, N) in enumerate([(16, 12288, 4096), (5, 8320, 700)]):   # second call smaller
        r = synth.rng_for(0, synth.WL_TEST, 64000 + t)
        x, W, S = synth.activations(r, M, K), synth.sign_words(r, N, K), synth.group_scales(r, N, K)
        assert b1.gemv_workspace_bytes(M, K, N) > 0            # the split path, which uses scratch
        xd, Wd, Sd = dev_tensors(dev, x, W, S)
        y_ws = b1.gemv_ws(xd, Wd, Sd)
        y = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = noalloc(xd.data_ptr(), Wd.data_ptr(), Sd.data_ptr(), y.data_ptr(), M, K, N, stream)
        assert st == 0, binding.lib().bin1_last_error()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ws), f"call {t}"
        ref, nrm = orc.gemv(x, W, S)
        assert norm_err(y, ref, nrm) <= TOL


def test_noalloc_rejects_shapes_beyond_its_scratch(noalloc):
    # 5 chunks x 16 tokens x 30000 rows x 4 bytes = 9.6 MB > 4 MiB; checked before any pointer is used
    assert b1.gemv_workspace_bytes(16, 20480, 30000) > 4 << 20
    st = noalloc(0x10000, 0x20000, 0x30000, 0x40000, 16, 20480, 30000, None)
    assert st == -2 and b"4 MiB" in binding.lib().bin1_last_error()
