"""Host-side checks of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments before touching the GPU (no kernel is launched by these tests)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bin1.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bin1_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    from bit_packed_sign_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from bit_packed_sign_amd import build
        build.build()
    return binding.lib()


def test_header_declares_the_entry_points():
    names = _declared()
    for fn in ["bin1_gemv", "bin1_gemv_group", "bin1_gemm_prefill", "bin1_gemv_pm1", "bin1_xor_patch_apply",
               "bin1_xor_patch_apply_multi", "bin1_xor_bits_apply", "bin1_rank_rows_by_scale",
               "bin1_gemv_t2", "bin1_gemm_prefill_t2", "bin1_gemv_group_t2",
               "bin1_status_string", "bin1_last_error", "bin1_abi_version"]:
        assert fn in names


def test_library_exports_every_declared_symbol(L):
    raw = ctypes.CDLL(os.path.join(ROOT, "bit_packed_sign_amd", "libbin1.so"))
    for fn in _declared():
        assert hasattr(raw, fn), fn


def test_binding_covers_every_declared_symbol():
    from bit_packed_sign_amd import binding
    assert sorted(binding._SIGS) == _declared()


def test_version_and_status_strings(L):
    assert L.bin1_abi_version() == 1
    for st in range(0, -7, -1):
        assert L.bin1_status_string(st).startswith(b"BIN1_")
    assert b"unknown" in L.bin1_status_string(42)


FAKE = 0x10000  # 16-byte-aligned fake address: never dereferenced, checks fail before use


@pytest.mark.parametrize("fn", ["bin1_gemv", "bin1_gemm_prefill", "bin1_gemv_t2", "bin1_gemm_prefill_t2"])
def test_product_validation(L, fn):
    f = getattr(L, fn)
    assert f(None, FAKE, FAKE, FAKE, 1, 128, 1, None) == -1
    assert b"non-NULL" in L.bin1_last_error()
    # a product with no outputs returns at once, its pointers unread (NULL allowed)
    assert f(None, None, None, None, 0, 128, 1, None) == 0
    assert f(None, None, None, None, 3, 128, 0, None) == 0
    assert f(None, None, None, None, 0, 100, 1, None) == -2     # K is checked first
    assert f(FAKE, FAKE, FAKE, FAKE * 2, -1, 128, 1, None) == -2
    assert f(FAKE, FAKE, FAKE, FAKE * 2, 1, 128, -1, None) == -2
    assert f(FAKE, FAKE, FAKE, FAKE * 2, 1, 100, 1, None) == -2
    assert f(FAKE, FAKE, FAKE, FAKE * 2, 1, 0, 1, None) == -2
    assert f(FAKE, FAKE, FAKE, FAKE * 2, 1, 128, 1 << 24, None) == -2            # rows past 24-bit
    assert f(FAKE, FAKE, FAKE, FAKE * 2, 1, 1 << 20, 1 << 14, None) == -2        # Wbits of 2 GiB
    assert b"2 GiB" in L.bin1_last_error()
    assert f(FAKE + 2, FAKE * 3, FAKE * 4, FAKE * 5, 1, 128, 1, None) == -3
    # y overlapping x (x occupies M*K*2 bytes from FAKE)
    assert f(FAKE, FAKE * 8, FAKE * 9, FAKE + 128, 1, 128, 1, None) == -4
    assert b"overlaps" in L.bin1_last_error()


def test_group_validation(L):
    arr = (ctypes.c_void_p * 2)
    n = (ctypes.c_int * 2)(8, 8)
    assert L.bin1_gemv_group(FAKE, 0, None, None, None, None, 1, 128, None) == -2
    assert L.bin1_gemv_group(FAKE, 5, None, None, None, None, 1, 128, None) == -2
    assert L.bin1_gemv_group(FAKE, 2, None, None, None, n, 1, 128, None) == -1
    # y[0] overlaps W[1]
    W = arr(FAKE * 4, FAKE * 8)
    S = arr(FAKE * 12, FAKE * 16)
    Y = arr(FAKE * 8 + 16, FAKE * 20)
    assert L.bin1_gemv_group(FAKE, 2, W, S, Y, n, 1, 128, None) == -4
    # Back-to-back matrices (weights, scales and outputs of matrix 1 each right after matrix 0's,
    # which a batch-1 call runs as one taller matrix) whose second output covers the first
    # matrix's weights: each output is clear of its own inputs, so only the check over the
    # caller's whole list (made before the merge) sees the overlap.
    n64 = (ctypes.c_int * 2)(64, 64)
    y0 = 0x1000000
    W0 = y0 + 128                        # y1 = y0 + 64 halves = W0
    Wm = arr(W0, W0 + 64 * 16)
    Sm = arr(0x2000000, 0x2000000 + 128)
    Ym = arr(y0, y0 + 128)
    assert L.bin1_gemv_group(0x3000000, 2, Wm, Sm, Ym, n64, 1, 128, None) == -4
    # every product empty: nothing to do
    assert L.bin1_gemv_group(None, 2, arr(None, None), arr(None, None), arr(None, None), n, 0, 128, None) == 0
    z = (ctypes.c_int * 2)(0, 0)
    assert L.bin1_gemv_group(None, 2, arr(None, None), arr(None, None), arr(None, None), z, 1, 128, None) == 0


def test_chain_validation(L):
    from bit_packed_sign_amd import binding
    assert L.bin1_chain_workspace_bytes(0) == 0
    assert L.bin1_chain_workspace_bytes(3) > 3 * 256 * 4
    plan = binding._Plan()
    assert L.bin1_chain_prepare(None, 1, FAKE, 1 << 20, ctypes.byref(plan)) == -1
    st = (binding._Stage * 1)()
    assert L.bin1_chain_prepare(ctypes.cast(st, ctypes.c_void_p), 0, FAKE, 1 << 20, ctypes.byref(plan)) == -2
    assert L.bin1_chain_prepare(ctypes.cast(st, ctypes.c_void_p), 1, FAKE, 16, ctypes.byref(plan)) == -2
    assert L.bin1_chain_prepare(ctypes.cast(st, ctypes.c_void_p), 1, FAKE + 16, 1 << 20, ctypes.byref(plan)) == -3
    assert L.bin1_gemv_chain(None, None) == -1
    assert L.bin1_gemv_chain(ctypes.byref(binding._Plan()), None) == -1


def test_pm1_and_patch_validation(L):
    assert L.bin1_gemv_pm1(None, FAKE, FAKE, 1, 128, 1, None) == -1
    assert L.bin1_gemv_pm1(None, None, None, 0, 128, 1, None) == 0          # no outputs
    assert L.bin1_gemv_pm1(None, None, None, 2, 128, 0, None) == 0
    assert L.bin1_gemv_pm1(FAKE, FAKE * 2, FAKE * 3, -1, 128, 1, None) == -2
    assert L.bin1_gemv_pm1(FAKE, FAKE * 2, FAKE * 3, 1, 96, 1, None) == -2
    assert L.bin1_gemv_pm1(FAKE, FAKE * 2, FAKE + 4, 1, 128, 1, None) == -3
    # an empty patch is a no-op that succeeds without touching anything
    assert L.bin1_xor_patch_apply(None, None, 0, 128, 1, None, None) == 0
    assert L.bin1_xor_patch_apply(FAKE, FAKE * 2, -1, 128, 1, None, None) == -2
    assert L.bin1_xor_patch_apply(None, FAKE, 3, 128, 1, None, None) == -1
    assert L.bin1_xor_patch_apply(FAKE + 4, FAKE * 2, 3, 128, 1, None, None) == -3
    assert L.bin1_xor_patch_apply(FAKE, FAKE, 3, 128, 1, None, None) == -4
    assert L.bin1_xor_patch_apply_multi(None, None, None, 1, None, 0, None, None) == 0
    assert L.bin1_xor_patch_apply_multi(FAKE, FAKE, FAKE, 0, FAKE, 1, None, None) == -2
    assert L.bin1_xor_patch_apply_multi(None, FAKE, FAKE, 1, FAKE, 1, None, None) == -1


def test_bit_patch_and_rank_validation(L):
    # bit patch: empty list is a no-op, bad counts and tables are rejected before launch
    assert L.bin1_xor_bits_apply(None, None, None, 1, None, 0, None, None) == 0
    assert L.bin1_xor_bits_apply(FAKE, FAKE, FAKE, 0, FAKE, 1, None, None) == -2
    assert L.bin1_xor_bits_apply(FAKE, FAKE, FAKE, 1, FAKE, -1, None, None) == -2
    assert L.bin1_xor_bits_apply(None, FAKE, FAKE, 1, FAKE, 1, None, None) == -1
    assert L.bin1_xor_bits_apply(FAKE + 4, FAKE, FAKE, 1, FAKE, 1, None, None) == -3
    # rank: NULLs, shapes, alignment and overlap
    assert L.bin1_rank_rows_by_scale(None, 1, 128, FAKE, FAKE * 2, None) == -1
    assert L.bin1_rank_rows_by_scale(None, 0, 128, None, None, None) == 0    # no rows
    assert L.bin1_rank_rows_by_scale(FAKE, -1, 128, FAKE * 2, FAKE * 3, None) == -2
    assert L.bin1_rank_rows_by_scale(FAKE, (1 << 20) + 1, 128, FAKE * 2, FAKE * 3, None) == -2
    assert L.bin1_rank_rows_by_scale(FAKE, 4, 96, FAKE * 2, FAKE * 3, None) == -2
    assert L.bin1_rank_rows_by_scale(FAKE + 2, 4, 128, FAKE * 2, FAKE * 3, None) == -3
    assert L.bin1_rank_rows_by_scale(FAKE, 4, 128, FAKE * 2 + 4, FAKE * 3, None) == -3
    assert L.bin1_rank_rows_by_scale(FAKE, 4, 1024, FAKE + 8, FAKE * 3, None) == -4     # score over scales
    assert L.bin1_rank_rows_by_scale(FAKE, 4, 128, FAKE * 2, FAKE * 2 + 16, None) == -4


def test_binding_rejects_cpu_tensors():
    import torch
    import bit_packed_sign_amd as b1
    x = torch.zeros(1, 128, dtype=torch.float16)
    W = torch.zeros(1, 4, dtype=torch.int32)
    S = torch.zeros(1, 1, dtype=torch.float16)
    with pytest.raises(ValueError):
        b1.gemv(x, W, S)
    with pytest.raises(ValueError):
        b1.xor_patch_apply(W, torch.zeros(1, dtype=torch.int32))


def test_workspace_product_validation(L):
    """bin1_gemv_ws: the workspace query, and a missing, short, misaligned or overlapping
    workspace rejected before anything is touched (fake addresses, never dereferenced)."""
    L.bin1_gemv_workspace_bytes.restype = ctypes.c_size_t
    need = L.bin1_gemv_workspace_bytes(16, 12288, 4096)
    assert need == 3 * 16 * 4096 * 4
    assert L.bin1_gemv_workspace_bytes(1, 12288, 4096) == 0          # batch 1: no split
    assert L.bin1_gemv_workspace_bytes(16, 4096, 4096) == 0          # one chunk: no split
    assert L.bin1_gemv_workspace_bytes(16, 100, 4096) == 0           # invalid shape
    f = L.bin1_gemv_ws
    x, W, S, y, ws = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000
    assert f(x, W, S, y, 16, 12288, 4096, None, 0, None) == -1
    assert f(x, W, S, y, 16, 12288, 4096, ws, need - 1, None) == -2
    assert f(x, W, S, y, 16, 12288, 4096, ws + 16, need, None) == -3
    assert f(x, W, S, y, 16, 12288, 4096, y - 256, need, None) == -4   # covers y
    assert f(x, W, S, y, 16, 12288, 4096, W, need, None) == -4         # covers the weights
    assert f(x, W, S, y, 0, 12288, 4096, None, 0, None) == 0           # no outputs: nothing to do



def test_calibration_validation(L):
    """The two measurement helpers reject bad sizes, NULL and misaligned pointers before launch."""
    assert L.bin1_stream_read(FAKE, 0, FAKE * 2, 1, 8, None) == -2            # no bytes
    assert L.bin1_stream_read(FAKE, 24, FAKE * 2, 1, 8, None) == -2           # not a multiple of 16
    assert L.bin1_stream_read(FAKE, 64, FAKE * 2, 0, 8, None) == -2           # grid
    assert L.bin1_stream_read(FAKE, 64, FAKE * 2, 1, 5, None) == -2           # unroll
    assert L.bin1_stream_read(None, 64, FAKE * 2, 1, 8, None) == -1
    assert L.bin1_stream_read(FAKE + 4, 64, FAKE * 2, 1, 8, None) == -3
    assert L.bin1_stream_read(FAKE, 64, FAKE + 32, 1, 8, None) == -4          # sink inside buf
    assert L.bin1_mfma_rate(FAKE, FAKE * 2, 0, 4, 10, None) == -2            # grid
    assert L.bin1_mfma_rate(FAKE, FAKE * 2, 1, 5, 10, None) == -2            # waves
    assert L.bin1_mfma_rate(FAKE, FAKE * 2, 1, 4, 0, None) == -2             # iters
    assert L.bin1_mfma_rate(None, FAKE * 2, 1, 4, 10, None) == -1
    assert L.bin1_mfma_rate(FAKE, None, 1, 4, 10, None) == -1
    assert L.bin1_mfma_rate(FAKE + 4, FAKE * 2, 1, 4, 10, None) == -3         # operands not 16-byte aligned
    assert L.bin1_mfma_rate(FAKE, FAKE * 2 + 2, 1, 4, 10, None) == -3
    assert L.bin1_mfma_rate(FAKE, FAKE + 1024, 1, 4, 10, None) == -4         # sink inside the operands
