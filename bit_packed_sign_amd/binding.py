"""Thin Python binding of libbin1 (include/bin1.h): argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI; this module
checks dtypes/shapes/devices of torch tensors, allocates outputs with torch and passes
raw device pointers plus torch's current HIP stream.  If libbin1.so is missing every
call raises -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbin1.so")

_lib = None
_lock = threading.Lock()

_p = ctypes.c_void_p
_i = ctypes.c_int

# name -> argtypes (all return int status unless listed in _RESTYPE)
_SIGS = {
    "bin1_gemv": [_p, _p, _p, _p, _i, _i, _i, _p],
    "bin1_gemm_prefill": [_p, _p, _p, _p, _i, _i, _i, _p],
    "bin1_gemv_group": [_p, _i, _p, _p, _p, _p, _i, _i, _p],
    "bin1_gemv_pm1": [_p, _p, _p, _i, _i, _i, _p],
    "bin1_xor_patch_apply": [_p, _p, _i, _i, _i, _p, _p],
    "bin1_xor_patch_apply_multi": [_p, _p, _p, _i, _p, _i, _p, _p],
    "bin1_status_string": [_i],
    "bin1_last_error": [],
    "bin1_abi_version": [],
}
_RESTYPE = {"bin1_status_string": ctypes.c_char_p, "bin1_last_error": ctypes.c_char_p}


class Bin1Error(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        self.status = status
        super().__init__(f"{fn} failed with status {status}: {detail}")


def lib():
    """Load libbin1.so (built by ``python -m bit_packed_sign_amd.build``)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is not built; run `python -m bit_packed_sign_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            for name, args in _SIGS.items():
                f = getattr(L, name)
                f.argtypes = args
                f.restype = _RESTYPE.get(name, _i)
            _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        L = lib()
        detail = (L.bin1_last_error() or b"").decode() or L.bin1_status_string(status).decode()
        raise Bin1Error(fn, status, detail)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, name: str, dtypes, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_BITS = (torch.int32, torch.uint32)


def _product(fn: str, x, Wbits, scales, out):
    _need(x, "x", (torch.float16,), 2)
    _need(Wbits, "Wbits", _BITS, 2)
    _need(scales, "scales", (torch.float16,), 2)
    M, K = x.shape
    N = Wbits.shape[0]
    if Wbits.shape[1] * 32 != K or tuple(scales.shape) != (N, K // 128):
        raise ValueError(f"shapes: x {tuple(x.shape)}, Wbits {tuple(Wbits.shape)}, scales {tuple(scales.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _need(out, "out", (torch.float16,), 2)
        if tuple(out.shape) != (M, N):
            raise ValueError("out has the wrong shape")
    with torch.cuda.device(x.device):
        _check(fn, getattr(lib(), fn)(x.data_ptr(), Wbits.data_ptr(), scales.data_ptr(), out.data_ptr(),
                                      M, K, N, _stream(x)))
    return out


def gemv(x: torch.Tensor, Wbits: torch.Tensor, scales: torch.Tensor, out: Optional[torch.Tensor] = None):
    """y[M][N] (fp16) = x[M][K] (fp16) times the 1-bit weights (Wbits [N][K/32], scales [N][K/128])."""
    return _product("bin1_gemv", x, Wbits, scales, out)


def gemv_group(x: torch.Tensor, Wbits: Sequence[torch.Tensor], scales: Sequence[torch.Tensor],
               outs: Optional[Sequence[torch.Tensor]] = None):
    """Products of several matrices with the same activations x (e.g. q/k/v), one launch at M=1.
    Returns the list of outputs y_i [M][N_i]."""
    _need(x, "x", (torch.float16,), 2)
    count = len(Wbits)
    if count < 1 or count > 4 or len(scales) != count:
        raise ValueError("need 1..4 matrices with one scale tensor each")
    M, K = x.shape
    Ns = []
    for i, (W, S) in enumerate(zip(Wbits, scales)):
        _need(W, f"Wbits[{i}]", _BITS, 2)
        _need(S, f"scales[{i}]", (torch.float16,), 2)
        if W.shape[1] * 32 != K or tuple(S.shape) != (W.shape[0], K // 128):
            raise ValueError(f"matrix {i}: shapes do not match x")
        Ns.append(W.shape[0])
    if outs is None:
        outs = [torch.empty((M, n), dtype=torch.float16, device=x.device) for n in Ns]
    else:
        for i, o in enumerate(outs):
            _need(o, f"outs[{i}]", (torch.float16,), 2)
            if tuple(o.shape) != (M, Ns[i]):
                raise ValueError(f"outs[{i}] has the wrong shape")
    arr_p = ctypes.c_void_p * count
    wp = arr_p(*[W.data_ptr() for W in Wbits])
    sp = arr_p(*[S.data_ptr() for S in scales])
    yp = arr_p(*[o.data_ptr() for o in outs])
    npv = (ctypes.c_int * count)(*Ns)
    with torch.cuda.device(x.device):
        _check("bin1_gemv_group", lib().bin1_gemv_group(x.data_ptr(), count, wp, sp, yp, npv, M, K,
                                                         _stream(x)))
    return list(outs)


def gemm_prefill(x: torch.Tensor, Wbits: torch.Tensor, scales: torch.Tensor, out: Optional[torch.Tensor] = None):
    """Same product as :func:`gemv`, on the matrix-core prefill kernel (for M >= 256)."""
    return _product("bin1_gemm_prefill", x, Wbits, scales, out)


def gemv_pm1(Abits: torch.Tensor, Wbits: torch.Tensor, out: Optional[torch.Tensor] = None):
    """Exact +-1 product: int32 [M][N] = K - 2*popcount(Abits[m] xor Wbits[n])."""
    _need(Abits, "Abits", _BITS, 2)
    _need(Wbits, "Wbits", _BITS, 2)
    M, KW = Abits.shape
    N = Wbits.shape[0]
    if Wbits.shape[1] != KW:
        raise ValueError("Abits and Wbits must have the same number of words per row")
    K = KW * 32
    if out is None:
        out = torch.empty((M, N), dtype=torch.int32, device=Abits.device)
    else:
        _need(out, "out", (torch.int32,), 2)
        if tuple(out.shape) != (M, N):
            raise ValueError("out has the wrong shape")
    with torch.cuda.device(Abits.device):
        _check("bin1_gemv_pm1", lib().bin1_gemv_pm1(Abits.data_ptr(), Wbits.data_ptr(), out.data_ptr(),
                                                     M, K, N, _stream(Abits)))
    return out


def xor_patch_apply(Wbits: torch.Tensor, rows: torch.Tensor, bad_rows: Optional[torch.Tensor] = None,
                    check_distinct: bool = True) -> None:
    """Flip (in place) every sign of the listed output rows of Wbits [N][K/32]; calling it again
    with the same rows removes the patch.  ``rows``: device int32 [nrows], distinct.  Rows out of
    range are skipped and counted into ``bad_rows`` (device int32 [1]) when given."""
    _need(Wbits, "Wbits", _BITS, 2)
    _need(rows, "rows", (torch.int32,), 1)
    if check_distinct and rows.numel() and torch.unique(rows).numel() != rows.numel():
        raise ValueError("patch rows must be distinct")
    N, KW = Wbits.shape
    bp = 0
    if bad_rows is not None:
        _need(bad_rows, "bad_rows", (torch.int32,), 1)
        bp = bad_rows.data_ptr()
    with torch.cuda.device(Wbits.device):
        _check("bin1_xor_patch_apply", lib().bin1_xor_patch_apply(
            Wbits.data_ptr(), rows.data_ptr(), rows.numel(), KW * 32, N, bp or None, _stream(Wbits)))


class PatchTable:
    """Device tables describing a set of weight matrices for multi-matrix patching
    ((layer, projection, row) records in one launch)."""

    def __init__(self, mats: Sequence[torch.Tensor]):
        if not mats:
            raise ValueError("need at least one matrix")
        dev = mats[0].device
        for i, w in enumerate(mats):
            _need(w, f"mats[{i}]", _BITS, 2)
            if w.device != dev:
                raise ValueError("all matrices must be on one device")
        self.mats = list(mats)
        self.ptrs = torch.tensor([w.data_ptr() for w in mats], dtype=torch.int64, device=dev)
        self.K = torch.tensor([w.shape[1] * 32 for w in mats], dtype=torch.int32, device=dev)
        self.N = torch.tensor([w.shape[0] for w in mats], dtype=torch.int32, device=dev)

    def __len__(self):
        return len(self.mats)


def xor_patch_apply_multi(table: PatchTable, entries: torch.Tensor, bad_rows: Optional[torch.Tensor] = None,
                          check_distinct: bool = True) -> None:
    """Patch many matrices in one launch.  ``entries``: device int32 [n][2] of (matrix id, row)."""
    _need(entries, "entries", (torch.int32,), 2)
    if entries.shape[1] != 2:
        raise ValueError("entries must be [n][2]")
    if check_distinct and entries.numel() and torch.unique(entries, dim=0).shape[0] != entries.shape[0]:
        raise ValueError("patch entries must be distinct")
    bp = 0
    if bad_rows is not None:
        _need(bad_rows, "bad_rows", (torch.int32,), 1)
        bp = bad_rows.data_ptr()
    dev = table.ptrs.device
    with torch.cuda.device(dev):
        _check("bin1_xor_patch_apply_multi", lib().bin1_xor_patch_apply_multi(
            table.ptrs.data_ptr(), table.K.data_ptr(), table.N.data_ptr(), len(table),
            entries.data_ptr(), entries.shape[0], bp or None, _stream(table.ptrs)))
