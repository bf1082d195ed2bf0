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

import numpy as np
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
    "bin1_gemv_t2": [_p, _p, _p, _p, _i, _i, _i, _p],
    "bin1_gemm_prefill_t2": [_p, _p, _p, _p, _i, _i, _i, _p],
    "bin1_gemv_group": [_p, _i, _p, _p, _p, _p, _i, _i, _p],
    "bin1_gemv_group_t2": [_p, _i, _p, _p, _p, _p, _i, _i, _p],
    "bin1_gemv_pm1": [_p, _p, _p, _i, _i, _i, _p],
    "bin1_xor_patch_apply": [_p, _p, _i, _i, _i, _p, _p],
    "bin1_xor_patch_apply_multi": [_p, _p, _p, _i, _p, _i, _p, _p],
    "bin1_xor_bits_apply": [_p, _p, _p, _i, _p, _i, _p, _p],
    "bin1_rank_rows_by_scale": [_p, _i, _i, _p, _p, _p],
    "bin1_chain_workspace_bytes": [_i],
    "bin1_chain_prepare": [_p, _i, _p, ctypes.c_size_t, _p],
    "bin1_gemv_chain": [_p, _p],
    "bin1_chain_status": [_p, _p, _p],
    "bin1_stream_read": [_p, ctypes.c_size_t, _p, _i, _i, _p],
    "bin1_mfma_rate": [_p, _p, _i, _i, _i, _p],
    "bin1_kernel_variant": [_i, _i, _i, _i, _p, _p, _i],
    "bin1_gemv_workspace_bytes": [_i, _i, _i],
    "bin1_gemv_ws": [_p, _p, _p, _p, _i, _i, _i, _p, ctypes.c_size_t, _p],
    "bin1_gemv_noalloc": [_p, _p, _p, _p, _i, _i, _i, _p],
    "bin1_status_string": [_i],
    "bin1_last_error": [],
    "bin1_abi_version": [],
}
_RESTYPE = {"bin1_status_string": ctypes.c_char_p, "bin1_last_error": ctypes.c_char_p,
            "bin1_chain_workspace_bytes": ctypes.c_size_t, "bin1_gemv_workspace_bytes": ctypes.c_size_t}


class _Stage(ctypes.Structure):
    _fields_ = [("x", _p), ("K", _i), ("count", _i), ("Wbits", _p * 4), ("scales", _p * 4),
                ("y", _p * 4), ("N", _i * 4)]


class _Plan(ctypes.Structure):
    _fields_ = [("workspace", _p), ("nstages", _i), ("spmax", _i), ("max_tiles", _i), ("spin_limit", _i)]


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


# the current stream of a device as a raw handle (torch's own accessor when it has one: no
# Stream object is built per call)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor) -> int:
    if _raw_stream is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _call(fn: str, device: int, *args) -> None:
    """Call `fn` of the library with `device` current (switching only when it is not already)."""
    f = getattr(_lib if _lib is not None else lib(), fn)
    if torch.cuda.current_device() == device:
        status = f(*args)
    else:
        with torch.cuda.device(device):
            status = f(*args)
    _check(fn, status)


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


def _product(fn: str, x, Wbits, scales, out, per_word: int = 32):
    _need(x, "x", (torch.float16,), 2)
    _need(Wbits, "Wbits", _BITS, 2)
    _need(scales, "scales", (torch.float16,), 2)
    M, K = x.shape
    N = Wbits.shape[0]
    if Wbits.shape[1] * per_word != K or tuple(scales.shape) != (N, K // 128):
        raise ValueError(f"shapes: x {tuple(x.shape)}, Wbits {tuple(Wbits.shape)}, scales {tuple(scales.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _need(out, "out", (torch.float16,), 2)
        if tuple(out.shape) != (M, N):
            raise ValueError("out has the wrong shape")
    _call(fn, x.get_device(), x.data_ptr(), Wbits.data_ptr(), scales.data_ptr(), out.data_ptr(), M, K, N,
          _stream(x))
    return out


def gemv(x: torch.Tensor, Wbits: torch.Tensor, scales: torch.Tensor, out: Optional[torch.Tensor] = None):
    """y[M][N] (fp16) = x[M][K] (fp16) times the 1-bit weights (Wbits [N][K/32], scales [N][K/128])."""
    return _product("bin1_gemv", x, Wbits, scales, out)


def gemv_workspace_bytes(M: int, K: int, N: int) -> int:
    """Bytes of workspace :func:`gemv_ws` uses for this shape (0: it takes no split path)."""
    return int(lib().bin1_gemv_workspace_bytes(M, K, N))


def gemv_ws(x: torch.Tensor, Wbits: torch.Tensor, scales: torch.Tensor, workspace: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None):
    """:func:`gemv` with a device workspace (uint8, at least :func:`gemv_workspace_bytes` bytes,
    256-byte aligned) that lets long small-batch products split K over workgroups.  The workspace
    is allocated here when not given."""
    _need(x, "x", (torch.float16,), 2)
    _need(Wbits, "Wbits", _BITS, 2)
    M, K = x.shape
    N = Wbits.shape[0]
    need = gemv_workspace_bytes(M, K, N) if M >= 1 and N >= 1 and K % 128 == 0 and K >= 128 else 0
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wp, wb = 0, 0
    if workspace is not None:
        _need(workspace, "workspace", (torch.uint8,), 1)
        wp, wb = workspace.data_ptr(), workspace.numel()
    return _product_ws("bin1_gemv_ws", x, Wbits, scales, out, wp or None, wb)


def gemv_noalloc(x: torch.Tensor, Wbits: torch.Tensor, scales: torch.Tensor, out: Optional[torch.Tensor] = None):
    """:func:`gemv_ws` on the library's own 4 MiB scratch per GPU (no workspace argument; calls
    overlapping in time on one GPU race).  Only the output is allocated here, when not given."""
    return _product("bin1_gemv_noalloc", x, Wbits, scales, out)


def _product_ws(fn, x, Wbits, scales, out, wp, wb):
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
    _call(fn, x.get_device(), x.data_ptr(), Wbits.data_ptr(), scales.data_ptr(), out.data_ptr(), M, K, N,
          wp, wb, _stream(x))
    return out


def gemv_t2(x: torch.Tensor, Tbits: torch.Tensor, scales: torch.Tensor, out: Optional[torch.Tensor] = None):
    """y[M][N] (fp16) = x[M][K] (fp16) times ternary weights in 2-bit slots (Tbits [N][K/16],
    scales [N][K/128])."""
    return _product("bin1_gemv_t2", x, Tbits, scales, out, per_word=16)


def gemm_prefill_t2(x: torch.Tensor, Tbits: torch.Tensor, scales: torch.Tensor, out: Optional[torch.Tensor] = None):
    """Ternary prefill product, tuned for M >= 256; same arguments as gemv_t2."""
    return _product("bin1_gemm_prefill_t2", x, Tbits, scales, out, per_word=16)


def gemv_group(x: torch.Tensor, Wbits: Sequence[torch.Tensor], scales: Sequence[torch.Tensor],
               outs: Optional[Sequence[torch.Tensor]] = None, _fn: str = "bin1_gemv_group", _per_word: int = 32):
    """Products of several matrices with the same activations x (e.g. q/k/v), one launch for M <= 16.
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
        if W.shape[1] * _per_word != K or tuple(S.shape) != (W.shape[0], K // 128):
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
    _call(_fn, x.get_device(), x.data_ptr(), count, wp, sp, yp, npv, M, K, _stream(x))
    return list(outs)



def gemv_group_t2(x: torch.Tensor, Tbits: Sequence[torch.Tensor], scales: Sequence[torch.Tensor],
                  outs: Optional[Sequence[torch.Tensor]] = None):
    """Same-input fusion for ternary weights (Tbits[i] [N_i][K/16]); one launch at M = 1."""
    return gemv_group(x, Tbits, scales, outs, _fn="bin1_gemv_group_t2", _per_word=16)

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
    _call("bin1_gemv_pm1", Abits.get_device(), Abits.data_ptr(), Wbits.data_ptr(), out.data_ptr(), M, K, N,
          _stream(Abits))
    return out


def xor_patch_apply(Wbits: torch.Tensor, rows: torch.Tensor, bad_rows: Optional[torch.Tensor] = None,
                    check_distinct: bool = False) -> None:
    """Flip (in place) every sign of the listed output rows of Wbits [N][K/32]; calling it again
    with the same rows removes the patch.  ``rows``: device int32 [nrows]; a row listed twice is
    flipped twice, i.e. unchanged.  Rows out of range are skipped and counted into ``bad_rows``
    (device int32 [1]) when given.  ``check_distinct=True`` rejects repeated rows first; that check
    reads the list back to the host (a synchronisation, so not inside graph capture)."""
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
                          check_distinct: bool = False) -> None:
    """Patch many matrices in one launch.  ``entries``: device int32 [n][2] of (matrix id, row);
    repeated entries commute as in :func:`xor_patch_apply` (``check_distinct=True`` rejects them,
    with a host synchronisation)."""
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


def xor_bits_apply(table: PatchTable, entries: torch.Tensor, bad: Optional[torch.Tensor] = None) -> None:
    """Bit-granular patch in one launch.  ``entries``: device int32 [n][3] of (matrix id, row, k);
    records may repeat (flips are XORs: an even count cancels)."""
    _need(entries, "entries", (torch.int32,), 2)
    if entries.shape[1] != 3:
        raise ValueError("entries must be [n][3]")
    bp = 0
    if bad is not None:
        _need(bad, "bad", (torch.int32,), 1)
        bp = bad.data_ptr()
    dev = table.ptrs.device
    with torch.cuda.device(dev):
        _check("bin1_xor_bits_apply", lib().bin1_xor_bits_apply(
            table.ptrs.data_ptr(), table.K.data_ptr(), table.N.data_ptr(), len(table),
            entries.data_ptr(), entries.shape[0], bp or None, _stream(table.ptrs)))


def rank_rows_by_scale(scales: torch.Tensor, score: Optional[torch.Tensor] = None,
                       order: Optional[torch.Tensor] = None):
    """Rows of a matrix by the exact sum of |scale| (units of 2^-24), largest first, ties by
    row.  ``scales``: device fp16 [N][K/128].  Returns (score int64 [N], order int32 [N])."""
    _need(scales, "scales", (torch.float16,), 2)
    N, G = scales.shape
    if score is None:
        score = torch.empty(N, dtype=torch.int64, device=scales.device)
    if order is None:
        order = torch.empty(N, dtype=torch.int32, device=scales.device)
    _need(score, "score", (torch.int64,), 1)
    _need(order, "order", (torch.int32,), 1)
    if score.shape[0] != N or order.shape[0] != N:
        raise ValueError("score and order must have N entries")
    with torch.cuda.device(scales.device):
        _check("bin1_rank_rows_by_scale", lib().bin1_rank_rows_by_scale(
            scales.data_ptr(), N, G * 128, score.data_ptr(), order.data_ptr(), _stream(scales)))
    return score, order


class ChainPlan:
    """A decode step as one persistent launch: ``stages`` is a sequence of
    (x [1][K] fp16, [Wbits...], [scales...], [y...]) -- 1..4 products per stage that share x.
    Stage s+1 starts after every output of stage s is written.  The device workspace is
    allocated here with torch; ``run()`` only enqueues the kernel (capturable in a graph)."""

    def __init__(self, stages):
        if not stages:
            raise ValueError("need at least one stage")
        dev = stages[0][0].device
        arr = (_Stage * len(stages))()
        self._keep = []
        for i, (x, Ws, Ss, ys) in enumerate(stages):
            _need(x, f"stage {i} x", (torch.float16,), 2)
            if x.shape[0] != 1:
                raise ValueError("chain stages take one activation row (batch 1)")
            K = x.shape[1]
            if not 1 <= len(Ws) <= 4 or len(Ss) != len(Ws) or len(ys) != len(Ws):
                raise ValueError(f"stage {i}: need 1..4 matrices with scales and outputs")
            st = arr[i]
            st.x = x.data_ptr()
            st.K = K
            st.count = len(Ws)
            for j, (W, S, y) in enumerate(zip(Ws, Ss, ys)):
                _need(W, "Wbits", _BITS, 2)
                _need(S, "scales", (torch.float16,), 2)
                _need(y, "y", (torch.float16,), 2)
                if W.shape[1] * 32 != K or tuple(S.shape) != (W.shape[0], K // 128) or \
                        tuple(y.shape) != (1, W.shape[0]):
                    raise ValueError(f"stage {i} matrix {j}: shapes do not match")
                st.Wbits[j] = W.data_ptr()
                st.scales[j] = S.data_ptr()
                st.y[j] = y.data_ptr()
                st.N[j] = W.shape[0]
            self._keep.append((x, list(Ws), list(Ss), list(ys)))
        nbytes = lib().bin1_chain_workspace_bytes(len(stages))
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.plan = _Plan()
        with torch.cuda.device(dev):
            _check("bin1_chain_prepare", lib().bin1_chain_prepare(
                ctypes.cast(arr, _p), len(stages), self.workspace.data_ptr(), nbytes, ctypes.byref(self.plan)))

    def set_spin_limit(self, polls: int):
        """Bound every stage wait to `polls` polls (0 = the library default)."""
        self.plan.spin_limit = int(polls)

    def run(self):
        with torch.cuda.device(self.workspace.device):
            _check("bin1_gemv_chain", lib().bin1_gemv_chain(ctypes.byref(self.plan), _stream(self.workspace)))

    def status(self):
        """(completed runs, error flag) -- synchronous."""
        runs, err = ctypes.c_int(0), ctypes.c_int(0)
        with torch.cuda.device(self.workspace.device):
            _check("bin1_chain_status", lib().bin1_chain_status(ctypes.byref(self.plan), ctypes.byref(runs),
                                                                  ctypes.byref(err)))
        return runs.value, err.value


def stream_read(buf: torch.Tensor, sink: Optional[torch.Tensor] = None, grid: int = 2048, unroll: int = 8):
    """Read every byte of the device tensor ``buf`` once (a measurement of the HBM read rate; no
    arithmetic of the method).  Returns the per-wave digest tensor (uint32 viewed as int32 [4 * grid])."""
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    if sink is None:
        sink = torch.empty(4 * grid, dtype=torch.int32, device=buf.device)
    _need(sink, "sink", (torch.int32,), 1)
    if sink.numel() < 4 * grid:
        raise ValueError("sink needs 4 * grid entries")
    nbytes = buf.numel() * buf.element_size()
    _call("bin1_stream_read", buf.get_device(), buf.data_ptr(), nbytes, sink.data_ptr(), grid, unroll, _stream(buf))
    return sink


def mfma_rate(operands: torch.Tensor, sink: torch.Tensor, grid: int = 1024, waves: int = 4, iters: int = 1000):
    """Issue grid * waves * iters * 12 independent fp16 32x32x16 matrix-core products on the lane
    fragments in ``operands`` (device float16 [2, 64, 8]: A then B) -- a measurement of the sustained
    MFMA rate, no arithmetic of the method.  ``sink``: device float32 [grid * waves], which receives
    12 * iters * (A B)[0, 0] per wave (exact for small integer operands)."""
    _need(operands, "operands", (torch.float16,), 3)
    if tuple(operands.shape) != (2, 64, 8):
        raise ValueError("operands must be [2, 64, 8]")
    _need(sink, "sink", (torch.float32,), 1)
    if sink.numel() < grid * waves:
        raise ValueError("sink needs grid * waves entries")
    _call("bin1_mfma_rate", sink.get_device(), operands.data_ptr(), sink.data_ptr(), grid, waves, iters, _stream(sink))
    return sink


_VARIANT_OPS = {"gemv": 0, "gemv_t2": 1, "prefill": 2, "prefill_t2": 3, "gemv_ws": 4}


def kernel_variant(op: str, M: int, K: int, N) -> str:
    """The kernel variant(s) and grid a product call would launch (no GPU needed).  ``op``: "gemv"
    (bin1_gemv / bin1_gemv_group), "gemv_t2", "prefill", "prefill_t2" or "gemv_ws"; ``N``: an int or the list
    of row counts of a group call, as it would launch them."""
    Ns = [int(N)] if isinstance(N, (int, np.integer)) else [int(n) for n in N]
    buf = ctypes.create_string_buffer(1024)
    arr = (ctypes.c_int * len(Ns))(*Ns)
    _check("bin1_kernel_variant", lib().bin1_kernel_variant(_VARIANT_OPS[op], M, K, len(Ns), arr, buf, len(buf)))
    return buf.value.decode()
