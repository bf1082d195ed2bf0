"""Shared helpers of the GPU parity tests (test infrastructure)."""
import numpy as np
import torch

# Parity bar for fp32-accumulated products: max over outputs of
# |y_gpu - y_ref| / sum_k |scale * x|  (normaliser computed by the oracle in fp64).
TOL = 2e-3


def norm_err(y_gpu, ref: np.ndarray, nrm: np.ndarray) -> float:
    """Max normalised error; an output whose normaliser is 0 must be exactly 0."""
    if isinstance(y_gpu, torch.Tensor):
        y_gpu = y_gpu.float().cpu().numpy()
    y = np.asarray(y_gpu, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.all(np.isfinite(y)), "non-finite output"
    zero = nrm == 0
    if np.any(zero):
        assert np.all(y[zero] == 0), "output with zero normaliser is not 0"
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.where(zero, 0.0, np.abs(y - ref) / np.where(zero, 1.0, nrm))
    return float(e.max()) if e.size else 0.0


def dev_tensors(device, x=None, W=None, S=None):
    out = []
    if x is not None:
        out.append(torch.from_numpy(np.ascontiguousarray(x)).to(device))
    if W is not None:
        out.append(torch.from_numpy(np.ascontiguousarray(W).view(np.int32)).to(device))
    if S is not None:
        out.append(torch.from_numpy(np.ascontiguousarray(S)).to(device))
    return out


def sample_rows(rng, N, k=256, edge=32):
    """Rows checked at full size: the first and last `edge` rows plus k random ones."""
    rows = set(range(min(edge, N))) | set(range(max(0, N - edge), N))
    rows |= set(rng.choice(N, size=min(k, N), replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)
