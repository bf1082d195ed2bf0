"""Exact-rational evaluation of the dequantise-and-dot (test infrastructure).

Used to pin the fp64 rounding of the C oracle: every fp16 value is a dyadic
rational, so ``fractions.Fraction`` gives the exact sum
    y[m][n] = sum_k s(n, k/G) * w(n, k) * x[m][k]
with w(n,k) = +1 if bit (k mod 32) of word k//32 of row n is set, else -1
("Bonsai 27B" page, binary weight format section).  The fp16 values are decoded
here by Python's own ``float`` conversion of numpy float16 (exact), not by the C
oracle's decoder.  Pure-Python loops: small cases only.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def gemv_exact(x: np.ndarray, W: np.ndarray, S: np.ndarray, group: int = 128):
    x = np.asarray(x, dtype=np.float16)
    S = np.asarray(S, dtype=np.float16)
    M, K = x.shape
    N = W.shape[0]
    xf = [[Fraction(float(v)) for v in row] for row in x]
    out = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        sf = [Fraction(float(v)) for v in S[n]]
        signs = [1 if (int(W[n][k // 32]) >> (k % 32)) & 1 else -1 for k in range(K)]
        for m in range(M):
            acc = Fraction(0)
            for k in range(K):
                acc += sf[k // group] * signs[k] * xf[m][k]
            out[m][n] = acc
    return out
