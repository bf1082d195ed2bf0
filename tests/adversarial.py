"""Adversarial activation patterns for the GPU parity tests (test infrastructure: input recipes
only, no arithmetic of the method).  Every pattern is fp16 [M][K], seeded.

* exponents -- each element from a random binade 2^-24 .. 2^15 (subnormals included), random
  fraction and sign, so every 32-element block mixes magnitudes over the whole fp16 range;
* max      -- one +-65504 (the largest fp16) in every 32-block, N(0,1) elsewhere;
* ratio    -- the block's maximum 2^a and the other elements 2^(a - r) N(0,1), r in
  {10, 12, 14, 16, 20, 24} (what is below the fp16 range rounds to 0);
* zeros    -- whole blocks of +0 and of -0 between N(0,1) blocks, and rows that are all -0;
* subnormal -- every element an fp16 subnormal (fraction * 2^-24).
"""
import numpy as np

KINDS = ["exponents", "max", "ratio", "zeros", "subnormal"]


def adversarial_x(rng, M, K, kind):
    if kind == "exponents":
        e = rng.integers(-24, 16, size=(M, K))
        frac = rng.integers(0, 1024, size=(M, K)).astype(np.float64)
        v = np.where(e < -14, np.maximum(frac, 1.0) * 2.0 ** -24, (1.0 + frac / 1024.0) * np.exp2(e.astype(np.float64)))
        x = v * rng.choice([-1.0, 1.0], size=(M, K))
    elif kind == "max":
        x = rng.standard_normal((M, K))
        pos = rng.integers(0, 32, size=(M, K // 32))
        sgn = rng.choice([-1.0, 1.0], size=(M, K // 32))
        blk = x.reshape(M, K // 32, 32)
        np.put_along_axis(blk, pos[..., None], (65504.0 * sgn)[..., None], axis=2)
        x = blk.reshape(M, K)
    elif kind == "ratio":
        nb = K // 32
        a = rng.integers(-4, 5, size=(M, nb)).astype(np.float64)
        r = np.array([10, 12, 14, 16, 20, 24], np.float64)[np.arange(nb) % 6][None, :]
        blk = rng.standard_normal((M, nb, 32)) * np.exp2(a - r)[..., None]
        pos = rng.integers(0, 32, size=(M, nb))
        np.put_along_axis(blk, pos[..., None], (np.exp2(a) * rng.choice([-1.0, 1.0], size=(M, nb)))[..., None],
                          axis=2)
        x = blk.reshape(M, K)
    elif kind == "zeros":
        x = rng.standard_normal((M, K))
        blk = x.reshape(M, K // 32, 32)
        which = rng.integers(0, 3, size=(M, K // 32))
        blk[which == 1] = 0.0
        blk[which == 2] = -0.0
        x = blk.reshape(M, K)
        if M > 1:
            x[M - 1] = -0.0
    elif kind == "subnormal":
        x = rng.integers(1, 1024, size=(M, K)).astype(np.float64) * 2.0 ** -24 * rng.choice([-1.0, 1.0], size=(M, K))
    else:
        raise ValueError(kind)
    return x.astype(np.float16)


def onehot_exact(rng, M, K, N, ternary=False):
    """Inputs whose product is exact in fp16: x holds one +-2^e (e in -2..0) per 128-group and zeros
    elsewhere, every scale is +-2^f (f in -2..1).  Each term is a multiple of 2^-4 of magnitude at
    most 2 and a row has at most K / 128 <= 64 of them here, so y is a multiple of 2^-4 below 2^7:
    exact in fp16, in fp32 and in fp64, whatever the summation order.  Returns (x, scales)."""
    assert K // 128 <= 64
    x = np.zeros((M, K), np.float64)
    g = K // 128
    pos = rng.integers(0, 128, size=(M, g)) + 128 * np.arange(g)[None, :]
    val = np.exp2(rng.integers(-2, 1, size=(M, g)).astype(np.float64)) * rng.choice([-1.0, 1.0], size=(M, g))
    np.put_along_axis(x, pos, val, axis=1)
    S = np.exp2(rng.integers(-2, 2, size=(N, g)).astype(np.float64)) * rng.choice([-1.0, 1.0], size=(N, g))
    return x.astype(np.float16), S.astype(np.float16)
