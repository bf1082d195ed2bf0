"""The activation split of the batch-1 decode kernel, checked exhaustively on the CPU from the number
formats' definitions (no GPU, no code shared with the kernel).

The kernel feeds the block-scaled fp8 x fp4 matrix cores, so each 32-element block of fp16
activations becomes three OCP fp8 e4m3 "limbs" with a shared power-of-two exponent:
  e0 = the exponent of the block's largest magnitude m (2^e0 <= m < 2^(e0+1); 0 for an all-zero
       block), u = x * 2^(7 - e0), and for r = 0, 1, 2:  L_r = e4m3(u), u <- 16 (u - L_r),
  so that x' = 2^(e0 - 7) (L_0 + L_1 / 16 + L_2 / 256).
e4m3 (1 sign, 4 exponent bits with bias 7, 3 fraction bits, no infinities): normal values
(1 + f/8) 2^E for E in -6..8, subnormal values f 2^-9, largest finite 448; conversion rounds to
nearest, ties to even.  The claims checked here, over every finite fp16 value and every block
exponent the value can occur under:
  (1) every element whose magnitude is at least 2^-10 of the block's maximum is represented exactly;
  (2) no element is off by more than 2^-25 of the block's maximum.
Together with fp32 accumulation these bound the limb error far below the 2e-3 parity bar (31
elements per block at 2^-25 of its maximum each)."""
import numpy as np


def e4m3_round(r: np.ndarray) -> np.ndarray:
    """Nearest e4m3 value of float64 r (|r| < 448), ties to even, from the format definition."""
    a = np.abs(r)
    _, ex = np.frexp(a)                           # a = f 2^ex with f in [0.5, 1): binade ex - 1
    E = np.maximum(ex.astype(np.float64) - 1.0, -6.0)   # below 2^-6 the subnormal spacing 2^-9 holds
    q = np.exp2(E - 3.0)                           # 3 fraction bits per binade
    out = np.sign(r) * np.round(a / q) * q         # numpy rounds halves to even
    assert np.all(np.abs(out) <= 448.0)
    return out


def all_finite_fp16() -> np.ndarray:
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16).astype(np.float64)
    return v[np.isfinite(v)]


def limbs(x: np.ndarray, e0: int) -> np.ndarray:
    """x' = 2^(e0 - 7) sum_r L_r 16^-r, the value the three limbs of x represent."""
    u = x * 2.0 ** (7 - e0)
    acc = np.zeros_like(x)
    for r in range(3):
        L = e4m3_round(u)
        acc += L * 16.0 ** -r
        u = 16.0 * (u - L)                         # exact: L is u rounded to 4 significant bits
    return acc * 2.0 ** (e0 - 7)


def test_e4m3_rounding_pins():
    # printed e4m3 facts: largest 448, smallest subnormal 2^-9, 3 fraction bits, ties to even
    assert e4m3_round(np.array([448.0]))[0] == 448.0
    assert e4m3_round(np.array([2.0 ** -9]))[0] == 2.0 ** -9
    assert e4m3_round(np.array([1.0 + 1 / 16]))[0] == 1.0            # tie -> even fraction 0
    assert e4m3_round(np.array([1.0 + 3 / 16]))[0] == 1.25           # tie -> even fraction 2
    assert e4m3_round(np.array([2.0 ** -10]))[0] == 0.0              # half the smallest subnormal: tie -> 0
    assert e4m3_round(np.array([3 * 2.0 ** -10]))[0] == 2.0 ** -8    # tie between 1 and 2 subnormal steps
    assert e4m3_round(np.array([-15.5]))[0] == -16.0                  # rounds into the next binade
    grid = np.array([(1 + f / 8) * 2.0 ** E for E in range(-6, 9) for f in range(8) if (E, f) != (8, 7)] +
                    [f * 2.0 ** -9 for f in range(8)])        # (E = 8, f = 7) is the NaN code
    assert np.array_equal(e4m3_round(grid), grid) and np.array_equal(e4m3_round(-grid), -grid)


def test_three_limbs_exact_within_2_pow_10_of_the_block_max():
    v = all_finite_fp16()
    worst_rel_err = 0.0
    for e0 in range(-24, 16):                     # every block exponent an fp16 maximum can have
        top = 2.0 ** (e0 + 1)
        x = v[np.abs(v) < top]                    # every value that can sit in such a block
        xr = limbs(x, e0)
        err = np.abs(xr - x)
        # (1) exact down to 2^-10 of the smallest possible maximum (2^e0) of this block class
        big = np.abs(x) >= 2.0 ** (e0 - 10)
        assert np.all(err[big] == 0.0), (e0, x[big][err[big] != 0][:5])
        # (2) everywhere within 2^-25 of 2^e0 <= the block maximum
        assert np.all(err <= 2.0 ** (e0 - 25)), (e0, err.max() / 2.0 ** e0)
        worst_rel_err = max(worst_rel_err, float(err.max() / 2.0 ** e0))
    assert 0.0 < worst_rel_err <= 2.0 ** -25


def test_two_limbs_would_not_do():
    """Why three limbs: two carry 8 significant bits, and an fp16 value needs up to 11."""
    e0 = 0
    x = np.array([1.0 + 429.0 / 1024.0])            # 0b1.0110101101: 181.625 after scaling
    u = x * 2.0 ** 7
    L0 = e4m3_round(u)
    L1 = e4m3_round(16.0 * (u - L0))
    two = (L0 + L1 / 16.0) * 2.0 ** -7
    assert np.any(two != x)
    assert np.array_equal(limbs(x, e0), x)
