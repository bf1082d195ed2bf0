"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than its own formula:
library routines (numpy float16 decode, unpackbits + BLAS, bitwise_count),
closed forms, exact rationals, invariants (involution, negation, scaling) and
exhaustive enumeration.  A plausible slip in the oracle -- a dropped term, a
wrong sign, a transposed operand, MSB-first bit order, a wrong group index --
fails at least one of them (test_planted_mistakes_are_caught checks that on CPU).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from bit_packed_sign_amd import synth
from oracle import exact

U = 2.0 ** -53
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(t):
    return synth.rng_for(0, synth.WL_TEST, t)


def _case(t, M, K, N, group=128):
    r = _rng(t)
    x = synth.activations(r, M, K)
    W = synth.sign_words(r, N, K)
    S = synth.group_scales(r, N, K, group)
    return x, W, S


def _fp64_bound(K, nrm):
    # Products s*x of two fp16 values are exact in fp64 (22 significant bits); only the
    # K-1 additions round, each by at most u times the running magnitude <= nrm.
    return (K + 1) * U * nrm


# ---------------------------------------------------------------- fp16 decode
def test_half_decode_matches_numpy_for_all_patterns(orc):
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([orc.half_to_double(int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero and subnormals are kept exactly (no flush to zero)
    assert np.signbit(orc.half_to_double(0x8000))
    assert orc.half_to_double(0x0001) == 2.0 ** -24


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("K", [128, 384, 4096])
def test_all_plus_and_all_minus_rows_closed_form(orc, K):
    r = _rng(1)
    M, N = 3, 4
    x = synth.activations(r, M, K)
    S = synth.group_scales(r, N, K)
    W = np.zeros((N, K // 32), np.uint32)
    W[0::2] = 0xFFFFFFFF                     # rows 0, 2: every weight +1; rows 1, 3: every weight -1
    y, nrm = orc.gemv(x, W, S)
    # closed form computed a different way: per-group sums of x first, then the scales
    gx = x.astype(np.float64).reshape(M, K // 128, 128).sum(axis=2)       # [M][G]
    cf = gx @ S.astype(np.float64).T                                        # [M][N]
    sign = np.array([1.0, -1.0, 1.0, -1.0])
    assert np.all(np.abs(y - sign * cf) <= 2 * _fp64_bound(K, nrm))
    # normaliser: sum |s x| = sum_g s_g * sum_{k in g} |x_k| for s >= 0
    ax = np.abs(x.astype(np.float64)).reshape(M, K // 128, 128).sum(axis=2)
    assert np.allclose(nrm, ax @ S.astype(np.float64).T, rtol=1e-12, atol=0)


def test_one_hot_rows_pin_lsb_first_bit_order(orc):
    K = 256
    r = _rng(2)
    x = synth.activations(r, 1, K)
    positions = list(range(32)) + [32 + 5, 64 + 31, 100, 127, 128, 200, 255]
    N = len(positions)
    S = synth.group_scales(r, N, K)
    W = np.zeros((N, K // 32), np.uint32)
    for n, k in enumerate(positions):
        W[n, k // 32] = np.uint32(1) << np.uint32(k % 32)
    y, nrm = orc.gemv(x, W, S)
    x64 = x[0].astype(np.float64)
    for n, k in enumerate(positions):
        s = S[n].astype(np.float64)
        base = -(np.repeat(s, 128) * x64).sum()
        expect = base + 2.0 * s[k // 128] * x64[k]
        assert abs(y[0, n] - expect) <= 2 * _fp64_bound(K, nrm[0, n]), (n, k)


def test_dense_numpy_expansion_matches(orc):
    # Special case reducing to library routines: numpy.unpackbits (little bit order) expands
    # the words to a dense +-1 matrix, BLAS does the product.
    M, K, N = 4, 1024, 37
    x, W, S = _case(3, M, K, N)
    bits = np.unpackbits(W.view(np.uint8).reshape(N, -1), axis=1, bitorder="little")[:, :K]
    dense = (2.0 * bits - 1.0) * np.repeat(S.astype(np.float64), 128, axis=1)
    ref = x.astype(np.float64) @ dense.T
    y, nrm = orc.gemv(x, W, S)
    assert np.all(np.abs(y - ref) <= 4 * _fp64_bound(K, nrm))


@pytest.mark.parametrize("K", [128, 256, 512])
def test_exact_rationals(orc, K):
    M, N = 2, 3
    x, W, S = _case(10 + K, M, K, N)
    y, nrm = orc.gemv(x, W, S)
    ex = exact.gemv_exact(x, W, S)
    for m in range(M):
        for n in range(N):
            err = abs(Fraction(float(y[m, n])) - ex[m][n])
            assert err <= Fraction(_fp64_bound(K, nrm[m, n])), (m, n)


@pytest.mark.parametrize("K,G", [(4, 4), (8, 4), (8, 8), (12, 4), (12, 12)])
def test_exhaustive_tiny_k(orc, K, G):
    """Every one of the 2^K sign patterns, with the group size generic (tiny K only)."""
    r = _rng(20 + K + G)
    N = 1 << K
    W = np.arange(N, dtype=np.uint32).reshape(N, 1)          # row n has sign bits = binary n
    x = synth.activations(r, 1, K)
    s_row = synth.group_scales(r, 1, K, G)
    S = np.repeat(s_row, N, axis=0)
    y, nrm = orc.gemv(x, W, S, group=G)
    yq = [Fraction(float(v)) for v in y[0]]
    # exact value of every pattern
    ex = exact.gemv_exact(x, W, S, group=G)[0]
    assert all(a == b for a, b in zip(yq, ex))                 # tiny sums are exact in fp64
    # linearity in each bit: setting bit k adds exactly 2 * s_g(k) * x_k
    xs = [Fraction(float(v)) for v in x[0]]
    ss = [Fraction(float(v)) for v in s_row[0]]
    for k in range(K):
        d = 2 * ss[k // G] * xs[k]
        for n in range(N):
            if not (n >> k) & 1:
                assert yq[n | (1 << k)] - yq[n] == d
    # complement symmetry
    for n in range(N):
        assert yq[n] == -yq[(N - 1) ^ n]


# ---------------------------------------------------------------- +-1 identity
@pytest.mark.parametrize("K", [128, 512, 4096])
def test_pm1_popcount_identity(orc, K):
    M, N = 3, 33
    r = _rng(40 + K)
    A = synth.pm1_words(r, M, K)
    W = synth.sign_words(r, N, K)
    # popcount identity via numpy.bitwise_count: dot = K - 2 * popcount(a xor w)
    pc = np.bitwise_count(A[:, None, :] ^ W[None, :, :]).sum(axis=2).astype(np.int64)
    ident = K - 2 * pc
    assert np.array_equal(orc.pm1(A, W, K), ident)
    # and the float oracle with x = +-1 (exact in fp16) and unit scales reproduces it exactly
    abits = np.unpackbits(A.view(np.uint8).reshape(M, -1), axis=1, bitorder="little")[:, :K]
    x = (2.0 * abits - 1.0).astype(np.float16)
    S = np.ones((N, K // 128), np.float16)
    y, _ = orc.gemv(x, W, S)
    assert np.array_equal(y, ident.astype(np.float64))


# ---------------------------------------------------------------- patch
def test_patch_definition_involution_and_negation(orc):
    M, K, N = 2, 512, 300
    x, W, S = _case(50, M, K, N)
    rows = synth.distinct_rows(_rng(51), N, 64)
    P, bad = orc.xor_patch(W, rows, K)
    assert bad == 0
    # definition: listed rows are the bitwise NOT, every other word unchanged
    expect = W.copy()
    expect[rows] = np.bitwise_not(W[rows])
    assert np.array_equal(P, expect)
    # involution: the same XOR removes the patch
    P2, _ = orc.xor_patch(P, rows, K)
    assert np.array_equal(P2, W)
    # flipping a whole output row negates that output exactly and leaves others alone
    y0, _ = orc.gemv(x, W, S)
    y1, _ = orc.gemv(x, P, S)
    mask = np.zeros(N, bool)
    mask[rows] = True
    assert np.array_equal(y1[:, mask], -y0[:, mask])
    assert np.array_equal(y1[:, ~mask], y0[:, ~mask])


def test_patch_out_of_range_rows_are_skipped_and_counted(orc):
    K, N = 128, 10
    W = synth.sign_words(_rng(52), N, K)
    P, bad = orc.xor_patch(W, np.array([-1, 3, 10, 11, 9], np.int32), K)
    assert bad == 3
    expect = W.copy()
    expect[[3, 9]] ^= np.uint32(0xFFFFFFFF)
    assert np.array_equal(P, expect)


# ---------------------------------------------------------------- scaling and signs
def test_power_of_two_scaling_and_scale_sign(orc):
    M, K, N = 2, 1024, 16
    x, W, S = _case(60, M, K, N)
    y, _ = orc.gemv(x, W, S)
    y2, _ = orc.gemv(x, W, (S.astype(np.float32) * 2).astype(np.float16))
    assert np.array_equal(y2, 2 * y)
    yn, _ = orc.gemv(x, W, -S)
    assert np.array_equal(yn, -y)


def test_zero_and_subnormal_scales_are_exact(orc):
    K, N = 256, 3
    r = _rng(61)
    x = synth.activations(r, 1, K)
    W = synth.sign_words(r, N, K)
    S = np.zeros((N, 2), np.float16)
    S[1, :] = np.float16(2.0 ** -24)          # smallest subnormal
    S[2, 0] = np.float16(6.0e-5)              # subnormal (below 2^-14)
    y, nrm = orc.gemv(x, W, S)
    assert y[0, 0] == 0.0 and nrm[0, 0] == 0.0
    bits = np.unpackbits(W.view(np.uint8).reshape(N, -1), axis=1, bitorder="little")
    w = 2.0 * bits - 1.0
    x64 = x[0].astype(np.float64)
    assert y[0, 1] == pytest.approx((2.0 ** -24) * (w[1] * x64).sum(), rel=1e-12)
    s2 = float(np.float16(6.0e-5))
    assert y[0, 2] == pytest.approx(s2 * (w[2, :128] * x64[:128]).sum(), rel=1e-12)


# ---------------------------------------------------------------- page figures
def test_byte_accounting_reproduces_page_figures():
    figs = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    bpw = figs["bits_per_weight_binary"]["value"]
    assert 1 + 16 / 128 == bpw
    assert round(16 / bpw, 1) == figs["compression_vs_fp16_binary"]["value"]
    wl = synth.decode_8b()
    g = synth.Gemv("x", 4096, 4096)
    assert g.weight_bytes * 8 / g.weights == bpw
    # 8B: the decode GEMVs plus a 151936 x 4096 embedding table = the model's matrix params
    params = wl.weights + 151936 * 4096
    assert round(params / 1e9, 1) == figs["bonsai_8b_params"]["value"] / 1e9
    assert round(params * bpw / 8 / 1e9, 2) == figs["bonsai_8b_gb"]["value"]
    assert wl.weight_bytes == 1_064_263_680
    # 27B: 64 blocks; page's parameter breakdown at 1.125 bits/weight gives its 3.9 GB
    assert len({s.layer for s in synth.decode_27b().stages}) == figs["bonsai_27b_blocks"]["value"]
    p27 = sum(figs["bonsai_27b_params_breakdown_b"]["value"]) * 1e9
    assert round(p27 * bpw / 8 / 1e9, 1) == figs["bonsai_27b_binary_gb"]["value"]
    assert synth.decode_27b().weight_bytes == 3_350_200_320
    assert len(synth.decode_8b().gemvs) == 253 and len(synth.decode_8b().stages) == 145
    assert len(synth.decode_27b().gemvs) == 448 and len(synth.decode_27b().stages) == 256


def test_patch_record_size_fits_page_range():
    # A row-flip entry stored as (u16 layer, u8 projection, u8 pad, u32 row) is 8 bytes; the
    # page's 840 B - 1.1 KB patches then hold about 100-140 entries.
    lo, hi = json.load(open(os.path.join(GOLDEN, "page_figures.json")))["bankai_patch_bytes"]["value"]
    assert 100 <= lo // 8 <= hi // 8 <= 140


# ---------------------------------------------------------------- the pins have teeth
def _planted(variant):
    """A deliberately wrong dequantise-and-dot (CPU only) standing in for the oracle."""
    def gemv(x, W, S, group=128):
        M, K = x.shape
        N = W.shape[0]
        order = "big" if variant == "msb_first" else "little"
        bits = np.unpackbits(W.view(np.uint8).reshape(N, -1), axis=1, bitorder=order)[:, :K]
        w = 2.0 * bits - 1.0
        if variant == "inverted_sign":
            w = -w
        s = S.astype(np.float64)
        if variant == "scale_groups_reversed":
            s = s[:, ::-1]
        sd = np.repeat(s, group, axis=1)
        x64 = x.astype(np.float64).copy()
        if variant == "dropped_last_term":
            x64[:, -1] = 0
        y = x64 @ (sd * w).T
        if variant == "transposed_output":
            y = y[::-1, :]
        return y, np.abs(x64) @ np.abs(sd).T
    return gemv


def _pins_pass(gemv):
    """The closed-form and one-hot pins, as predicates over any gemv implementation."""
    ok = True
    r = _rng(80)
    K, M = 256, 2
    x = synth.activations(r, M, K)
    S = synth.group_scales(r, 2, K)
    W = np.zeros((2, K // 32), np.uint32)
    W[0] = 0xFFFFFFFF
    y, nrm = gemv(x, W, S)
    gx = x.astype(np.float64).reshape(M, K // 128, 128).sum(axis=2)
    cf = gx @ S.astype(np.float64).T
    ok &= bool(np.all(np.abs(y - cf * np.array([1.0, -1.0])) <= 2 * _fp64_bound(K, nrm)))
    positions = [0, 7, 31, 32, 127, 128, 255]
    S1 = synth.group_scales(r, len(positions), K)
    W1 = np.zeros((len(positions), K // 32), np.uint32)
    for n, k in enumerate(positions):
        W1[n, k // 32] = np.uint32(1) << np.uint32(k % 32)
    y1, n1 = gemv(x, W1, S1)
    x64 = x.astype(np.float64)
    for n, k in enumerate(positions):
        s = S1[n].astype(np.float64)
        expect = -(x64 * np.repeat(s, 128)).sum(axis=1) + 2.0 * s[k // 128] * x64[:, k]
        ok &= bool(np.all(np.abs(y1[:, n] - expect) <= 2 * _fp64_bound(K, n1[:, n])))
    return ok


def test_pins_accept_the_oracle(orc):
    assert _pins_pass(orc.gemv)


@pytest.mark.parametrize("variant", ["msb_first", "inverted_sign", "scale_groups_reversed",
                                     "dropped_last_term", "transposed_output"])
def test_planted_mistakes_are_caught(variant):
    assert not _pins_pass(_planted(variant))


# ---------------------------------------------------------------- bit patch (Bankai experiments)
def _bits_pins_pass(xor_bits, gemv):
    """Pins of the bit-granular patch, as a predicate over any implementation."""
    ok = True
    r = _rng(90)
    mats = [synth.sign_words(r, 40, 256), synth.sign_words(r, 7, 384)]
    # one flip of weight (row, k) changes output row `row` by -2 s w x_k and nothing else
    # (the rank-one closed form, checked through the pinned dequantise-and-dot)
    x = synth.activations(r, 2, 256)
    S = synth.group_scales(r, 40, 256)
    for row, k in [(0, 0), (5, 31), (5, 32), (39, 255), (17, 128)]:
        P, bad = xor_bits(mats, np.array([[0, row, k]], np.int32))
        y0, _ = gemv(x, mats[0], S)
        y1, _ = gemv(x, P[0], S)
        w = 1.0 if (int(mats[0][row, k // 32]) >> (k % 32)) & 1 else -1.0
        delta = -2.0 * float(S[row, k // 128]) * w * x[:, k].astype(np.float64)
        expect = y0.copy()
        expect[:, row] += delta
        ok &= bad == 0 and bool(np.allclose(y1, expect, rtol=0, atol=1e-9))
        ok &= bool(np.array_equal(P[1], mats[1]))
    # every bit of a row listed == the row patch of that row
    row = 3
    full = np.array([[1, row, k] for k in range(384)], np.int32)
    P, _ = xor_bits(mats, full)
    expect = mats[1].copy()
    expect[row] = np.bitwise_not(mats[1][row])
    ok &= bool(np.array_equal(P[1], expect))
    # a multiset of flips: duplicates cancel in pairs, order is irrelevant, and the same list
    # applied twice restores both matrices
    e = np.array([[0, 1, 2], [1, 6, 383], [0, 1, 2], [0, 1, 2], [1, 0, 0]], np.int32)
    P, _ = xor_bits(mats, e)
    expect0 = mats[0].copy()
    expect0[1, 0] ^= np.uint32(1 << 2)
    expect1 = mats[1].copy()
    expect1[6, 11] ^= np.uint32(1 << 31)
    expect1[0, 0] ^= np.uint32(1)
    ok &= bool(np.array_equal(P[0], expect0)) and bool(np.array_equal(P[1], expect1))
    P2, _ = xor_bits(P, e[::-1])
    ok &= bool(np.array_equal(P2[0], mats[0])) and bool(np.array_equal(P2[1], mats[1]))
    # out-of-range entries are skipped and counted
    bad_e = np.array([[2, 0, 0], [-1, 0, 0], [0, 40, 0], [0, -1, 0], [0, 0, 256], [1, 0, -1], [1, 6, 0]],
                     np.int32)
    P, bad = xor_bits(mats, bad_e)
    expect1 = mats[1].copy()
    expect1[6, 0] ^= np.uint32(1)
    ok &= bad == 6 and bool(np.array_equal(P[0], mats[0])) and bool(np.array_equal(P[1], expect1))
    return ok


def _planted_bits(variant):
    def xor_bits(mats, entries):
        outs = [np.array(m, copy=True) for m in mats]
        bad = 0
        for mid, row, k in np.asarray(entries).reshape(-1, 3):
            if not (0 <= mid < len(outs)) or not (0 <= row < outs[mid].shape[0]) or \
                    not (0 <= k < outs[mid].shape[1] * 32):
                bad += 1
                continue
            if variant == "msb_first":
                outs[mid][row, k // 32] ^= np.uint32(1 << (31 - k % 32))
            elif variant == "set_not_flip":
                outs[mid][row, k // 32] |= np.uint32(1 << (k % 32))
            elif variant == "row_major_swapped":
                kk = k % (outs[mid].shape[0] * 32)
                outs[mid][kk // 32 % outs[mid].shape[0], (row * 32 + k % 32) // 32 % outs[mid].shape[1]] ^= \
                    np.uint32(1 << (k % 32))
            else:
                outs[mid][row, k // 32] ^= np.uint32(1 << (k % 32))
        if variant == "uncounted":
            bad = 0
        return outs, bad
    return xor_bits


def test_bit_patch_pins_accept_the_oracle(orc):
    assert _bits_pins_pass(orc.xor_bits, orc.gemv)


@pytest.mark.parametrize("variant", ["msb_first", "set_not_flip", "row_major_swapped", "uncounted"])
def test_bit_patch_planted_mistakes_are_caught(orc, variant):
    assert not _bits_pins_pass(_planted_bits(variant), orc.gemv)


# ---------------------------------------------------------------- scale ranking of rows
def _rank_pins_pass(rank_rows, half_to_double):
    ok = True
    r = _rng(95)
    S = synth.group_scales(r, 300, 1024)                 # 8 groups per row
    S[7] = S[3]                                          # exact ties, resolved by row index
    S[250] = S[3]
    S[11, :] = np.float16(0.0)
    S[12, 0] = np.float16(-0.0)                          # sign ignored
    S[12, 1:] = S[11, 1:]
    S[13] = -S[5]                                        # magnitude only: same score as row 5
    S[20, 0] = np.float16(np.ldexp(1.0, -24))            # subnormals and the largest finite value
    S[21, 0] = np.float16(65504.0)
    score, order = rank_rows(S)
    # the score is sum |s| * 2^24, with |s| from the pinned fp16 decode
    for n in range(S.shape[0]):
        ref = sum(abs(half_to_double(int(h))) for h in S[n].view(np.uint16)) * 2.0 ** 24
        ok &= float(score[n]) == ref
    # the order is the comparison sort (score descending, row ascending), brute force
    ranked = sorted(range(S.shape[0]), key=lambda n: (-int(score[n]), n))
    ok &= bool(np.array_equal(order, np.array(ranked, np.int32)))
    ok &= list(order[list(order).index(3):list(order).index(3) + 2]) == [3, 7]
    ok &= int(order[0]) == 21
    # hand-worked example: rows of two groups
    S2 = np.array([[1.0, 2.0], [-3.0, 0.0], [0.5, 2.5], [0.0, 0.0]], np.float16)
    sc2, or2 = rank_rows(S2)
    ok &= list(sc2) == [3 << 24, 3 << 24, 3 << 24, 0] and list(or2) == [0, 1, 2, 3]
    S3 = np.array([[0.25, 0.0], [1.0, 1.0], [0.0, 0.5]], np.float16)
    sc3, or3 = rank_rows(S3)
    ok &= list(sc3) == [1 << 22, 1 << 25, 1 << 23] and list(or3) == [1, 2, 0]
    return ok


def _planted_rank(variant):
    def rank_rows(S):
        s = S.astype(np.float64)
        if variant == "signed_sum":
            sc = (s.sum(axis=1) * 2.0 ** 24).astype(np.int64)
        elif variant == "max_not_sum":
            sc = (np.abs(s).max(axis=1) * 2.0 ** 24).astype(np.int64)
        else:
            sc = (np.abs(s).sum(axis=1) * 2.0 ** 24).astype(np.int64)
        if variant == "ascending":
            order = sorted(range(len(sc)), key=lambda n: (int(sc[n]), n))
        elif variant == "ties_reversed":
            order = sorted(range(len(sc)), key=lambda n: (-int(sc[n]), -n))
        else:
            order = sorted(range(len(sc)), key=lambda n: (-int(sc[n]), n))
        return sc, np.array(order, np.int32)
    return rank_rows


def test_rank_pins_accept_the_oracle(orc):
    assert _rank_pins_pass(orc.rank_rows, orc.half_to_double)


@pytest.mark.parametrize("variant", ["signed_sum", "max_not_sum", "ascending", "ties_reversed"])
def test_rank_planted_mistakes_are_caught(orc, variant):
    assert not _rank_pins_pass(_planted_rank(variant), orc.half_to_double)


# ---------------------------------------------------------------- ternary g128 in 2-bit slots
def _binary_as_ternary(W, K):
    """The 2-bit-slot words holding +1 (code 01) for every set sign bit and -1 (code 11) for
    every clear one."""
    bits = np.unpackbits(W.view(np.uint8).reshape(W.shape[0], -1), axis=1, bitorder="little")[:, :K]
    codes = np.where(bits == 1, 1, 3).astype(np.uint32).reshape(W.shape[0], K // 16, 16)
    return np.bitwise_or.reduce(codes << (2 * np.arange(16, dtype=np.uint32)), axis=2).astype(np.uint32)


def _t2_pins_pass(gemv_t2, gemv):
    ok = True
    r = _rng(97)
    M, K, N = 2, 512, 24
    x = synth.activations(r, M, K)
    S = synth.group_scales(r, N, K)
    S[3] = -S[3]
    W = synth.sign_words(r, N, K)
    # with no zero codes, the ternary product is the binary product of the same signs, term for
    # term (both ascending k, same products), so bit-identical
    yt, nt = gemv_t2(x, _binary_as_ternary(W, K), S)
    yb, nb = gemv(x, W, S)
    ok &= bool(np.array_equal(yt, yb)) and bool(np.array_equal(nt, nb))
    # all-zero codes, and the never-written code 10, add nothing
    for code in (0, 2):
        Tz = np.full((N, K // 16), sum(code << (2 * i) for i in range(16)), np.uint32)
        yz, nz = gemv_t2(x, Tz, S)
        ok &= bool(np.all(yz == 0.0)) and bool(np.all(nz == 0.0))
    # one nonzero slot at k: y = t * s_{k/128} * x_k exactly (pins LSB-first 2-bit placement)
    x64 = x.astype(np.float64)
    for k, code, t in [(0, 1, 1.0), (1, 3, -1.0), (15, 1, 1.0), (16, 3, -1.0), (127, 1, 1.0), (128, 3, -1.0),
                       (511, 1, 1.0)]:
        T1 = np.zeros((N, K // 16), np.uint32)
        T1[:, k // 16] = np.uint32(code << (2 * (k % 16)))
        y1, _ = gemv_t2(x, T1, S)
        expect = t * S[:, k // 128].astype(np.float64)[None, :] * x64[:, k:k + 1]
        ok &= bool(np.array_equal(y1, expect))
    # exhaustive: every ternary row of K = 8 (3^8 rows, groups of 4) against exact rationals
    Kt, G = 8, 4
    vals = np.array(np.meshgrid(*[[0, 1, -1]] * Kt, indexing="ij")).reshape(Kt, -1).T      # [6561][8]
    codes = np.where(vals == 0, 0, np.where(vals > 0, 1, 3)).astype(np.uint32)
    Te = np.bitwise_or.reduce(codes << (2 * np.arange(Kt, dtype=np.uint32)), axis=1).astype(np.uint32)[:, None]
    xe = synth.activations(_rng(98), 1, Kt)
    Se = synth.group_scales(_rng(99), vals.shape[0], Kt, group=G)
    ye, _ = gemv_t2(xe, Te, Se, group=G)
    xf = [Fraction(float(v)) for v in xe[0]]
    for n in range(vals.shape[0]):
        ref = sum(Fraction(float(Se[n, k // G])) * int(vals[n, k]) * xf[k] for k in range(Kt))
        ok &= abs(Fraction(ye[0, n]) - ref) <= Fraction(2 ** -40) * (abs(ref) + 1)
    return ok


def _planted_t2(variant):
    def gemv_t2(x, T, S, group=128):
        M, K = x.shape
        N = T.shape[0]
        sh = 2 * np.arange(16, dtype=np.uint32)
        if variant == "msb_first":
            sh = sh[::-1]
        codes = ((T[:, :, None] >> sh[None, None, :]) & 3).reshape(N, -1)[:, :K]
        if variant == "sign_magnitude_swapped":
            t = np.where(codes & 2, np.where(codes & 1, -1.0, 1.0), 0.0)
        elif variant == "code10_is_minus_one":
            t = np.where(codes == 1, 1.0, np.where(codes == 0, 0.0, -1.0))
        else:
            t = np.where(codes & 1, np.where(codes & 2, -1.0, 1.0), 0.0)
        sd = np.repeat(S.astype(np.float64), group, axis=1)
        if variant == "scale_off_by_one_group":
            sd = np.roll(sd, group, axis=1)
        terms = x.astype(np.float64)[:, None, :] * (sd * t)[None, :, :]
        return terms.sum(axis=2), np.abs(terms).sum(axis=2)
    return gemv_t2


def test_ternary_pins_accept_the_oracle(orc):
    assert _t2_pins_pass(orc.gemv_t2, orc.gemv)


@pytest.mark.parametrize("variant", ["msb_first", "sign_magnitude_swapped", "code10_is_minus_one",
                                     "scale_off_by_one_group"])
def test_ternary_planted_mistakes_are_caught(orc, variant):
    assert not _t2_pins_pass(_planted_t2(variant), orc.gemv)


def test_ternary_byte_accounting_reproduces_page_figures():
    figs = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    bits = np.log2(3) + 16 / 128                                  # information content + scale
    assert round(bits, 2) == figs["bits_per_weight_ternary"]["value"]
    assert round(16 / figs["bits_per_weight_ternary"]["value"], 1) == figs["compression_vs_fp16_ternary"]["value"]
    lm, vision, emb = figs["bonsai_27b_params_breakdown_b"]["value"]
    assert round((lm + vision + emb) * figs["bits_per_weight_ternary"]["value"] / 8, 1) == \
        figs["bonsai_27b_ternary_gb"]["value"]
    # 2-bit slots: 2 + 16/128 bits per weight for the language model and embedding/head (the
    # vision tower is stored at 4 bits separately), about the page's deployed 7.2 GB
    slot_bits = 2 + 16 / 128
    assert synth.ternary_words(_rng(1), 4, 256).nbytes * 8 / (4 * 256) == 2.0
    assert abs((lm + emb) * slot_bits / 8 - figs["bonsai_27b_ternary_deployed_gb"]["value"]) < 0.1
