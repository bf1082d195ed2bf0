"""Shapes that reach every branch of the product dispatch (test infrastructure).

Each case is (op, M, K, Ns, expected variant): ``op`` as in ``bit_packed_sign_amd.kernel_variant``
("gemv" covers bin1_gemv and bin1_gemv_group, "gemv_t2" their ternary forms), ``Ns`` the row
counts of the matrices of one call, and the expected text the variant query returns for them.
The shapes are derived from the dispatch thresholds of the batch-1 decode kernel (tiles of 16
rows against the workgroups that fit 256 compute units at one, two or more 1024-wide pairs per
wave), of the small-batch kernel (tiles per workgroup, 4096-wide K chunks) and of the prefill
kernel (256-row tiles only when they fill the GPU twice over).  Every decode branch appears with
an even and an odd number of scale groups per row (K / 128 odd: the scale pair of a lane is read
as two halves), with a last 1024-wide pair that is only partly inside K, and with three or four
matrices (no scalar tile table) as well as one or two.
"""

# K values: EVEN = K / 128 even and K a whole number of 1024-wide pairs; ODD = K / 128 odd;
# PART = the last pair partly inside K
SP_K = {
    1: {"even": 4096, "odd": 3968, "part": 3200},
    2: {"even": 8192, "odd": 4224, "part": 6400},
    3: {"even": 12288, "odd": 8320, "part": 10496},
    4: {"even": 16384, "odd": 12416, "part": 14592},
    5: {"even": 20480, "odd": 16512, "part": 18688},
}


def _mx(sp, p, r, odd, t2, nw, two, tt=1, al=False):
    tail = (f",{tt}" if tt > 1 or al else "") + (",AL" if al else "")
    return f"gemv_mx<{sp},{p},{r},{int(odd)},{int(t2)},{nw},{int(two)}{tail}>"


def _decode_cases(t2):
    op = "gemv_t2" if t2 else "gemv"
    cases = []
    for kind, K in [(k, v) for sp in SP_K for k, v in SP_K[sp].items()]:
        sp = ((K + 1023) // 1024 + 3) // 4
        odd = (K // 128) % 2 == 1
        # (Ns, expected (SP, P, R, NW)) per branch of this pairs-per-wave class
        if sp == 1:
            # up to 256 16-row tiles one per workgroup; then one 32-row tile per workgroup; then
            # three groups of four waves per workgroup (TT = 3) on 16-row tiles; a three-slot ring
            # of 16-row tiles; past that 32-row tiles in three wave groups on a one-slot ring
            # (ternary rows: 16-row tiles in two wave groups).
            # Three or four matrices: one group of four waves in the same tiles.
            big = (1, 1, 1, 8, 2) if t2 else (1, 1, 2, 12, 3)
            big3 = (1, 1, 1, 4) if t2 else (1, 1, 2, 4)
            branches = [([100], (1, 1, 1, 4)), ([6000], (1, 1, 2, 4)), ([20000], (1, 1, 1, 12, 3)),
                        ([30000], (1, 3, 1, 4)), ([40000], big), ([100, 200, 300], (1, 1, 1, 4)),
                        ([2000, 2000, 2000], (1, 1, 2, 4)), ([7000, 7000, 7000], (1, 1, 1, 4)),
                        ([10000, 10000, 10000], (1, 3, 1, 4)), ([15000, 15000, 15000], big3)]
        elif sp == 2 and not t2:
            # binary: eight waves of one pair on 32-row tiles; a two-slot ring past 1536 of them
            branches = [([1000], (1, 1, 2, 8)), ([30000], (1, 1, 2, 8)), ([60000], (1, 2, 2, 8)),
                        ([3000, 3000, 3000], (1, 1, 2, 8)), ([20000, 20000, 20000], (1, 2, 2, 8))]
        elif sp == 2:
            branches = [([1000], (1, 1, 1, 8)), ([10000], (2, 1, 2, 4)), ([20000], (2, 2, 1, 4)),
                        ([30000], (2, 2, 2, 4)), ([3000, 3000, 3000], (2, 1, 2, 4))]
        elif sp == 3:
            branches = [([1000], (1, 1, 1, 12)), ([6000], (3, 1, 2, 4)), ([10000], (3, 2, 2, 4)),
                        ([500, 600, 700, 800], (1, 1, 1, 12))]
        elif sp == 4:
            branches = [([1000], (1, 1, 1, 16)), ([6000], (4, 1, 1 if t2 else 2, 4)),
                        ([2000, 2000, 2000], (4, 1, 1 if t2 else 2, 4))]
        elif t2:
            branches = [([1000], (5, 1, 1, 4)), ([300, 400, 500], (5, 1, 1, 4))]
        else:
            # binary: twelve waves of up to two pairs, A operands read per pair (AL), on 16-row
            # tiles: a one-slot ring up to 256 32-row tiles, two slots past that
            branches = [([1000], (2, 1, 1, 12, 1, True)), ([6000], (2, 1, 1, 12, 1, True)),
                        ([300, 400, 500], (2, 1, 1, 12, 1, True)),
                        ([10000], (2, 2, 1, 12, 1, True)), ([3000, 3000, 3000], (2, 2, 1, 12, 1, True))]
        # the even-K class carries every branch; the odd and partial-pair classes every branch too,
        # but with smaller matrices where a branch allows it
        for Ns, br in branches:
            s_, p_, r_, nw_ = br[:4]
            tt = br[4] if len(br) > 4 else 1
            al = br[5] if len(br) > 5 else False
            cases.append((op, 1, K, Ns, _mx(s_, p_, r_, odd, t2, nw_, len(Ns) <= 2, tt, al), f"{kind}"))
    return cases


DECODE_CASES = _decode_cases(False)
DECODE_T2_CASES = _decode_cases(True)

# rows past the block-scaled kernel's K range (K > 20480): the select/accumulate kernel
SELECT_CASES = [("gemv", 1, 20608, [70], "gemv_select<1>", "long")]

# small batch (2 <= M <= 16): tiles per workgroup TB and K chunks in flight D (D = 0: one chunk)
SMALLM_CASES = [
    ("gemv", 16, 4096, [4096], "gemv_smallm<2,0>", "tb2"),
    ("gemv", 12, 4096, [12288], "gemv_smallm<4,0>", "tb4"),
    ("gemv", 16, 4096, [12288, 12288], "gemv_smallm<6,0>", "tb6"),
    ("gemv", 16, 12288, [4096], "gemv_smallm<1,4>", "tb1d4"),
    ("gemv", 2, 8192, [8192], "gemv_smallm<2,3>", "tb2d3"),
    ("gemv", 8, 8192, [16384], "gemv_smallm<4,2>", "tb4d2"),
    ("gemv", 3, 3968, [1000, 2000, 3000], "gemv_smallm<2,0>", "group3"),
]

# 2 <= M <= 8 with K a multiple of 1024 (and K <= 4096 without a workspace) and at least 4096
# tiles of 16 rows: the block-scaled small-batch kernel, MB token blocks of four (MB = 1 for
# M <= 4), a four-slot ring (every such product gives a workgroup 16 tiles or more); past 43 tiles
# per workgroup (MB = 2) the grid grows.  One tile fewer stays on the fp16 kernel.
MXM_CASES = [
    ("gemv", 2, 4096, [65536], "gemv_mxm<1,4>", "tall"),
    ("gemv", 3, 1024, [70000], "gemv_mxm<1,4>", "k1024"),
    ("gemv", 5, 4096, [70000], "gemv_mxm<2,4>", "m5"),
    ("gemv", 6, 2048, [30000, 30000, 10000], "gemv_mxm<2,4>", "group3"),
    ("gemv", 7, 4096, [20000, 20000, 20000, 10000], "gemv_mxm<2,4>", "group4"),
    ("gemv", 8, 4096, [180000], "gemv_mxm<2,4>", "capped"),
    ("gemv", 8, 4096, [65520], "gemv_smallm<6,0>", "below"),
]

MXM_WS_CASES = [
    ("gemv_ws", 2, 8192, [65536], "gemv_mxm_split<1,4>", "split2"),
    ("gemv_ws", 5, 12288, [70000], "gemv_mxm_split<2,4>", "split3"),
    ("gemv_ws", 3, 5120, [66000], "gemv_mxm_split<1,4>", "onepair"),
    ("gemv_ws", 3, 8192, [300], "gemv_smallm_split<1>", "ragged"),
]

# two tokens on short products (at most 256 tiles of 16 rows): two copies of the one-token grid,
# workgroup b serving token b / grid (the variant's " tokens=2" is checked beside its name)
TOKEN_CASES = [
    ("gemv", 2, 4096, [4096], "gemv_mx<1,1,1,0,0,4,1>", "o"),
    ("gemv", 2, 4096, [4112], "gemv_smallm<2,0>", "past256"),
    ("gemv", 2, 12288, [4096], "gemv_mx<1,1,1,0,0,12,1>", "down"),
    ("gemv", 2, 3968, [1000], "gemv_mx<1,1,1,1,0,4,1>", "odd"),
    ("gemv", 2, 4096, [1000, 2000, 1000], "gemv_mx<1,1,1,0,0,4,0>", "group3"),
    ("gemv", 2, 4096, [2000, 2000], "gemv_mx<1,1,1,0,0,4,1>", "group2"),
    ("gemv_ws", 2, 12288, [4096], "gemv_mx<1,1,1,0,0,12,1>", "ws"),
    ("gemv", 2, 17408, [4000], "gemv_mx<2,1,1,0,0,12,1,1,AL>", "al"),
]

# prefill: 128-row tiles (two workgroups per CU) at every M; a short and a full-width M
PREFILL_CASES = [
    ("prefill", 300, 1024, [777], "prefill<128,2,0>", "small"),
    ("prefill", 2048, 1024, [12288], "prefill<128,2,0>", "large"),
    ("prefill_t2", 300, 1024, [777], "prefill<128,2,1>", "small"),
    ("prefill_t2", 2048, 1024, [12288], "prefill<128,2,1>", "large"),
]

# small batch with a workspace: K split into 4096-wide chunks over workgroups (G tile groups per
# chunk, TB tiles each) then the chunk reduction; shapes without a split run as bin1_gemv
WS_CASES = [
    ("gemv_ws", 16, 12288, [4096], "gemv_smallm_split<4>", "down"),
    ("gemv_ws", 12, 20480, [5000], "gemv_smallm_split<8>", "tb8"),
    ("gemv_ws", 16, 17408, [5120], "gemv_smallm_split<8>", "down27b"),
    ("gemv_ws", 9, 4224, [1000], "gemv_smallm_split<1>", "partial"),
    ("gemv_ws", 16, 4096, [4096], "gemv_smallm<2,0>", "nosplit"),
    ("gemv_ws", 1, 12288, [4096], "gemv_mx<1,1,1,0,0,12,1>", "m1"),
    ("gemv_ws", 1, 4096, [151936], "gemv_mx<1,1,2,0,0,12,1,3>", "lmhead"),
]

ALL_CASES = (DECODE_CASES + DECODE_T2_CASES + SELECT_CASES + SMALLM_CASES + MXM_CASES + PREFILL_CASES + WS_CASES
             + MXM_WS_CASES + TOKEN_CASES)


def case_id(c):
    op, M, K, Ns, exp, kind = c
    return f"{op}-M{M}-K{K}-{'x'.join(map(str, Ns))}"
