"""The variant query (bin1_kernel_variant) names, for every shape of tests/variants.py, the kernel
variant the dispatch code picks; the GPU tests then run exactly those shapes against the oracle.
Here (no GPU) the table is checked against the query, and the table is checked to reach every
branch of the dispatch."""
import numpy as np
import pytest

from variants import ALL_CASES, DECODE_CASES, DECODE_T2_CASES, case_id


@pytest.fixture(scope="module")
def b1():
    import bit_packed_sign_amd as b1
    from bit_packed_sign_amd import binding, build
    import os
    if not os.path.exists(binding.LIB_PATH):
        build.build()
    return b1


@pytest.mark.parametrize("case", ALL_CASES, ids=case_id)
def test_query_names_the_expected_variant(b1, case):
    op, M, K, Ns, expect, _ = case
    got = b1.kernel_variant(op, M, K, Ns)
    assert got.split(" ")[0] == expect, (got, expect)
    if expect.startswith("gemv_mx<"):                # batch-1 kernel: one grid copy per token
        assert (f" tokens={M} " in got) == (M > 1), got
    if "split" in expect:                       # the partial-sum kernel, then the chunk reduction
        assert got.count(";") == 1 and got.split(";")[1].startswith("smallm_reduce")
    else:
        assert ";" not in got                   # one launch for the whole call


def test_every_decode_branch_is_reached():
    """Each (pairs per wave, ring slots, rows per tile, waves) branch of the batch-1 kernel occurs
    with even and odd K / 128, with a partial last pair, and with one/two and three/four matrices."""
    for cases, expected_branches in ((DECODE_CASES, 5 + 2 + 3 + 2 + 2), (DECODE_T2_CASES, 5 + 4 + 3 + 2 + 1)):
        # (binary rows of 5..8 and 17..20 pairs have layouts of their own)
        seen = {}
        for op, M, K, Ns, exp, kind in cases:
            core = exp.split("<")[1].rstrip(">").split(",")
            branch = tuple(core[i] for i in (0, 1, 2, 5)) + (core[7] if len(core) > 7 else "1",)   # SP, P, R, NW, TT
            seen.setdefault(branch, set()).add((kind, core[3], core[6]))
        assert len(seen) == expected_branches, sorted(seen)
        for branch, kinds in seen.items():
            assert {k for k, _, _ in kinds} == {"even", "odd", "part"}, (branch, kinds)
            assert {o for _, o, _ in kinds} == {"0", "1"}, (branch, kinds)
    # matrices past the scalar tile table occur in every pairs-per-wave class
    for cases in (DECODE_CASES, DECODE_T2_CASES):
        table = [c for c in cases if c[4].split("<")[1].split(",")[6].rstrip(">") == "0"]
        classes = {((c[2] + 1023) // 1024 + 3) // 4 for c in table}
        nws = {c[4].split(",")[5] for c in table}
        assert classes == {1, 2, 3, 4, 5} and nws >= {"4", "12"}


def test_query_rejects_bad_arguments(b1):
    from bit_packed_sign_amd.binding import Bin1Error
    with pytest.raises(Bin1Error):
        b1.kernel_variant("gemv", 1, 100, [10])               # K % 128 != 0
    with pytest.raises(Bin1Error):
        b1.kernel_variant("gemv", 0, 128, [10])               # M < 1
    with pytest.raises(Bin1Error):
        b1.kernel_variant("prefill", 4, 128, [10, 20])        # prefill takes one matrix
    with pytest.raises(Bin1Error):
        b1.kernel_variant("gemv", 1, 128, [1, 2, 3, 4, 5])    # at most four matrices


def test_batch1_launches_fit_the_lds(b1):
    """The batch-1 kernel holds a K-long slice of limbs, a tile table and one fp32 partial per
    (row, wave) of its tiles in LDS; the launcher bounds the tiles per workgroup so that this stays
    within the 160 KB a workgroup can have, also at the longest rows (K = 20480) and the tallest
    matrices the argument rules allow (N < 2^24 - 64, the bits under 2 GiB).  Every launch of a
    sweep over K and N must describe an LDS size within the limit."""
    lim = 160 * 1024
    seen = 0
    for op, bits in (("gemv", 1), ("gemv_t2", 2)):
        for K in (128, 1024, 3968, 4096, 5120, 8192, 12288, 16384, 17408, 19456, 20352, 20480):
            nmax = min((1 << 24) - 65, ((1 << 31) - 1) // (K * bits // 8))
            Ns = sorted({int(n) for n in np.geomspace(1, nmax, 48)} | {nmax})
            for N in Ns:
                for group in ([N], [N // 2 + 1, N // 2 + 1], [N // 3 + 1] * 3):
                    desc = b1.kernel_variant(op, 1, K, group)
                    for launch in desc.split(";"):
                        if launch.startswith("gemv_mx<"):
                            lds = int(launch.split("lds=")[1].split()[0])
                            assert 0 < lds <= lim, (op, K, group, launch)
                            seen += 1
    assert seen > 1000
