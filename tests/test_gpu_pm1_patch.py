"""GPU checks of the exact paths: +-1 popcount product and XOR row patches (bit-exact)."""
import numpy as np
import pytest
import torch

import bit_packed_sign_amd as b1
from bit_packed_sign_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32))


# every lanes-per-row class (rows of 1, 2, 4, ... 64+ sixteen-byte chunks), chunk counts that are not
# a power of two, ragged row counts, batches above and below the 8-row activation block
@pytest.mark.parametrize("M,K,N", [(1, 128, 1), (1, 128, 131), (2, 256, 67), (3, 512, 77), (1, 640, 99),
                                   (1, 1024, 513), (5, 2048, 130), (1, 4096, 4096), (1, 4096, 4099),
                                   (16, 12288, 300), (9, 17408, 65), (1, 4096, 151936), (1, 8192, 1000)])
def test_pm1_bit_exact(orc, dev, M, K, N):
    r = synth.rng_for(0, synth.WL_TEST, 6000 + M + K + N)
    A = synth.pm1_words(r, M, K)
    W = synth.sign_words(r, N, K)
    y = b1.gemv_pm1(_i32(A).to(dev), _i32(W).to(dev)).cpu().numpy()
    assert np.array_equal(y, orc.pm1(A, W, K))


def test_pm1_extremes(orc, dev):
    K = 256
    A = np.array([[0xFFFFFFFF] * 8, [0] * 8], np.uint32)
    W = np.array([[0xFFFFFFFF] * 8, [0] * 8, [0xAAAAAAAA] * 8], np.uint32)
    y = b1.gemv_pm1(_i32(A).to(dev), _i32(W).to(dev)).cpu().numpy()
    assert np.array_equal(y, orc.pm1(A, W, K))
    assert y[0, 0] == K and y[0, 1] == -K and y[0, 2] == 0


def test_single_matrix_patch_apply_remove(orc, dev):
    """4096x4096 weights, 64 distinct rows: apply then remove, bit-exact against the oracle."""
    K = N = 4096
    W = synth.sign_words(synth.rng_for(0, synth.WL_SINGLE, 0), N, K)
    rows = synth.patch_rows_single()
    Wd = _i32(W).to(dev)
    rd = torch.from_numpy(rows).to(dev)
    bad = torch.zeros(1, dtype=torch.int32, device=dev)
    b1.xor_patch_apply(Wd, rd, bad_rows=bad)
    expect, nbad = orc.xor_patch(W, rows, K)
    assert np.array_equal(Wd.cpu().numpy().view(np.uint32), expect)
    b1.xor_patch_apply(Wd, rd, bad_rows=bad)
    assert np.array_equal(Wd.cpu().numpy().view(np.uint32), W)
    assert int(bad.item()) == 0 and nbad == 0


def test_patch_out_of_range_and_empty(orc, dev):
    K, N = 256, 40
    W = synth.sign_words(synth.rng_for(0, synth.WL_TEST, 6100), N, K)
    rows = np.array([-5, 0, 39, 40, 1000, 7], np.int32)
    Wd = _i32(W).to(dev)
    bad = torch.zeros(1, dtype=torch.int32, device=dev)
    b1.xor_patch_apply(Wd, torch.from_numpy(rows).to(dev), bad_rows=bad)
    expect, nbad = orc.xor_patch(W, rows, K)
    assert np.array_equal(Wd.cpu().numpy().view(np.uint32), expect)
    assert int(bad.item()) == nbad == 3
    b1.xor_patch_apply(Wd, torch.zeros(0, dtype=torch.int32, device=dev))
    assert np.array_equal(Wd.cpu().numpy().view(np.uint32), expect)
    with pytest.raises(ValueError):                  # the opt-in host check of repeated rows
        b1.xor_patch_apply(Wd, torch.tensor([1, 1], dtype=torch.int32, device=dev), check_distinct=True)


def test_patch_repeated_rows_commute(orc, dev):
    """Rows listed several times in one call: each listing is one complement, applied as atomic
    XORs, so an even count leaves the row unchanged and an odd count complements it -- the same
    as the oracle's one-after-another application -- on both patch calls, every run."""
    K, N = 4096, 64
    W = synth.sign_words(synth.rng_for(0, synth.WL_TEST, 6150), N, K)
    rows = np.array([3, 3, 5, 9, 9, 9, 11, 11, 11, 11, 20] * 8, np.int32)   # many workgroups per row
    expect, _ = orc.xor_patch(W, rows, K)
    for _ in range(3):
        Wd = _i32(W).to(dev)
        b1.xor_patch_apply(Wd, torch.from_numpy(rows).to(dev))
        assert np.array_equal(Wd.cpu().numpy().view(np.uint32), expect)
        table = b1.PatchTable([Wd])
        ent = torch.from_numpy(np.stack([np.zeros_like(rows), rows], axis=1)).to(dev)
        b1.xor_patch_apply_multi(table, ent)
        assert np.array_equal(Wd.cpu().numpy().view(np.uint32), W)


def test_patch_in_a_graph(orc, dev):
    """The patch calls enqueue work only (no host synchronisation), so they can be captured; every
    replay of apply-then-remove leaves the weights as they were, and one apply matches the oracle."""
    K, N = 1024, 300
    W = synth.sign_words(synth.rng_for(0, synth.WL_TEST, 6160), N, K)
    rows = synth.distinct_rows(synth.rng_for(0, synth.WL_TEST, 6161), N, 40)
    Wd = _i32(W).to(dev)
    rd = torch.from_numpy(rows).to(dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        b1.xor_patch_apply(Wd, rd)
        b1.xor_patch_apply(Wd, rd)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g1, g2 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        b1.xor_patch_apply(Wd, rd)
    with torch.cuda.graph(g2):
        b1.xor_patch_apply(Wd, rd)
    expect, _ = orc.xor_patch(W, rows, K)
    for _ in range(3):
        g1.replay()
        torch.cuda.synchronize()
        assert np.array_equal(Wd.cpu().numpy().view(np.uint32), expect)
        g2.replay()
        torch.cuda.synchronize()
        assert np.array_equal(Wd.cpu().numpy().view(np.uint32), W)


def test_multi_matrix_patch_27b_mlp(orc, dev):
    """2000 distinct (layer, projection, row) flips over all 192 MLP matrices of the 27B
    decode workload in one launch; every matrix bit-exact after apply and after removal."""
    mats = synth.mlp_rows_27b()
    r = synth.rng_for(0, synth.WL_TEST, 6200)
    host = []
    for (_, p, n) in mats:
        K = 5120 if p in ("gate", "up") else 17408
        host.append(synth.sign_words(r, n, K))
    devm = [_i32(h).to(dev) for h in host]
    table = b1.PatchTable(devm)
    ent = synth.patch_entries_27b()
    ed = torch.from_numpy(ent).to(dev)
    bad = torch.zeros(1, dtype=torch.int32, device=dev)
    b1.xor_patch_apply_multi(table, ed, bad_rows=bad)
    torch.cuda.synchronize()
    for mid, (h, d) in enumerate(zip(host, devm)):
        rows = ent[ent[:, 0] == mid, 1]
        expect, _ = orc.xor_patch(h, rows, h.shape[1] * 32)
        assert np.array_equal(d.cpu().numpy().view(np.uint32), expect), mid
    b1.xor_patch_apply_multi(table, ed, bad_rows=bad)
    for h, d in zip(host, devm):
        assert np.array_equal(d.cpu().numpy().view(np.uint32), h)
    assert int(bad.item()) == 0


def test_multi_patch_bad_entries_counted(dev):
    W = synth.sign_words(synth.rng_for(0, synth.WL_TEST, 6300), 10, 128)
    Wd = _i32(W).to(dev)
    table = b1.PatchTable([Wd])
    ent = torch.tensor([[0, 2], [1, 0], [-1, 0], [0, 10], [0, -1]], dtype=torch.int32, device=dev)
    bad = torch.zeros(1, dtype=torch.int32, device=dev)
    b1.xor_patch_apply_multi(table, ent, bad_rows=bad)
    got = Wd.cpu().numpy().view(np.uint32)
    expect = W.copy()
    expect[2] ^= np.uint32(0xFFFFFFFF)
    assert np.array_equal(got, expect) and int(bad.item()) == 4


# ---------------------------------------------------------------- bit-granular patch
def test_bit_patch_matches_oracle_with_duplicates_and_bad_entries(orc, dev):
    r = synth.rng_for(0, synth.WL_TEST, 6400)
    host = [synth.sign_words(r, 37, 128), synth.sign_words(r, 300, 4096), synth.sign_words(r, 5, 12288)]
    devm = [_i32(h).to(dev) for h in host]
    table = b1.PatchTable(devm)
    ent = synth.bit_flip_entries(1, [(h.shape[0], h.shape[1] * 32) for h in host], 5000)
    ent = np.concatenate([ent, ent[:700], ent[:300],                              # repeats
                          np.array([[3, 0, 0], [-1, 0, 0], [0, 37, 0], [1, 0, 4096], [2, 4, -1]], np.int32)])
    ed = torch.from_numpy(ent).to(dev)
    bad = torch.zeros(1, dtype=torch.int32, device=dev)
    b1.xor_bits_apply(table, ed, bad=bad)
    expect, nbad = orc.xor_bits(host, ent)
    torch.cuda.synchronize()
    for mid, (e, d) in enumerate(zip(expect, devm)):
        assert np.array_equal(d.cpu().numpy().view(np.uint32), e), mid
    assert int(bad.item()) == nbad == 5
    b1.xor_bits_apply(table, ed[torch.randperm(ed.shape[0], device=dev)])   # any order removes it
    for h, d in zip(host, devm):
        assert np.array_equal(d.cpu().numpy().view(np.uint32), h)


def test_bit_patch_500k_random_flips_8b_mlp(orc, dev):
    """500K random single-bit flips over all 108 MLP matrices of the 8B workload (the page's
    robustness experiment, mechanics only), one launch; every matrix bit-exact, then removed."""
    mats = synth.mlp_mats_8b()
    r = synth.rng_for(0, synth.WL_TEST, 6500)
    host = [synth.sign_words(r, n, k) for (_, _, n, k) in mats]
    devm = [_i32(h).to(dev) for h in host]
    table = b1.PatchTable(devm)
    ent = synth.bit_flip_entries(0, [(n, k) for (_, _, n, k) in mats], 500_000)
    ed = torch.from_numpy(ent).to(dev)
    bad = torch.zeros(1, dtype=torch.int32, device=dev)
    b1.xor_bits_apply(table, ed, bad=bad)
    expect, nbad = orc.xor_bits(host, ent)
    torch.cuda.synchronize()
    assert nbad == 0 and int(bad.item()) == 0
    for mid, (e, d) in enumerate(zip(expect, devm)):
        assert np.array_equal(d.cpu().numpy().view(np.uint32), e), mid
    b1.xor_bits_apply(table, ed)
    for h, d in zip(host, devm):
        assert np.array_equal(d.cpu().numpy().view(np.uint32), h)


# ---------------------------------------------------------------- scale ranking of rows
@pytest.mark.parametrize("N,K", [(1, 128), (300, 1024), (2500, 4096), (17408, 5120), (5120, 17408)])
def test_rank_rows_matches_oracle(orc, dev, N, K):
    r = synth.rng_for(0, synth.WL_TEST, 6600 + N)
    S = synth.group_scales(r, N, K)
    if N >= 300:
        S[N - 1] = S[0]                                  # ties across LDS tiles of the ranking
        S[N // 2] = -S[1]                                # sign ignored
        S[5] = np.float16(0.0)
        S[6, 0] = np.float16(np.ldexp(1.0, -24))
        S[7, :] = np.float16(65504.0)
    score_ref, order_ref = orc.rank_rows(S)
    Sd = torch.from_numpy(S).to(dev)
    score, order = b1.rank_rows_by_scale(Sd)
    torch.cuda.synchronize()
    assert np.array_equal(score.cpu().numpy(), score_ref)
    assert np.array_equal(order.cpu().numpy(), order_ref)
