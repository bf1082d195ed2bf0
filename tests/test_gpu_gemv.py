"""GPU parity of bin1_gemv (decode / small-batch) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import bit_packed_sign_amd as b1
from bit_packed_sign_amd import synth
from parity import TOL, dev_tensors, norm_err, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _case(t, M, K, N):
    r = synth.rng_for(0, synth.WL_TEST, t)
    return synth.activations(r, M, K), synth.sign_words(r, N, K), synth.group_scales(r, N, K)


SMALL = [(128, 1), (128, 7), (256, 64), (512, 300), (1024, 1000), (4096, 1024), (12288, 130), (13440, 90),
         (16384, 48), (17408, 33), (24576, 40)]


@pytest.mark.parametrize("K,N", SMALL)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 16])
def test_gemv_matches_oracle(orc, dev, M, K, N):
    x, W, S = _case(1000 + K + N + M, M, K, N)
    ref, nrm = orc.gemv(x, W, S)
    xd, Wd, Sd = dev_tensors(dev, x, W, S)
    y = b1.gemv(xd, Wd, Sd)
    assert norm_err(y, ref, nrm) <= TOL


FULL = [(4096, 4096), (4096, 1024), (4096, 12288), (12288, 4096), (4096, 151936),
        (5120, 5120), (5120, 17408), (17408, 5120)]


@pytest.mark.parametrize("K,N", FULL)
@pytest.mark.parametrize("M", [1, 16])
def test_gemv_full_size(orc, dev, M, K, N):
    """Projection shapes of the 8B and 27B decode steps: every output at batch 1, and at batch 16
    all tokens of every fourth row plus sampled ones, checked against the oracle."""
    x, W, S = _case(2000 + K + N + M, M, K, N)
    xd, Wd, Sd = dev_tensors(dev, x, W, S)
    y = b1.gemv(xd, Wd, Sd).float().cpu().numpy()
    rows = np.arange(N) if M == 1 else np.union1d(np.arange(0, N, 4),
                                                 sample_rows(synth.rng_for(0, synth.WL_TEST, 3000 + N), N))
    ref, nrm = orc.gemv_rows(x, W, S, rows)
    assert norm_err(y[:, rows], ref, nrm) <= TOL
    assert np.all(np.isfinite(y))


def test_closed_form_and_one_hot_rows(orc, dev):
    K = 512
    r = synth.rng_for(0, synth.WL_TEST, 4000)
    x = synth.activations(r, 2, K)
    positions = [0, 1, 31, 32, 63, 127, 128, 300, 511]
    N = 2 + len(positions)
    W = np.zeros((N, K // 32), np.uint32)
    W[0] = 0xFFFFFFFF
    for n, k in enumerate(positions):
        W[2 + n, k // 32] = np.uint32(1) << np.uint32(k % 32)
    S = synth.group_scales(r, N, K)
    ref, nrm = orc.gemv(x, W, S)
    y = b1.gemv(*dev_tensors(dev, x, W, S))
    assert norm_err(y, ref, nrm) <= TOL


def test_scale_edge_cases(orc, dev):
    """Zero, subnormal and negative scales; zero activations."""
    K, N = 1024, 64
    x, W, S = _case(4100, 3, K, N)
    S = S.copy()
    S[0] = 0
    S[1] = np.float16(2.0 ** -24)
    S[2, ::2] = np.float16(3.0e-6)
    S[3] = -S[3]
    S[4, 3] = np.float16(-0.0)
    x = x.copy()
    x[1] = 0
    ref, nrm = orc.gemv(x, W, S)
    y = b1.gemv(*dev_tensors(dev, x, W, S))
    assert norm_err(y, ref, nrm) <= TOL
    yn = y.float().cpu().numpy()
    assert np.all(yn[:, 0] == 0) and np.all(yn[1] == 0)


def test_patched_rows_negate_output(dev):
    """Flipping whole rows negates those outputs bit for bit and leaves the rest unchanged."""
    M, K, N = 1, 4096, 4096
    x, W, S = _case(4200, M, K, N)
    xd, Wd, Sd = dev_tensors(dev, x, W, S)
    y0 = b1.gemv(xd, Wd, Sd).clone()
    rows = torch.from_numpy(synth.patch_rows_single()).to(dev)
    b1.xor_patch_apply(Wd, rows)
    y1 = b1.gemv(xd, Wd, Sd)
    b1.xor_patch_apply(Wd, rows)
    mask = torch.zeros(N, dtype=torch.bool, device=dev)
    mask[rows.long()] = True
    assert torch.equal(y1[:, mask], -y0[:, mask])
    assert torch.equal(y1[:, ~mask], y0[:, ~mask])
    assert torch.equal(Wd.cpu(), torch.from_numpy(W.view(np.int32)))


def test_output_is_fully_overwritten_and_out_argument(orc, dev):
    M, K, N = 2, 256, 77
    x, W, S = _case(4300, M, K, N)
    ref, nrm = orc.gemv(x, W, S)
    xd, Wd, Sd = dev_tensors(dev, x, W, S)
    out = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
    b1.gemv(xd, Wd, Sd, out=out)
    assert norm_err(out, ref, nrm) <= TOL


@pytest.mark.parametrize("M,K,Ns", [(1, 4096, (4096, 1024, 1024)), (1, 4096, (12288, 12288)),
                                    (1, 5120, (5120, 5120, 5120)), (1, 384, (7, 33, 100, 16)),
                                    (1, 17408, (5120,)), (2, 512, (64, 65)),
                                    (16, 4096, (12288, 12288)), (5, 384, (7, 33, 100, 16)),
                                    (16, 4352, (300, 1000, 17)), (9, 12288, (4096, 1500))])
def test_gemv_group_matches_oracle(orc, dev, M, K, Ns):
    """Same-input fusion (q/k/v, gate/up): one launch, each output checked against the oracle."""
    r = synth.rng_for(0, synth.WL_TEST, 7000 + K + sum(Ns) + M)
    x = synth.activations(r, M, K)
    Ws = [synth.sign_words(r, n, K) for n in Ns]
    Ss = [synth.group_scales(r, n, K) for n in Ns]
    xd = dev_tensors(dev, x)[0]
    Wd = [dev_tensors(dev, W=W)[0] for W in Ws]
    Sd = [dev_tensors(dev, S=S)[0] for S in Ss]
    outs = b1.gemv_group(xd, Wd, Sd)
    for W, S, y in zip(Ws, Ss, outs):
        N = W.shape[0]
        rows = sample_rows(r, N, k=128) if N > 2048 else np.arange(N)
        ref, nrm = orc.gemv_rows(x, W, S, rows)
        assert norm_err(y.float().cpu().numpy()[:, rows], ref, nrm) <= TOL


@pytest.mark.parametrize("M", [1, 3, 16])
def test_gemv_group_equals_separate_calls(dev, M):
    """One grouped launch gives bit-identical outputs to one call per matrix."""
    r = synth.rng_for(0, synth.WL_TEST, 7300 + M)
    K, Ns = 4352, (300, 1000, 17, 2048)
    x = synth.activations(r, M, K)
    xd = dev_tensors(dev, x)[0]
    Wd = [dev_tensors(dev, W=synth.sign_words(r, n, K))[0] for n in Ns]
    Sd = [dev_tensors(dev, S=synth.group_scales(r, n, K))[0] for n in Ns]
    outs = b1.gemv_group(xd, Wd, Sd)
    for W, S, y in zip(Wd, Sd, outs):
        assert torch.equal(b1.gemv(xd, W, S), y)


def _same_row_order(K, Ns_a, Ns_b):
    """Whether two batch-1 launches sum every row in the same order: the same pairs per wave and
    waves per workgroup (the split of K over waves), from the variant query."""
    def key(Ns):
        v = b1.kernel_variant("gemv", 1, K, Ns).split(" ")[0].split("<")[1].rstrip(">").split(",")
        return v[0], v[5]
    return key(Ns_a) == key(Ns_b)


def _back_to_back(dev, mats, M, widths):
    """Device views of one allocation each for weights, scales and outputs, matrix i's rows right
    after matrix i-1's (a fused q/k/v layout)."""
    W_all = dev_tensors(dev, W=np.concatenate([W for W, _ in mats]))[0]
    S_all = dev_tensors(dev, S=np.concatenate([S for _, S in mats]))[0]
    y_all = torch.full((M, sum(widths)), float("nan"), dtype=torch.float16, device=dev)
    offs = np.concatenate([[0], np.cumsum(widths)])
    return ([W_all[a:b] for a, b in zip(offs[:-1], offs[1:])], [S_all[a:b] for a, b in zip(offs[:-1], offs[1:])],
            [y_all[:, a:b] for a, b in zip(offs[:-1], offs[1:])])


@pytest.mark.parametrize("K,Ns", [(4096, (4096, 1024, 1024)), (4096, (12288, 12288)), (4352, (296, 1000, 24, 2047)),
                                  (384, (8, 40, 104, 17)), (12288, (1000, 24))])
def test_gemv_group_back_to_back(orc, dev, K, Ns):
    """Matrices stored back to back (weights, scales and outputs) run as one taller matrix at
    M == 1: every output matches the oracle and the one-call-per-matrix results; a mixed group
    (only some neighbours adjacent, or adjacent weights with separate outputs) as well."""
    r = synth.rng_for(0, synth.WL_TEST, 7500 + K + sum(Ns))
    x = synth.activations(r, 1, K)
    mats = [(synth.sign_words(r, n, K), synth.group_scales(r, n, K)) for n in Ns]
    xd = dev_tensors(dev, x)[0]
    Wv, Sv, yv = _back_to_back(dev, mats, 1, Ns)
    outs = [y.clone() for y in b1.gemv_group(xd, Wv, Sv, outs=yv)]
    for (W, S), y, Wd, Sd in zip(mats, outs, Wv, Sv):
        N = W.shape[0]
        rows = sample_rows(r, N, k=128) if N > 2048 else np.arange(N)
        ref, nrm = orc.gemv_rows(x, W, S, rows)
        assert norm_err(y.float().cpu().numpy()[:, rows], ref, nrm) <= TOL
        if _same_row_order(K, [sum(Ns)], [N]):      # same split of a row over waves: identical bits
            assert torch.equal(y, b1.gemv(xd, Wd, Sd))
    separate = b1.gemv_group(xd, Wv, Sv)         # adjacent weights, outputs allocated per matrix
    mixed = list(Wv), list(Sv), list(yv)
    if len(Ns) > 2:                              # matrix 1 moved out: 0, 1 no longer adjacent, 2, 3 still
        mixed[0][1], mixed[1][1] = Wv[1].clone(), Sv[1].clone()
    for y in yv:
        y.fill_(float("nan"))
    mixed_out = b1.gemv_group(xd, mixed[0], mixed[1], outs=mixed[2])
    mixed_ns = [Ns[0], Ns[1], sum(Ns[2:])] if len(Ns) > 2 else [sum(Ns)]
    for (W, S), a, b, c in zip(mats, outs, separate, mixed_out):
        if _same_row_order(K, [sum(Ns)], list(Ns)) and _same_row_order(K, [sum(Ns)], mixed_ns):
            assert torch.equal(a, b) and torch.equal(a, c)
        else:                                    # the launches split a row over waves differently
            ref, nrm = orc.gemv(x, W, S)
            assert norm_err(b, ref, nrm) <= TOL and norm_err(c, ref, nrm) <= TOL


@pytest.mark.parametrize("M", [1, 2])
def test_gemv_largest_row_count(orc, dev, M):
    """The largest accepted N (2^24 - 65 rows, K = 128): row offsets near the 24-bit limit of the
    kernels' row products, sampled rows (the last ones included) checked against the oracle."""
    K, N = 128, (1 << 24) - 65
    r = synth.rng_for(0, synth.WL_TEST, 7600 + M)
    x = synth.activations(r, M, K)
    W = r.integers(0, 1 << 32, size=(N, K // 32), dtype=np.uint32)
    S = synth.group_scales(r, N, K)
    xd, Wd, Sd = dev_tensors(dev, x, W, S)
    y = b1.gemv(xd, Wd, Sd)
    rows = sample_rows(synth.rng_for(0, synth.WL_TEST, 7601), N, k=256, edge=64)
    ref, nrm = orc.gemv_rows(x, W, S, rows)
    assert norm_err(y.float().cpu().numpy()[:, rows], ref, nrm) <= TOL
    with pytest.raises(b1.Bin1Error):
        b1.gemv(xd, torch.zeros((N + 1, K // 32), dtype=torch.int32, device=dev),
                torch.zeros((N + 1, K // 128), dtype=torch.float16, device=dev))


def test_gemv_repeated_calls_are_deterministic(dev):
    """The same inputs give bit-identical outputs on every call (fixed accumulation order)."""
    x, W, S = _case(7100, 1, 4096, 12288)
    xd, Wd, Sd = dev_tensors(dev, x, W, S)
    y0 = b1.gemv(xd, Wd, Sd)
    for _ in range(3):
        assert torch.equal(b1.gemv(xd, Wd, Sd), y0)


def test_empty_products_are_no_ops(orc, dev):
    """Degenerate shapes: M == 0 or N == 0 products return at once (nothing is written), and a
    grouped call with an empty matrix among others equals the calls on the non-empty ones."""
    K = 512
    x, W, S = _case(7400, 3, K, 40)
    xd, Wd, Sd = dev_tensors(dev, x, W, S)
    for fn in (b1.gemv, b1.gemm_prefill):
        y = fn(xd[:0], Wd, Sd)                                   # M == 0
        assert tuple(y.shape) == (0, 40)
        y = fn(xd, Wd[:0], Sd[:0])                               # N == 0
        assert tuple(y.shape) == (3, 0)
    outs = b1.gemv_group(xd, [Wd, Wd[:0], Wd], [Sd, Sd[:0], Sd])
    ref, nrm = orc.gemv(x, W, S)
    assert tuple(outs[1].shape) == (3, 0)
    assert norm_err(outs[0], ref, nrm) <= TOL and torch.equal(outs[0], outs[2])
    assert torch.equal(outs[0], b1.gemv(xd, Wd, Sd))
    assert tuple(b1.gemv_pm1(torch.zeros((0, K // 32), dtype=torch.int32, device=dev),
                             Wd).shape) == (0, 40)
    score, order = b1.rank_rows_by_scale(Sd[:0])
    assert score.numel() == 0 and order.numel() == 0


def _tile_rows(grid, locals_, wgs, N):
    """Rows of the workgroups' local tiles (tile = local * grid + workgroup, 16 rows each)."""
    rows = [r for k in locals_ for b in wgs for r in range((k * grid + b) * 16, (k * grid + b) * 16 + 16)]
    return np.array(sorted({r for r in rows if r < N}))


@pytest.mark.parametrize("op,K,N", [("gemv", 17408, 139264), ("gemv_t2", 16384, 139264)])
def test_tall_matrix_every_tile_of_a_workgroup(orc, dev, op, K, N):
    """Tall products on the 16-row-tile layouts give a workgroup 34 tiles, so the last merge pass
    covers tiles 32 and 33 with only lanes 0..31 active, and those lanes need the table entries of
    tiles 32 and 33 (held by lanes 32 and 33 of the tile table, read from its LDS copy).  Every
    output must be written (the buffer starts as NaN), and the rows of local tiles 31..33 of
    several workgroups match the oracle."""
    t2 = op == "gemv_t2"
    desc = b1.kernel_variant(op, 1, K, [N])
    grid = int(desc.split("grid=")[1])
    assert (N // 16 + grid - 1) // grid == 34, desc
    r = synth.rng_for(0, synth.WL_TEST, 7700 + K)
    x = synth.activations(r, 1, K)
    W = synth.ternary_words_fast(r, N, K) if t2 else synth.sign_words(r, N, K)
    S = synth.group_scales(r, N, K)
    xd, Wd, Sd = dev_tensors(dev, x, W, S)
    y = torch.full((1, N), float("nan"), dtype=torch.float16, device=dev)
    (b1.gemv_t2 if t2 else b1.gemv)(xd, Wd, Sd, out=y)
    yy = y.float().cpu().numpy()
    assert np.all(np.isfinite(yy)), f"{int(np.sum(~np.isfinite(yy)))} outputs not written"
    rows = np.union1d(_tile_rows(grid, [0, 31, 32, 33], [0, 1, grid // 2, grid - 1], N),
                      sample_rows(synth.rng_for(0, synth.WL_TEST, 7701 + K), N))
    ref, nrm = (orc.gemv_t2_rows if t2 else orc.gemv_rows)(x, W, S, rows)
    assert norm_err(yy[:, rows], ref, nrm) <= TOL


@pytest.mark.parametrize("M", [2, 5, 7])
def test_small_batch_many_tiles_per_workgroup(orc, dev, M):
    """The block-scaled small-batch kernel at an lm_head shape gives each workgroup 37 or 38 tiles;
    with M not a multiple of 4 the last token block leaves lanes idle at the store, and the merge
    must still read every tile's output pointer and rows with all lanes.  Every output written,
    sampled rows of tiles 15..37 against the oracle."""
    K, N = 4096, 151936
    desc = b1.kernel_variant("gemv", M, K, [N])
    assert desc.startswith("gemv_mxm<"), desc
    grid = int(desc.split("grid=")[1])
    r = synth.rng_for(0, synth.WL_TEST, 7800 + M)
    x, W, S = synth.activations(r, M, K), synth.sign_words(r, N, K), synth.group_scales(r, N, K)
    xd, Wd, Sd = dev_tensors(dev, x, W, S)
    y = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
    b1.gemv(xd, Wd, Sd, out=y)
    yy = y.float().cpu().numpy()
    assert np.all(np.isfinite(yy)), f"{int(np.sum(~np.isfinite(yy)))} outputs not written"
    rows = np.union1d(_tile_rows(grid, [0, 15, 16, 17, 31, 36, 37], [0, 1, 23, grid - 1], N),
                      sample_rows(synth.rng_for(0, synth.WL_TEST, 7801 + M), N))
    ref, nrm = orc.gemv_rows(x, W, S, rows)
    assert norm_err(yy[:, rows], ref, nrm) <= TOL
