"""GPU parity of the decode steps exactly as the benchmark times them (bench.Step): each stage's
projections stored back to back (q|k|v and gate|up run as one matrix each), one launch per stage,
captured into a HIP graph and replayed.

* the 8B step (145 stages, 253 products), every output against the fp64 oracle;
* the 27B step (256 stages, 448 products), every output; its fused q|k|v (15360 x 5120) and
  gate|up (34816 x 5120) launches and the long-row down launches (K = 17408, operands read per
  pair) are the variants the benchmark runs for it;
* the ternary 8B step (2-bit slots), every output;
* the 8B MLP at batch 16 (72 stages on the small-batch kernel; down splits K over workgroups with
  the step's workspace), all 16 tokens of every eighth row plus the edge rows of every product;
* the 8B step at M = 5, every 16th row of every product; its lm_head launch runs on the
  block-scaled small-batch kernel with 38 tiles per workgroup (the merge's tile-table shuffles
  past lane 16 with part of a token block idle).
Every replay must reproduce the eager outputs bit for bit, with eager work between replays.
Concurrent calls on two streams give the same outputs as one stream."""
import numpy as np
import pytest
import torch

import bench
import bit_packed_sign_amd as b1
from bit_packed_sign_amd import synth
from parity import TOL, norm_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _rows(N, stride):
    if stride == 1:
        return np.arange(N)
    return np.unique(np.concatenate([np.arange(0, N, stride), np.arange(min(16, N)), np.arange(max(0, N - 16), N)]))


def _check_step(orc, dev, wl, ternary, row_stride, expect_variants=None):
    step = bench.Step(wl, dev, ternary=ternary)
    if expect_variants:
        for s, want in expect_variants.items():
            x, Ws, Ss, ys, _ = step.stages[s]
            op = "gemv_t2" if ternary else "gemv_ws" if step.workspace is not None and len(Ws) == 1 else "gemv"
            got = b1.kernel_variant(op, wl.M, x.shape[1], [sum(W.shape[0] for W in Ws)] if wl.M == 1
                                    else [W.shape[0] for W in Ws])
            assert got.split(" ")[0] == want, (s, got, want)
    outs = [y for _, _, _, ys, _ in step.stages for y in ys]
    for y in outs:
        y.fill_(float("nan"))
    step.run_eager()
    torch.cuda.synchronize()
    eager = [y.clone() for y in outs]
    gen = synth.ternary_gemv_tensors if ternary else synth.gemv_tensors
    ref_fn = orc.gemv_t2 if ternary else orc.gemv
    gi = 0
    worst = 0.0
    for s, stage in enumerate(wl.stages):
        x = synth.stage_activations(0, wl, s)
        for g in stage.gemvs:
            W, S = gen(0, wl, gi)
            rows = _rows(g.N, row_stride)
            ref, nrm = ref_fn(x, W[rows], S[rows])
            e = norm_err(eager[gi].float().cpu().numpy()[:, rows], ref, nrm)
            assert e <= TOL, f"stage {s} product {gi} ({g.name}): {e}"
            worst = max(worst, e)
            gi += 1
    assert gi == len(wl.gemvs)
    step.capture()
    for rep in range(3):
        for y in outs:                          # eager work between replays
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        step.graph.replay()
        torch.cuda.synchronize()
        for i, (a, y) in enumerate(zip(eager, outs)):
            assert torch.equal(a, y), f"graph replay {rep}: product {i} differs"
    return worst


def test_step_8b_every_output(orc, dev):
    _check_step(orc, dev, synth.decode_8b(), False, 1,
                {0: "gemv_mx<1,1,2,0,0,4,1>", 1: "gemv_mx<1,1,1,0,0,4,1>", 2: "gemv_mx<1,1,1,0,0,12,1,3>",
                 3: "gemv_mx<1,1,1,0,0,12,1>", 144: "gemv_mx<1,1,2,0,0,12,1,3>"})


def test_step_27b_every_output(orc, dev):
    _check_step(orc, dev, synth.decode_27b(), False, 1,
                {0: "gemv_mx<1,1,2,0,0,8,1>", 1: "gemv_mx<1,1,2,0,0,8,1>", 2: "gemv_mx<1,1,2,0,0,8,1>",
                 3: "gemv_mx<2,1,1,0,0,12,1,1,AL>"})


def test_step_ternary_8b_every_output(orc, dev):
    _check_step(orc, dev, synth.decode_8b(), True, 1,
                {0: "gemv_mx<1,1,2,0,1,4,1>", 2: "gemv_mx<1,1,1,0,1,12,1,3>", 3: "gemv_mx<1,1,1,0,1,12,1>",
                 144: "gemv_mx<1,1,1,0,1,8,1,2>"})


def test_step_mlp16_every_product(orc, dev):
    _check_step(orc, dev, synth.mlp_8b_m16(), False, 8,
                {0: "gemv_smallm<6,0>", 1: "gemv_smallm_split<4>"})


def test_step_8b_m5_sampled_rows(orc, dev):
    """The 8B decode step at M = 5 tokens (the verify pass of speculative decoding with four drafted
    tokens) as the benchmark times it: all five tokens of every 16th row of every product."""
    wl = synth._decoder(synth.WL_DECODE_8B, "decode-8b-m5", 5, 36, 4096, 4096, 1024, 4096, 12288,
                        lm_vocab=151936)
    _check_step(orc, dev, wl, False, 16,
                {0: "gemv_smallm<2,0>", 1: "gemv_smallm<2,0>", 2: "gemv_smallm<6,0>", 3: "gemv_smallm_split<4>",
                 144: "gemv_mxm<2,4>"})


def test_concurrent_streams_match_one_stream(dev):
    """The library keeps no state between calls: the same products issued on two streams at once
    (batch 1 and batch 16, decode and prefill shapes) equal the results of one stream."""
    r = synth.rng_for(0, synth.WL_TEST, 8900)
    cases = []
    for M, K, N in [(1, 4096, 12288), (16, 4096, 4096), (1, 12288, 4096), (300, 1024, 777)]:
        x = torch.from_numpy(synth.activations(r, M, K)).to(dev)
        W = torch.from_numpy(synth.sign_words(r, N, K).view(np.int32)).to(dev)
        S = torch.from_numpy(synth.group_scales(r, N, K)).to(dev)
        cases.append((x, W, S))
    ref = [b1.gemv(x, W, S) for x, W, S in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.full_like(y, float("nan")) for y in ref] for _ in streams]
    for rep in range(4):
        for st, o in zip(streams, outs):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                for (x, W, S), y in zip(cases, o):
                    b1.gemv(x, W, S, out=y)
        torch.cuda.synchronize()
        for o in outs:
            for a, b in zip(ref, o):
                assert torch.equal(a, b)
