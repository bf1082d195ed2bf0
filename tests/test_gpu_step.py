"""GPU parity of the decode steps exactly as the benchmark times them: the 8B step's 145 stages with
each stage's projections stored back to back (q|k|v and gate|up run as one matrix each), and the
8B MLP at batch 16 (72 stages on the small-batch kernel), one launch per stage, captured into a
HIP graph and replayed.  Sampled outputs of a spread of products (the first layers' fused stages
included, and lm_head) are checked against the fp64 oracle, and every replay must reproduce the
eager outputs bit for bit.  Concurrent calls on two streams give the same outputs as one stream."""
import numpy as np
import pytest
import torch

import bench
import bit_packed_sign_amd as b1
from bit_packed_sign_amd import synth
from parity import TOL, norm_err, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.mark.parametrize("name,n_gemvs", [("decode_8b", 253), ("mlp_8b_m16", 108)])
def test_step_graph_full_size_sampled(orc, dev, name, n_gemvs):
    wl = getattr(synth, name)()
    step = bench.Step(wl, dev)
    outs = [y for _, _, _, ys, _ in step.stages for y in ys]
    for y in outs:
        y.fill_(float("nan"))
    step.run_eager()
    torch.cuda.synchronize()
    eager = [y.clone() for y in outs]
    for y in eager:
        assert bool(torch.isfinite(y).all())

    gi = 0
    checked = 0
    for s, stage in enumerate(wl.stages):
        x = synth.stage_activations(0, wl, s)
        for g in stage.gemvs:
            if gi % 5 == 0 or s % 4 in (0, 2) and s < 8 or g.N > 100000:
                W, S = synth.gemv_tensors(0, wl, gi)
                rows = sample_rows(synth.rng_for(0, synth.WL_TEST, 8800 + gi), g.N, k=32 if wl.M > 1 else 48, edge=16)
                ref, nrm = orc.gemv_rows(x, W, S, rows)
                e = norm_err(eager[gi].float().cpu().numpy()[:, rows], ref, nrm)
                assert e <= TOL, f"stage {s} product {gi}: {e}"
                checked += 1
            gi += 1
    assert gi == n_gemvs and checked >= 20

    step.capture()
    for rep in range(3):
        for y in outs:                          # eager work between replays
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        step.graph.replay()
        torch.cuda.synchronize()
        for i, (a, y) in enumerate(zip(eager, outs)):
            assert torch.equal(a, y), f"graph replay {rep}: product {i} differs"


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
