"""GPU parity of the decode step exactly as the benchmark times it: the 8B step's 145 stages with
each stage's projections stored back to back (q|k|v and gate|up run as one matrix each), one
launch per stage, captured into a HIP graph and replayed.  Sampled outputs of a spread of
products (every layer's q|k|v and gate|up included, and lm_head) are checked against the fp64
oracle, and every replay must reproduce the eager outputs bit for bit."""
import numpy as np
import pytest
import torch

import bench
from bit_packed_sign_amd import synth
from parity import TOL, norm_err, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def test_decode_8b_step_graph_full_size_sampled(orc, dev):
    wl = synth.decode_8b()
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
                rows = sample_rows(synth.rng_for(0, synth.WL_TEST, 8800 + gi), g.N, k=48, edge=16)
                ref, nrm = orc.gemv_rows(x, W, S, rows)
                e = norm_err(eager[gi].float().cpu().numpy()[:, rows], ref, nrm)
                assert e <= TOL, f"stage {s} product {gi}: {e}"
                checked += 1
            gi += 1
    assert gi == 253 and checked >= 50

    step.capture()
    for rep in range(3):
        for y in outs:                          # eager work between replays
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        step.graph.replay()
        torch.cuda.synchronize()
        for i, (a, y) in enumerate(zip(eager, outs)):
            assert torch.equal(a, y), f"graph replay {rep}: product {i} differs"
