"""GPU parity of the decode-step chain (bin1_chain_prepare / bin1_gemv_chain) against the
fp64 oracle: every stage of a chain, each kernel variant, a chain whose stages feed each other,
replays (eager and from a captured graph), the bounded-wait failure path, and the 8B decode
step at full size with every output checked."""
import numpy as np
import pytest
import torch

import bit_packed_sign_amd as b1
from bit_packed_sign_amd import synth
from parity import TOL, dev_tensors, norm_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _mat(t, K, N):
    r = synth.rng_for(0, synth.WL_TEST, t)
    return synth.sign_words(r, N, K), synth.group_scales(r, N, K)


def _x(t, K):
    return synth.activations(synth.rng_for(0, synth.WL_TEST, t), 1, K)


def _build(dev, spec, t0):
    """spec: list of (K, [N...]); every stage has its own seeded x.  Returns host data,
    device stages for ChainPlan, and the output tensors."""
    host, stages = [], []
    for s, (K, Ns) in enumerate(spec):
        x = _x(t0 + 100 * s, K)
        mats = [_mat(t0 + 100 * s + 1 + i, K, N) for i, N in enumerate(Ns)]
        xd, = dev_tensors(dev, x)
        Wd = [dev_tensors(dev, W=W)[0] for W, _ in mats]
        Sd = [dev_tensors(dev, S=S)[0] for _, S in mats]
        yd = [torch.full((1, N), float("nan"), dtype=torch.float16, device=dev) for N in Ns]
        host.append((x, mats))
        stages.append((xd, Wd, Sd, yd))
    return host, stages


def _check_all(orc, host, stages):
    for s, ((x, mats), (_, _, _, ys)) in enumerate(zip(host, stages)):
        for i, ((W, S), y) in enumerate(zip(mats, ys)):
            ref, nrm = orc.gemv(x, W, S)
            e = norm_err(y, ref, nrm)
            assert e <= TOL, f"stage {s} matrix {i}: normalised error {e}"


# One chain per kernel variant (the widest K selects it: ceil(K/1024) pairs over 4 waves).
# Stages mix K values that leave the last 1024-wide pair partly filled (1280, 2304, ...),
# ragged N, 1..4 products per stage, and a 1-row stage that leaves 255 workgroups idle.
VARIANTS = {
    "sp1": [(1024, [4096, 17, 1000]), (256, [1]), (768, [300, 2049, 64, 5000])],
    "sp2": [(4096, [4096, 1024, 1024]), (8192, [777]), (1280, [12288])],
    "sp3": [(12288, [4096]), (2304, [333, 4096]), (4096, [12288, 12288]), (10240, [1])],
    "sp4": [(16384, [1500]), (5120, [5120, 1024, 1024]), (13312, [4096])],
    "sp5": [(17408, [5120]), (20480, [700, 31]), (5120, [17408, 17408])],
}


@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_chain_stages_match_oracle(orc, dev, name):
    spec = VARIANTS[name]
    host, stages = _build(dev, spec, 5000 + 1000 * sorted(VARIANTS).index(name))
    plan = b1.ChainPlan(stages)
    want_sp = (max(K for K, _ in spec) // 1024 + (max(K for K, _ in spec) % 1024 > 0) + 3) // 4
    assert plan.plan.spmax == want_sp
    plan.run()
    torch.cuda.synchronize()
    assert plan.status() == (1, 0)
    _check_all(orc, host, stages)


def test_chain_replays_bit_identical_and_in_graph(orc, dev):
    host, stages = _build(dev, VARIANTS["sp3"], 7000)
    plan = b1.ChainPlan(stages)
    plan.run()
    torch.cuda.synchronize()
    first = [[y.clone() for y in st[3]] for st in stages]
    _check_all(orc, host, stages)
    for rep in range(2):
        for st in stages:
            for y in st[3]:
                y.fill_(float("nan"))
        plan.run()
        torch.cuda.synchronize()
        for a, st in zip(first, stages):
            for y0, y in zip(a, st[3]):
                assert torch.equal(y0, y), f"eager replay {rep} differs"
    assert plan.status() == (3, 0)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run()
    torch.cuda.synchronize()
    for rep in range(3):
        for st in stages:                      # eager work between replays
            for y in st[3]:
                y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, st in zip(first, stages):
            for y0, y in zip(a, st[3]):
                assert torch.equal(y0, y), f"graph replay {rep} differs"
    runs, err = plan.status()
    assert err == 0 and runs >= 6       # capture itself does not run the kernel


def test_chain_stages_feed_each_other(orc, dev):
    """x of stage s+1 is an output of stage s, so a stage that started before its predecessor
    finished would read the NaN fill (and give non-finite outputs).  Each stage is checked on its
    own: the oracle takes the fp16 activations the GPU actually fed that stage (the previous
    stage's output as stored), so every stage meets the single-product bar."""
    dims = [(1024, [2048, 512, 512]), (2048, [4096]), (4096, [1280, 3000]), (1280, [12288]),
            (12288, [1024]), (1024, [17, 300, 5000, 256])]
    mats = [[_mat(9000 + 10 * s + i, K, N) for i, N in enumerate(Ns)] for s, (K, Ns) in enumerate(dims)]
    x0 = _x(8999, dims[0][0])
    ys = [[torch.empty((1, N), dtype=torch.float16, device=dev) for N in Ns] for _, Ns in dims]
    stages = []
    for s, (K, Ns) in enumerate(dims):
        xd = dev_tensors(dev, x0)[0] if s == 0 else ys[s - 1][0]
        stages.append((xd, [dev_tensors(dev, W=W)[0] for W, _ in mats[s]],
                       [dev_tensors(dev, S=S)[0] for _, S in mats[s]], ys[s]))
    plan = b1.ChainPlan(stages)
    for rep in range(2):
        for row in ys:
            for y in row:
                y.fill_(float("nan"))
        plan.run()
        torch.cuda.synchronize()
        x = x0
        for s in range(len(dims)):
            for i, (W, S) in enumerate(mats[s]):
                y = ys[s][i].cpu().numpy()
                assert np.all(np.isfinite(y)), f"run {rep} stage {s} matrix {i}: read an unfinished input"
                ref, nrm = orc.gemv(x, W, S)
                e = norm_err(y, ref, nrm)
                assert e <= TOL, f"run {rep} stage {s} matrix {i}: {e}"
            x = ys[s][0].cpu().numpy()                # what stage s + 1 read
    assert plan.status() == (2, 0)


def test_chain_bounded_wait_reports_error(orc, dev):
    """Workgroup 0 is told (through the workspace header's fault-injection word) never to
    publish stage 0; every wait then ends by its spin limit, the kernel exits normally and
    the status reports the failure.  Preparing the chain again clears it."""
    host, stages = _build(dev, VARIANTS["sp1"], 7500)
    plan = b1.ChainPlan(stages)
    plan.set_spin_limit(64)
    hdr = plan.workspace[:64].view(torch.int32)
    hdr[6] = 1                                       # ChainHeader.withhold
    plan.run()
    torch.cuda.synchronize()
    assert plan.status() == (1, 1)
    plan = b1.ChainPlan(stages)
    plan.run()
    torch.cuda.synchronize()
    assert plan.status() == (1, 0)
    _check_all(orc, host, stages)


def test_chain_rejects_bad_plans(dev):
    K, N = 1024, 256
    W, S = _mat(7700, K, N)
    Wd, Sd = dev_tensors(dev, W=W, S=S)
    x = torch.zeros((1, K), dtype=torch.float16, device=dev)
    y = torch.empty((1, N), dtype=torch.float16, device=dev)
    Wb, Sb = _mat(7702, K, N)
    Wbd, Sbd = dev_tensors(dev, W=Wb, S=Sb)
    over = Wbd.view(torch.float16).view(-1)[:N].view(1, N)
    with pytest.raises(b1.Bin1Error) as ei:                   # output over a later stage's weights
        b1.ChainPlan([(x, [Wd], [Sd], [over]), (x, [Wbd], [Sbd], [y])])
    assert ei.value.status == -4
    with pytest.raises(b1.Bin1Error) as ei:                   # output over its own stage's x
        b1.ChainPlan([(x, [Wd], [Sd], [x[:, :N]])])
    assert ei.value.status == -4
    x128 = torch.zeros((1, 1152), dtype=torch.float16, device=dev)
    W2, S2 = _mat(7701, 1152, 64)
    W2d, S2d = dev_tensors(dev, W=W2, S=S2)
    with pytest.raises(b1.Bin1Error) as ei:                   # K % 256 != 0
        b1.ChainPlan([(x128, [W2d], [S2d], [torch.empty((1, 64), dtype=torch.float16, device=dev)])])
    assert ei.value.status == -2
    with pytest.raises(ValueError):
        b1.ChainPlan([(torch.zeros((2, K), dtype=torch.float16, device=dev), [Wd], [Sd], [y])])


def test_chain_decode_8b_every_output(orc, dev):
    """The whole 8B decode step (145 stages, 253 products) as one chain, in the configuration
    the benchmark times; every output of every product checked against the oracle."""
    wl = synth.decode_8b()
    stages, checks = [], []
    gi = 0
    for s, st in enumerate(wl.stages):
        x = synth.stage_activations(0, wl, s)
        xd, = dev_tensors(dev, x)
        Wd, Sd, yd = [], [], []
        for g in st.gemvs:
            W, S = synth.gemv_tensors(0, wl, gi)
            a, b = dev_tensors(dev, W=W, S=S)
            Wd.append(a)
            Sd.append(b)
            yd.append(torch.full((1, g.N), float("nan"), dtype=torch.float16, device=dev))
            checks.append((s, yd[-1], gi))
            gi += 1
        stages.append((xd, Wd, Sd, yd))
    plan = b1.ChainPlan(stages)
    plan.run()
    torch.cuda.synchronize()
    assert plan.status() == (1, 0)
    for s, y, gi in checks:
        W, S = synth.gemv_tensors(0, wl, gi)
        ref, nrm = orc.gemv(synth.stage_activations(0, wl, s), W, S)
        e = norm_err(y, ref, nrm)
        assert e <= TOL, f"product {gi}: {e}"
