"""Benchmark of the 1-bit sign GEMV decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]
                    [--only NAME]

Headline step: one batch-1 decode pass of the 8B-class model's GEMVs -- 36 layers of
q 4096x4096, k/v 4096x1024, o 4096x4096, gate/up 4096x12288, down 12288x4096, then
lm_head 4096x151936: 253 products in 145 dependent stages (q/k/v and gate/up each share
one activation vector), every stage reading its own fp16 activation vector (norms/attention
omitted), all weights and activations resident in HBM.  Two complete implementations of the
dependent step are timed on the same tensors:
  graph  -- one decode launch per stage (same-input products fused), captured once into a HIP
            graph and replayed;
  chain  -- the whole step as one persistent launch (bin1_gemv_chain): stage s+1 reads its x
            only after every output of stage s is visible device-wide.
K steps of each are timed between HIP events after W warm-up steps; the faster one is the
headline (named in config.workload) and the other is reported under extra.step_paths.

Metric: weight-GB/s = bytes of packed bits + fp16 scales per step (1,064,263,680 B)
divided by the step time; implied tokens/s = 1 / step time.

The other workloads run after the headline and are reported under "extra": one
4096x4096 GEMV (cache-cold over a >1 GiB pool of copies, and cache-hot) with a 64-row
patch; the 8B MLP at batch 16; the prefill contraction M=2048, K=4096, N=12288; the 27B
decode step with a 2000-row multi-matrix patch; and the +-1 popcount product.
One JSON line on stdout; progress on stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP16_MFMA_PEAK_TFLOPS = 2500.0 # MI355X dense fp16/bf16 matrix peak, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--only", default=None,
                    help="run one workload alone (for profiling): step8b, chain8b, lmhead, single, mlp16, "
                         "prefill, step27b, pm1, bits, ternary, copy")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def graph_launch_floor_us(device, n, reps=20):
    """Per-launch time of a replayed graph of n dependent launches of a one-element fill (one
    workgroup, no traffic): the launch cost that every dependent stage pays."""
    import torch
    t = torch.zeros(1, device=device)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(n):
            t.fill_(float(i))
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            t.fill_(float(i))
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = events()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps / n


def stream_read_gbs(device, nbytes=2 << 30, reps=10):
    """A reference read rate for this GPU's HBM: torch's row sums over a 2 GiB fp32 tensor in
    8192-wide rows (reads every byte once, writes 1/8192 of it); of the plain torch reductions
    and copies tried on this GPU it reads fastest."""
    import torch
    t = torch.ones(nbytes // 4, dtype=torch.float32, device=device).view(-1, 8192)
    out = torch.empty(t.shape[0], dtype=torch.float32, device=device)
    ms = time_fn(lambda: torch.sum(t, dim=1, out=out), reps)
    del t
    torch.cuda.empty_cache()
    return nbytes / (ms * 1e-3) / 1e9


# Matrix-core work reaches its steady clock only after some milliseconds of load: the prefill
# timings (and the dense GEMMs beside them) run this many untimed calls first (~20 ms at M = 2048).
PREFILL_WARM = 100


def time_fn(fn, reps, warm=2):
    """Average ms per call of fn() over `reps` calls, HIP events on the current stream."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = events()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


class Step:
    """Device-resident weights/activations of a staged workload and a graph of one pass."""

    def __init__(self, wl, device, ternary=False):
        import torch
        from bit_packed_sign_amd import synth
        self.wl = wl
        self.ternary = ternary
        self.stages = []                      # (x, [W...], [S...], [y...], bytes)
        t0 = time.time()
        gi = 0
        for s, stage in enumerate(wl.stages):
            xs = torch.from_numpy(synth.stage_activations(0, wl, s)).to(device)
            # The projections of one stage (q/k/v, gate/up) live back to back in one allocation
            # each for weights, scales and (at batch 1) outputs, the usual fused layout.
            bits_l, scales_l = [], []
            for g in stage.gemvs:
                bits, scales = (synth.ternary_gemv_tensors if ternary else synth.gemv_tensors)(0, wl, gi)
                bits_l.append(bits.view(np.int32))
                scales_l.append(scales)
                gi += 1
            W_all = torch.from_numpy(np.concatenate(bits_l)).to(device)
            S_all = torch.from_numpy(np.concatenate(scales_l)).to(device)
            ntot = sum(g.N for g in stage.gemvs)
            y_all = torch.empty((wl.M, ntot), dtype=torch.float16, device=device) if wl.M == 1 else None
            Ws, Ss, ys = [], [], []
            r = 0
            for g in stage.gemvs:
                Ws.append(W_all[r:r + g.N])
                Ss.append(S_all[r:r + g.N])
                ys.append(y_all[:, r:r + g.N] if y_all is not None
                          else torch.empty((wl.M, g.N), dtype=torch.float16, device=device))
                r += g.N
            del bits_l, scales_l
            nbytes = sum(round(g.N * g.K * synth.TERNARY_BYTES_PER_WEIGHT) if ternary else g.weight_bytes
                         for g in stage.gemvs)
            self.stages.append((xs, Ws, Ss, ys, nbytes))
        # one workspace for the split-K small-batch products (stages run one after another)
        import bit_packed_sign_amd as b1
        need = max([b1.gemv_workspace_bytes(wl.M, st[0].shape[1], st[1][0].shape[0])
                    for st in self.stages if len(st[1]) == 1] + [0])
        self.workspace = torch.empty(need, dtype=torch.uint8, device=device) if need and not ternary else None
        torch.cuda.synchronize()
        self.weight_bytes = sum(st[4] for st in self.stages)
        log(f"[bench] {wl.name}{' (ternary)' if ternary else ''}: {gi} GEMVs in {len(self.stages)} stages, "
            f"{self.weight_bytes / 1e9:.3f} GB "
            f"resident (generated in {time.time() - t0:.1f} s)")
        self.graph = None

    def run_stage(self, st):
        import bit_packed_sign_amd as b1
        x, Ws, Ss, ys, _ = st
        if self.ternary:
            if len(Ws) == 1:
                b1.gemv_t2(x, Ws[0], Ss[0], out=ys[0])
            else:
                b1.gemv_group_t2(x, Ws, Ss, outs=ys)
        elif len(Ws) == 1:
            if self.workspace is not None:    # small batch: K split over workgroups where it pays
                b1.gemv_ws(x, Ws[0], Ss[0], workspace=self.workspace, out=ys[0])
            else:
                b1.gemv(x, Ws[0], Ss[0], out=ys[0])
        else:                                 # q/k/v or gate/up: same-input fusion
            b1.gemv_group(x, Ws, Ss, outs=ys)

    def run_eager(self):
        for st in self.stages:
            self.run_stage(st)

    def capture(self):
        import torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.run_eager()                  # warm the path outside capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.run_eager()
        torch.cuda.synchronize()

    def timed(self, steps, warmup):
        import torch
        for _ in range(warmup):
            self.graph.replay()
        torch.cuda.synchronize()
        e0, e1 = events()
        e0.record()
        for _ in range(steps):
            self.graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def replay_percentiles_us(self, reps=50):
        """p10 / p50 / p90 of single graph replays (each bracketed by its own HIP events)."""
        import torch
        ev = [events() for _ in range(reps)]
        for _ in range(3):
            self.graph.replay()
        torch.cuda.synchronize()
        for a, b in ev:
            a.record()
            self.graph.replay()
            b.record()
        torch.cuda.synchronize()
        t = np.sort([a.elapsed_time(b) * 1e3 for a, b in ev])
        return {f"p{q}": round(float(np.percentile(t, q)), 1) for q in (10, 50, 90)}

    def per_launch_ms(self, reps=3):
        """Per-launch kernel durations (one launch per stage) from HIP events recorded on the
        stream the kernels are launched on (eager launches)."""
        import torch
        st = torch.cuda.current_stream()
        n = len(self.stages)
        ev = [events() for _ in range(n)]
        tot = np.zeros(n)
        for _ in range(reps):
            for i, stage in enumerate(self.stages):
                ev[i][0].record(st)
                self.run_stage(stage)
                ev[i][1].record(st)
            torch.cuda.synchronize()
            tot += np.array([a.elapsed_time(b) for a, b in ev])
        return tot / reps


class ChainStep:
    """The same stages as one persistent chain launch per step."""

    def __init__(self, step):
        import bit_packed_sign_amd as b1
        self.step = step
        self.plan = b1.ChainPlan([(x, Ws, Ss, ys) for x, Ws, Ss, ys, _ in step.stages])

    def timed(self, steps, warmup):
        import torch
        for _ in range(warmup):
            self.plan.run()
        torch.cuda.synchronize()
        e0, e1 = events()
        st = torch.cuda.current_stream()
        e0.record(st)
        for _ in range(steps):
            self.plan.run()
        e1.record(st)
        torch.cuda.synchronize()
        runs, err = self.plan.status()
        if err:
            raise RuntimeError("the chain reported a stage wait that gave up")
        return e0.elapsed_time(e1) / steps


def kernel_source_sha(*names):
    """Hash of the kernel sources (and of the build script, which holds the compile flags) a
    stored counter summary was taken with."""
    import hashlib
    h = hashlib.sha256()
    for n in (*names, "../build.py"):
        with open(os.path.join(ROOT, "bit_packed_sign_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel_key, sources, bytes_per_launch):
    """HBM traffic per launch from the committed rocprofv3 counter summary of `kernel_key`
    (FETCH_SIZE / WRITE_SIZE scaled by a plain copy of known size), or None when the summary
    is missing or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)[kernel_key]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha") != kernel_source_sha(*sources):
        return None
    return {"fetch_bytes_per_launch": rec["fetch_bytes_per_launch"],
            "write_bytes_per_launch": rec["write_bytes_per_launch"],
            "over_algorithmic": round((rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]) /
                                      bytes_per_launch, 3),
            "copy_scale": rec["copy_scale"], "source": "profiles/traffic.json"}


def cpu_baseline(wl):
    """The fp64 oracle over every output of the whole 8B decode step, on the host cores."""
    from bit_packed_sign_amd import synth
    from oracle import oracle
    oracle.lib()
    gi, nbytes, secs = 0, 0, 0.0
    for s, stage in enumerate(wl.stages):
        x = synth.stage_activations(0, wl, s)
        for g in stage.gemvs:
            bits, scales = synth.gemv_tensors(0, wl, gi)
            t0 = time.perf_counter()
            oracle.gemv(x, bits, scales)
            secs += time.perf_counter() - t0
            nbytes += g.weight_bytes
            gi += 1
    return {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"the whole 8B decode step: {gi} GEMVs, {nbytes / 1e9:.3f} GB of weights, every output, "
                      f"fp64 dequantise-and-dot with OpenMP over rows; {secs:.1f} s wall",
            "ms_per_step": round(secs * 1e3, 1)}


# ----------------------------------------------------------------------------------- extras
def extra_single(dev):
    """One 4096x4096 GEMV: cache-cold over a pool of copies larger than the 256 MB cache, and
    cache-hot; plus the 64-row patch applied and removed."""
    import torch
    import bit_packed_sign_amd as b1
    from bit_packed_sign_amd import synth
    wl = synth.single_gemv()
    bits, scales = synth.gemv_tensors(0, wl, 0)
    x = torch.from_numpy(synth.stage_activations(0, wl, 0)).to(dev)
    W0 = torch.from_numpy(bits.view(np.int32)).to(dev)
    S0 = torch.from_numpy(scales).to(dev)
    g = wl.gemvs[0]
    copies = int(np.ceil((1 << 30) / g.weight_bytes))
    Ws = [W0.clone() for _ in range(copies)]
    Ss = [S0.clone() for _ in range(copies)]
    y = torch.empty((1, 4096), dtype=torch.float16, device=dev)
    it = iter(range(10 ** 9))

    def cold():
        i = next(it) % copies
        b1.gemv(x, Ws[i], Ss[i], out=y)
    ms_cold = time_fn(cold, reps=copies)
    ms_hot = time_fn(lambda: b1.gemv(x, W0, S0, out=y), reps=200)
    rows = torch.from_numpy(synth.patch_rows_single()).to(dev)
    ms_patch = time_fn(lambda: b1.xor_patch_apply(W0, rows), reps=200)
    del Ws, Ss
    return {"workload": "4096x4096 GEMV, M=1", "pool_copies": copies,
            "us_cold": round(ms_cold * 1e3, 2), "gbs_cold": round(g.weight_bytes / ms_cold / 1e6, 1),
            "us_hot": round(ms_hot * 1e3, 2), "gbs_hot_cache": round(g.weight_bytes / ms_hot / 1e6, 1),
            "patch_64_rows_us": round(ms_patch * 1e3, 2),
            "note": "eager launches back to back: each time includes the launch gap"}


def extra_step(wl, dev, steps, label, chain=False):
    st = Step(wl, dev)
    st.capture()
    ms = st.timed(max(5, steps // 2), 2)
    out = {"workload": label, "ms_per_step": round(ms, 4),
           "gbs": round(wl.weight_bytes / ms / 1e6, 1), "tok_s": round(1e3 / ms, 1),
           "pct_hbm_peak": round(100 * wl.weight_bytes / ms / 1e6 / HBM_PEAK_GBS, 2), "path": "graph"}
    if chain:
        c = ChainStep(st)
        msc = c.timed(max(5, steps // 2), 2)
        out["chain"] = {"ms_per_step": round(msc, 4), "gbs": round(wl.weight_bytes / msc / 1e6, 1)}
        del c
    return st, out


def extra_patch27b(st, dev):
    """2000 distinct (layer, projection, row) flips over the 27B MLP matrices, one launch."""
    import bit_packed_sign_amd as b1
    import torch
    from bit_packed_sign_amd import synth
    mlp = []
    for l in range(64):                       # stages per layer: q|k|v, o, gate|up, down
        gu = st.stages[4 * l + 2][1]
        dn = st.stages[4 * l + 3][1]
        mlp += [gu[0], gu[1], dn[0]]
    table = b1.PatchTable(mlp)
    ent_np = synth.patch_entries_27b()
    ent = torch.from_numpy(ent_np).to(dev)
    ms = time_fn(lambda: b1.xor_patch_apply_multi(table, ent), reps=200)
    row_bytes = np.array([m.shape[1] * 4 for m in mlp])[ent_np[:, 0]].sum()
    return {"patch_2000_rows_us": round(ms * 1e3, 2), "patch_bytes_read_and_written": int(2 * row_bytes)}


def extra_bits_8b(st, dev):
    """500K random single-bit flips over the 108 MLP matrices of the 8B batch-16 workload (the
    Bankai robustness experiment's data movement), one launch; each timed call flips them again."""
    import bit_packed_sign_amd as b1
    import torch
    from bit_packed_sign_amd import synth
    mlp = []
    for l in range(36):                       # stages per layer: gate|up, down
        gu = st.stages[2 * l][1]
        dn = st.stages[2 * l + 1][1]
        mlp += [gu[0], gu[1], dn[0]]
    table = b1.PatchTable(mlp)
    ent = torch.from_numpy(synth.bit_flip_entries(0, [(m.shape[0], m.shape[1] * 32) for m in mlp],
                                                  500_000)).to(dev)
    ms = time_fn(lambda: b1.xor_bits_apply(table, ent), reps=50)
    return {"bit_flips_500k_us": round(ms * 1e3, 2), "flips_per_s": round(500_000 / (ms * 1e-3), 0)}


def extra_rank27b(st, dev):
    """Scale ranking of the rows of one 27B gate matrix (17408 x 5120), exact."""
    import bit_packed_sign_amd as b1
    S = st.stages[2][2][0]                    # layer 0: gate|up stage, gate scales
    score, order = b1.rank_rows_by_scale(S)
    ms = time_fn(lambda: b1.rank_rows_by_scale(S, score, order), reps=20)
    return {"rank_rows_17408x5120_us": round(ms * 1e3, 1)}


def extra_ternary(dev, steps):
    """Ternary g128 (2-bit slots): the 8B decode step (one launch per stage, q/k/v and gate/up
    fused, HIP graph), the lm_head product alone, and the prefill contraction."""
    import torch
    import bit_packed_sign_amd as b1
    from bit_packed_sign_amd import synth
    out = {"bytes_per_weight": synth.TERNARY_BYTES_PER_WEIGHT}
    st = Step(synth.decode_8b(), dev, ternary=True)
    st.capture()
    ms = st.timed(steps, 3)
    out["decode_8b"] = {"ms_per_step": round(ms, 4), "gbs": round(st.weight_bytes / ms / 1e6, 1),
                        "tok_s": round(1e3 / ms, 1), "launches": len(st.stages),
                        "weight_bytes": st.weight_bytes}
    x, Ws, Ss, ys, nb = st.stages[-1]                 # lm_head 4096 x 151936
    ms = time_fn(lambda: b1.gemv_t2(x, Ws[0], Ss[0], out=ys[0]), reps=20)
    out["lm_head"] = {"us": round(ms * 1e3, 2), "gbs": round(nb / ms / 1e6, 1)}
    del st
    torch.cuda.empty_cache()
    M, K, N = synth.PREFILL_M, synth.PREFILL_K, synth.PREFILL_N
    r = synth.rng_for(0, synth.WL_PREFILL, 1)
    x = torch.from_numpy(synth.activations(r, M, K)).to(dev)
    T = torch.from_numpy(synth.ternary_words_fast(r, N, K).view(np.int32)).to(dev)
    S = torch.from_numpy(synth.group_scales(r, N, K)).to(dev)
    y = torch.empty((M, N), dtype=torch.float16, device=dev)
    ms = time_fn(lambda: b1.gemm_prefill_t2(x, T, S, out=y), reps=50, warm=PREFILL_WARM)
    tf = 2.0 * M * K * N / (ms * 1e-3) / 1e12
    out["prefill"] = {"us": round(ms * 1e3, 2), "tflops": round(tf, 1),
                      "frac_of_fp16_mfma_peak": round(tf / FP16_MFMA_PEAK_TFLOPS, 4)}
    return out


def extra_prefill(dev):
    import torch
    import bit_packed_sign_amd as b1
    from bit_packed_sign_amd import synth
    M, K, N = synth.PREFILL_M, synth.PREFILL_K, synth.PREFILL_N
    r = synth.rng_for(0, synth.WL_PREFILL, 0)
    x = torch.from_numpy(synth.activations(r, M, K)).to(dev)
    W = torch.from_numpy(synth.sign_words(r, N, K).view(np.int32)).to(dev)
    S = torch.from_numpy(synth.group_scales(r, N, K)).to(dev)
    y = torch.empty((M, N), dtype=torch.float16, device=dev)
    ms = time_fn(lambda: b1.gemm_prefill(x, W, S, out=y), reps=50, warm=PREFILL_WARM)
    tf = 2.0 * M * K * N / (ms * 1e-3) / 1e12
    # a 512-token prompt (the pages' pp512 point) on the same weights: the first 512 rows of x
    m5 = 512
    y5 = torch.empty((m5, N), dtype=torch.float16, device=dev)
    ms5 = time_fn(lambda: b1.gemm_prefill(x[:m5], W, S, out=y5), reps=50, warm=4 * PREFILL_WARM)
    tf5 = 2.0 * m5 * K * N / (ms5 * 1e-3) / 1e12
    # context only: a dense fp16 GEMM of the same shape through torch (the vendor BLAS), with
    # the weights as a plain fp16 matrix (row-major [K][N] and transposed [N][K])
    del W, S
    a = torch.randn((M, K), dtype=torch.float16, device=dev)
    b = torch.randn((K, N), dtype=torch.float16, device=dev)
    bt = b.t().contiguous()
    ref = {}
    for name, fn in (("b_row_major", lambda: a @ b), ("b_transposed", lambda: a @ bt.t())):
        rms = time_fn(fn, reps=50, warm=PREFILL_WARM)
        ref[name] = {"us": round(rms * 1e3, 2), "tflops": round(2.0 * M * K * N / (rms * 1e-3) / 1e12, 1)}
    return {"workload": "prefill M=2048 K=4096 N=12288", "us": round(ms * 1e3, 2),
            "tflops": round(tf, 1), "frac_of_fp16_mfma_peak": round(tf / FP16_MFMA_PEAK_TFLOPS, 4),
            "m512": {"us": round(ms5 * 1e3, 2), "tflops": round(tf5, 1),
                     "frac_of_fp16_mfma_peak": round(tf5 / FP16_MFMA_PEAK_TFLOPS, 4)},
            "dense_fp16_gemm_same_shape_torch": ref}


def extra_pm1(dev):
    import torch
    import bit_packed_sign_amd as b1
    from bit_packed_sign_amd import synth
    K, N = 4096, 151936
    r = synth.rng_for(0, synth.WL_TEST, 424242)
    A = torch.from_numpy(synth.pm1_words(r, 1, K).view(np.int32)).to(dev)
    W = torch.from_numpy(synth.sign_words(r, N, K).view(np.int32)).to(dev)
    y = torch.empty((1, N), dtype=torch.int32, device=dev)
    ms = time_fn(lambda: b1.gemv_pm1(A, W, out=y), reps=50)
    return {"workload": "+-1 popcount product K=4096 N=151936 M=1", "us": round(ms * 1e3, 2),
            "gbs": round(N * K / 8 / ms / 1e6, 1)}


# ------------------------------------------------------------------------------------ main
def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU only: the products here run on one "
                                   "GPU's share of the weights, and no multi-GPU path is provided",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    from bit_packed_sign_amd import synth
    dev = torch.device("cuda:0")

    if args.only:
        run_only(args, dev)
        return

    wl = synth.decode_8b()
    wbytes = wl.weight_bytes
    step = Step(wl, dev)
    step.capture()
    ms_graph = step.timed(args.steps, args.warmup)
    log(f"[bench] graph step {ms_graph * 1e3:.1f} us, {wbytes / ms_graph / 1e6:.0f} GB/s")
    chain = ChainStep(step)
    ms_chain = chain.timed(args.steps, args.warmup)
    log(f"[bench] chain step {ms_chain * 1e3:.1f} us, {wbytes / ms_chain / 1e6:.0f} GB/s")

    # eager per-launch HIP events (on the launch stream) give each stage's share; in the replayed
    # graph the launches run back to back, so the kernel's average duration there is the step
    # time over the launches (rocprofv3 kernel traces of the same command agree)
    per = step.per_launch_ms()
    nl = len(step.stages)
    floor_us = graph_launch_floor_us(dev, nl)
    log(f"[bench] graph of {nl} dependent one-workgroup launches: {floor_us:.2f} us per launch")
    pct = step.replay_percentiles_us()
    read_gbs = stream_read_gbs(dev)
    log(f"[bench] single replays {pct} us; stream read {read_gbs:.0f} GB/s")
    big = max(range(nl), key=lambda i: step.stages[i][4])
    paths = {
        "graph": {"ms_per_step": round(ms_graph, 5), "gbs": round(wbytes / ms_graph / 1e6, 1),
                  "tok_s": round(1e3 / ms_graph, 1),
                  "launches": nl, "avg_launch_us_in_graph": round(ms_graph * 1e3 / nl, 3),
                  "eager_launch_sum_us": round(float(per.sum() * 1e3), 1),
                  "graph_floor_us_per_launch": round(floor_us, 3),
                  "single_replay_us": pct,
                  "largest_launch_eager": {"stage": "lm_head 4096x151936", "bytes": step.stages[big][4],
                                           "us": round(float(per[big] * 1e3), 2),
                                           "gbs": round(step.stages[big][4] / (per[big] * 1e-3) / 1e9, 1)}},
        "chain": {"ms_per_step": round(ms_chain, 5), "gbs": round(wbytes / ms_chain / 1e6, 1),
                  "tok_s": round(1e3 / ms_chain, 1)},
    }
    if ms_chain <= ms_graph:
        head, ms = "chain", ms_chain
        achieved = wbytes / (ms_chain * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": stored_traffic("gemv_chain_kernel", ["gemv_chain.hip", "mx_common.hpp"], wbytes),
                "kernel": "gemv_chain_kernel (one launch per step)",
                "bytes_per_launch": wbytes, "avg_launch_us": round(ms_chain * 1e3, 2),
                "timing": "HIP events around the timed launches (back to back on one stream)"}
    else:
        head, ms = "graph", ms_graph
        achieved = wbytes / (ms_graph * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": stored_traffic("gemv_mx_kernel", ["gemv_mx.hip", "mx_common.hpp"], wbytes / nl),
                "kernel": "gemv_mx_kernel, all 145 launches of the 8B step",
                "bytes_per_launch": round(wbytes / nl, 1), "avg_launch_us": round(ms_graph * 1e3 / nl, 3),
                "timing": "HIP events around the timed graph replays on the replay stream; launches run "
                          "back to back, so the average launch is the step time over 145 launches"}
    gbs = wbytes / (ms * 1e-3) / 1e9
    log(f"[bench] headline {head}: {ms * 1e3:.1f} us, {gbs:.0f} GB/s, {1e3 / ms:.0f} tok/s")
    del chain, step
    torch.cuda.empty_cache()

    extra = {"step_paths": paths}
    if not args.no_extra:
        t0 = time.time()
        extra["single_gemv"] = extra_single(dev)
        log(f"[bench] single GEMV: {extra['single_gemv']}")
        st, extra["mlp_8b_m16"] = extra_step(synth.mlp_8b_m16(), dev, args.steps,
                                             "8B MLP batch 16: 36 x (gate/up 4096x12288, down 12288x4096)")
        extra["mlp_8b_m16"].update(extra_bits_8b(st, dev))
        log(f"[bench] mlp m16: {extra['mlp_8b_m16']}")
        del st
        torch.cuda.empty_cache()
        extra["prefill"] = extra_prefill(dev)
        log(f"[bench] prefill: {extra['prefill']}")
        st, extra["decode_27b"] = extra_step(synth.decode_27b(), dev, args.steps,
                                             "27B decode batch 1: 64 x (q/k/v/o 5120x5120, gate/up "
                                             "5120x17408, down 17408x5120)", chain=True)
        extra["decode_27b"].update(extra_patch27b(st, dev))
        extra["decode_27b"].update(extra_rank27b(st, dev))
        log(f"[bench] 27b: {extra['decode_27b']}")
        del st
        torch.cuda.empty_cache()
        extra["ternary"] = extra_ternary(dev, args.steps)
        log(f"[bench] ternary: {extra['ternary']}")
        extra["pm1"] = extra_pm1(dev)
        log(f"[bench] pm1: {extra['pm1']} ({time.time() - t0:.0f} s of extras)")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl)
        log(f"[bench] cpu baseline {cpu['value']:.3f} GB/s on {cpu['cores']} threads")
    out = {
        "metric": "1-bit decode GEMV weight-GB/s (% of HBM peak) and implied tok/s at 8B shape",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "decode-8b-m1: 36 x (q 4096x4096, k/v 4096x1024, o 4096x4096, "
                               "gate/up 4096x12288, down 12288x4096) + lm_head 4096x151936, batch 1, "
                               "253 GEMVs in 145 dependent stages (q/k/v and gate/up fused per stage); "
                               + ("one persistent chain launch per step" if head == "chain" else
                                  "one launch per stage, HIP-graph replay"),
                   "step_path": head,
                   "weight_bytes_per_step": wbytes, "global_batch": 1, "parallelism": "none (1 GPU)"},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "pct_of_stream_read": round(100 * gbs / read_gbs, 2),
        "stream_read_gbs": round(read_gbs, 1),
        "implied_tok_s": round(1e3 / ms, 1),
        "roofline": roof,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


def run_only(args, dev):
    """One workload alone, for profiler runs (rocprofv3 kernel traces and counters)."""
    import torch
    import bit_packed_sign_amd as b1
    from bit_packed_sign_amd import synth
    name = args.only
    if name == "step8b":
        st = Step(synth.decode_8b(), dev)
        st.capture()
        ms = st.timed(args.steps, args.warmup)
        log(f"[bench] step8b {ms * 1e3:.1f} us")
    elif name == "chain8b":
        st = Step(synth.decode_8b(), dev)
        ms = ChainStep(st).timed(args.steps, args.warmup)
        log(f"[bench] chain8b {ms * 1e3:.1f} us")
    elif name == "lmhead":
        wl = synth.decode_8b()
        i = len(wl.gemvs) - 1
        bits, scales = synth.gemv_tensors(0, wl, i)
        x = torch.from_numpy(synth.stage_activations(0, wl, len(wl.stages) - 1)).to(dev)
        W = torch.from_numpy(bits.view(np.int32)).to(dev)
        S = torch.from_numpy(scales).to(dev)
        y = torch.empty((1, W.shape[0]), dtype=torch.float16, device=dev)
        ms = time_fn(lambda: b1.gemv(x, W, S, out=y), reps=args.steps)
        log(f"[bench] lm_head {ms * 1e3:.1f} us")
    elif name == "single":
        log(f"[bench] {extra_single(dev)}")
    elif name == "mlp16":
        st, o = extra_step(synth.mlp_8b_m16(), dev, args.steps, "mlp16")
        log(f"[bench] {o}")
    elif name == "bits":
        st, _ = extra_step(synth.mlp_8b_m16(), dev, 2, "mlp16")
        log(f"[bench] {extra_bits_8b(st, dev)}")
    elif name == "prefill":
        log(f"[bench] {extra_prefill(dev)}")
    elif name == "step27b":
        st, o = extra_step(synth.decode_27b(), dev, args.steps, "27b")
        log(f"[bench] {o} patch {extra_patch27b(st, dev)} rank {extra_rank27b(st, dev)}")
    elif name == "pm1":
        log(f"[bench] {extra_pm1(dev)}")
    elif name == "ternary":
        log(f"[bench] {extra_ternary(dev, args.steps)}")
    elif name == "copy":
        # a plain device copy of known size, to scale the HBM traffic counters
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        ms = time_fn(lambda: dst.copy_(src), reps=args.steps)
        log(f"[bench] copy 256 MiB {ms * 1e3:.1f} us")
    else:
        raise SystemExit(f"unknown workload {name}")
    torch.cuda.synchronize()


if __name__ == "__main__":
    main()
