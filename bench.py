"""Benchmark of the 1-bit sign GEMV decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--extra]

A step is one batch-1 decode pass of the 8B-class model's GEMVs: 36 layers of
q 4096x4096, k/v 4096x1024, o 4096x4096, gate/up 4096x12288, down 12288x4096, then
lm_head 4096x151936 -- 253 products in 145 dependent stages, every stage reading its own
fp16 activation vector (norms/attention omitted), all weights and activations resident
in HBM.  The step is captured once into a HIP graph and replayed.

Metric: weight-GB/s = bytes of packed bits + fp16 scales per step (1,064,263,680 B)
divided by the step time; implied tokens/s = 1 / step time.  One JSON line on stdout.
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=6,
                    help="decode layers of the 8B step the oracle runs for the CPU baseline")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class DecodeStep:
    """Device-resident weights/activations of a workload and a graph of one step."""

    def __init__(self, wl, device):
        import torch
        from bit_packed_sign_amd import synth
        self.wl = wl
        self.dev = device
        # one entry per stage: (x, [W...], [S...], [y...], bytes)
        self.stages = []
        t0 = time.time()
        gi = 0
        for s, stage in enumerate(wl.stages):
            xs = torch.from_numpy(synth.stage_activations(0, wl, s)).to(device)
            Ws, Ss, ys = [], [], []
            for g in stage.gemvs:
                bits, scales = synth.gemv_tensors(0, wl, gi)
                Ws.append(torch.from_numpy(bits.view(np.int32)).to(device))
                Ss.append(torch.from_numpy(scales).to(device))
                ys.append(torch.empty((wl.M, g.N), dtype=torch.float16, device=device))
                gi += 1
            self.stages.append((xs, Ws, Ss, ys, sum(g.weight_bytes for g in stage.gemvs)))
        torch.cuda.synchronize()
        log(f"[bench] {wl.name}: {gi} GEMVs in {len(self.stages)} stages, {wl.weight_bytes / 1e9:.3f} GB resident "
            f"(generated in {time.time() - t0:.1f} s)")
        self.graph = None

    @staticmethod
    def run_stage(st):
        import bit_packed_sign_amd as b1
        x, Ws, Ss, ys, _ = st
        if len(Ws) == 1:
            b1.gemv(x, Ws[0], Ss[0], out=ys[0])
        else:                                     # q/k/v or gate/up: same-input fusion
            b1.gemv_group(x, Ws, Ss, outs=ys)

    def run_eager(self):
        for st in self.stages:
            self.run_stage(st)

    def capture(self):
        import torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.run_eager()                      # warm the path outside capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.run_eager()
        torch.cuda.synchronize()

    def replay(self):
        self.graph.replay()

    def per_launch_ms(self, reps=3):
        """Per-launch kernel durations (one launch per stage) with HIP events recorded on the
        stream the kernels are launched on (eager launches)."""
        import torch
        st = torch.cuda.current_stream()
        n = len(self.stages)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        tot = np.zeros(n)
        for _ in range(reps):
            for i, stage in enumerate(self.stages):
                ev[i][0].record(st)
                self.run_stage(stage)
                ev[i][1].record(st)
            torch.cuda.synchronize()
            tot += np.array([a.elapsed_time(b) for a, b in ev])
        return tot / reps


def cpu_baseline(wl, layers):
    """The fp64 oracle on the first `layers` decode layers of the step (all their outputs)."""
    from bit_packed_sign_amd import synth
    from oracle import oracle
    oracle.lib()
    gi, nbytes, secs = 0, 0, 0.0
    for s, stage in enumerate(wl.stages):
        if stage.layer >= layers:
            break
        x = synth.stage_activations(0, wl, s)
        for g in stage.gemvs:
            bits, scales = synth.gemv_tensors(0, wl, gi)
            t0 = time.perf_counter()
            oracle.gemv(x, bits, scales)
            secs += time.perf_counter() - t0
            nbytes += g.weight_bytes
            gi += 1
    return {"value": nbytes / secs / 1e9, "unit": "GB/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"first {layers} of 36 decode layers of the 8B step ({gi} GEMVs, "
                      f"{nbytes / 1e9:.3f} GB of weights), every output, fp64; {secs:.1f} s wall"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; multi-GPU runs are not part of "
                                   "this build (see the sharding note in the design document)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    from bit_packed_sign_amd import synth
    dev = torch.device("cuda:0")
    wl = synth.decode_8b()
    step = DecodeStep(wl, dev)
    step.capture()
    for _ in range(args.warmup):
        step.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    wbytes = wl.weight_bytes
    gbs = wbytes / (ms * 1e-3) / 1e9
    log(f"[bench] step {ms * 1e3:.1f} us, {gbs:.0f} GB/s, {1e3 / ms:.0f} tok/s")

    # dominant kernel: the decode GEMV kernel; per-launch durations by HIP events
    per = step.per_launch_ms()
    kern_gbs = wbytes / (per.sum() * 1e-3) / 1e9
    log(f"[bench] kernel-sum {per.sum() * 1e3:.1f} us over {len(per)} launches -> {kern_gbs:.0f} GB/s")
    big = max(range(len(step.stages)), key=lambda i: step.stages[i][4])
    log(f"[bench] largest launch (lm_head): {per[big] * 1e3:.1f} us -> "
        f"{step.stages[big][4] / (per[big] * 1e-3) / 1e9:.0f} GB/s")
    roof = {"bound": "hbm", "achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(kern_gbs / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "gemv_mx_kernel (all 145 launches of the step)",
            "bytes_per_launch": wbytes / len(per), "avg_launch_us": float(per.mean() * 1e3)}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_layers)
        log(f"[bench] cpu baseline {cpu['value']:.3f} GB/s on {cpu['cores']} threads")
    out = {
        "metric": "1-bit decode GEMV weight-GB/s (% of HBM peak) and implied tok/s at 8B shape",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "decode-8b-m1: 36 x (q 4096x4096, k/v 4096x1024, o 4096x4096, "
                               "gate/up 4096x12288, down 12288x4096) + lm_head 4096x151936, batch 1, "
                               "253 GEMVs in 145 dependent stages (q/k/v and gate/up fused per stage), "
                               "HIP-graph replay",
                   "weight_bytes_per_step": wbytes, "global_batch": 1, "parallelism": "none (1 GPU)"},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "implied_tok_s": round(1e3 / ms, 1),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
