"""Seeded synthetic inputs and workload shapes for the 1-bit GEMV / XOR-patch path.

This module only draws random numbers and lists shapes.  It holds none of the
method's arithmetic (no unpacking, no dot products, no patching), so both the
HIP path and the CPU oracle can be fed from it without sharing any code.

Distributions (one per tensor kind):

* sign bits  -- uniform 32-bit words, i.e. i.i.d. Bernoulli(0.5) bits; bit 1
  stands for +1 and bit 0 for -1, 32 weights per uint32 along K, LSB first.
* scales     -- fp16(|N(0,1)| * 0.02), one per 128 consecutive weights along K.
* activations -- fp16(N(0,1)), rounded to nearest even from float64.
* patch rows -- distinct rows drawn uniformly without replacement.

Seeding: tensor ``t`` of workload ``w`` is drawn from
``PCG64(SeedSequence(entropy=seed, spawn_key=(w, t)))``.  That is the child
``SeedSequence.spawn`` would hand out, but addressable directly, so any single
tensor of a large workload can be regenerated without drawing the others.

Shapes follow the model families on the pages: the 1-bit Bonsai 8B model
("1-bit Bonsai" page on news.hada.io) and Bonsai 27B, 64 blocks with hidden
width 5120 ("Bonsai 27B" page on discuss.pytorch.kr, section on the
representation).  The matrices are written K x N: K is the input width and N
the number of output rows.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

GROUP = 128          # weights per fp16 scale
WORD_BITS = 32       # weights per packed uint32

# Workload ids used in the seeding key.
WL_SINGLE = 0        # one 4096x4096 GEMV + 64-row patch
WL_DECODE_8B = 1     # 8B-class decode step, batch 1
WL_MLP_8B_M16 = 2    # 8B-class MLP, batch 16
WL_PREFILL = 3       # prefill contraction M=2048, K=4096, N=12288
WL_DECODE_27B = 4    # 27B-class decode step + 2000-row patch
WL_TEST = 9          # ad-hoc test tensors


def rng_for(seed: int, workload: int, tensor: int) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(workload, tensor))
    return np.random.Generator(np.random.PCG64(ss))


def sign_words(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """uint32 [N][ceil(K/32)] of i.i.d. fair bits (bits past K in the last word are random too)."""
    return rng.integers(0, 1 << 32, size=(N, (K + WORD_BITS - 1) // WORD_BITS), dtype=np.uint32)


def ternary_words(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """uint32 [N][K/16]: 2-bit slots, LSB first, each weight drawn uniformly from {0, +1, -1}
    as the codes 00, 01, 11 (code 10 is never drawn)."""
    codes = np.array([0, 1, 3], np.uint32)[rng.integers(0, 3, size=(N, K), dtype=np.int64)]
    shifts = (2 * np.arange(16, dtype=np.uint32))[None, None, :]
    return np.bitwise_or.reduce(codes.reshape(N, K // 16, 16) << shifts, axis=2).astype(np.uint32)


def group_scales(rng: np.random.Generator, N: int, K: int, group: int = GROUP) -> np.ndarray:
    """fp16 [N][K/group] = fp16(|N(0,1)| * 0.02)."""
    return (np.abs(rng.standard_normal((N, K // group))) * 0.02).astype(np.float16)


def activations(rng: np.random.Generator, M: int, K: int) -> np.ndarray:
    """fp16 [M][K] = fp16(N(0,1))."""
    return rng.standard_normal((M, K)).astype(np.float16)


def pm1_words(rng: np.random.Generator, M: int, K: int) -> np.ndarray:
    """uint32 [M][K/32]: +-1 activations packed like the weights (bit 1 = +1)."""
    return sign_words(rng, M, K)


def distinct_rows(rng: np.random.Generator, n_total: int, count: int) -> np.ndarray:
    """int32 [count]: rows drawn uniformly without replacement from range(n_total)."""
    return rng.choice(n_total, size=count, replace=False).astype(np.int32)


# --------------------------------------------------------------------------------------
# Workload shapes
# --------------------------------------------------------------------------------------

@dataclass
class Gemv:
    name: str
    K: int
    N: int

    @property
    def weights(self) -> int:
        return self.K * self.N

    @property
    def weight_bytes(self) -> int:
        """Packed bits plus fp16 scales: K*N/8 + 2*K*N/128 (1.125 bits per weight)."""
        return self.K * self.N // 8 + 2 * (self.K * self.N // GROUP)


@dataclass
class Stage:
    """GEMVs that read the same activation vector; stages run one after another."""
    layer: int
    gemvs: List[Gemv] = field(default_factory=list)

    @property
    def K(self) -> int:
        return self.gemvs[0].K


@dataclass
class Workload:
    wid: int
    name: str
    M: int
    stages: List[Stage]

    @property
    def gemvs(self) -> List[Gemv]:
        return [g for s in self.stages for g in s.gemvs]

    @property
    def weight_bytes(self) -> int:
        return sum(g.weight_bytes for g in self.gemvs)

    @property
    def weights(self) -> int:
        return sum(g.weights for g in self.gemvs)


def _decoder(wid, name, M, layers, hidden, q_out, kv_out, o_in, inter, lm_vocab=None, mlp_only=False):
    stages: List[Stage] = []
    for l in range(layers):
        if not mlp_only:
            stages.append(Stage(l, [Gemv(f"L{l}.q", hidden, q_out), Gemv(f"L{l}.k", hidden, kv_out),
                                    Gemv(f"L{l}.v", hidden, kv_out)]))
            stages.append(Stage(l, [Gemv(f"L{l}.o", o_in, hidden)]))
        stages.append(Stage(l, [Gemv(f"L{l}.gate", hidden, inter), Gemv(f"L{l}.up", hidden, inter)]))
        stages.append(Stage(l, [Gemv(f"L{l}.down", inter, hidden)]))
    if lm_vocab:
        stages.append(Stage(layers, [Gemv("lm_head", hidden, lm_vocab)]))
    return Workload(wid, name, M, stages)


def single_gemv() -> Workload:
    return Workload(WL_SINGLE, "single-gemv-4096x4096-m1", 1, [Stage(0, [Gemv("W", 4096, 4096)])])


def decode_8b() -> Workload:
    """36 layers of q 4096x4096, k/v 4096x1024, o 4096x4096, gate/up 4096x12288, down 12288x4096,
    then lm_head 4096x151936; batch 1.  253 GEMVs in 145 dependent stages."""
    return _decoder(WL_DECODE_8B, "decode-8b-m1", 1, 36, 4096, 4096, 1024, 4096, 12288, lm_vocab=151936)


def mlp_8b_m16() -> Workload:
    """36 layers of gate/up 4096x12288 then down 12288x4096 at batch 16 (108 GEMVs, 72 stages)."""
    return _decoder(WL_MLP_8B_M16, "mlp-8b-m16", 16, 36, 4096, 0, 0, 0, 12288, mlp_only=True)


def decode_27b() -> Workload:
    """64 layers of q/k/v/o 5120x5120, gate/up 5120x17408, down 17408x5120; batch 1
    (448 GEMVs in 256 stages; no lm_head)."""
    return _decoder(WL_DECODE_27B, "decode-27b-m1", 1, 64, 5120, 5120, 5120, 5120, 17408)


PREFILL_M, PREFILL_K, PREFILL_N = 2048, 4096, 12288


def mlp_rows_27b() -> List[Tuple[int, str, int]]:
    """(layer, projection, N) of every MLP matrix of the 27B workload, in patch-table order."""
    out = []
    for l in range(64):
        out += [(l, "gate", 17408), (l, "up", 17408), (l, "down", 5120)]
    return out


# --------------------------------------------------------------------------------------
# Tensor draws for a workload.  Tensor index layout per workload:
#   GEMV i (in stage order):   bits -> 2*i, scales -> 2*i+1
#   stage s activations:       10_000 + s
#   patch rows:                20_000
# --------------------------------------------------------------------------------------

def gemv_tensors(seed: int, wl: Workload, i: int) -> Tuple[np.ndarray, np.ndarray]:
    g = wl.gemvs[i]
    return (sign_words(rng_for(seed, wl.wid, 2 * i), g.N, g.K),
            group_scales(rng_for(seed, wl.wid, 2 * i + 1), g.N, g.K))


def ternary_words_fast(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """uint32 [N][K/16] of 2-bit slots from uniform random words, every never-written code 10
    turned into 00: weights 0 with probability 1/2, +1 and -1 with 1/4 each.  For large
    workloads (the benchmark), where drawing each weight separately would not fit in memory."""
    w = rng.integers(0, 2 ** 32, size=(N, K // 16), dtype=np.uint32)
    lo = w & np.uint32(0x55555555)
    return (lo | (w & np.uint32(0xAAAAAAAA) & (lo << np.uint32(1)))).astype(np.uint32)


def ternary_gemv_tensors(seed: int, wl: Workload, i: int) -> Tuple[np.ndarray, np.ndarray]:
    """Ternary weights (2-bit slots) and scales of GEMV i of a workload, for the benchmark."""
    g = wl.gemvs[i]
    return (ternary_words_fast(rng_for(seed, wl.wid, 30_000 + 2 * i), g.N, g.K),
            group_scales(rng_for(seed, wl.wid, 30_000 + 2 * i + 1), g.N, g.K))


TERNARY_BYTES_PER_WEIGHT = 2 / 8 + 2 / GROUP        # 2-bit slot + the fp16 group scale


def stage_activations(seed: int, wl: Workload, s: int) -> np.ndarray:
    return activations(rng_for(seed, wl.wid, 10_000 + s), wl.M, wl.stages[s].K)


def patch_rows_single(seed: int = 0, count: int = 64, N: int = 4096) -> np.ndarray:
    return distinct_rows(rng_for(seed, WL_SINGLE, 20_000), N, count)


def patch_entries_27b(seed: int = 0, count: int = 2000) -> np.ndarray:
    """int32 [count][2] = (matrix id into mlp_rows_27b(), row), drawn uniformly without replacement
    from all 2,555,904 MLP output rows of the 27B workload."""
    mats = mlp_rows_27b()
    sizes = np.array([n for (_, _, n) in mats], dtype=np.int64)
    offs = np.concatenate([[0], np.cumsum(sizes)])
    flat = rng_for(seed, WL_DECODE_27B, 20_000).choice(int(offs[-1]), size=count, replace=False)
    mid = np.searchsorted(offs, flat, side="right") - 1
    return np.stack([mid, flat - offs[mid]], axis=1).astype(np.int32)


def mlp_mats_8b() -> List[Tuple[int, str, int, int]]:
    """(layer, projection, N, K) of every MLP matrix of the 8B workload (36 x gate, up, down)."""
    out = []
    for l in range(36):
        out += [(l, "gate", 12288, 4096), (l, "up", 12288, 4096), (l, "down", 4096, 12288)]
    return out


def bit_flip_entries(seed: int, shapes: List[Tuple[int, int]], count: int, workload: int = WL_TEST,
                     tensor: int = 21_000) -> np.ndarray:
    """int32 [count][3] = (matrix id, row, k): `count` weights drawn uniformly (with replacement,
    as independent random flips are) from all weights of the matrices of `shapes` [(N, K), ...]."""
    sizes = np.array([n * k for (n, k) in shapes], dtype=np.int64)
    offs = np.concatenate([[0], np.cumsum(sizes)])
    flat = rng_for(seed, workload, tensor).integers(0, int(offs[-1]), size=count, dtype=np.int64)
    mid = np.searchsorted(offs, flat, side="right") - 1
    local = flat - offs[mid]
    Ks = np.array([k for (_, k) in shapes], dtype=np.int64)[mid]
    return np.stack([mid, local // Ks, local % Ks], axis=1).astype(np.int32)
