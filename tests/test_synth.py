"""The seeded input generators: determinism, distributions and workload shapes."""
import numpy as np

from bit_packed_sign_amd import synth


def test_seeded_draws_are_deterministic_and_addressable():
    wl = synth.decode_8b()
    a1, s1 = synth.gemv_tensors(0, wl, 1)
    a2, s2 = synth.gemv_tensors(0, wl, 1)
    assert np.array_equal(a1, a2) and np.array_equal(s1, s2)
    b, _ = synth.gemv_tensors(1, wl, 1)
    assert not np.array_equal(a1, b)
    assert a1.shape == (1024, 4096 // 32) and s1.shape == (1024, 4096 // 128)


def test_distributions():
    r = synth.rng_for(0, synth.WL_TEST, 1000)
    W = synth.sign_words(r, 512, 4096)
    frac = np.unpackbits(W.view(np.uint8)).mean()
    assert abs(frac - 0.5) < 0.002
    S = synth.group_scales(r, 512, 4096)
    assert S.dtype == np.float16 and (S >= 0).all()
    # |N(0,1)| * 0.02 has mean 0.02 * sqrt(2/pi)
    assert abs(S.astype(np.float64).mean() - 0.02 * np.sqrt(2 / np.pi)) < 3e-4
    x = synth.activations(r, 16, 4096)
    assert x.dtype == np.float16
    assert abs(x.astype(np.float64).std() - 1.0) < 0.02


def test_patch_draws_are_distinct_and_in_range():
    rows = synth.patch_rows_single()
    assert rows.size == 64 and np.unique(rows).size == 64 and rows.min() >= 0 and rows.max() < 4096
    ent = synth.patch_entries_27b()
    mats = synth.mlp_rows_27b()
    assert ent.shape == (2000, 2)
    assert len({(int(a), int(b)) for a, b in ent}) == 2000
    assert all(0 <= r < mats[m][2] for m, r in ent)
    assert sum(n for _, _, n in mats) == 2_555_904


def test_workload_shapes():
    assert synth.decode_8b().weight_bytes == 1_064_263_680
    assert synth.mlp_8b_m16().weight_bytes == 764_411_904
    assert len(synth.mlp_8b_m16().gemvs) == 108 and len(synth.mlp_8b_m16().stages) == 72
    assert synth.single_gemv().weight_bytes == 2_359_296
