"""Seeded input generators: determinism, recipe and quantisation (CPU only)."""
import numpy as np
import torch

from bwd_rmsnorm_fwd_amd import synth


def test_bf16_quantisation_matches_library():
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(100000) * 10.0 ** rng.integers(-20, 20, 100000)).astype(np.float32)
    bits = synth.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    back = synth.bf16_bits_to_f32(bits)
    assert np.array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_seeded_and_deterministic():
    wl = synth.small_case(33, 96, synth.BF16, seed=3, outlier_frac=0.01)
    assert np.array_equal(wl.x(), wl.x())
    assert not np.array_equal(wl.x(), synth.small_case(33, 96, synth.BF16, seed=4).x())
    assert wl.x().dtype == np.uint16 and wl.x().shape == (33, 96)
    f = synth.small_case(5, 7, synth.F32)
    assert f.x().dtype == np.float32


def test_recipe_distributions():
    wl = synth.WORKLOADS["c2_bf16_4096x4096"]
    small = synth.Workload("t", synth.BF16, 512, 4096, 1e-6, 201, 202, 203,
                           x_outlier_frac=0.01, seed_outlier=205)
    x = synth.to_f64(small.x(), synth.BF16)
    col_rms = np.sqrt(np.mean(x * x, axis=0))
    outliers = np.flatnonzero(col_rms > 10)
    assert len(outliers) == 41                       # ceil(1% of 4096) feature columns
    assert np.all(np.abs(col_rms[outliers] / 50 - 1) < 0.15)
    assert abs(np.delete(col_rms, outliers).mean() - 1) < 0.01
    w = synth.to_f64(wl.w(), synth.BF16)
    assert w.min() >= 0.5 and w.max() <= 1.5
    dy = synth.to_f64(small.dy(), synth.BF16)
    assert abs(dy.std() / 1e-2 - 1) < 0.01


def test_workload_table():
    names = set(synth.WORKLOADS)
    assert {"c1_f32_64x896", "c2_bf16_4096x4096", "c3_bf16_decode_1x896",
            "c4_bf16_residual_16384x4096", "c5a_bf16_262144x128", "c5b_bf16_8192x8192"} == names
    assert synth.WORKLOADS["c4_bf16_residual_16384x4096"].residual
    assert synth.WORKLOADS["c3_bf16_decode_1x896"].decode_splits == (4, 8, 16)
