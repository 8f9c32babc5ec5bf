"""Seeded input generators: reproducibility, shapes, bf16 rounding, workload structure."""
import numpy as np
import pytest

from efficient_long_sequence_lsh_amd import workloads as W


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e38, 1e-40, 0.0, -0.0], np.float32)
    bits = W.f32_to_bf16_bits(vals)
    back = W.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is exactly halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert back[1] == 1.0
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6: even is 1 + 2^-6
    assert back[2] == np.float32(1.015625)
    assert back[3] == -2.5 and back[6] == 0.0
    assert np.signbit(back[7])
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    err = np.abs(W.bf16_bits_to_f32(W.f32_to_bf16_bits(x)) - x) / np.abs(x)
    assert err.max() <= 2.0 ** -8   # half an ulp at 8 significant bits


def test_generation_is_reproducible_and_shaped():
    a = W.make_inputs("small_4k_bf16", seq_len=256)
    b = W.make_inputs("small_4k_bf16", seq_len=256)
    assert np.array_equal(a.qk_bits, b.qk_bits) and np.array_equal(a.v_bits, b.v_bits)
    assert a.qk.shape == (2, 4, 256, 64) and a.rotations.shape == (2, 64, 32)
    assert a.qk.dtype == np.float32 and a.qk_bits.dtype == np.uint16
    assert np.array_equal(W.bf16_bits_to_f32(a.qk_bits), a.qk)
    f = W.make_inputs("tiny_1k_full")
    assert f.rotations.shape == (1, 64, 0)


def test_mixture_workload_is_clustered():
    inp = W.make_inputs("text_64k", seq_len=4096)
    x = inp.qk[0, 0].astype(np.float64)
    norms = np.linalg.norm(x, axis=1)
    # centre of norm 3 plus noise of expected norm 1: norms concentrate near sqrt(10)
    assert 2.5 < np.median(norms) < 3.7
    # many pairs share a centre: cosine similarity close to 1 for a visible fraction of pairs
    xn = x[:512] / norms[:512, None]
    cos = xn @ xn.T
    assert (cos > 0.85).mean() > 1.0 / 256


def test_ar1_workload_is_smooth_along_position():
    inp = W.make_inputs("image_12k", seq_len=2048)
    x = inp.qk[0, 0].astype(np.float64)
    c = np.corrcoef(x[1:, 0], x[:-1, 0])[0, 1]
    assert 0.85 < c < 0.95
    assert x.var() == pytest.approx(1 / (1 - 0.81), rel=0.25)
