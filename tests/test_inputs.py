"""Seeded input generator: reproducibility and the storage roundings."""

import hashlib

import numpy as np

from dense_gemm_transformer_amd import inputs


def test_reproducible():
    a = inputs.normal(1234, (64, 33), 0.02, "bf16")
    b = inputs.normal(1234, (64, 33), 0.02, "bf16")
    assert a.dtype == np.uint16 and np.array_equal(a, b)
    assert not np.array_equal(a, inputs.normal(1235, (64, 33), 0.02, "bf16"))
    h = hashlib.sha256(inputs.uniform(7, (16, 16), -1, 1, "f16").tobytes()).hexdigest()
    assert h == hashlib.sha256(inputs.uniform(7, (16, 16), -1, 1, "f16").tobytes()).hexdigest()


def test_bf16_round_nearest_even():
    # 1 + 2^-8 is exactly halfway between bf16 neighbours 1 and 1 + 2^-7: ties to even -> 1
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even) -> 1 + 2^-6
    vals = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -(1 + 2 ** -8)], np.float32)
    got = inputs.widen(inputs.f32_to_bf16_bits(vals), "bf16")
    assert list(got) == [1.0, 1 + 2 ** -6, 1 + 2 ** -7, -1.0]
    assert inputs.f32_to_bf16_bits(np.array([np.inf, -np.inf], np.float32)).tolist() == [0x7F80, 0xFF80]
    nan = inputs.f32_to_bf16_bits(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


def test_f16_storage_is_double_rounded_through_f32():
    v = np.array([0.1, 1 / 3, 65519.0, 1e-7])
    s = inputs.store(v, "f16")
    assert s.dtype == np.float16
    assert np.array_equal(s, v.astype(np.float32).astype(np.float16))


def test_workload_shapes():
    c = inputs.workload_fp16_narrow()
    assert c.X.shape == (16, 4096) and c.W.shape == (4096, 4096) and c.b is None
    assert np.max(np.abs(c.W.astype(np.float64))) <= 0.05
    layer = inputs.workload_gpt2_layer(M=128)
    assert [(l.M, l.N, l.K, l.gelu) for l in layer] == [
        (128, 2304, 768, False), (128, 768, 768, False), (128, 3072, 768, True), (128, 768, 3072, False)]
    sq = inputs.workload_square(n=64, dtype="bf16")
    assert sq.layout == "KN" and sq.out_dtype == "f32" and sq.W.dtype == np.uint16
    w = inputs.workload_fp32_linear_128x768().W.astype(np.float64)
    assert 0.015 < w.std() < 0.025


def test_periodic_normal_repeats_one_prime_block():
    """The multi-GiB generator repeats one seeded block with prime sides, seeded like ``normal``."""
    a = inputs.periodic_normal(9, (2500, 3000), 0.05, "bf16")
    b = inputs.normal(9, (1021, 1031), 0.05, "bf16")
    assert a.shape == (2500, 3000) and a.dtype == b.dtype and a.flags.c_contiguous
    for i, j in [(0, 0), (1020, 1030), (1021, 1031), (2499, 2999), (2042 + 5, 7)]:
        assert a[i, j] == b[i % 1021, j % 1031]
    small = inputs.periodic_normal(9, (10, 20), 1.0, "f32")  # smaller than a block: one draw of that shape
    assert np.array_equal(small, inputs.normal(9, (10, 20), 1.0, "f32"))
    c = inputs.large_case(3, 64, 96, 128, "f16", "f32", "KN")
    assert c.X.shape == (64, 128) and c.W.shape == (128, 96) and c.b is None and c.out_dtype == "f32"
