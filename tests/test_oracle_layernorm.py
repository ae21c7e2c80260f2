"""Pins for the oracle's modulated layer normalization (the LayerNorm form
of the producer in front of a transformer block's linears; TurboT2VA paper,
architecture-aware inference stack, fused-kernels paragraph).

Hand-worked rows (tests/golden/layernorm_modulate_examples.json: the mean
subtracted, eps, an off-centre row, bf16 ties, the zero row, the batch entry
each row takes its modulation from), exact invariants (a shift of every
value by a constant, power-of-two scaling), rows of zero mean reducing to
the RMS normalization bit for bit, the unit variance of an unmodulated row,
and agreement with the independent numpy oracle.
"""
import numpy as np

import oracle
from oracle import ref_tiny
from conftest import load_golden
from block_quantized_int8_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits, random_bf16


def hx(v):
    return np.array([int(s, 16) for s in v], np.uint16)


def test_golden_rows():
    for c in load_golden("layernorm_modulate_examples.json")["cases"]:
        B, L, K = c["B"], c["L"], c["K"]
        x = hx(c["x"]).reshape(B * L, K)
        sc, sh = hx(c["scale"]).reshape(B, K), hx(c["shift"]).reshape(B, K)
        want = hx(c["y"]).reshape(B * L, K)
        assert np.array_equal(oracle.layernorm_modulate(x, L, sc, sh, c["eps"]), want), c["note"]
        assert np.array_equal(ref_tiny.layernorm_modulate(x, L, sc, sh, c["eps"]), want), c["note"]


def _mod(seed, B, K):
    return random_bf16(seed, (B, K), 0.2), random_bf16(seed + 1, (B, K), 0.2)


def test_constant_shift_of_the_row_is_exact():
    # integer values |x| <= 64 and K = 256: the mean is exact in fp32, the
    # deviations and their squares exact in fp64, so adding 64 to every value
    # (still exact in bf16) changes nothing downstream
    rng = np.random.default_rng(70)
    K = 256
    xi = rng.integers(-64, 65, (12, K)).astype(np.float32)
    sc, sh = _mod(71, 1, K)
    y = oracle.layernorm_modulate(f32_to_bf16_bits(xi), 12, sc, sh, 1e-6)
    ys = oracle.layernorm_modulate(f32_to_bf16_bits(xi + np.float32(64.0)), 12, sc, sh, 1e-6)
    assert np.array_equal(y, ys)


def test_power_of_two_scaling_is_exact():
    x = random_bf16(72, (16, 256))
    sc, sh = _mod(73, 1, 256)
    y = oracle.layernorm_modulate(x, 16, sc, sh, 1e-30)
    xf = bf16_bits_to_f32(x)
    for j in (-6, -1, 1, 4):
        xs = f32_to_bf16_bits(xf * np.float32(2.0 ** j))
        assert np.array_equal(oracle.layernorm_modulate(xs, 16, sc, sh, 1e-30), y), j


def test_zero_mean_rows_equal_the_rms_normalization():
    # rows made of +-v pairs have an exactly zero sum: the mean is 0 and the
    # variance is the mean square, so both normalizations agree bit for bit
    half = random_bf16(74, (8, 128), 2.0)
    x = np.concatenate([half, half ^ np.uint16(0x8000)], axis=1)
    sc, sh = _mod(75, 2, 256)
    y, st = oracle.layernorm_modulate(x, 4, sc, sh, 1e-6, want_stats=True)
    yr, r = oracle.rmsnorm_modulate(x, 4, sc, sh, 1e-6, want_r=True)
    assert np.all(st[:, 0] == 0) and np.array_equal(st[:, 1], r)
    assert np.array_equal(y, yr)


def test_unmodulated_rows_have_zero_mean_and_unit_variance():
    x = random_bf16(76, (32, 1024), 3.0)
    x = f32_to_bf16_bits(bf16_bits_to_f32(x) + np.float32(5.0))   # off-centre rows
    zero = np.zeros((1, 1024), np.uint16)
    y = bf16_bits_to_f32(oracle.layernorm_modulate(x, 32, zero, zero, 1e-12)).astype(np.float64)
    assert np.all(np.abs(y.mean(axis=1)) < 1e-2)
    assert np.all(np.abs(y.var(axis=1) - 1.0) < 1e-2)


def test_matches_ref_tiny():
    for B, L, K, seed in [(1, 3, 8, 80), (2, 4, 40, 81), (3, 2, 128, 82)]:
        x = random_bf16(seed, (B * L, K), 3.0)
        x[0] = f32_to_bf16_bits(bf16_bits_to_f32(x[0]) + np.float32(7.0))
        sc, sh = _mod(seed + 1, B, K)
        for eps in (1e-6, 0.5):
            assert np.array_equal(oracle.layernorm_modulate(x, L, sc, sh, eps),
                                  ref_tiny.layernorm_modulate(x, L, sc, sh, eps)), (B, L, K, eps)
