"""Pins for the oracle's modulated RMS normalization (the producer in front
of a transformer block's linears; TurboT2VA paper, architecture-aware
inference stack, fused-kernels paragraph).

Hand-worked rows (tests/golden/rmsnorm_modulate_examples.json: exact
intermediates, bf16 ties, eps, the zero row), invariants that hold exactly
(power-of-two scaling of a row, sign symmetry, row locality, the batch entry
each row takes its modulation from), the unit mean square of an unmodulated
row, and agreement with the independent numpy oracle.
"""
import numpy as np
import pytest

import oracle
from oracle import ref_tiny
from conftest import load_golden
from block_quantized_int8_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits, random_bf16


def hx(v):
    return np.array([int(s, 16) for s in v], np.uint16)


def test_golden_rows():
    for c in load_golden("rmsnorm_modulate_examples.json")["cases"]:
        y = oracle.rmsnorm_modulate(hx(c["x"])[None, :], 1, hx(c["scale"])[None, :], hx(c["shift"])[None, :], c["eps"])
        assert np.array_equal(y[0], hx(c["y"])), c["note"]


def _mod(seed, B, K):
    return random_bf16(seed, (B, K), 0.2), random_bf16(seed + 1, (B, K), 0.2)


def test_power_of_two_scaling_is_exact():
    # with eps far below S/K, scaling a row by 2^j scales S by 4^j, the root by
    # 2^j and r by 2^-j exactly, so x * r and everything after it is unchanged
    x = random_bf16(11, (16, 256))
    sc, sh = _mod(12, 1, 256)
    y = oracle.rmsnorm_modulate(x, 16, sc, sh, 1e-30)
    xf = bf16_bits_to_f32(x)
    for j in (-7, -1, 1, 5):
        xs = f32_to_bf16_bits(xf * np.float32(2.0 ** j))
        assert np.array_equal(oracle.rmsnorm_modulate(xs, 16, sc, sh, 1e-30), y), j


def test_sign_symmetry_without_shift():
    x = random_bf16(13, (8, 384))
    sc, _ = _mod(14, 1, 384)
    zero = np.zeros((1, 384), np.uint16)
    y = oracle.rmsnorm_modulate(x, 8, sc, zero, 1e-6)
    yn = oracle.rmsnorm_modulate(x ^ np.uint16(0x8000), 8, sc, zero, 1e-6)
    assert np.array_equal(yn, y ^ np.uint16(0x8000))


def test_unmodulated_rows_have_unit_mean_square():
    # scale 0, shift 0, eps tiny: mean(y^2) = 1 up to the bf16 rounding of y
    x = random_bf16(15, (32, 1024), 3.0)
    zero = np.zeros((1, 1024), np.uint16)
    y = bf16_bits_to_f32(oracle.rmsnorm_modulate(x, 32, zero, zero, 1e-12)).astype(np.float64)
    ms = np.mean(y * y, axis=1)
    assert np.all(np.abs(ms - 1.0) < 2.0 ** -8), ms


def test_rows_are_independent_and_take_their_batch_modulation():
    B, L, K = 3, 5, 128
    x = random_bf16(16, (B * L, K))
    sc, sh = _mod(17, B, K)
    y, r = oracle.rmsnorm_modulate(x, L, sc, sh, 1e-6, want_r=True)
    for b in range(B):
        rows = slice(b * L, (b + 1) * L)
        yb, rb = oracle.rmsnorm_modulate(x[rows], L, sc[b:b + 1], sh[b:b + 1], 1e-6, want_r=True)
        assert np.array_equal(y[rows], yb) and np.array_equal(r[rows], rb)
    # changing one row changes no other row
    x2 = x.copy()
    x2[7] = random_bf16(18, (K,), 5.0)
    y2 = oracle.rmsnorm_modulate(x2, L, sc, sh, 1e-6)
    keep = np.arange(B * L) != 7
    assert np.array_equal(y2[keep], y[keep]) and not np.array_equal(y2[7], y[7])


def test_agrees_with_independent_oracle():
    B, L, K = 2, 3, 256
    x = random_bf16(19, (B * L, K), 2.0)
    sc, sh = _mod(20, B, K)
    for eps in (1e-6, 0.5):
        assert np.array_equal(oracle.rmsnorm_modulate(x, L, sc, sh, eps), ref_tiny.rmsnorm_modulate(x, L, sc, sh, eps))


def test_fused_result_is_the_block_quantization_of_the_bf16_output():
    B, L, K = 2, 128, 256
    x = random_bf16(21, (B * L, K))
    sc, sh = _mod(22, B, K)
    q, s = oracle.rmsnorm_modulate_quantize_block(x, L, sc, sh, 1e-6)
    q2, s2 = oracle.quantize_block(oracle.rmsnorm_modulate(x, L, sc, sh, 1e-6))
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_argument_errors():
    x = random_bf16(23, (4, 8))
    sc, sh = _mod(24, 2, 8)
    with pytest.raises(ValueError):
        oracle.rmsnorm_modulate(x, 3, sc, sh)             # rows not a multiple of L
    with pytest.raises(ValueError):
        oracle.rmsnorm_modulate(x, 2, sc, sh, 0.0)        # eps must be positive
