"""Pins for the oracle's gated residual update (the consumer of a linear's
output in a transformer block; TurboT2VA paper, architecture-aware inference
stack, fused-kernels paragraph).

Hand-worked cases (tests/golden/gated_residual_examples.json: exact sums,
bf16 ties, signed zeros, cancellation, the batch entry each row takes its
gate from, spacing at a large residual, a sum whose fp32 rounding lands on a
bf16 tie), the exact rational h + g*o rounded to fp32 and then to bf16 on
random triples over a wide exponent range, the special gates 0 and 1, sign
symmetry, and the numpy twin.
"""
import math
from fractions import Fraction

import numpy as np

import oracle
from oracle import ref_tiny
from conftest import load_golden
from block_quantized_int8_amd.workloads import bf16_bits_to_f32, random_bf16


def hx(v):
    return np.array([int(s, 16) for s in v], np.uint16)


def test_golden_cases():
    for c in load_golden("gated_residual_examples.json")["cases"]:
        B, L, N = c["B"], c["L"], c["N"]
        h, o = hx(c["h"]).reshape(B * L, N), hx(c["o"]).reshape(B * L, N)
        g, want = hx(c["gate"]).reshape(B, N), hx(c["y"]).reshape(B * L, N)
        assert np.array_equal(oracle.gated_residual(h, o, g, L), want), c["note"]
        assert np.array_equal(ref_tiny.gated_residual(h, o, g, L), want), c["note"]


def _bits_to_fraction(b):
    v = float(bf16_bits_to_f32(np.array([b], np.uint16))[0])
    return Fraction(v)


def _round(v: Fraction, bits: int) -> Fraction:
    """Nearest (ties to even) rational with `bits` significant bits, exponent
    floor at the fp32 normal range (so subnormal spacing below 2^-126)."""
    if v == 0:
        return v
    a = abs(v)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (max(e, -126) - bits + 1)
    q = a / ulp
    f = math.floor(q)
    d = q - f
    if d > Fraction(1, 2) or (d == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return (f * ulp) if v > 0 else -(f * ulp)


def _bf16_of(v: Fraction) -> int:
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    return sign | int(np.array([float(abs(v))], np.float32).view(np.uint32)[0] >> 16)


def _wide_bf16(rng, n):
    # sign, exponent over 2^-40 .. 2^40, any mantissa
    e = rng.integers(127 - 40, 127 + 40, n).astype(np.uint16)
    m = rng.integers(0, 128, n).astype(np.uint16)
    s = rng.integers(0, 2, n).astype(np.uint16)
    return (s << 15) | (e << 7) | m


def test_is_the_exact_value_rounded_to_fp32_then_bf16():
    # the product of two bf16 is exact in fp32, so the oracle's steps amount to
    # rounding the exact rational h + g*o to fp32 and that to bf16 (which is
    # not always the exact value rounded once: see the golden case with a
    # bf16 tie)
    rng = np.random.default_rng(40)
    n = 4000
    h, o, g = _wide_bf16(rng, n), _wide_bf16(rng, n), _wide_bf16(rng, n)
    # push a quarter of the products next to h, where rounding and cancellation bite
    k = n // 4
    o[:k] = h[:k]
    g[:k] = (g[:k] & 0x807F) | 0x3F80  # gate in +-[1, 2)
    y = oracle.gated_residual(h[:, None], o[:, None], g[:, None], 1)[:, 0]
    for i in range(n):
        exact = _bits_to_fraction(h[i]) + _bits_to_fraction(g[i]) * _bits_to_fraction(o[i])
        assert int(y[i]) == _bf16_of(_round(_round(exact, 24), 8)), (hex(h[i]), hex(g[i]), hex(o[i]))


def test_special_gates_and_sign_symmetry():
    B, L, N = 3, 5, 64
    h = random_bf16(41, (B * L, N), 4.0)
    o = random_bf16(42, (B * L, N), 4.0)
    g = random_bf16(43, (B, N), 0.5)
    h[(h & 0x7FFF) == 0] = 0x3F80
    o[(o & 0x7FFF) == 0] = 0x3F80
    zero = np.zeros((B, N), np.uint16)
    one = np.full((B, N), 0x3F80, np.uint16)
    assert np.array_equal(oracle.gated_residual(h, o, zero, L), h)
    assert np.array_equal(oracle.gated_residual(np.zeros_like(h), o, one, L), o)
    y = oracle.gated_residual(h, o, g, L)
    neg = np.uint16(0x8000)
    yn = oracle.gated_residual(h ^ neg, o ^ neg, g, L)
    nz = (y & 0x7FFF) != 0
    assert np.array_equal(yn[nz], y[nz] ^ neg)
    # the sign may sit on the gate or on the output
    assert np.array_equal(oracle.gated_residual(h, o ^ neg, g ^ neg, L), y)


def test_matches_ref_tiny():
    for B, L, N, seed in [(1, 3, 8, 50), (2, 4, 33, 51), (3, 2, 128, 52)]:
        h = random_bf16(seed, (B * L, N), 3.0)
        o = random_bf16(seed + 1, (B * L, N), 3.0)
        g = random_bf16(seed + 2, (B, N), 1.0)
        assert np.array_equal(oracle.gated_residual(h, o, g, L), ref_tiny.gated_residual(h, o, g, L))
