"""Pins for the oracle's bf16/fp16 conversions and the guard.

bf16 rounding is checked against hand-worked cases (tests/golden) and against
torch's fp32 -> bf16 conversion (a library routine, round to nearest even) on
values that fp32 holds exactly; fp16 decoding against numpy's float16.
"""
import numpy as np
import torch

import oracle
from conftest import load_golden


def test_bf16_golden():
    g = load_golden("bf16_rounding.json")
    for v, want in g["cases"]:
        assert oracle.f64_to_bf16(float.fromhex(v)) == int(want, 16), (v, want)


def test_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    # add specials: subnormals, near max, ties
    extra = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 2 ** -130, -2 ** -140, 3.3e38, -0.0, 0.0,
                      2 ** -126 * (1 - 2 ** -9)], np.float32)
    vals = np.concatenate([vals, extra])
    want = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f64_to_bf16(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, want)


def test_fp16_decode_all_values():
    h = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16_to_f64(int(v)) for v in h])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def test_route_golden():
    g = load_golden("route_cases.json")
    for dt, M, K, N, hq, want, note in g["cases"]:
        assert oracle.route(dt, M, K, N, hq) == want, note


def test_gelu_reference_points():
    import math
    xs = np.array([0.0, 1.0, -1.0, 3.0, -3.0, 0.5, -10.0, 10.0], np.float32)
    from block_quantized_int8_amd.workloads import f32_to_bf16_bits, bf16_bits_to_f32
    y = bf16_bits_to_f32(oracle.gelu_bf16(f32_to_bf16_bits(xs)))
    ref = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in xs.astype(float)])
    assert y[0] == 0.0 and y[-1] == 10.0 and y[-2] == 0.0
    assert np.all(np.abs(y - ref) <= 2 ** -8 * np.abs(ref) + 1e-30)
