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

