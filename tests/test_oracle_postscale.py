"""Pins for the oracle's post-scale W8A8 variant (row-wise scales with the
1e-4 floor, INT32 over all of K, scales and bias once in the epilogue)."""
import numpy as np
import pytest
import torch

import oracle
from block_quantized_int8_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits, random_bf16
from conftest import load_golden


def test_rows_golden():
    g = load_golden("quantize_rows_examples.json")
    x = np.zeros((len(g["rows"]), 256), np.float32)
    rng = np.random.default_rng(3)
    pos = []
    for i, row in enumerate(g["rows"]):
        p = rng.choice(256, len(row["values"]), replace=False)
        x[i, p] = [v for v, _ in row["values"]]
        pos.append(p)
    xb = f32_to_bf16_bits(x)
    assert np.array_equal(bf16_bits_to_f32(xb), x)
    q, s = oracle.quantize_rows(xb)
    for i, row in enumerate(g["rows"]):
        assert int(s.view(np.uint32)[i]) == int(row["s_bits"], 16), i
        assert q[i, pos[i]].tolist() == [c for _, c in row["values"]], i
        assert not np.delete(q[i], pos[i]).any()


def test_rows_invariants():
    x = random_bf16(21, (64, 384), 2.0)
    q, s = oracle.quantize_rows(x)
    xf = bf16_bits_to_f32(x)
    a = np.abs(xf).max(axis=1)
    assert np.array_equal(s, a / np.float32(127))  # no row is below the floor here
    hit = np.abs(xf) == a[:, None]
    assert np.all(np.abs(q[hit]) == 127)
    err = np.abs(q.astype(np.float64) * s[:, None] - xf.astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 1e-5))
    qn, sn = oracle.quantize_rows(x ^ np.uint16(0x8000))
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    # rows are independent
    y = x.copy()
    y[7] = random_bf16(22, (384,), 100.0)
    q2, s2 = oracle.quantize_rows(y)
    keep = np.arange(64) != 7
    assert np.array_equal(q2[keep], q[keep]) and np.array_equal(s2[keep], s[keep])


def test_postscale_unit_scales_integer_gemm():
    rng = np.random.default_rng(23)
    M, N, K = 96, 80, 384
    x = rng.integers(-126, 127, size=(M, K)).astype(np.float32)
    w = rng.integers(-126, 127, size=(N, K)).astype(np.float32)
    x[np.arange(M), rng.integers(0, K, M)] = 127.0
    w[np.arange(N), rng.integers(0, K, N)] = -127.0
    qx, sx = oracle.quantize_rows(f32_to_bf16_bits(x))
    qw, sw = oracle.quantize_rows(f32_to_bf16_bits(w))
    assert np.all(sx == 1) and np.all(sw == 1)
    b = (np.arange(N) % 50 - 25).astype(np.float32)
    y = oracle.linear_postscale(qx, sx, qw, sw, bias=f32_to_bf16_bits(b))
    exact = (x.astype(np.int64) @ w.astype(np.int64).T + b.astype(np.int64)).astype(np.float32)
    want = torch.from_numpy(exact).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y, want)


def test_postscale_error_bound():
    rng = np.random.default_rng(24)
    M, N, K = 128, 96, 512
    xf = rng.standard_normal((M, K), dtype=np.float32) * (np.float32(2.0) ** rng.integers(-6, 6, (M, 1)).astype(np.float32))
    wf = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02) * (np.float32(2.0) ** rng.integers(-6, 6, (N, 1)).astype(np.float32))
    xb, wb = f32_to_bf16_bits(xf), f32_to_bf16_bits(wf)
    x, w = bf16_bits_to_f32(xb).astype(np.float64), bf16_bits_to_f32(wb).astype(np.float64)
    qx, sx = oracle.quantize_rows(xb)
    qw, sw = oracle.quantize_rows(wb)
    y = bf16_bits_to_f32(oracle.linear_postscale(qx, sx, qw, sw)).astype(np.float64)
    exact = x @ w.T
    dx = sx.astype(np.float64)[:, None] * (0.5 + 1e-5)
    dw = sw.astype(np.float64)[:, None] * (0.5 + 1e-5)
    bound = (np.abs(x).sum(1)[:, None] * dw.T + dx * np.abs(w).sum(1)[None, :] + K * dx * dw.T)
    assert np.all(np.abs(y - exact) <= bound + 2.0 ** -8 * np.abs(exact) + 1e-30)
    rows = np.array([5, 0, 127])
    assert np.array_equal(oracle.linear_postscale(qx, sx, qw, sw, rows=rows),
                          oracle.linear_postscale(qx, sx, qw, sw)[rows])
