"""Pins for the oracle's INT8 partials, dequantized output and bf16 fallback.

* partials: int64 brute force with numpy on tiny shapes, and closed-form
  extremes (128 * 127^2);
* dequantized output: the special case where every block's absmax is 127 on
  integer inputs (all scales exactly 1) reduces to a textbook integer GEMM;
  on random data the result must sit within the brute-force quantization
  error bound of the exact fp64 product of the original inputs, with block
  scales that differ strongly so that a transposed or mis-indexed scale fails;
* fallback: fp64 matmul of the bf16 inputs, rounded by torch on exactly
  representable sums, and the bf16 rounding bound otherwise.
"""
import numpy as np
import pytest
import torch

import oracle
from block_quantized_int8_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits, random_bf16


def _int_blocks(rng, rows, cols):
    """Integer values in [-126, 126] with one +-127 per 128x128 block."""
    a = rng.integers(-126, 127, size=(rows, cols)).astype(np.float32)
    for i in range(rows // 128):
        for j in range(cols // 128):
            a[i * 128 + rng.integers(128), j * 128 + rng.integers(128)] = rng.choice([-127.0, 127.0])
    return a


def _torch_bf16_bits(a_f32):
    return torch.from_numpy(np.ascontiguousarray(a_f32, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def test_partials_bruteforce():
    rng = np.random.default_rng(1)
    M, N, K = 160, 96, 384
    qx = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    qw = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    p = oracle.kblock_partials(qx, qw)
    ref = np.einsum("mbk,nbk->mnb", qx.astype(np.int64).reshape(M, K // 128, 128),
                    qw.astype(np.int64).reshape(N, K // 128, 128))
    assert p.shape == (M, N, K // 128)
    assert np.array_equal(p.astype(np.int64), ref)
    # window
    pw = oracle.kblock_partials(qx, qw, m0=32, mt=50, n0=7, nt=60)
    assert np.array_equal(pw, p[32:82, 7:67])


def test_partials_extremes():
    qx = np.full((128, 256), 127, np.int8)
    qw = np.full((128, 256), 127, np.int8)
    p = oracle.kblock_partials(qx, qw)
    assert np.all(p == 2064512)
    p = oracle.kblock_partials(qx, -qw)
    assert np.all(p == -2064512)


def test_unit_scale_reduces_to_integer_gemm():
    rng = np.random.default_rng(2)
    M, N, K = 256, 384, 512
    x = _int_blocks(rng, M, K)
    w = _int_blocks(rng, N, K)
    qx, sx = oracle.quantize_block(f32_to_bf16_bits(x))
    qw, sw = oracle.quantize_block(f32_to_bf16_bits(w))
    assert np.all(sx == 1.0) and np.all(sw == 1.0)
    assert np.array_equal(qx.astype(np.float32), x) and np.array_equal(qw.astype(np.float32), w)
    bias = (np.arange(N) % 200 - 100).astype(np.float32)   # |b| < 128: bf16-exact integers
    assert np.array_equal(bf16_bits_to_f32(f32_to_bf16_bits(bias)), bias)
    y = oracle.linear_int8(qx, sx, qw, sw, bias=f32_to_bf16_bits(bias))
    exact = x.astype(np.int64) @ w.astype(np.int64).T + bias.astype(np.int64)
    assert np.abs(exact).max() < 2 ** 24
    want = _torch_bf16_bits(exact.astype(np.float32))  # int -> fp32 exact, torch rounds to bf16
    assert np.array_equal(y, want)
    # row selection returns the same rows
    rows = np.array([0, 5, 255, 128], np.int64)
    assert np.array_equal(oracle.linear_int8(qx, sx, qw, sw, bias=f32_to_bf16_bits(bias), rows=rows),
                          want[rows])


@pytest.mark.parametrize("seed", [0, 1])
def test_error_bound_vs_exact_product(seed):
    rng = np.random.default_rng(seed)
    M, N, K = 256, 384, 640
    xf = rng.standard_normal((M, K), dtype=np.float32)
    wf = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    # make block scales differ by large, block-specific factors so that a
    # transposed or mis-indexed scale gives a large error
    fx = np.float32(2.0) ** rng.integers(-4, 5, size=(M // 128, K // 128)).astype(np.float32)
    fw = np.float32(2.0) ** rng.integers(-4, 5, size=(N // 128, K // 128)).astype(np.float32)
    xf *= np.kron(fx, np.ones((128, 128), np.float32)) * rng.uniform(0.5, 1.5, size=(M, 1)).astype(np.float32)
    wf *= np.kron(fw, np.ones((128, 128), np.float32))
    xb, wb = f32_to_bf16_bits(xf), f32_to_bf16_bits(wf)
    x, w = bf16_bits_to_f32(xb).astype(np.float64), bf16_bits_to_f32(wb).astype(np.float64)
    qx, sx = oracle.quantize_block(xb)
    qw, sw = oracle.quantize_block(wb)
    y, y64 = oracle.linear_int8(qx, sx, qw, sw, want_f64=True)
    exact = x @ w.T
    dx = np.kron(sx.astype(np.float64), np.ones((128, 128))) * (0.5 + 1e-5)
    dw = np.kron(sw.astype(np.float64), np.ones((128, 128))) * (0.5 + 1e-5)
    bound = np.abs(x) @ dw.T + dx @ np.abs(w).T + dx @ dw.T
    assert np.all(np.abs(y64 - exact) <= bound * (1 + 1e-9) + 1e-300)
    # bf16 rounding of the fp64 sum: within half an ulp (<= 2^-8 relative)
    yf = bf16_bits_to_f32(y).astype(np.float64)
    assert np.all(np.abs(yf - y64) <= 2.0 ** -8 * np.abs(y64) + 2.0 ** -134)
    # and the quantization error is far below the signal (sanity of the bound)
    assert np.linalg.norm(y64 - exact) / np.linalg.norm(exact) < 0.05


def test_output_rounded_once_from_the_full_sum():
    """Hand-worked: the K-block sum is rounded to bf16 once, not through fp32.

    K-block 0 has unit scales and partial 127*2 + 3*1 = 257; K-block 1 has
    combined scale 2^-10 * 2^-10 and partial 1, so Y = 257 + 2^-20 exactly.
    bf16 spacing in [256, 512) is 2: 257 is the midpoint of 256 (0x4380) and
    258 (0x4381), and Y lies just above it, so Y -> 258.  Through fp32 (ulp
    2^-15 there) Y would first become 257, a tie that goes to the even 256.
    Column 1 has the same partials with the weight code of K-block 1 negated:
    257 - 2^-20 -> 256 either way.
    """
    qx = np.zeros((128, 256), np.int8)
    qw = np.zeros((128, 256), np.int8)
    qx[0, 0], qw[0, 0] = 127, 2
    qx[0, 1], qw[0, 1] = 3, 1
    qx[0, 128], qw[0, 128] = 1, 1
    qw[1, 0], qw[1, 1], qw[1, 128] = 2, 1, -1
    sx = np.array([[1.0, 2.0 ** -10]], np.float32)
    sw = np.array([[1.0, 2.0 ** -10]], np.float32)
    y, y64 = oracle.linear_int8(qx, sx, qw, sw, rows=[0], want_f64=True)
    assert y64[0, 0] == 257 + 2.0 ** -20 and y64[0, 1] == 257 - 2.0 ** -20
    assert y[0, 0] == 0x4381 and y[0, 1] == 0x4380
    assert np.all(y[0, 2:] == 0)


def test_kblock_separability():
    # Y (fp64, before rounding) is the sum over K-blocks of the contributions
    # of each K-block alone: quantizing a matrix with all other K-blocks
    # zeroed leaves that K-block's codes and scales unchanged.
    x = random_bf16(3, (128, 384))
    w = random_bf16(4, (256, 384), 0.02)
    qx, sx = oracle.quantize_block(x)
    qw, sw = oracle.quantize_block(w)
    _, y64 = oracle.linear_int8(qx, sx, qw, sw, want_f64=True)
    total = np.zeros_like(y64)
    for kb in range(3):
        xs = np.zeros_like(x); xs[:, kb * 128:(kb + 1) * 128] = x[:, kb * 128:(kb + 1) * 128]
        ws = np.zeros_like(w); ws[:, kb * 128:(kb + 1) * 128] = w[:, kb * 128:(kb + 1) * 128]
        a, b = oracle.quantize_block(xs)
        c, d = oracle.quantize_block(ws)
        _, part = oracle.linear_int8(a, b, c, d, want_f64=True)
        total += part
    assert np.allclose(total, y64, rtol=1e-12, atol=1e-300)


def test_fallback_exact_small_integers():
    rng = np.random.default_rng(5)
    M, N, K = 37, 53, 71
    x = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    w = rng.integers(-8, 9, size=(N, K)).astype(np.float32)
    b = rng.integers(-8, 9, size=(N,)).astype(np.float32)
    y = oracle.linear_bf16(f32_to_bf16_bits(x), oracle.DTYPE_BF16, f32_to_bf16_bits(w),
                           bias=f32_to_bf16_bits(b))
    exact = (x.astype(np.int64) @ w.astype(np.int64).T + b.astype(np.int64)).astype(np.float32)
    assert np.array_equal(y, _torch_bf16_bits(exact))


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_fallback_vs_fp64_matmul(dtype):
    rng = np.random.default_rng(6)
    M, N, K = 45, 70, 131
    xf = rng.standard_normal((M, K), dtype=np.float32)
    wb = random_bf16(8, (N, K), 0.02)
    if dtype == "bf16":
        xin, code = f32_to_bf16_bits(xf), oracle.DTYPE_BF16
    elif dtype == "fp16":
        xin, code = xf.astype(np.float16).view(np.uint16), oracle.DTYPE_FP16
    else:
        xin, code = xf, oracle.DTYPE_FP32
    # the input rounded to bf16 by torch (nearest even), independent of the oracle
    src = torch.from_numpy(xin.view(np.float16)) if dtype == "fp16" else \
        (torch.from_numpy(xf) if dtype == "fp32" else None)
    if src is None:
        xb = bf16_bits_to_f32(xin)
    else:
        xb = src.float().to(torch.bfloat16).float().numpy()
    ref = xb.astype(np.float64) @ bf16_bits_to_f32(wb).astype(np.float64).T
    y = bf16_bits_to_f32(oracle.linear_bf16(xin, code, wb)).astype(np.float64)
    assert np.all(np.abs(y - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)
    rows = np.array([44, 0, 17], np.int64)
    y2 = bf16_bits_to_f32(oracle.linear_bf16(xin, code, wb, rows=rows)).astype(np.float64)
    assert np.array_equal(y2, y[rows])
