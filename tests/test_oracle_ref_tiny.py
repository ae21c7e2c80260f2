"""The C oracle against the independent numpy oracle (oracle/ref_tiny.py).

Two implementations written separately from the same definitions must agree
bit for bit on small seeded inputs: codes, scales, int32 partials, and the
bf16 outputs of the block-scaled product, the fallback and the post-scale
form, plus INT8 attention Q/K and the guard.  Inputs carry block-to-block
scale variation, an all-zero block and a block of tiny values, so that a
transposed or shifted scale index, a skipped zero case or a lost subnormal
on either side shows up.
"""
import numpy as np
import pytest

import oracle
from oracle import ref_tiny
from block_quantized_int8_amd.workloads import f32_to_bf16_bits, random_bf16


def varied_matrix(seed: int, rows: int, cols: int, scale: float = 1.0) -> np.ndarray:
    """N(0, scale^2) with every 128x128 block multiplied by its own power of
    two, block (0, 1) all zero and block (last, 0) scaled down to ~2^-128."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(scale)
    for i in range(rows // 128):
        for j in range(cols // 128):
            x[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128] *= np.float32(2.0 ** ((3 * i + 5 * j) % 7 - 3))
    if cols >= 256:
        x[0:128, 128:256] = 0
    if rows >= 256:
        x[rows - 128:rows, 0:128] *= np.float32(2.0 ** -126)
    return f32_to_bf16_bits(x)


@pytest.fixture(scope="module")
def operands():
    x = varied_matrix(101, 256, 384)
    w = varied_matrix(102, 256, 384, 0.02)
    b = random_bf16(103, (256,), 0.1)
    return x, w, b


def test_block_quantization_agrees(operands):
    x, w, _ = operands
    for m in (x, w):
        q1, s1 = oracle.quantize_block(m)
        q2, s2 = ref_tiny.quantize_block(m)
        assert np.array_equal(q1, q2)
        assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    # the fixture really has a zero block and a subnormal-range scale
    _, s = ref_tiny.quantize_block(x)
    assert s[0, 1] == 0 and 0 < s[1, 0] < np.float32(2.0 ** -120)


def test_partials_and_outputs_agree(operands):
    x, w, b = operands
    qx, sx = oracle.quantize_block(x)
    qw, sw = oracle.quantize_block(w)
    assert np.array_equal(oracle.kblock_partials(qx, qw), ref_tiny.kblock_partials(qx, qw))
    for bias in (None, b):
        assert np.array_equal(oracle.linear_int8(qx, sx, qw, sw, bias=bias),
                              ref_tiny.linear_int8(qx, sx, qw, sw, bias=bias))


def test_fallback_agrees(operands):
    x, w, b = operands
    xs, ws = x[:77, :130], w[:45, :130]      # odd shapes, as the guard sends them
    assert np.array_equal(oracle.linear_bf16(xs, oracle.DTYPE_BF16, ws, bias=b[:45]),
                          ref_tiny.linear_bf16(xs, ws, bias=b[:45]))


def test_postscale_agrees(operands):
    x, w, b = operands
    qx1, sx1 = oracle.quantize_rows(x)
    qx2, sx2 = ref_tiny.quantize_rows(x)
    assert np.array_equal(qx1, qx2) and np.array_equal(sx1.view(np.uint32), sx2.view(np.uint32))
    qw, sw = oracle.quantize_rows(w)
    for bias in (None, b):
        assert np.array_equal(oracle.linear_postscale(qx1, sx1, qw, sw, bias=bias),
                              ref_tiny.linear_postscale(qx1, sx1, qw, sw, bias=bias))


def test_qk_agrees():
    B, L, H, D = 2, 200, 3, 64
    ld = H * D + 16                           # padded rows, as a column slice of a wider output
    x = random_bf16(104, (B * L, ld))
    q1, s1 = oracle.quantize_qk(x, B, L, H, D, ld)
    q2, s2 = ref_tiny.quantize_qk(x, B, L, H, D, ld)
    assert np.array_equal(q1, q2) and np.array_equal(s1.view(np.uint32), s2.view(np.uint32))


def test_route_agrees():
    for dt in (oracle.DTYPE_BF16, oracle.DTYPE_FP16, oracle.DTYPE_FP32):
        for M in (1, 127, 128, 256, 4000, 4096):
            for K in (64, 128, 130, 4096):
                for N in (45, 128, 384):
                    for hq in (0, 1):
                        assert oracle.route(dt, M, K, N, hq) == \
                            ref_tiny.route(dt == oracle.DTYPE_BF16, M, K, N, bool(hq)), (dt, M, K, N, hq)


def test_bf16_rounding_agrees():
    rng = np.random.default_rng(105)
    vals = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 38, 3000),
                           [2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, -(1 + 2.0 ** -8), 1 + 3 * 2.0 ** -9]])
    for v in vals:
        assert oracle.f64_to_bf16(float(v)) == ref_tiny.f64_to_bf16_bits(float(v)), v
