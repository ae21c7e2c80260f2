"""GPU INT8 GEMM vs the oracle: per-K-block int32 partials bit-exact,
dequantized bf16 output within tolerance."""
import numpy as np
import pytest
import torch

import block_quantized_int8_amd as w8a8
import oracle
from block_quantized_int8_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits, random_bf16, single_linear_256
from parity import assert_bf16_close, bf16_bits, to_dev_bf16

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_partials_single_linear_256_full():
    d = single_linear_256()
    qx, sx = oracle.quantize_block(d["x"])
    qw, sw = oracle.quantize_block(d["w"])
    p = w8a8.debug_kblock_partials(_dev(qx), _dev(qw), 0, 256, 0, 256)
    torch.cuda.synchronize()
    assert np.array_equal(p.cpu().numpy(), oracle.kblock_partials(qx, qw))


@pytest.mark.parametrize("M,N,K,win", [(384, 256, 640, (128, 256, 0, 256)),
                                       (256, 512, 384, (0, 256, 384, 128)),
                                       (128, 128, 128, (0, 128, 0, 128))])
def test_partials_windows(M, N, K, win):
    rng = np.random.default_rng(M + N + K)
    qx = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    qw = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    m0, mt, n0, nt = win
    p = w8a8.debug_kblock_partials(_dev(qx), _dev(qw), m0, mt, n0, nt)
    torch.cuda.synchronize()
    assert np.array_equal(p.cpu().numpy(), oracle.kblock_partials(qx, qw, m0, mt, n0, nt))


def test_partials_extremes():
    qx = np.full((128, 256), 127, np.int8)
    qw = np.full((128, 256), -127, np.int8)
    qw[:, 128:] = 127
    p = w8a8.debug_kblock_partials(_dev(qx), _dev(qw), 0, 128, 0, 128).cpu().numpy()
    assert np.all(p[:, :, 0] == -2064512) and np.all(p[:, :, 1] == 2064512)


def _gemm_case(M, N, K, seed, bias=False):
    x = random_bf16(seed, (M, K))
    w = random_bf16(seed + 1, (N, K), 0.02)
    b = random_bf16(seed + 2, (N,), 0.5) if bias else None
    qx, sx = oracle.quantize_block(x)
    qw, sw = oracle.quantize_block(w)
    y = w8a8.gemm_blockscale(_dev(qx), _dev(sx), _dev(qw), _dev(sw),
                             bias=None if b is None else to_dev_bf16(b))
    torch.cuda.synchronize()
    yo = oracle.linear_int8(qx, sx, qw, sw, bias=b)
    return assert_bf16_close(bf16_bits(y), yo, f"gemm {M}x{N}x{K}")


# K = 128: a single K-block, so every sub-tile's dequantization is the one
# carried out of the main loop (the degenerate case of the pipeline)
@pytest.mark.parametrize("M,N,K,bias", [(256, 256, 256, False), (384, 640, 512, True),
                                        (1024, 256, 1024, False), (128, 1152, 384, True),
                                        (128, 128, 128, False), (384, 384, 128, True)])
def test_gemm_vs_oracle(M, N, K, bias):
    _gemm_case(M, N, K, M * 7 + N, bias)


def test_gemm_zero_rows():
    # an all-zero activation block row gives exactly-zero output rows
    x = random_bf16(9, (256, 256))
    x[128:] = 0
    w = random_bf16(10, (256, 256), 0.02)
    qx, sx = oracle.quantize_block(x)
    qw, sw = oracle.quantize_block(w)
    y = bf16_bits(w8a8.gemm_blockscale(_dev(qx), _dev(sx), _dev(qw), _dev(sw)))
    assert not y[128:].any()
    assert_bf16_close(y, oracle.linear_int8(qx, sx, qw, sw), "zero rows")


def test_block_gemm_long_k_scale_reload():
    # K = 65536: 512 K-blocks, the per-lane scale preload is refilled every 64
    M = N = 128
    K = 65536
    x = random_bf16(91, (M, K))
    w = random_bf16(92, (N, K), 0.02)
    # scales vary strongly along K so that a stale or shifted scale shows
    x = (bf16_bits_to_f32(x).reshape(M, K // 128, 128) * np.float32(2.0) ** (np.arange(K // 128) % 7)[None, :, None])
    x = f32_to_bf16_bits(x.reshape(M, K))
    qx, sx = oracle.quantize_block(x)
    qw, sw = oracle.quantize_block(w)
    y = w8a8.gemm_blockscale(_dev(qx), _dev(sx), _dev(qw), _dev(sw))
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(y), oracle.linear_int8(qx, sx, qw, sw), "block GEMM K=65536")


def test_block_gemm_at_max_k():
    # K = 2^22, the largest K the block kernel accepts: 32768 K-blocks (the
    # per-lane scale preload refilled 512 times) and operand byte offsets up
    # to 255 * K inside a full 256 x 256 tile; output rows sampled
    M = N = 256
    K = w8a8.BLOCK_MAX_K
    kbs = K // 128
    rng = np.random.default_rng(4242)
    qx = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    qw = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    # scales spread over a few binades and different in every K-block, so a
    # stale, shifted or transposed scale shows in the result
    sx = (rng.uniform(0.5, 1.0, (M // 128, kbs)) * 2.0 ** -rng.integers(4, 12, (M // 128, kbs))).astype(np.float32)
    sw = (rng.uniform(0.5, 1.0, (N // 128, kbs)) * 2.0 ** -rng.integers(4, 12, (N // 128, kbs))).astype(np.float32)
    y = w8a8.gemm_blockscale(_dev(qx), _dev(sx), _dev(qw), _dev(sw))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 63, 64, 127, 128, 191, 200, 255])
    assert_bf16_close(bf16_bits(y)[rows], oracle.linear_int8(qx, sx, qw, sw, rows=rows), "block GEMM at the K limit")
