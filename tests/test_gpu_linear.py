"""Guarded linear on the GPU: routing and results vs the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import block_quantized_int8_amd as w8a8
import oracle
from block_quantized_int8_amd.workloads import single_linear_256, random_bf16
from parity import assert_bf16_close, bf16_bits, to_dev_bf16

pytestmark = pytest.mark.gpu


def test_single_linear_256_int8_path():
    d = single_linear_256()
    x, w = to_dev_bf16(d["x"]), to_dev_bf16(d["w"])
    layer = w8a8.W8A8Linear(w)
    y = layer(x)
    torch.cuda.synchronize()
    assert layer.last_path == w8a8.PATH_INT8
    oqx, osx = oracle.quantize_block(d["x"])
    oqw, osw = oracle.quantize_block(d["w"])
    assert np.array_equal(layer.qweight.cpu().numpy(), oqw)
    assert np.array_equal(layer.wscale.cpu().numpy(), osw)
    assert_bf16_close(bf16_bits(y), oracle.linear_int8(oqx, osx, oqw, osw), "single linear 256^3")


def test_linear_with_bias_and_leading_dims():
    x = random_bf16(1, (2, 128, 384))
    w = random_bf16(2, (256, 384), 0.02)
    b = random_bf16(3, (256,), 0.1)
    layer = w8a8.W8A8Linear(to_dev_bf16(w), to_dev_bf16(b))
    y = layer(to_dev_bf16(x))
    assert y.shape == (2, 128, 256) and layer.last_path == w8a8.PATH_INT8
    qx, sx = oracle.quantize_block(x.reshape(256, 384))
    qw, sw = oracle.quantize_block(w)
    assert_bf16_close(bf16_bits(y.reshape(256, 256)), oracle.linear_int8(qx, sx, qw, sw, bias=b), "bias")


@pytest.mark.parametrize("M,K,N", [(4000 // 8, 512, 256), (1, 128, 128), (1000, 256, 384),
                                   (77, 130, 45), (128, 129, 128), (3, 7, 5), (300, 1000, 200)])
def test_fallback_shapes(M, K, N):
    x = random_bf16(M + K, (M, K))
    w = random_bf16(N + K, (N, K), 0.02)
    b = random_bf16(N, (N,), 0.1)
    wd = to_dev_bf16(w)
    qw = sw = None
    if N % 128 == 0 and K % 128 == 0:
        qw, sw = w8a8.quantize_weight(wd)
    y, path = w8a8.linear(to_dev_bf16(x), wd, qw, sw, bias=to_dev_bf16(b))
    torch.cuda.synchronize()
    assert path == w8a8.PATH_BF16
    assert_bf16_close(bf16_bits(y), oracle.linear_bf16(x, oracle.DTYPE_BF16, w, bias=b),
                      f"fallback {M}x{K}x{N}")


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_fallback_other_dtypes(dtype):
    rng = np.random.default_rng(5)
    xf = rng.standard_normal((256, 256), dtype=np.float32)
    w = random_bf16(6, (256, 256), 0.02)
    wd = to_dev_bf16(w)
    qw, sw = w8a8.quantize_weight(wd)
    xt = torch.from_numpy(xf).to(dtype)
    y, path = w8a8.linear(xt.cuda(), wd, qw, sw)
    torch.cuda.synchronize()
    assert path == w8a8.PATH_BF16
    if dtype == torch.float16:
        xin, code = xt.numpy().view(np.uint16), oracle.DTYPE_FP16
    else:
        xin, code = xf, oracle.DTYPE_FP32
    assert_bf16_close(bf16_bits(y), oracle.linear_bf16(xin, code, w), str(dtype))


def test_misaligned_input_falls_back():
    x = random_bf16(7, (128 * 256 + 8,))
    w = random_bf16(8, (128, 256), 0.02)
    wd = to_dev_bf16(w)
    qw, sw = w8a8.quantize_weight(wd)
    xd = to_dev_bf16(x)[1:1 + 128 * 256].view(128, 256)  # 2-byte offset: not 16-byte aligned
    assert xd.data_ptr() % 16 != 0
    y, path = w8a8.linear(xd, wd, qw, sw)
    torch.cuda.synchronize()
    assert path == w8a8.PATH_BF16
    xo = x[1:1 + 128 * 256].reshape(128, 256)
    assert_bf16_close(bf16_bits(y), oracle.linear_bf16(xo, oracle.DTYPE_BF16, w), "misaligned")


def test_errors_on_host_pointers_and_small_workspace():
    L = w8a8.lib()
    host = np.zeros(128 * 128, np.uint16)
    dev = torch.zeros(128 * 128, dtype=torch.int16, device="cuda")
    qd = torch.zeros(128 * 128, dtype=torch.int8, device="cuda")
    sd = torch.zeros(1, dtype=torch.float32, device="cuda")
    hp = ctypes.c_void_p(host.ctypes.data)
    dp = ctypes.c_void_p(dev.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # host input pointer -> INVALID_ARG, nothing launched
    assert L.w8a8_quantize_act(hp, 128, 128, ctypes.c_void_p(qd.data_ptr()),
                               ctypes.c_void_p(sd.data_ptr()), stream) == 1
    path = ctypes.c_int(-1)
    assert L.w8a8_linear(hp, 0, 128, 128, 128, dp, None, None, None, dp, None, 0, stream,
                         ctypes.byref(path)) == 1
    # INT8 route with too small a workspace -> INVALID_ARG
    assert L.w8a8_linear(dp, 0, 128, 128, 128, dp, ctypes.c_void_p(qd.data_ptr()),
                         ctypes.c_void_p(sd.data_ptr()), None, dp, dp, 16, stream,
                         ctypes.byref(path)) == 1
    with pytest.raises(ValueError):
        w8a8.quantize_act(torch.zeros(128, 128, dtype=torch.bfloat16))  # CPU tensor
    torch.cuda.synchronize()


def test_repeat_calls_are_deterministic():
    x = to_dev_bf16(random_bf16(11, (512, 512)))
    layer = w8a8.W8A8Linear(to_dev_bf16(random_bf16(12, (384, 512), 0.02)))
    y1 = layer(x).clone()
    y2 = layer(x)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


# bf16 input with K % 64 == 0, N % 128 == 0 and at least 256 output tiles of
# 256x256 runs the 256x256-tile kernel's bf16 mode: ragged M (a partial last
# tile, a wavefront half inside it), a partial N tile, 1 to 64 K-blocks of 64
@pytest.mark.parametrize("M,K,N", [(4000, 64, 4096), (4001, 192, 4224), (8191, 4096, 2048),
                                   (4100, 128, 4096)])
def test_fallback_large_tiled(M, K, N):
    x = random_bf16(M + K + 1, (M, K))
    w = random_bf16(N + K + 1, (N, K), 0.02)
    b = random_bf16(N + 1, (N,), 0.1)
    y, path = w8a8.linear(to_dev_bf16(x), to_dev_bf16(w), bias=to_dev_bf16(b))
    torch.cuda.synchronize()
    assert path == w8a8.PATH_BF16
    rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(M - 200, M),
                                     np.random.default_rng(M).integers(0, M, 200)]))
    assert_bf16_close(bf16_bits(y)[rows], oracle.linear_bf16(x, oracle.DTYPE_BF16, w, bias=b, rows=rows),
                      f"fallback {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N", [(1000, 2048, 2048), (999, 64, 200), (65, 128, 8), (129, 320, 1000),
                                   (3000, 1024, 1032), (64, 384, 128)])
def test_fallback_pipelined(M, K, N):
    # bf16 input, K a multiple of 64, N of 8, too few 256x256 tiles for the
    # tiled kernel: the pipelined 64x128-tile kernel, from fewer K steps than
    # its ring has stages (K = 64) to many more (K = 2048), ragged M and N
    x = random_bf16(M + 2 * K, (M, K))
    w = random_bf16(N + 2 * K, (N, K), 0.02)
    b = random_bf16(N + 2, (N,), 0.1)
    for bias in (None, b):
        y, path = w8a8.linear(to_dev_bf16(x), to_dev_bf16(w), bias=None if bias is None else to_dev_bf16(bias))
        torch.cuda.synchronize()
        assert path == w8a8.PATH_BF16
        rows = np.unique(np.concatenate([np.arange(0, min(M, 40)), np.arange(max(0, M - 40), M),
                                         np.random.default_rng(M).integers(0, M, 60)]))
        assert_bf16_close(bf16_bits(y)[rows], oracle.linear_bf16(x, oracle.DTYPE_BF16, w, bias=bias, rows=rows),
                          f"pipelined fallback {M}x{K}x{N} bias={bias is not None}")


def test_block_gemm_k_limit_routes_to_fallback():
    # K just past the block GEMM's limit: the guarded linear takes the bf16
    # fallback (never a silently wrong INT8 result); one output row vs the oracle
    from block_quantized_int8_amd._lib import BLOCK_MAX_K
    M, N, K = 128, 128, BLOCK_MAX_K + 128
    x = random_bf16(71, (M, K))
    w = random_bf16(72, (N, K), 0.02)
    wd = to_dev_bf16(w)
    qw, sw = w8a8.quantize_weight(wd)
    y, path = w8a8.linear(to_dev_bf16(x), wd, qw, sw)
    torch.cuda.synchronize()
    assert path == w8a8.PATH_BF16
    rows = np.array([0, 77], np.int64)
    assert_bf16_close(bf16_bits(y)[rows], oracle.linear_bf16(x, oracle.DTYPE_BF16, w, rows=rows), "K past the limit")
