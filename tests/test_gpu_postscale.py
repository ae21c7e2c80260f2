"""Post-scale W8A8 form on the GPU vs the oracle: row codes and scales
bit-exact, bf16 outputs within tolerance, guard routing."""
import numpy as np
import pytest
import torch

import block_quantized_int8_amd as w8a8
import oracle
from block_quantized_int8_amd import workloads
from block_quantized_int8_amd.workloads import f32_to_bf16_bits, random_bf16
from conftest import load_golden
from parity import assert_bf16_close, bf16_bits, to_dev_bf16

pytestmark = pytest.mark.gpu


def _rows_same(bits, what):
    q, s = w8a8.quantize_rows(to_dev_bf16(bits))
    torch.cuda.synchronize()
    oq, os_ = oracle.quantize_rows(bits)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32)), f"{what}: scales differ"
    qg = q.cpu().numpy()
    if not np.array_equal(qg, oq):
        bad = np.argwhere(qg != oq)
        raise AssertionError(f"{what}: {len(bad)} codes differ, first at {tuple(bad[0])}")
    return oq, os_


@pytest.mark.parametrize("shape,scale,seed", [((256, 256), 1.0, 1), ((77, 8), 3.0, 2),
                                              ((300, 4096), 0.02, 3), ((64, 8200), 1.0, 4),
                                              ((40, 16384), 5.0, 5), ((128, 1000), 1e-6, 6),
                                              ((16, 20008), 2.0, 7), ((200, 4088), 1.0, 8)])
def test_quantize_rows_random(shape, scale, seed):
    _rows_same(random_bf16(seed, shape, scale), f"rows {shape} x{scale}")


def test_quantize_rows_golden_and_floor():
    g = load_golden("quantize_rows_examples.json")
    x = np.zeros((len(g["rows"]), 256), np.float32)
    rng = np.random.default_rng(3)
    for i, row in enumerate(g["rows"]):
        p = rng.choice(256, len(row["values"]), replace=False)
        x[i, p] = [v for v, _ in row["values"]]
    oq, os_ = _rows_same(f32_to_bf16_bits(x), "golden rows")
    for i, row in enumerate(g["rows"]):
        assert int(os_.view(np.uint32)[i]) == int(row["s_bits"], 16)
    # every bf16 magnitude below the floor, both signs, in one row each
    tiny = np.arange(0, 0x38D1, dtype=np.uint16)  # bf16 values below 1e-4
    tiny = np.concatenate([tiny, tiny | 0x8000])
    n = -(-tiny.size // 512) * 512
    rows = np.zeros(n, np.uint16)
    rows[:tiny.size] = tiny
    _rows_same(rows.reshape(-1, 512), "every sub-floor bf16 value")


@pytest.mark.parametrize("M,N,K,bias", [(256, 256, 256, False), (384, 640, 512, True),
                                        (128, 1152, 4096, True), (256, 256, 16384, False),
                                        (384, 384, 128, True)])
def test_gemm_postscale(M, N, K, bias):
    x = random_bf16(M + K, (M, K))
    w = random_bf16(N + K, (N, K), 0.02)
    b = random_bf16(N, (N,), 0.3) if bias else None
    qx, sx = oracle.quantize_rows(x)
    qw, sw = oracle.quantize_rows(w)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    y = w8a8.gemm_postscale(dev(qx), dev(sx), dev(qw), dev(sw), bias=None if b is None else to_dev_bf16(b))
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(y), oracle.linear_postscale(qx, sx, qw, sw, bias=b), f"postscale {M}x{N}x{K}")


def test_gemm_postscale_extremes():
    # |sum| = K * 127^2 at K = 16384: 264,257,536 < 2^31, exact in int32
    K = 16384
    x = np.full((128, K), 127.0, np.float32)
    w = np.full((128, K), -127.0, np.float32)
    w[1::2] = 127.0
    qx, sx = oracle.quantize_rows(f32_to_bf16_bits(x))
    qw, sw = oracle.quantize_rows(f32_to_bf16_bits(w))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    y = bf16_bits(w8a8.gemm_postscale(dev(qx), dev(sx), dev(qw), dev(sw)))
    # all scales are 1: both sides round the same exact integer once
    assert np.array_equal(y, oracle.linear_postscale(qx, sx, qw, sw))
    yf = y.astype(np.uint32) << 16
    assert np.all(yf.view(np.float32)[:, 0::2] < -2.6e8) and np.all(yf.view(np.float32)[:, 1::2] > 2.6e8)


def test_linear_postscale_attention_projection():
    d = workloads.attention_projection()
    xd, wd = to_dev_bf16(d["x"]), to_dev_bf16(d["w"])
    layer = w8a8.W8A8Linear(wd, scaling="postscale")
    y = layer(xd)
    torch.cuda.synchronize()
    assert layer.last_path == w8a8.PATH_INT8
    oqw, osw = _rows_same(d["w"], "weight channels")
    assert np.array_equal(layer.qweight.cpu().numpy(), oqw)
    oqx, osx = oracle.quantize_rows(d["x"])
    rows = workloads.sample_rows(16, 32768)
    rel = assert_bf16_close(bf16_bits(y)[rows], oracle.linear_postscale(oqx, osx, oqw, osw, rows=rows),
                            "post-scale attention projection")
    print(f"post-scale 32768x4096x4096: {rows.size} rows rel err {rel:.2e}", flush=True)


def test_linear_postscale_guard_and_bias():
    x = random_bf16(31, (1000, 512))
    w = random_bf16(32, (256, 512), 0.02)
    b = random_bf16(33, (256,), 0.1)
    layer = w8a8.W8A8Linear(to_dev_bf16(w), to_dev_bf16(b), scaling="postscale")
    y = layer(to_dev_bf16(x))
    torch.cuda.synchronize()
    assert layer.last_path == w8a8.PATH_BF16  # M = 1000
    assert_bf16_close(bf16_bits(y), oracle.linear_bf16(x, oracle.DTYPE_BF16, w, bias=b), "post-scale guard")
    y2 = layer(to_dev_bf16(x[:896]))
    torch.cuda.synchronize()
    assert layer.last_path == w8a8.PATH_INT8
    qx, sx = oracle.quantize_rows(x[:896])
    qw, sw = oracle.quantize_rows(w)
    assert_bf16_close(bf16_bits(y2), oracle.linear_postscale(qx, sx, qw, sw, bias=b), "post-scale with bias")


def test_gemm_postscale_max_k_at_the_int32_limit():
    # K = 133120 is the largest K accepted: all codes +-127 give |sum| =
    # 133120 * 127^2 = 2,147,092,480, just below 2^31, exact in int32
    K = w8a8.POSTSCALE_MAX_K
    assert K * 127 * 127 < 2 ** 31 <= (K + 128) * 127 * 127
    x = np.full((128, K), 127.0, np.float32)
    w = np.full((128, K), 127.0, np.float32)
    w[1::2] = -127.0
    qx, sx = oracle.quantize_rows(f32_to_bf16_bits(x))
    qw, sw = oracle.quantize_rows(f32_to_bf16_bits(w))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    y = bf16_bits(w8a8.gemm_postscale(dev(qx), dev(sx), dev(qw), dev(sw)))
    assert np.array_equal(y, oracle.linear_postscale(qx, sx, qw, sw))
    # one K-block more is refused (the guarded linear falls back instead)
    big = torch.zeros((128, K + 128), dtype=torch.int8, device="cuda")
    sc = torch.ones(128, dtype=torch.float32, device="cuda")
    with pytest.raises(w8a8.W8A8Error):
        w8a8.gemm_postscale(big, sc, big, sc)
