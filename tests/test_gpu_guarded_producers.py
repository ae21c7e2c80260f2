"""The guarded producer linears (w8a8_linear_gelu, w8a8_linear_rmsnorm_modulate,
w8a8_linear_layernorm_modulate) and the routing rules every guarded entry
shares, on the GPU, against the oracle.

* INT8 path: equal, bit for bit, to the fused producer + quantizer followed by
  the block GEMM (the library's route takes the decision, not Python);
* fallback (rows not a multiple of 128, a misaligned bias, the
  W8A8_FORCE_FALLBACK test switch): the producer's bf16 output through the
  bf16 linear, within the bf16 tolerance of the oracle's fallback;
* a misaligned input with no workspace takes the fallback instead of failing.
"""
import ctypes

import numpy as np
import pytest
import torch

import block_quantized_int8_amd as w8a8
import oracle
from block_quantized_int8_amd.workloads import random_bf16
from parity import assert_bf16_close, bf16_bits, to_dev_bf16

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _misaligned_copy(bits):
    """A device bf16 copy of `bits` that starts 2 bytes past a 16-byte boundary."""
    buf = to_dev_bf16(np.concatenate([np.zeros(1, np.uint16), bits.ravel()]))
    t = buf[1:].view(bits.shape)
    assert t.data_ptr() % 16 == 2
    return t


def test_linear_gelu_int8_equals_fused_chain_and_oracle():
    M, K, N = 256, 384, 256
    u = random_bf16(301, (M, K), 1.28)
    w = random_bf16(302, (N, K), 0.02)
    b = random_bf16(303, (N,), 0.5)
    wd, bd = to_dev_bf16(w), to_dev_bf16(b)
    qw, sw = w8a8.quantize_weight(wd)
    y, path = w8a8.linear_gelu(to_dev_bf16(u), wd, qw, sw, bd)
    q, s = w8a8.gelu_quantize_act(to_dev_bf16(u))
    chain = w8a8.gemm_blockscale(q, s, qw, sw, bd)
    torch.cuda.synchronize()
    assert path == w8a8.PATH_INT8
    assert torch.equal(y.view(torch.int16), chain.view(torch.int16))
    oq, os_ = oracle.quantize_block(oracle.gelu_bf16(u))
    oqw, osw = oracle.quantize_block(w)
    assert_bf16_close(bf16_bits(y), oracle.linear_int8(oq, os_, oqw, osw, b), "linear_gelu int8")
    _say("linear_gelu 256x256x384: INT8 path equals the fused chain bit for bit")


@pytest.mark.parametrize("M", [300, 1])
def test_linear_gelu_fallback_rows(M):
    K, N = 256, 384
    u = random_bf16(310 + M, (M, K), 1.28)
    w = random_bf16(311, (N, K), 0.02)
    wd = to_dev_bf16(w)
    qw, sw = w8a8.quantize_weight(wd)
    y, path = w8a8.linear_gelu(to_dev_bf16(u), wd, qw, sw)
    torch.cuda.synchronize()
    assert path == w8a8.PATH_BF16
    assert_bf16_close(bf16_bits(y), oracle.linear_bf16(oracle.gelu_bf16(u), oracle.DTYPE_BF16, w),
                      f"linear_gelu fallback M={M}")


def test_misaligned_bias_takes_the_fallback_on_every_guarded_entry():
    M, K, N = 256, 256, 256
    u = random_bf16(320, (M, K), 1.28)
    w = random_bf16(321, (N, K), 0.02)
    b = random_bf16(322, (N,), 0.5)
    wd = to_dev_bf16(w)
    bmis = _misaligned_copy(b)
    layer = w8a8.W8A8Linear(wd, bmis)
    out = layer.forward_gelu(to_dev_bf16(u))
    torch.cuda.synchronize()
    assert layer.last_path == w8a8.PATH_BF16
    assert_bf16_close(bf16_bits(out), oracle.linear_bf16(oracle.gelu_bf16(u), oracle.DTYPE_BF16, w, b),
                      "forward_gelu with a misaligned bias")
    y = layer(to_dev_bf16(u))
    torch.cuda.synchronize()
    assert layer.last_path == w8a8.PATH_BF16
    assert_bf16_close(bf16_bits(y), oracle.linear_bf16(u, oracle.DTYPE_BF16, w, b), "forward, misaligned bias")
    sc, sh = random_bf16(323, (2, K), 0.3), random_bf16(324, (2, K), 0.3)
    x = random_bf16(325, (M, K), 2.0)
    ym = layer.forward_modulated(to_dev_bf16(x).view(2, 128, K), to_dev_bf16(sc), to_dev_bf16(sh), 1e-6)
    torch.cuda.synchronize()
    assert layer.last_path == w8a8.PATH_BF16
    xn = oracle.rmsnorm_modulate(x, 128, sc, sh, 1e-6)
    assert_bf16_close(bf16_bits(ym).reshape(M, N), oracle.linear_bf16(xn, oracle.DTYPE_BF16, w, b),
                      "forward_modulated, misaligned bias")


@pytest.mark.parametrize("norm", ["rms", "layer"])
@pytest.mark.parametrize("B,L", [(2, 128), (2, 100)])
def test_linear_modulated_paths(norm, B, L):
    K, N = 512, 384
    x = random_bf16(330 + L, (B * L, K), 2.0)
    sc, sh = random_bf16(331, (B, K), 0.3), random_bf16(332, (B, K), 0.3)
    w = random_bf16(333, (N, K), 0.02)
    wd = to_dev_bf16(w)
    qw, sw = w8a8.quantize_weight(wd)
    xd, scd, shd = to_dev_bf16(x).view(B, L, K), to_dev_bf16(sc), to_dev_bf16(sh)
    y, path = w8a8.linear_modulated(xd, scd, shd, wd, qw, sw, None, 1e-6, norm)
    torch.cuda.synchronize()
    ofn = oracle.rmsnorm_modulate if norm == "rms" else oracle.layernorm_modulate
    xn = ofn(x, L, sc, sh, 1e-6)
    if (B * L) % 128 == 0:
        assert path == w8a8.PATH_INT8
        fused = (w8a8.rmsnorm_modulate_quantize_act if norm == "rms" else w8a8.layernorm_modulate_quantize_act)
        q, s = fused(xd, scd, shd, 1e-6)
        chain = w8a8.gemm_blockscale(q, s, qw, sw)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16).reshape(B * L, N), chain.view(torch.int16))
        oq, os_ = oracle.quantize_block(xn)
        oqw, osw = oracle.quantize_block(w)
        assert_bf16_close(bf16_bits(y).reshape(B * L, N), oracle.linear_int8(oq, os_, oqw, osw), f"{norm} int8")
    else:
        assert path == w8a8.PATH_BF16
        assert_bf16_close(bf16_bits(y).reshape(B * L, N), oracle.linear_bf16(xn, oracle.DTYPE_BF16, w),
                          f"{norm} fallback")
    _say(f"linear_modulated {norm} B={B} L={L}: path {path}")


def test_force_fallback_switch(monkeypatch):
    M, K, N = 256, 256, 256
    x = random_bf16(340, (M, K), 1.0)
    w = random_bf16(341, (N, K), 0.02)
    layer = w8a8.W8A8Linear(to_dev_bf16(w))
    y8 = layer(to_dev_bf16(x))
    assert layer.last_path == w8a8.PATH_INT8
    monkeypatch.setenv("W8A8_FORCE_FALLBACK", "1")
    y = layer(to_dev_bf16(x))
    torch.cuda.synchronize()
    assert layer.last_path == w8a8.PATH_BF16
    assert_bf16_close(bf16_bits(y), oracle.linear_bf16(x, oracle.DTYPE_BF16, w), "forced fallback")
    assert not torch.equal(y.view(torch.int16), y8.view(torch.int16))   # really the other path
    yg = layer.forward_gelu(to_dev_bf16(x))
    torch.cuda.synchronize()
    assert layer.last_path == w8a8.PATH_BF16
    assert_bf16_close(bf16_bits(yg), oracle.linear_bf16(oracle.gelu_bf16(x), oracle.DTYPE_BF16, w), "forced gelu")
    sc, sh = random_bf16(342, (2, K), 0.3), random_bf16(343, (2, K), 0.3)
    ym = layer.forward_modulated(to_dev_bf16(x).view(2, 128, K), to_dev_bf16(sc), to_dev_bf16(sh), 1e-6, "layer")
    torch.cuda.synchronize()
    assert layer.last_path == w8a8.PATH_BF16
    h, g = random_bf16(344, (M, N), 2.0), random_bf16(345, (2, N), 0.5)
    yr = layer.forward_gated_residual(to_dev_bf16(x), to_dev_bf16(h), to_dev_bf16(g))
    torch.cuda.synchronize()
    assert layer.last_path == w8a8.PATH_BF16
    _, path = w8a8.linear(to_dev_bf16(x), layer.weight, layer.qweight, layer.wscale)
    assert path == w8a8.PATH_BF16
    monkeypatch.delenv("W8A8_FORCE_FALLBACK")
    layer(to_dev_bf16(x))
    assert layer.last_path == w8a8.PATH_INT8
    _say("W8A8_FORCE_FALLBACK=1 sends every guarded entry to the bf16 fallback")


def test_misaligned_input_needs_no_workspace():
    L = w8a8.lib()
    x = random_bf16(350, (128 * 128,), 1.0)
    w = random_bf16(351, (128, 128), 0.02)
    xd = _misaligned_copy(x)
    wd = to_dev_bf16(w)
    qw, sw = w8a8.quantize_weight(wd)
    y = torch.empty((128, 128), dtype=torch.bfloat16, device="cuda")
    path = ctypes.c_int(-1)
    st = L.w8a8_linear(ctypes.c_void_p(xd.data_ptr()), 0, 128, 128, 128, ctypes.c_void_p(wd.data_ptr()),
                       ctypes.c_void_p(qw.data_ptr()), ctypes.c_void_p(sw.data_ptr()), None,
                       ctypes.c_void_p(y.data_ptr()), None, 0, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream),
                       ctypes.byref(path))
    torch.cuda.synchronize()
    assert st == 0 and path.value == w8a8.PATH_BF16
    assert_bf16_close(bf16_bits(y), oracle.linear_bf16(x.reshape(128, 128), oracle.DTYPE_BF16, w), "no workspace")


def test_hip_error_is_reported_through_the_abi():
    """A real HIP failure, forced from the host: the launch goes to a stream
    handle that was created and destroyed, which the runtime rejects before
    any work is enqueued.  The call returns W8A8_ERR_HIP with the HIP code
    kept per thread, the binding raises W8A8Error, and the library keeps
    working on a valid stream afterwards."""
    hip = ctypes.CDLL("libamdhip64.so")
    dead = ctypes.c_void_p()
    assert hip.hipStreamCreate(ctypes.byref(dead)) == 0
    assert hip.hipStreamDestroy(dead) == 0
    L = w8a8.lib()
    x = to_dev_bf16(random_bf16(360, (128, 128), 1.0))
    q = torch.empty((128, 128), dtype=torch.int8, device="cuda")
    s = torch.empty((1, 1), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    st = L.w8a8_quantize_act(ctypes.c_void_p(x.data_ptr()), 128, 128, ctypes.c_void_p(q.data_ptr()),
                             ctypes.c_void_p(s.data_ptr()), dead)
    assert st == 3 and L.w8a8_last_hip_error() != 0
    assert L.w8a8_status_string(st).decode() == "W8A8_ERR_HIP"
    err = w8a8.W8A8Error("w8a8_quantize_act", st)
    assert err.status == 3 and "hipError" in str(err)
    q2, s2 = w8a8.quantize_act(x)          # the current stream still works
    oq, os_ = oracle.quantize_block(bf16_bits(x))
    torch.cuda.synchronize()
    assert np.array_equal(q2.cpu().numpy(), oq) and np.array_equal(s2.cpu().numpy(), os_)
