"""Gated residual update on the GPU (TurboT2VA paper, architecture-aware
inference stack, fused-kernels paragraph), alone and in the epilogue of the
block-scaled GEMM.

The update is a fixed pair of fp32 operations and one bf16 rounding, so the
standalone kernel is compared with the oracle bit for bit (golden cases,
random shapes, in place).  The fused GEMM is compared bit for bit with the
update applied to the plain GEMM's output on the GPU (same accumulation,
same bf16 o), and end to end with the oracle (linear, then update) within
the output tolerance; likewise the guarded layer on both paths and the
32768 x 4096 x 4096 attention-projection size.
"""
import numpy as np
import pytest
import torch

import block_quantized_int8_amd as w8a8
import oracle
from block_quantized_int8_amd import workloads
from block_quantized_int8_amd.workloads import random_bf16, sample_rows
from conftest import load_golden
from parity import assert_bf16_close, bf16_bits, to_dev_bf16

pytestmark = pytest.mark.gpu


def hx(v):
    return np.array([int(s, 16) for s in v], np.uint16)


def test_golden_cases_on_gpu():
    # each case's rows padded to 8 channels with (h, o, g) = (1, 1, 0) columns
    for c in load_golden("gated_residual_examples.json")["cases"]:
        B, L, N = c["B"], c["L"], c["N"]
        h = np.full((B * L, 8), 0x3F80, np.uint16)
        o = np.full((B * L, 8), 0x3F80, np.uint16)
        g = np.zeros((B, 8), np.uint16)
        h[:, :N] = hx(c["h"]).reshape(B * L, N)
        o[:, :N] = hx(c["o"]).reshape(B * L, N)
        g[:, :N] = hx(c["gate"]).reshape(B, N)
        y = w8a8.gated_residual(to_dev_bf16(h), to_dev_bf16(o), to_dev_bf16(g))
        torch.cuda.synchronize()
        got = bf16_bits(y)
        assert np.array_equal(got[:, :N], hx(c["y"]).reshape(B * L, N)), c["note"]
        assert np.all(got[:, N:] == 0x3F80)


@pytest.mark.parametrize("B,L,N", [(1, 1, 8), (2, 37, 64), (3, 129, 4096), (4, 5, 1000)])
def test_update_bit_exact(B, L, N):
    h = random_bf16(B * 100 + L, (B * L, N), 4.0)
    o = random_bf16(B * 100 + L + 1, (B * L, N), 4.0)
    g = random_bf16(B * 100 + L + 2, (B, N), 0.5)
    want = oracle.gated_residual(h, o, g, L)
    hd, od, gd = to_dev_bf16(h), to_dev_bf16(o), to_dev_bf16(g)
    y = w8a8.gated_residual(hd, od, gd)
    w8a8.gated_residual(hd, od, gd, out=od)          # in place on o
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y), want)
    assert np.array_equal(bf16_bits(od), want)
    w8a8.gated_residual(hd, to_dev_bf16(o), gd, out=hd)  # in place on h
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(hd), want)


def _layer_case(M, N, K, L, seed, bias=True):
    x = random_bf16(seed, (M, K))
    w = random_bf16(seed + 1, (N, K), 0.02)
    b = random_bf16(seed + 2, (N,), 0.1) if bias else None
    h = random_bf16(seed + 3, (M, N), 2.0)
    g = random_bf16(seed + 4, (M // L, N), 0.5)
    return x, w, b, h, g


@pytest.mark.parametrize("M,N,K,L,bias", [(256, 256, 256, 128, True), (384, 512, 640, 96, False),
                                          (512, 384, 256, 1, True)])
def test_fused_epilogue_equals_unfused_and_oracle(M, N, K, L, bias):
    x, w, b, h, g = _layer_case(M, N, K, L, M + N + K, bias)
    xd, wd, hd, gd = to_dev_bf16(x), to_dev_bf16(w), to_dev_bf16(h), to_dev_bf16(g)
    bd = to_dev_bf16(b) if bias else None
    qx, sx = w8a8.quantize_act(xd)
    qw, sw = w8a8.quantize_weight(wd)
    y = w8a8.gemm_blockscale_gated_residual(qx, sx, qw, sw, hd, gd, bias=bd)
    o = w8a8.gemm_blockscale(qx, sx, qw, sw, bd)
    yu = w8a8.gated_residual(hd, o, gd)
    hin = hd.clone()
    w8a8.gemm_blockscale_gated_residual(qx, sx, qw, sw, hin, gd, bias=bd, out=hin)  # in place on h
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), yu.view(torch.int16)), "fused != unfused"
    assert torch.equal(hin.view(torch.int16), y.view(torch.int16)), "in place != out of place"
    assert np.array_equal(bf16_bits(y), oracle.gated_residual(h, bf16_bits(o), g, L))
    oq, os_ = oracle.quantize_block(x)
    wq, ws = oracle.quantize_block(w)
    want = oracle.gated_residual(h, oracle.linear_int8(oq, os_, wq, ws, b), g, L)
    assert_bf16_close(bf16_bits(y), want, f"gated residual GEMM {M}x{N}x{K}")


def test_guarded_layer_both_paths():
    for (M, N, K, L) in [(512, 256, 384, 128), (4000, 256, 512, 1000)]:   # INT8; M not a multiple of 128 -> bf16
        x, w, b, h, g = _layer_case(M, N, K, L, M + 7)
        layer = w8a8.W8A8Linear(to_dev_bf16(w), to_dev_bf16(b))
        hd, gd = to_dev_bf16(h), to_dev_bf16(g)
        y = layer.forward_gated_residual(to_dev_bf16(x), hd, gd)
        path = layer.last_path
        yu = w8a8.gated_residual(hd, layer(to_dev_bf16(x)), gd)
        torch.cuda.synchronize()
        assert path == (w8a8.PATH_INT8 if M % 128 == 0 else w8a8.PATH_BF16)
        assert torch.equal(y.view(torch.int16), yu.view(torch.int16)), (M, "fused != unfused")
        if path == w8a8.PATH_INT8:
            oq, os_ = oracle.quantize_block(x)
            wq, ws = oracle.quantize_block(w)
            o = oracle.linear_int8(oq, os_, wq, ws, b)
        else:
            o = oracle.linear_bf16(x, oracle.DTYPE_BF16, w, b)
        assert_bf16_close(bf16_bits(y), oracle.gated_residual(h, o, g, L), f"guarded layer M={M}")


def test_attention_projection_size():
    # 32768 x 4096 x 4096, 4 batch entries of 8192 tokens: fused == unfused on
    # the whole output; oracle (linear then update) on sampled rows
    d = workloads.attention_projection()
    M, N, K, L = 32768, 4096, 4096, 8192
    h = random_bf16(90, (M, N), 2.0)
    g = random_bf16(91, (M // L, N), 0.5)
    xd, wd, hd, gd = to_dev_bf16(d["x"]), to_dev_bf16(d["w"]), to_dev_bf16(h), to_dev_bf16(g)
    qx, sx = w8a8.quantize_act(xd)
    qw, sw = w8a8.quantize_weight(wd)
    y = w8a8.gemm_blockscale_gated_residual(qx, sx, qw, sw, hd, gd)
    yu = w8a8.gated_residual(hd, w8a8.gemm_blockscale(qx, sx, qw, sw), gd)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), yu.view(torch.int16))
    rows = sample_rows(92, M)
    oq, os_ = oracle.quantize_block(d["x"])
    wq, ws = oracle.quantize_block(d["w"])
    o = oracle.linear_int8(oq, os_, wq, ws, rows=rows)
    want = np.stack([oracle.gated_residual(h[r:r + 1], o[i:i + 1], g[r // L:r // L + 1], 1)[0]
                     for i, r in enumerate(rows)])
    assert_bf16_close(bf16_bits(y)[rows], want, "attention projection + gated residual")
    print(f"gated residual GEMM 32768x4096x4096: fused == unfused bit-exact; {len(rows)} rows vs oracle", flush=True)


def test_argument_errors():
    h = torch.zeros((256, 256), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((3, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        w8a8.gated_residual(h, h.clone(), g)                     # 3 does not divide 256 rows
    with pytest.raises(w8a8.W8A8Error):
        o = torch.zeros((256, 12), dtype=torch.bfloat16, device="cuda")
        w8a8.gated_residual(torch.zeros_like(o), o, torch.zeros((1, 12), dtype=torch.bfloat16, device="cuda"))
    layer = w8a8.W8A8Linear(torch.zeros((256, 256), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(w8a8.W8A8Error):                          # out overlapping h
        layer.forward_gated_residual(h, h, torch.zeros((1, 256), dtype=torch.bfloat16, device="cuda"), out=h)
