"""Modulated layer normalization on the GPU against the oracle, alone and
fused with the 128x128 block quantization (TurboT2VA paper, architecture-
aware inference stack, fused-kernels paragraph: LayerNorm replaced).

The bf16 output is compared bit for bit, the fused codes and scales bit for
bit: off-centre rows (means far from zero, where the centring matters),
ragged row counts, 128-row blocks that straddle two batch entries, extreme
magnitudes, constant rows, and the full 32768 x 4096 transformer-block
input (oracle on sampled 128-row blocks, fused == unfused on the whole
matrix); the layer's forward with the fused producer equals the chain.
"""
import numpy as np
import pytest
import torch

import block_quantized_int8_amd as w8a8
import oracle
from block_quantized_int8_amd.workloads import bf16_bits_to_f32, block_hidden, f32_to_bf16_bits, random_bf16
from parity import bf16_bits, to_dev_bf16

pytestmark = pytest.mark.gpu


def dev(a):
    return to_dev_bf16(a)


def off_centre(seed, R, K, spread=2.0):
    # each row gets its own mean in [-40, 40]
    x = bf16_bits_to_f32(random_bf16(seed, (R, K), spread))
    mu = np.random.default_rng(seed + 1).uniform(-40, 40, (R, 1)).astype(np.float32)
    return f32_to_bf16_bits(x + mu)


def gpu_y(x, L, sc, sh, eps):
    B = x.shape[0] // L
    y = w8a8.layernorm_modulate_bf16(dev(x).view(B, L, -1), dev(sc), dev(sh), eps)
    torch.cuda.synchronize()
    return bf16_bits(y).reshape(x.shape)


@pytest.mark.parametrize("B,L,K,eps", [(2, 300, 512, 1e-6), (3, 77, 136, 1e-6), (1, 5, 8, 0.5), (4, 96, 4096, 1e-5),
                                       # the widths whose rows stay in registers for the statistics
                                       (2, 64, 1024, 1e-6), (1, 40, 2048, 1e-6), (1, 33, 3072, 1e-6),
                                       (1, 17, 5120, 1e-6), (1, 16, 6144, 1e-6), (1, 13, 8192, 1e-6)])
def test_bf16_output_bit_exact(B, L, K, eps):
    x = off_centre(B * 1000 + L, B * L, K)
    sc = random_bf16(K + 1, (B, K), 0.3)
    sh = random_bf16(K + 2, (B, K), 0.3)
    assert np.array_equal(gpu_y(x, L, sc, sh, eps), oracle.layernorm_modulate(x, L, sc, sh, eps))


def test_extreme_magnitudes_and_constant_rows():
    B, L, K = 2, 8, 256
    xf = bf16_bits_to_f32(random_bf16(31, (B * L, K)))
    xf[0] *= np.float32(2.0 ** -100)    # tiny row
    xf[1] *= np.float32(2.0 ** 100)     # huge row
    xf[2] = 0.0                         # zero row: y = shift
    xf[3] = 7.0                         # constant row: x - m = 0, y = shift
    xf[9, :5] = np.float32(1e30)        # a few huge values in an otherwise normal row
    xf[10] += np.float32(1e4)           # mean far above the spread
    x = f32_to_bf16_bits(xf)
    sc = random_bf16(32, (B, K), 0.3)
    sh = random_bf16(33, (B, K), 0.3)
    for eps in (1e-6, 1e-30):
        assert np.array_equal(gpu_y(x, L, sc, sh, eps), oracle.layernorm_modulate(x, L, sc, sh, eps)), eps
    y = gpu_y(x, L, sc, sh, 1e-6)
    assert np.array_equal(y[2], sh[0]) and np.array_equal(y[3], sh[0])


def test_fused_extreme_rows():
    """The fused entry on rows that stress the statistics: tiny and huge
    magnitudes, zero and constant rows, a few huge values, a mean far above
    the spread, and halves of a row with different means (K = 1024)."""
    B, L, K = 1, 128, 1024
    xf = bf16_bits_to_f32(random_bf16(35, (B * L, K)))
    xf[0] *= np.float32(2.0 ** -100)
    xf[1] *= np.float32(2.0 ** 100)
    xf[2] = 0.0
    xf[3] = 7.0
    xf[9, :5] = np.float32(1e30)
    xf[10] += np.float32(1e4)
    xf[11, 512:] += np.float32(300.0)
    x = f32_to_bf16_bits(xf)
    sc = random_bf16(36, (B, K), 0.3)
    sh = random_bf16(37, (B, K), 0.3)
    for eps in (1e-6, 1e-30):
        q, s = w8a8.layernorm_modulate_quantize_act(dev(x).view(B, L, K), dev(sc), dev(sh), eps)
        torch.cuda.synchronize()
        oq, os_ = oracle.layernorm_modulate_quantize_block(x, L, sc, sh, eps)
        assert np.array_equal(q.cpu().numpy(), oq), eps
        assert np.array_equal(s.cpu().numpy(), os_), eps


@pytest.mark.parametrize("B,L,K", [(2, 384, 512), (4, 96, 256), (1, 128, 128), (4, 96, 1024), (2, 192, 2560),
                                   (1, 256, 384)])
def test_fused_codes_bit_exact(B, L, K):
    # L = 96, 192: some 128-row blocks hold rows of two batch entries
    x = off_centre(B * 7 + L, B * L, K)
    sc = random_bf16(K + 3, (B, K), 0.3)
    sh = random_bf16(K + 4, (B, K), 0.3)
    q, s = w8a8.layernorm_modulate_quantize_act(dev(x).view(B, L, K), dev(sc), dev(sh), 1e-6)
    torch.cuda.synchronize()
    oq, os_ = oracle.layernorm_modulate_quantize_block(x, L, sc, sh, 1e-6)
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(s.cpu().numpy(), os_)


def test_transformer_block_input_full_size():
    d = block_hidden()
    x, sc, sh, L = d["x"], d["scale"], d["shift"], d["L"]
    B, K = sc.shape
    xd = dev(x).view(B, L, K)
    scd, shd = dev(sc), dev(sh)
    q, s = w8a8.layernorm_modulate_quantize_act(xd, scd, shd, 1e-6)
    y = w8a8.layernorm_modulate_bf16(xd, scd, shd, 1e-6).view(B * L, K)
    q2, s2 = w8a8.quantize_act(y)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s, s2), "fused differs from the unfused chain"
    for blk in (0, L // 128 - 1, L // 128, 2 * L // 128 + 17, B * L // 128 - 1):
        rows = slice(blk * 128, blk * 128 + 128)
        b = blk * 128 // L
        oy = oracle.layernorm_modulate(x[rows], 128, sc[b:b + 1], sh[b:b + 1], 1e-6)
        assert np.array_equal(bf16_bits(y[rows]), oy), blk
        oq, os_ = oracle.quantize_block(oy)
        assert np.array_equal(q[rows].cpu().numpy(), oq) and np.array_equal(s[blk].cpu().numpy(), os_[0]), blk


def test_layer_forward_modulated_layer_norm():
    B, L, K, N = 2, 256, 512, 384
    x = dev(off_centre(51, B * L, K)).view(B, L, K)
    sc = dev(random_bf16(52, (B, K), 0.3))
    sh = dev(random_bf16(53, (B, K), 0.3))
    layer = w8a8.W8A8Linear(dev(random_bf16(54, (N, K), 0.02)))
    fused = layer.forward_modulated(x, sc, sh, 1e-6, norm="layer")
    assert layer.last_path == w8a8.PATH_INT8
    chained = layer(w8a8.layernorm_modulate_bf16(x, sc, sh, 1e-6))
    torch.cuda.synchronize()
    assert fused.shape == (B, L, N)
    assert torch.equal(fused.view(torch.int16), chained.view(torch.int16))
