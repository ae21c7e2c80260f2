"""Fused producer on the GPU vs the oracle: exact GELU rounded to bf16
(every finite bf16 input, bit for bit) and the block quantization of that
result (codes and scales bit for bit), up to the MLP pair's hidden size."""
import numpy as np
import pytest
import torch

import block_quantized_int8_amd as w8a8
import oracle
from block_quantized_int8_amd import workloads
from block_quantized_int8_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits, random_bf16
from parity import bf16_bits, to_dev_bf16

pytestmark = pytest.mark.gpu

FINITE = np.array([u for u in range(1 << 16) if (u >> 7) & 0xFF != 0xFF], np.uint16)


def _say(msg):
    print(msg, flush=True)


def _same_codes(q, s, oq, os_, what):
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32)), f"{what}: scales differ"
    qg = q.cpu().numpy()
    if not np.array_equal(qg, oq):
        bad = np.argwhere(qg != oq)
        raise AssertionError(f"{what}: {len(bad)} codes differ, first at {tuple(bad[0])}")


def test_gelu_every_bf16_value():
    x = to_dev_bf16(FINITE)
    y = bf16_bits(w8a8.gelu_bf16(x))
    ref = oracle.gelu_bf16(FINITE)
    bad = np.flatnonzero(y != ref)
    assert bad.size == 0, [(hex(FINITE[i]), hex(y[i]), hex(ref[i])) for i in bad[:10]]
    # in place, on a permuted copy
    perm = np.random.default_rng(1).permutation(FINITE.size)
    xp = to_dev_bf16(FINITE[perm])
    w8a8.gelu_bf16(xp, out=xp)
    assert np.array_equal(bf16_bits(xp), ref[perm])
    _say(f"GELU: all {FINITE.size} finite bf16 inputs bit-exact")


@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 4095, 1000003])
def test_gelu_ragged_and_misaligned(n):
    rng = np.random.default_rng(n)
    bits = FINITE[rng.integers(0, FINITE.size, n + 1)]
    buf = to_dev_bf16(bits)
    ref = oracle.gelu_bf16(bits)
    y = torch.empty(n + 1, dtype=torch.bfloat16, device="cuda")
    assert np.array_equal(bf16_bits(w8a8.gelu_bf16(buf[:n], out=y[:n])), ref[:n])
    if n:  # both pointers 2 bytes off 16-byte alignment: element-wise path
        assert np.array_equal(bf16_bits(w8a8.gelu_bf16(buf[1:], out=y[1:])), ref[1:])


def _hidden_like(seed, shape):
    """N(0, 1.28^2) plus blocks that hit every branch of the map."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32) * np.float32(1.28)
    R, C = shape
    if R >= 256 and C >= 384:
        a[0:128, 128:256] *= np.float32(2.0 ** -14)        # |x| < 2^-10 only: x/2
        a[128:256, 0:128] = -np.abs(a[128:256, 0:128]) - 16  # x <= -16 only: all -0, s = 0
        a[128:256, 128:256] = -np.abs(a[128:256, 128:256]) * 0.5 - 12.5  # GELU ~ -1e-35: tiny scale
        a[0:128, 256:384] *= np.float32(1e37)               # near the top of the bf16 range
    return f32_to_bf16_bits(a)


@pytest.mark.parametrize("shape,seed", [((128, 128), 1), ((256, 384), 2), ((384, 1024), 3),
                                        ((640, 256), 4)])
def test_gelu_quantize_vs_oracle(shape, seed):
    y = _hidden_like(seed, shape)
    q, s = w8a8.gelu_quantize_act(to_dev_bf16(y))
    torch.cuda.synchronize()
    oq, os_ = oracle.gelu_quantize_block(y)
    _same_codes(q, s, oq, os_, f"gelu+quantize {shape}")
    if shape == (256, 384):
        sc = os_.reshape(2, 3)
        assert sc[1, 0] == 0 and sc[1, 1] < 2 ** -60 and sc[0, 2] > 1e35  # the branches were hit


def test_gelu_quantize_equals_unfused_chain():
    y = to_dev_bf16(random_bf16(9, (512, 768), 1.28))
    q, s = w8a8.gelu_quantize_act(y)
    q2, s2 = w8a8.quantize_act(w8a8.gelu_bf16(y))
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s.view(torch.int32), s2.view(torch.int32))


def test_gelu_quantize_mlp_hidden_32768x16384():
    M, K = 32768, 16384
    y = workloads.mlp_hidden(M, K)
    yd = to_dev_bf16(y)
    q, s = w8a8.gelu_quantize_act(yd)
    torch.cuda.synchronize()
    blocks = [0, M // 256, M // 128 - 1]
    rows = np.concatenate([np.arange(b * 128, (b + 1) * 128) for b in blocks])
    oq, os_ = oracle.gelu_quantize_block(y[rows])
    _same_codes(q[torch.from_numpy(rows).cuda()], s[torch.tensor(blocks).cuda()], oq, os_,
                "gelu+quantize 32768x16384, row blocks first/middle/last")
    # every other tile: scales agree with the unfused GPU chain, and each
    # scale is GELU's block absmax / 127 (largest |code| is 127)
    s2 = w8a8.quantize_act(w8a8.gelu_bf16(yd))[1]
    assert torch.equal(s.view(torch.int32), s2.view(torch.int32))
    amax = q.view(M // 128, 128, K // 128, 128).abs().amax(dim=(1, 3))
    assert bool((amax == 127).all())
    _say(f"gelu+quantize 32768x16384: {rows.size} rows bit-exact vs oracle; all {s.numel()} scales consistent")


def test_forward_gelu_paths():
    N, K = 256, 384
    w = random_bf16(41, (N, K), 0.02)
    layer = w8a8.W8A8Linear(to_dev_bf16(w))
    y = random_bf16(42, (3, 128, K), 1.28)
    out = layer.forward_gelu(to_dev_bf16(y))
    torch.cuda.synchronize()
    assert layer.last_path == w8a8.PATH_INT8 and out.shape == (3, 128, N)
    xo = oracle.gelu_bf16(y.reshape(-1, K))
    oq, os_ = oracle.quantize_block(xo)
    oqw, osw = oracle.quantize_block(w)
    from parity import assert_bf16_close
    assert_bf16_close(bf16_bits(out).reshape(-1, N), oracle.linear_int8(oq, os_, oqw, osw), "forward_gelu int8")
    # M = 300: GELU alone, then the guarded linear falls back to bf16
    y2 = random_bf16(43, (300, K), 1.28)
    out2 = layer.forward_gelu(to_dev_bf16(y2))
    torch.cuda.synchronize()
    assert layer.last_path == w8a8.PATH_BF16
    assert_bf16_close(bf16_bits(out2), oracle.linear_bf16(oracle.gelu_bf16(y2), oracle.DTYPE_BF16, w),
                      "forward_gelu fallback")
