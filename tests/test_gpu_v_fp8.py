"""Attention V in FP8 E4M3 on the GPU vs the oracle (TurboT2VA paper,
architecture-aware inference stack, sparse-attention paragraph: FP8
values beside INT8 Q/K): codes and scales bit for bit.

The conversion itself is checked exhaustively: in a block whose max-abs is
448 the scale is exactly 1, so the quotient is the input, and every bf16
value of magnitude <= 448 (both signs, subnormals of bf16 included) goes
through the kernel's E4M3 rounding once.  Then random, ragged, strided,
tiny-scale and zero blocks, and the video self-attention's V.
"""
import numpy as np
import pytest
import torch

import block_quantized_int8_amd as w8a8
import oracle
from block_quantized_int8_amd import workloads
from block_quantized_int8_amd.workloads import f32_to_bf16_bits, random_bf16
from parity import to_dev_bf16

pytestmark = pytest.mark.gpu


def _check(xbits, B, L, H, D, ld, col0=0, what=""):
    dev = to_dev_bf16(xbits)
    view = dev[:, col0:col0 + H * D].view(B, L, H * D)
    q, s = w8a8.quantize_v_fp8(view, H)
    torch.cuda.synchronize()
    oq, os_ = oracle.quantize_v_fp8(np.ascontiguousarray(xbits[:, col0:col0 + H * D]), B, L, H, D, H * D)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32)), f"{what}: scales differ"
    g = q.cpu().numpy()
    if not np.array_equal(g, oq):
        bad = np.argwhere(g != oq)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} codes differ, first at {i}: {g[i]:#x} vs {oq[i]:#x}")
    return g, s.cpu().numpy()


def test_every_bf16_magnitude_up_to_448():
    mags = np.arange(0, 0x43E1, dtype=np.uint16)          # +0 .. 448 (0x43E0), every bf16 pattern between
    vals = np.concatenate([mags, mags | np.uint16(0x8000)])
    D = 128
    per_block = 128 * D - 1                                # one slot per block holds 448 itself
    nb = -(-vals.size // per_block)
    x = np.zeros((nb * 128, D), np.uint16)
    flat = x.reshape(nb, 128 * D)
    for b in range(nb):
        chunk = vals[b * per_block:(b + 1) * per_block]
        flat[b, 0] = 0x43E0
        flat[b, 1:1 + chunk.size] = chunk
    g, s = _check(x, 1, nb * 128, 1, D, D, what="bf16 sweep")
    assert np.all(s == 1.0)


@pytest.mark.parametrize("B,L,H,D,extra,col0", [(1, 128, 1, 128, 0, 0), (2, 200, 3, 64, 8, 0),
                                                (1, 1, 4, 128, 0, 0), (3, 257, 2, 128, 128, 128),
                                                (2, 384, 4, 64, 512, 256)])
def test_v_random_vs_oracle(B, L, H, D, extra, col0):
    ld = col0 + H * D + extra
    x = random_bf16(B * 2000 + L, (B * L, ld), 1.5)
    _check(x, B, L, H, D, ld, col0, f"V B={B} L={L} H={H} D={D} ld={ld}")


def test_v_edge_blocks():
    # all-zero block (with -0 values), tiny-scale block, huge block, one value in a ragged tail
    B, L, H, D = 1, 300, 2, 64
    x = np.zeros((L, H * D), np.float32)
    rng = np.random.default_rng(15)
    x[128:256, :D] = rng.standard_normal((128, D)).astype(np.float32) * np.float32(1e-30)
    x[0:128, D:] = rng.standard_normal((128, D)).astype(np.float32) * np.float32(1e37)
    x[299, D + 63] = -3.0
    xb = f32_to_bf16_bits(x)
    xb[0:128:3, :D] = 0x8000                                # -0 inside the all-zero block
    g, s = _check(xb, B, L, H, D, H * D, what="V edge blocks")
    assert s[0, 0, 0] == 0 and not g[0, 0, :128].any()
    assert s[0, 0, 1] < 2 ** -60 and s[0, 1, 0] > 1e34
    assert g[0, 1, 299, 63] == 0xFE and np.count_nonzero(g[0, 1, 256:]) == 1


def test_v_video_self_attention_size():
    d = workloads.attention_qk()
    L, H, D = 28672, 32, 128
    _check(d["k"], 1, L, H, D, H * D, what=f"video self-attention V stand-in [{L}, {H}x{D}]")
    print("V FP8: video self-attention 28672 x 32 x 128 bit-exact", flush=True)
