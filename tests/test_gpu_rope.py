"""Split-halves rotary embedding of Q/K on the GPU, alone (bf16) and fused
into the INT8 Q/K quantizer, vs the oracle.  The rotation is a fixed sequence
of fp32 operations and one bf16 rounding, so the bf16 output is compared bit
for bit, like the codes and scales."""
import numpy as np
import pytest
import torch

import block_quantized_int8_amd as w8a8
import oracle
from block_quantized_int8_amd import workloads
from block_quantized_int8_amd.workloads import random_bf16, rope_tables
from conftest import load_golden
from parity import bf16_bits, to_dev_bf16

pytestmark = pytest.mark.gpu


def _tables_dev(cs, sn):
    return torch.from_numpy(cs).cuda(), torch.from_numpy(sn).cuda()


def _run(xbits, B, L, H, D, col0, cs, sn, what):
    """xbits [B*L, ld_total]; the tensor is the column slice [col0, col0 + H*D)."""
    dev = to_dev_bf16(xbits)
    view = dev[:, col0:col0 + H * D].view(B, L, H * D)
    c, s = _tables_dev(cs, sn)
    y = w8a8.rope_bf16(view, H, c, s)
    qf, sf = w8a8.rope_quantize_qk(view, H, c, s)
    qu, su = w8a8.quantize_qk(y, H)
    torch.cuda.synchronize()
    xs = np.ascontiguousarray(xbits[:, col0:col0 + H * D])
    oy = oracle.rope(xs, B, L, H, D, H * D, cs, sn)
    gy = bf16_bits(y).reshape(B * L, H * D)
    if not np.array_equal(gy, oy):
        bad = np.argwhere(gy != oy)
        raise AssertionError(f"{what}: {len(bad)} rotated values differ, first at {tuple(bad[0])}")
    oq, os_ = oracle.quantize_qk(oy, B, L, H, D, H * D)
    assert np.array_equal(sf.cpu().numpy().reshape(B, H, -1).view(np.uint32), os_.view(np.uint32)), what
    assert np.array_equal(qf.cpu().numpy().reshape(B, H, L, D), oq), what
    # the fused kernel equals the two-kernel chain on the device as well
    assert torch.equal(qf, qu) and torch.equal(sf.view(torch.int32), su.view(torch.int32)), what
    return gy


def test_rope_golden_pairs_on_gpu():
    # each single-pair golden case embedded as pair 0 of a 64-wide head
    # (elements 0 and 32, table column 0) among random pairs
    for n, c in enumerate(load_golden("rope_examples.json")["cases"]):
        if c["D"] != 2 or c["B"] * c["L"] * c["H"] != 1:
            continue
        x = random_bf16(700 + n, (1, 64))
        x[0, 0], x[0, 32] = (int(v, 16) for v in c["x"])
        cs, sn = rope_tables(1, 64)
        cs[0, 0] = np.uint32(int(c["cos"][0], 16)).view(np.float32)
        sn[0, 0] = np.uint32(int(c["sin"][0], 16)).view(np.float32)
        gy = _run(x, 1, 1, 1, 64, 0, cs, sn, c["note"][:40])
        assert [int(gy[0, 0]), int(gy[0, 32])] == [int(v, 16) for v in c["y"]], c["note"]


@pytest.mark.parametrize("B,L,H,D,extra,col0", [(1, 128, 1, 128, 0, 0), (2, 200, 3, 64, 8, 0),
                                                (1, 1, 4, 128, 0, 0), (3, 257, 2, 128, 128, 128),
                                                (2, 384, 4, 64, 512, 256), (1, 1000, 16, 64, 0, 0)])
def test_rope_random_vs_oracle(B, L, H, D, extra, col0):
    ld = col0 + H * D + extra
    x = random_bf16(B * 3000 + L, (B * L, ld), 1.5)
    cs, sn = rope_tables(L, D)
    _run(x, B, L, H, D, col0, cs, sn, f"rope B={B} L={L} H={H} D={D} ld={ld} col0={col0}")


def test_rope_special_angles_and_edges():
    # identity and rotate-half angles in alternate tokens, a zero block, a
    # tiny-scale block, a huge block, one nonzero value in a ragged tail
    B, L, H, D = 1, 300, 2, 64
    rng = np.random.default_rng(9)
    x = np.zeros((L, H * D), np.float32)
    x[128:256, :D] = rng.standard_normal((128, D)).astype(np.float32) * np.float32(1e-30)
    x[0:128, D:] = rng.standard_normal((128, D)).astype(np.float32) * np.float32(1e37)
    x[299, D + 63] = -3.0
    cs = np.zeros((L, D // 2), np.float32)
    sn = np.zeros((L, D // 2), np.float32)
    cs[0::2] = 1.0
    sn[1::2] = 1.0
    _run(workloads.f32_to_bf16_bits(x), B, L, H, D, 0, cs, sn, "special angles and edge blocks")


def test_rope_video_self_attention_size():
    # Q and K as column slices of a fused Q/K/V output [28672, 3 x 4096], the
    # latent grid 16 x 56 x 32 driving a three-axis table
    d = workloads.attention_qk()
    L, H, D = 28672, 32, 128
    cs, sn = rope_tables(L, D, grid=(16, 56, 32))
    qkv = np.zeros((L, 3 * H * D), np.uint16)
    qkv[:, :H * D] = d["q"]
    qkv[:, H * D:2 * H * D] = d["k"]
    for name, col0 in (("q", 0), ("k", H * D)):
        _run(qkv, 1, L, H, D, col0, cs, sn, f"video self-attention {name} [{L}, {H}x{D}]")
    print("rotary embedding (+ Q/K INT8): video self-attention 28672 x 32 x 128 bit-exact", flush=True)


def test_rope_argument_errors():
    x = torch.zeros((256, 2 * 128), dtype=torch.bfloat16, device="cuda")
    c = torch.zeros((256, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        w8a8.rope_bf16(x, 2, c[:, :32].contiguous(), c)        # wrong table shape
    with pytest.raises(ValueError):
        w8a8.rope_quantize_qk(x, 2, c.double(), c)             # wrong table dtype
    with pytest.raises(w8a8.W8A8Error):
        w8a8.rope_bf16(torch.zeros((256, 2 * 96), dtype=torch.bfloat16, device="cuda"), 2,
                       torch.zeros((256, 48), device="cuda"), torch.zeros((256, 48), device="cuda"))
