"""INT8 attention Q/K on the GPU vs the oracle: codes and scales bit for bit,
sequence-major input (strided views included) to head-major output, ragged
token counts, and the video self-attention size."""
import numpy as np
import pytest
import torch

import block_quantized_int8_amd as w8a8
import oracle
from block_quantized_int8_amd import workloads
from block_quantized_int8_amd.workloads import f32_to_bf16_bits, random_bf16
from conftest import load_golden
from parity import to_dev_bf16

pytestmark = pytest.mark.gpu


def _check(xbits, B, L, H, D, ld, col0=0, what=""):
    """xbits: [B*L, ld_total] bf16 bits; the tensor is the column slice
    [col0, col0 + H*D) (row stride ld_total)."""
    dev = to_dev_bf16(xbits)
    view = dev[:, col0:col0 + H * D].view(B, L, H * D) if B > 1 else dev[:, col0:col0 + H * D]
    q, s = w8a8.quantize_qk(view, H)
    torch.cuda.synchronize()
    oq, os_ = oracle.quantize_qk(np.ascontiguousarray(xbits[:, col0:col0 + H * D]), B, L, H, D, H * D)
    qg, sg = q.cpu().numpy().reshape(B, H, L, D), s.cpu().numpy().reshape(B, H, -1)
    assert np.array_equal(sg.view(np.uint32), os_.view(np.uint32)), f"{what}: scales differ"
    if not np.array_equal(qg, oq):
        bad = np.argwhere(qg != oq)
        raise AssertionError(f"{what}: {len(bad)} codes differ, first at {tuple(bad[0])}")
    return qg, sg


def test_qk_golden_on_gpu():
    g = load_golden("quantize_qk_examples.json")
    B, L, H, D, ld = g["B"], g["L"], g["H"], g["D"], g["ld"]
    x = np.zeros((B * L, ld), np.float32)
    x[:, H * D:] = g["padding_value"]
    for r, c, v in g["values"]:
        x[r, c] = v
    xb = f32_to_bf16_bits(x)
    q, s = w8a8.quantize_qk(to_dev_bf16(xb)[:, :H * D], H)  # 2-D view: [L, H*D], row stride ld
    torch.cuda.synchronize()
    q, s = q.cpu().numpy(), s.cpu().numpy()
    for b, h, j, bits in g["scales"]:
        assert int(s.view(np.uint32)[h, j]) == int(bits, 16), (b, h, j)
    want = np.zeros((H, L, D), np.int8)
    for b, h, l, d, v in g["codes"]:
        want[h, l, d] = v
    assert np.array_equal(q, want)


@pytest.mark.parametrize("B,L,H,D,extra,col0", [(1, 128, 1, 128, 0, 0), (2, 200, 3, 64, 8, 0),
                                                (1, 1, 4, 128, 0, 0), (3, 257, 2, 128, 128, 128),
                                                (2, 384, 4, 64, 512, 256), (1, 1000, 16, 64, 0, 0)])
def test_qk_random_vs_oracle(B, L, H, D, extra, col0):
    ld = col0 + H * D + extra
    x = random_bf16(B * 1000 + L, (B * L, ld), 1.5)
    _check(x, B, L, H, D, ld, col0, f"qk B={B} L={L} H={H} D={D} ld={ld} col0={col0}")


def test_qk_edge_blocks():
    # all-zero block, tiny-scale block, huge block, one nonzero in a ragged tail
    B, L, H, D = 1, 300, 2, 64
    x = np.zeros((L, H * D), np.float32)
    rng = np.random.default_rng(5)
    x[128:256, :D] = rng.standard_normal((128, D)).astype(np.float32) * np.float32(1e-30)
    x[0:128, D:] = rng.standard_normal((128, D)).astype(np.float32) * np.float32(1e37)
    x[299, D + 63] = -3.0
    qg, sg = _check(f32_to_bf16_bits(x), B, L, H, D, H * D, 0, "qk edge blocks")
    assert sg[0, 0, 0] == 0 and sg[0, 0, 1] < 2 ** -60 and sg[0, 1, 0] > 1e35
    assert qg[0, 1, 299, 63] == -127 and np.count_nonzero(qg[0, 1, 256:]) == 1


def test_qk_from_projection_group():
    # Q and K views of a fused Q/K/V output (row stride 3 * H * D) quantize
    # exactly like contiguous copies of themselves
    H, D, K = 4, 64, 256
    ws = [to_dev_bf16(random_bf16(60 + i, (H * D, K), 0.02)) for i in range(3)]
    grp = w8a8.W8A8ProjectionGroup(ws)
    q, k, v = grp(to_dev_bf16(random_bf16(63, (2, 384, K))))
    for t in (q, k):
        a = w8a8.quantize_qk(t, H)
        b = w8a8.quantize_qk(t.contiguous(), H)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))
        assert a[0].shape == (2, H, 384, D) and a[1].shape == (2, H, 3)


def test_qk_video_self_attention_size():
    d = workloads.attention_qk()
    L, H, D = 28672, 32, 128
    for name in ("q", "k"):
        _check(d[name], 1, L, H, D, H * D, 0, f"video self-attention {name} [{L}, {H}x{D}]")
    a = workloads.attention_qk(l=251, heads=16, d=64, seed=7)  # short, ragged audio-like sequence
    _check(a["k"], 1, 251, 16, 64, 16 * 64, 0, "audio-like K [251, 16x64]")
    print("Q/K INT8: video self-attention 28672 x 32 x 128 and a ragged 251-token sequence bit-exact", flush=True)
