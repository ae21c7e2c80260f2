"""GPU block quantization vs the oracle: codes and scales bit-exact."""
import numpy as np
import pytest
import torch

import block_quantized_int8_amd as w8a8
import oracle
from block_quantized_int8_amd.workloads import single_linear_256, f32_to_bf16_bits, random_bf16
from conftest import load_golden
from parity import to_dev_bf16

pytestmark = pytest.mark.gpu


def _gpu_quant(bits, weight=False):
    x = to_dev_bf16(bits)
    q, s = (w8a8.quantize_weight if weight else w8a8.quantize_act)(x)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def _assert_same(bits, weight=False, what=""):
    q, s = _gpu_quant(bits, weight)
    oq, os_ = oracle.quantize_block(bits)
    assert np.array_equal(s.view(np.uint32), os_.view(np.uint32)), f"{what}: scales differ"
    if not np.array_equal(q, oq):
        bad = np.argwhere(q != oq)
        r, c = bad[0]
        raise AssertionError(f"{what}: {len(bad)} codes differ, first at {r},{c}: "
                             f"gpu {q[r, c]} oracle {oq[r, c]} x_bits {bits[r, c]:#06x}")


def test_single_linear_256_weight_and_activation():
    d = single_linear_256()
    _assert_same(d["x"], False, "single linear 256^3: x")
    _assert_same(d["w"], True, "single linear 256^3: w")


@pytest.mark.parametrize("shape,scale,seed", [((384, 640), 1.0, 1), ((128, 128), 3e-3, 2),
                                              ((1024, 256), 1e4, 3), ((256, 1152), 0.02, 4)])
def test_random_shapes(shape, scale, seed):
    _assert_same(random_bf16(seed, shape, scale), False, f"random {shape}")


def test_golden_blocks_on_gpu():
    g = load_golden("quantize_examples.json")
    rng = np.random.default_rng(11)
    blocks = []
    for blk in g["blocks"]:
        x = np.zeros((128, 128), np.uint16)
        pos = rng.choice(128 * 128, len(blk["cases"]), replace=False)
        x.reshape(-1)[pos] = f32_to_bf16_bits(np.array([c[0] for c in blk["cases"]], np.float32))
        blocks.append((x, pos, blk))
    big = np.concatenate([b[0] for b in blocks], axis=1)  # 128 x (128 * nblocks)
    q, s = _gpu_quant(big)
    for i, (x, pos, blk) in enumerate(blocks):
        qb = q[:, i * 128:(i + 1) * 128]
        assert qb.reshape(-1)[pos].tolist() == [c[1] for c in blk["cases"]], blk["absmax"]
        if blk["s_bits"] is not None:
            assert int(s.view(np.uint32)[0, i]) == int(blk["s_bits"], 16)


def test_zero_subnormal_and_huge_blocks():
    x = np.zeros((256, 512), np.float32)
    x[0:128, 128:256] = 2.0 ** -130                  # subnormal absmax
    x[3, 130] = -(2.0 ** -128)
    x[128:256, 0:128] = np.float32(3.0e38)           # near the bf16 maximum
    x[200, 5] = -3.3e38
    x[0:128, 256:384] = np.linspace(-1, 1, 128 * 128, dtype=np.float32).reshape(128, 128) * 2.0 ** -100
    x[128:256, 384:512] = 2.0 ** -133                # smallest subnormal only
    bits = f32_to_bf16_bits(x)
    _assert_same(bits, False, "edge blocks")
    q, s = _gpu_quant(bits)
    assert s[0, 0] == 0 and not q[0:128, 0:128].any()  # all-zero block


def _exhaustive_pairs():
    """Every positive finite bf16 absmax a with every bf16 magnitude x <= a
    (both signs alternating), one absmax per tile group: ~5.3e8 elements."""
    per = 128 * 128 - 1
    tiles = []
    for ab in range(1, 0x7F80):
        xs = np.arange(0, ab + 1, dtype=np.uint16)
        xs[1::2] |= 0x8000
        n = -(-xs.size // per)
        buf = np.zeros((n, per + 1), np.uint16)
        buf[:, 0] = ab | (0x8000 if ab & 1 else 0)
        flat = buf[:, 1:].reshape(-1)
        flat[:xs.size] = xs
        tiles.append(buf)
    return np.concatenate(tiles).reshape(-1, 128)


def test_exhaustive_bf16_domain():
    bits = _exhaustive_pairs()
    print(f"exhaustive domain: {bits.shape[0] // 128} tiles, {bits.size} elements", flush=True)
    _assert_same(bits, False, "exhaustive bf16 (absmax, x) domain")
