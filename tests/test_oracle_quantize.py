"""Pins for the oracle's 128x128 block-absmax INT8 quantization.

The oracle is checked against hand-worked examples (tests/golden), against
invariants that the rule s = max|x|/127, q = rint(x/s) implies, and against a
brute-force error bound; none of these re-types the oracle's own code.
"""
import numpy as np
import pytest

import oracle
from block_quantized_int8_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits, random_bf16
from conftest import load_golden


def _bf16(vals):
    v = np.asarray(vals, np.float32)
    b = f32_to_bf16_bits(v)
    assert np.array_equal(bf16_bits_to_f32(b), v), "fixture value not bf16-exact"
    return b


def test_golden_examples():
    g = load_golden("quantize_examples.json")
    rng = np.random.default_rng(11)
    for blk in g["blocks"]:
        x = np.zeros((128, 128), np.uint16)
        pos = rng.choice(128 * 128, len(blk["cases"]), replace=False)
        vals = [c[0] for c in blk["cases"]]
        x.reshape(-1)[pos] = _bf16(vals)
        q, s = oracle.quantize_block(x)
        assert s.shape == (1, 1)
        if blk["s_bits"] is not None:
            assert int(s.view(np.uint32)[0, 0]) == int(blk["s_bits"], 16), blk
        got = q.reshape(-1)[pos].tolist()
        want = [c[1] for c in blk["cases"]]
        assert got == want, (blk["absmax"], got, want)
        # everything else in the block is zero
        rest = np.delete(q.reshape(-1), pos)
        assert not rest.any()


def test_zero_block_and_layout():
    # 256 x 384: 2 x 3 blocks; block (1, 2) all zero, others with distinct absmax
    x = np.zeros((256, 384), np.float32)
    absmax = {(0, 0): 1.0, (0, 1): 2.0, (0, 2): 4.0, (1, 0): 8.0, (1, 1): 16.0}
    for (i, j), a in absmax.items():
        x[i * 128 + 5, j * 128 + 7] = -a  # negative absmax element
        x[i * 128 + 100, j * 128 + 1] = a / 4
    q, s = oracle.quantize_block(f32_to_bf16_bits(x))
    assert s.shape == (2, 3)
    for (i, j), a in absmax.items():
        assert s[i, j] == np.float32(a) / np.float32(127)
        assert q[i * 128 + 5, j * 128 + 7] == -127
        # a/4 / (a/127) = 31.75 -> 32
        assert q[i * 128 + 100, j * 128 + 1] == 32
    assert s[1, 2] == 0.0
    assert not q[128:, 256:].any()


def test_invariants_random():
    x = random_bf16(3, (384, 256), 1.5)
    q, s = oracle.quantize_block(x)
    xf = bf16_bits_to_f32(x)
    assert q.dtype == np.int8 and q.min() >= -127 and q.max() <= 127
    for i in range(3):
        for j in range(2):
            blk = xf[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            qb = q[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            a = np.abs(blk).max()
            # exactly +-127 wherever |x| attains the block absmax
            hit = np.abs(blk) == a
            assert np.all(np.abs(qb[hit]) == 127)
            assert np.all(np.sign(qb[hit]) == np.sign(blk[hit]))
            # brute-force reconstruction error: |q*s - x| <= s/2 (plus the
            # fp32 quotient's half-ulp, scaled back)
            sc = float(s[i, j])
            err = np.abs(qb.astype(np.float64) * sc - blk.astype(np.float64))
            assert err.max() <= sc * (0.5 + 1e-5)
    # sign symmetry
    qn, sn = oracle.quantize_block(x ^ np.uint16(0x8000))
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)


@pytest.mark.parametrize("e", [-7, -1, 3, 20])
def test_power_of_two_scaling(e):
    x = random_bf16(5, (256, 256))
    xf = bf16_bits_to_f32(x)
    x2 = f32_to_bf16_bits(xf * np.float32(2.0 ** e))
    assert np.array_equal(bf16_bits_to_f32(x2), xf * np.float32(2.0 ** e))
    q, s = oracle.quantize_block(x)
    q2, s2 = oracle.quantize_block(x2)
    assert np.array_equal(q2, q)
    assert np.array_equal(s2, s * np.float32(2.0 ** e))


def test_block_locality():
    x = random_bf16(6, (256, 384))
    q, s = oracle.quantize_block(x)
    y = x.copy()
    y[128:256, 128:256] = random_bf16(7, (128, 128), 50.0)
    q2, s2 = oracle.quantize_block(y)
    mask = np.ones((256, 384), bool)
    mask[128:256, 128:256] = False
    assert np.array_equal(q[mask], q2[mask])
    smask = np.ones((2, 3), bool)
    smask[1, 1] = False
    assert np.array_equal(s[smask], s2[smask])
    assert s2[1, 1] != s[1, 1]


def test_subnormal_block():
    # absmax in the bf16 subnormal range: s = a/127 is an fp32 subnormal
    a = np.float32(2.0 ** -130)
    x = np.zeros((128, 128), np.float32)
    x[0, 0] = a
    x[3, 3] = -a
    x[7, 9] = np.float32(2.0 ** -133)
    q, s = oracle.quantize_block(f32_to_bf16_bits(x))
    assert s[0, 0] == a / np.float32(127)
    assert q[0, 0] == 127 and q[3, 3] == -127
    # 2^-133 / (2^-130/127) = 127/8 = 15.875 (up to the fp32 rounding of s) -> 16
    assert q[7, 9] == 16


def test_rejects_unaligned_shape():
    with pytest.raises(ValueError):
        oracle.quantize_block(np.zeros((128, 130), np.uint16))
