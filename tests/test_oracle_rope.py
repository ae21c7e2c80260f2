"""Pins for the oracle's split-halves rotary position embedding (applied to
attention queries and keys ahead of their INT8 quantization; TurboT2VA paper,
architecture-aware inference stack, fused-kernels paragraph).

Hand-worked cases (tests/golden/rope_examples.json: a 3-4-5 angle, the
absence of fused multiply-adds, bf16 ties, the split pairing, the table
indexed by position and shared by heads), the special angles that reduce it
to identity, negation and the rotate-half map exactly, the complex product
it computes (checked in fp64 within the fp32 and bf16 rounding bound), the
locality of rows, heads and padding columns, and agreement with the
independent numpy oracle.
"""
import numpy as np

import oracle
from oracle import ref_tiny
from conftest import load_golden
from block_quantized_int8_amd.workloads import bf16_bits_to_f32, random_bf16, rope_tables


def hx16(v):
    return np.array([int(s, 16) for s in v], np.uint16)


def hx32(v):
    return np.array([int(s, 16) for s in v], np.uint32).view(np.float32)


def test_golden_cases():
    for c in load_golden("rope_examples.json")["cases"]:
        B, L, H, D = c["B"], c["L"], c["H"], c["D"]
        x = hx16(c["x"]).reshape(B * L, H * D)
        cs = hx32(c["cos"]).reshape(L, D // 2)
        sn = hx32(c["sin"]).reshape(L, D // 2)
        want = hx16(c["y"]).reshape(B * L, H * D)
        assert np.array_equal(oracle.rope(x, B, L, H, D, H * D, cs, sn), want), c["note"]
        assert np.array_equal(ref_tiny.rope(x, B, L, H, D, H * D, cs, sn), want), c["note"]


def _nonzero(seed, shape):
    x = random_bf16(seed, shape)
    x[(x & 0x7FFF) == 0] = 0x3F80  # +-0 would make -0 - (+0) style sign cases
    return x


def _const(L, D, c, s):
    return np.full((L, D // 2), c, np.float32), np.full((L, D // 2), s, np.float32)


def test_special_angles():
    B, L, H, D = 2, 5, 3, 64
    ld = H * D + 16
    x = _nonzero(21, (B * L, ld))
    xh = x[:, :H * D].reshape(B * L, H, 2, D // 2)
    lo, hi = xh[:, :, 0], xh[:, :, 1]
    neg = np.uint16(0x8000)
    cases = {(1.0, 0.0): (lo, hi), (-1.0, 0.0): (lo ^ neg, hi ^ neg),
             (0.0, 1.0): (hi ^ neg, lo), (0.0, -1.0): (hi, lo ^ neg)}
    for (c, s), (a, b) in cases.items():
        y = oracle.rope(x, B, L, H, D, ld, *_const(L, D, c, s)).reshape(B * L, H, 2, D // 2)
        assert np.array_equal(y[:, :, 0], a), (c, s)
        assert np.array_equal(y[:, :, 1], b), (c, s)


def test_is_the_complex_rotation():
    # (x_d + i x_{d+D/2}) * (c + i s), exact in fp64; the oracle's result
    # differs from it by at most the fp32 roundings of two products and one
    # sum, then one bf16 rounding
    B, L, H, D = 2, 37, 2, 128
    x = random_bf16(22, (B * L, H * D), 2.0)
    cs, sn = rope_tables(L, D)
    y = bf16_bits_to_f32(oracle.rope(x, B, L, H, D, H * D, cs, sn)).astype(np.float64)
    xf = bf16_bits_to_f32(x).astype(np.float64).reshape(B, L, H, 2, D // 2)
    z = (xf[:, :, :, 0] + 1j * xf[:, :, :, 1]) * (cs.astype(np.float64) + 1j * sn.astype(np.float64))[None, :, None, :]
    want = np.stack([z.real, z.imag], axis=3).reshape(B * L, H * D)
    mag = np.stack([np.abs(xf[:, :, :, 0] * cs[None, :, None, :]) + np.abs(xf[:, :, :, 1] * sn[None, :, None, :]),
                    np.abs(xf[:, :, :, 1] * cs[None, :, None, :]) + np.abs(xf[:, :, :, 0] * sn[None, :, None, :])],
                   axis=3).reshape(B * L, H * D)
    bound = np.abs(want) * 2.0 ** -8 + mag * 2.0 ** -22 + 2.0 ** -133
    assert np.all(np.abs(y - want) <= bound)
    # and a real rotation: the mean pair norm is kept (c^2 + s^2 = 1)
    assert abs(np.sum(y * y) / np.sum(want * want) - 1.0) < 1e-3


def test_rows_heads_and_padding_are_independent():
    B, L, H, D = 3, 9, 4, 64
    ld = H * D + 8
    x = random_bf16(23, (B * L, ld))
    cs, sn = rope_tables(L, D)
    y = oracle.rope(x, B, L, H, D, ld, cs, sn)
    # padding columns are never read
    xp = x.copy()
    xp[:, H * D:] = 0x7F80
    assert np.array_equal(oracle.rope(xp, B, L, H, D, ld, cs, sn), y)
    # each batch entry alone, each head alone
    for b in range(B):
        yb = oracle.rope(x[b * L:(b + 1) * L], 1, L, H, D, ld, cs, sn)
        assert np.array_equal(yb, y[b * L:(b + 1) * L])
    for h in range(H):
        xh = np.ascontiguousarray(x[:, h * D:(h + 1) * D])
        assert np.array_equal(oracle.rope(xh, B, L, 1, D, D, cs, sn), y[:, h * D:(h + 1) * D])


def test_identity_angle_leaves_qk_quantization_unchanged():
    B, L, H, D = 1, 200, 2, 128
    x = _nonzero(24, (B * L, H * D))
    q0, s0 = oracle.quantize_qk(x, B, L, H, D, H * D)
    q1, s1 = oracle.rope_quantize_qk(x, B, L, H, D, H * D, *_const(L, D, 1.0, 0.0))
    assert np.array_equal(q0, q1) and np.array_equal(s0, s1)


def test_matches_ref_tiny():
    for (B, L, H, D, ld, seed) in [(1, 7, 1, 8, 8, 30), (2, 5, 3, 64, 200, 31), (1, 3, 2, 128, 256, 32)]:
        x = random_bf16(seed, (B * L, ld), 4.0)
        cs, sn = rope_tables(L, D)
        assert np.array_equal(oracle.rope(x, B, L, H, D, ld, cs, sn), ref_tiny.rope(x, B, L, H, D, ld, cs, sn))
