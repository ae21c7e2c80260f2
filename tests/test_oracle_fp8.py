"""Pins for the oracle's FP8 E4M3 conversion and the FP8 quantization of
attention V (TurboT2VA paper, architecture-aware inference stack,
sparse-attention paragraph).

Hand-worked codes (tests/golden/fp8_e4m3_examples.json: normals, the
largest value and the tie beyond it, mantissa ties, subnormals and their
ties), every finite code decoded and re-encoded to itself, the midpoints
between neighbouring codes and the floats next to them, a nearest-code
search over the whole table on random values, and for the V quantizer:
+-448 at each block's max-abs element, sign symmetry, exact power-of-two
scaling, block locality, the zero block and the numpy twin.
"""
import numpy as np

import oracle
from oracle import ref_tiny
from conftest import load_golden
from block_quantized_int8_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits, random_bf16


def test_golden_codes():
    for c in load_golden("fp8_e4m3_examples.json")["cases"]:
        assert oracle.f32_to_e4m3(c["x"]) == int(c["code"], 16), c["note"]
        assert oracle.f32_to_e4m3(-c["x"]) == int(c["code"], 16) ^ 0x80, c["note"]
        assert ref_tiny.e4m3_code(c["x"]) == int(c["code"], 16), c["note"]


def test_every_finite_code_round_trips():
    for code in range(256):
        if code & 0x7F == 0x7F:
            assert np.isnan(oracle.e4m3_to_f64(code))
            continue
        v = oracle.e4m3_to_f64(code)
        assert oracle.f32_to_e4m3(v) == code, hex(code)


def test_midpoints_and_their_neighbours():
    vals = [(oracle.e4m3_to_f64(c), c) for c in range(0x7F)]
    for (lo, clo), (hi, chi) in zip(vals, vals[1:]):
        mid = np.float32((lo + hi) / 2)          # exact: neighbours differ by one quantum
        even = clo if clo % 2 == 0 else chi
        assert oracle.f32_to_e4m3(float(mid)) == even, (lo, hi)
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(np.inf))
        assert oracle.f32_to_e4m3(float(below)) == clo and oracle.f32_to_e4m3(float(above)) == chi, (lo, hi)


def test_nearest_code_search():
    rng = np.random.default_rng(90)
    xs = np.concatenate([rng.uniform(-460, 460, 3000), rng.uniform(-0.02, 0.02, 2000),
                         rng.standard_normal(3000) * 4]).astype(np.float32)
    for v in xs:
        assert oracle.f32_to_e4m3(float(v)) == ref_tiny.e4m3_code(float(v)), float(v)


def test_v_quantizer_invariants():
    B, L, H, D = 2, 200, 3, 64
    ld = H * D + 8
    x = random_bf16(91, (B * L, ld), 1.5)
    q, s = oracle.quantize_v_fp8(x, B, L, H, D, ld)
    xf = bf16_bits_to_f32(x)[:, :H * D].reshape(B, L, H, D).transpose(0, 2, 1, 3)   # [B, H, L, D]
    for b in range(B):
        for h in range(H):
            for j in range(2):
                blk = xf[b, h, j * 128:(j + 1) * 128]
                k = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
                code = q[b, h, j * 128 + k[0], k[1]]
                assert code & 0x7F == 0x7E and (code >> 7) == (blk[k] < 0)
                assert s[b, h, j] == np.float32(np.float32(np.max(np.abs(blk))) / np.float32(448.0))
    qn, sn = oracle.quantize_v_fp8(x ^ np.uint16(0x8000), B, L, H, D, ld)
    assert np.array_equal(sn, s) and np.array_equal(qn, q ^ np.uint8(0x80))
    for e in (-3, 5):
        xe = f32_to_bf16_bits(bf16_bits_to_f32(x) * np.float32(2.0 ** e))
        qe, se = oracle.quantize_v_fp8(xe, B, L, H, D, ld)
        assert np.array_equal(qe, q) and np.array_equal(se, s * np.float32(2.0 ** e))
    # a zero block and block locality (padding columns never read)
    x2 = x.copy()
    x2[:128, :D] = 0
    x2[:, H * D:] = 0x7F7F
    q2, s2 = oracle.quantize_v_fp8(x2, B, L, H, D, ld)
    assert s2[0, 0, 0] == 0 and not q2[0, 0, :128].any()
    assert np.array_equal(q2[:, 1:], q[:, 1:]) and np.array_equal(q2[1], q[1])


def test_matches_ref_tiny():
    for B, L, H, D, seed in [(1, 130, 2, 8, 92), (2, 40, 1, 16, 93)]:
        x = random_bf16(seed, (B * L, H * D), 3.0)
        q, s = oracle.quantize_v_fp8(x, B, L, H, D, H * D)
        q2, s2 = ref_tiny.quantize_v_fp8(x, B, L, H, D, H * D)
        assert np.array_equal(s, s2) and np.array_equal(q, q2)
