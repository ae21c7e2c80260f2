"""Parity on the five synthetic transformer-linear workloads at full size.

Each test runs the guarded linear exactly as bench.py calls it (w8a8.linear
with a preallocated workspace) and checks against the oracle:
* activation and weight codes and scales: bit-exact, in full;
* per-K-block int32 partials: bit-exact on 8 output tiles of 128x128 (the
  first, the last and 6 seeded ones);
* bf16 output: within tolerance on a deterministic row sample (every row of
  the first, middle and last 128-row block plus seeded rows), which the
  oracle computes row by row.
Oracle inputs always come from the shared input generator or from the
oracle itself, never from the GPU.
"""
import numpy as np
import pytest
import torch

import block_quantized_int8_amd as w8a8
import oracle
from block_quantized_int8_amd import workloads
from parity import assert_bf16_close, bf16_bits, to_dev_bf16

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _check_codes(dev_q, dev_s, bits, what):
    oq, os_ = oracle.quantize_block(bits)
    assert np.array_equal(dev_s.cpu().numpy().view(np.uint32), os_.view(np.uint32)), f"{what}: scales differ"
    q = dev_q.cpu().numpy()
    if not np.array_equal(q, oq):
        bad = np.argwhere(q != oq)
        raise AssertionError(f"{what}: {len(bad)} codes differ, first at {tuple(bad[0])}")
    return oq, os_


def _tiles(seed, M, N, n=6):
    rng = np.random.default_rng(seed)
    mb, nb = M // 128, N // 128
    t = {(0, 0), (mb - 1, nb - 1)}
    while len(t) < min(n + 2, mb * nb):
        t.add((int(rng.integers(mb)), int(rng.integers(nb))))
    return sorted(t)


def _check_partials(qx_d, qw_d, oqx, oqw, seed, what):
    M, N = oqx.shape[0], oqw.shape[0]
    for (i, j) in _tiles(seed, M, N):
        p = w8a8.debug_kblock_partials(qx_d, qw_d, i * 128, 128, j * 128, 128).cpu().numpy()
        po = oracle.kblock_partials(oqx, oqw, i * 128, 128, j * 128, 128)
        assert np.array_equal(p, po), f"{what}: partials differ in tile ({i}, {j})"


def _int8_linear_case(x_bits, w_bits, seed, what, bias_bits=None):
    """Full INT8-path check of one linear; returns GPU output and oracle codes."""
    M, K = x_bits.shape
    N = w_bits.shape[0]
    _say(f"{what}: M={M} N={N} K={K}")
    xd, wd = to_dev_bf16(x_bits), to_dev_bf16(w_bits)
    qw, sw = w8a8.quantize_weight(wd)
    ws = torch.empty(w8a8.workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    bd = None if bias_bits is None else to_dev_bf16(bias_bits)
    _, path = w8a8.linear(xd, wd, qw, sw, bias=bd, out=y, workspace=ws)
    torch.cuda.synchronize()
    assert path == w8a8.PATH_INT8
    # the activation codes the linear used are in the workspace
    qx = ws[:M * K].view(torch.int8).view(M, K)
    so = (M * K + 255) // 256 * 256
    sx = ws[so:so + (M // 128) * (K // 128) * 4].view(torch.float32).view(M // 128, K // 128)
    oqx, osx = _check_codes(qx, sx, x_bits, f"{what} activations")
    oqw, osw = _check_codes(qw, sw, w_bits, f"{what} weights")
    _check_partials(qx, qw, oqx, oqw, seed, what)
    rows = workloads.sample_rows(seed, M)
    yo = oracle.linear_int8(oqx, osx, oqw, osw, bias=bias_bits, rows=rows)
    rel = assert_bf16_close(bf16_bits(y)[rows], yo, what)
    _say(f"{what}: codes, scales and 8 partial tiles bit-exact; {rows.size} rows rel err {rel:.2e}")
    return y, (oqx, osx, oqw, osw)


def test_single_linear_256():
    d = workloads.single_linear_256()
    y, (oqx, osx, oqw, osw) = _int8_linear_case(d["x"], d["w"], 10, "single linear 256^3")
    # small enough for the whole output and all partials
    assert_bf16_close(bf16_bits(y), oracle.linear_int8(oqx, osx, oqw, osw), "single linear, all rows")


def test_square_4096_and_guard():
    d = workloads.square_4096()
    _int8_linear_case(d["x"], d["w"], 11, "square 4096^3")
    # guard case: M = 4000 is not a multiple of 128 -> bf16 fallback
    wd = to_dev_bf16(d["w"])
    qw, sw = w8a8.quantize_weight(wd)
    y, path = w8a8.linear(to_dev_bf16(d["x_guard"]), wd, qw, sw)
    torch.cuda.synchronize()
    assert path == w8a8.PATH_BF16
    rows = np.unique(np.concatenate([np.arange(0, 128), np.arange(3872, 4000),
                                     np.random.default_rng(12).integers(0, 4000, 128)]))
    yo = oracle.linear_bf16(d["x_guard"], oracle.DTYPE_BF16, d["w"], rows=rows)
    rel = assert_bf16_close(bf16_bits(y)[rows], yo, "square guard M=4000")
    _say(f"guard case routed to bf16 fallback; {rows.size} rows rel err {rel:.2e}")


def test_attention_projection_32768():
    d = workloads.attention_projection()
    _int8_linear_case(d["x"], d["w"], 13, "attention projection 32768x4096x4096")


def test_mlp_pair():
    d = workloads.mlp_pair()
    M = 32768
    y_up, (oqx, osx, oqw_up, osw_up) = _int8_linear_case(d["x"], d["w_up"], 14, "MLP up 32768x16384x4096")
    # producer between the two linears: the library's exact GELU fused into
    # the down projection's activation quantization
    wd_down = to_dev_bf16(d["w_down"])
    down = w8a8.W8A8Linear(wd_down)
    qw_down, sw_down = down.qweight, down.wscale
    oqw_down, osw_down = _check_codes(qw_down, sw_down, d["w_down"], "MLP down weights")
    y_down = down.forward_gelu(y_up)
    torch.cuda.synchronize()
    assert down.last_path == w8a8.PATH_INT8
    # the unfused library chain (GELU written out, then the guarded linear) is bit-identical
    y_unfused, path = w8a8.linear(w8a8.gelu_bf16(y_up), wd_down, qw_down, sw_down)
    torch.cuda.synchronize()
    assert path == w8a8.PATH_INT8 and torch.equal(y_down.view(torch.int16), y_unfused.view(torch.int16))
    del y_up, y_unfused
    # oracle chain on three 128-row blocks: its own up-projection rows, its
    # own GELU, its own requantization, then the down projection
    blocks = [0, M // 256, M // 128 - 1]
    rows = np.concatenate([np.arange(b * 128, (b + 1) * 128) for b in blocks])
    yo_up = oracle.linear_int8(oqx, osx, oqw_up, osw_up, rows=rows)
    xo = oracle.gelu_bf16(yo_up)                       # [384, 16384] bf16 bits
    oqx2, osx2 = oracle.quantize_block(xo)
    # the GPU quantizer on the oracle's X' rows: bit-exact requantization
    q2, s2 = w8a8.quantize_act(to_dev_bf16(xo))
    _check_codes(q2, s2, xo, "MLP down requantization of X'")
    # the fused GELU + quantize on the oracle's up-projection rows: bit-exact too
    q3, s3 = w8a8.gelu_quantize_act(to_dev_bf16(yo_up))
    _check_codes(q3, s3, xo, "MLP fused GELU + quantize of the oracle's up-projection rows")
    # the GPU GEMM on those codes vs the oracle's down projection
    yg_blocks = w8a8.gemm_blockscale(q2, s2, qw_down, sw_down)
    yo_down = oracle.linear_int8(oqx2, osx2, oqw_down, osw_down)
    rel1 = assert_bf16_close(bf16_bits(yg_blocks), yo_down, "MLP down on the oracle's X'")
    # the GPU's own end-to-end chain on the same rows
    rel2 = assert_bf16_close(bf16_bits(y_down)[rows], yo_down, "MLP chained end to end")
    _say(f"MLP pair: down on oracle X' rel {rel1:.2e}; chained rel {rel2:.2e}")


def test_two_stream_step():
    d = workloads.two_stream()
    xa, wa = to_dev_bf16(d["x_a"]), to_dev_bf16(d["w_a"])
    xb, wb = to_dev_bf16(d["x_b"]), to_dev_bf16(d["w_b"])
    la, lb = w8a8.W8A8Linear(wa), w8a8.W8A8Linear(wb)
    assert lb.qweight is not None  # B's weight is 2048x2048: quantized, yet M=1000 falls back
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(sa):
        ya = la(xa)
    with torch.cuda.stream(sb):
        yb = lb(xb)
    torch.cuda.synchronize()
    assert la.last_path == w8a8.PATH_INT8 and lb.last_path == w8a8.PATH_BF16
    oqx, osx = oracle.quantize_block(d["x_a"])
    oqw, osw = oracle.quantize_block(d["w_a"])
    rows = workloads.sample_rows(15, 65536)
    rel_a = assert_bf16_close(bf16_bits(ya)[rows], oracle.linear_int8(oqx, osx, oqw, osw, rows=rows),
                              "two-stream A 65536x4096x4096")
    rel_b = assert_bf16_close(bf16_bits(yb), oracle.linear_bf16(d["x_b"], oracle.DTYPE_BF16, d["w_b"]),
                              "two-stream B 1000x2048x2048 (fallback)")
    _say(f"two-stream step: A (INT8) rel {rel_a:.2e}, B (bf16 fallback) rel {rel_b:.2e}")
