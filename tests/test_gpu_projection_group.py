"""Shared-input projection group (Q/K/V, cross-attention K/V) on the GPU: one
quantize and one GEMM over the concatenated output channels; each view is
bit-identical to its projection run alone and within tolerance of the
oracle; misaligned groups take the bf16 fallback."""
import numpy as np
import pytest
import torch

import block_quantized_int8_amd as w8a8
import oracle
from block_quantized_int8_amd import workloads
from block_quantized_int8_amd.workloads import random_bf16
from parity import assert_bf16_close, bf16_bits, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("scaling", ["block", "postscale"])
def test_qkv_group_equals_separate_projections(scaling):
    K, splits = 512, [256, 128, 384]
    ws = [random_bf16(10 + i, (n, K), 0.02) for i, n in enumerate(splits)]
    bs = [random_bf16(20, (splits[0],), 0.1), None, random_bf16(22, (splits[2],), 0.1)]
    x = random_bf16(30, (2, 256, K), 1.0)
    grp = w8a8.W8A8ProjectionGroup([to_dev_bf16(w) for w in ws],
                                   [None if b is None else to_dev_bf16(b) for b in bs], scaling=scaling)
    outs = grp(to_dev_bf16(x))
    assert grp.last_path == w8a8.PATH_INT8
    assert [o.shape for o in outs] == [(2, 256, n) for n in splits]
    for i, (w, b, o) in enumerate(zip(ws, bs, outs)):
        alone = w8a8.W8A8Linear(to_dev_bf16(w), None if b is None else to_dev_bf16(b), scaling=scaling)
        ya = alone(to_dev_bf16(x))
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(o), bf16_bits(ya)), f"projection {i} differs from running it alone"
    # vs the oracle on the concatenated weight
    wcat = np.concatenate(ws, 0)
    bcat = np.concatenate([b if b is not None else np.zeros(n, np.uint16) for b, n in zip(bs, splits)])
    xf = x.reshape(-1, K)
    if scaling == "block":
        oq, os_ = oracle.quantize_block(xf)
        oqw, osw = oracle.quantize_block(wcat)
        assert np.array_equal(grp.linear.qweight.cpu().numpy(), oqw)
        yo = oracle.linear_int8(oq, os_, oqw, osw, bias=bcat)
    else:
        oq, os_ = oracle.quantize_rows(xf)
        oqw, osw = oracle.quantize_rows(wcat)
        yo = oracle.linear_postscale(oq, os_, oqw, osw, bias=bcat)
    yg = np.concatenate([bf16_bits(o).reshape(-1, n) for o, n in zip(outs, splits)], 1)
    assert_bf16_close(yg, yo, f"QKV group ({scaling})")


def test_cross_attention_kv_group_and_guards():
    K = 256
    wk, wv = random_bf16(40, (256, K), 0.02), random_bf16(41, (256, K), 0.02)
    grp = w8a8.W8A8ProjectionGroup([to_dev_bf16(wk), to_dev_bf16(wv)])
    ctx = random_bf16(42, (384, K))
    k, v = grp(to_dev_bf16(ctx))
    torch.cuda.synchronize()
    assert grp.last_path == w8a8.PATH_INT8
    oq, os_ = oracle.quantize_block(ctx)
    oqw, osw = oracle.quantize_block(np.concatenate([wk, wv], 0))
    yo = oracle.linear_int8(oq, os_, oqw, osw)
    assert_bf16_close(np.concatenate([bf16_bits(k), bf16_bits(v)], 1), yo, "cross-attention KV group")
    # a ragged context length (M = 77 text tokens) falls back, views still split
    ctx2 = random_bf16(43, (77, K))
    k2, v2 = grp(to_dev_bf16(ctx2))
    torch.cuda.synchronize()
    assert grp.last_path == w8a8.PATH_BF16 and k2.shape == (77, 256) and v2.shape == (77, 256)
    yo2 = oracle.linear_bf16(ctx2, oracle.DTYPE_BF16, np.concatenate([wk, wv], 0))
    assert_bf16_close(np.concatenate([bf16_bits(k2), bf16_bits(v2)], 1), yo2, "KV group fallback")
    # a projection width that is not a multiple of 128 (block boundaries would
    # straddle projections): the whole group stays on the bf16 path
    wa, wb = random_bf16(44, (192, K), 0.02), random_bf16(45, (64, K), 0.02)
    g2 = w8a8.W8A8ProjectionGroup([to_dev_bf16(wa), to_dev_bf16(wb)])
    a, b = g2(to_dev_bf16(ctx))
    torch.cuda.synchronize()
    assert g2.last_path == w8a8.PATH_BF16 and g2.linear.qweight is None
    yo3 = oracle.linear_bf16(ctx, oracle.DTYPE_BF16, np.concatenate([wa, wb], 0))
    assert_bf16_close(np.concatenate([bf16_bits(a), bf16_bits(b)], 1), yo3, "misaligned group fallback")


def test_qkv_group_attention_projection_shape():
    # Q, K, V of the attention-projection workload's input: 32768 x 4096 -> 3 x 4096
    d = workloads.attention_projection()
    wq = d["w"]
    wk = random_bf16(51, (4096, 4096), 0.02)
    wv = random_bf16(52, (4096, 4096), 0.02)
    grp = w8a8.W8A8ProjectionGroup([to_dev_bf16(w) for w in (wq, wk, wv)])
    q, k, v = grp(to_dev_bf16(d["x"]))
    torch.cuda.synchronize()
    assert grp.last_path == w8a8.PATH_INT8
    rows = workloads.sample_rows(17, 32768, extra=256)
    oq, os_ = oracle.quantize_block(d["x"])
    for name, w, o in (("Q", wq, q), ("K", wk, k), ("V", wv, v)):
        oqw, osw = oracle.quantize_block(w)
        assert_bf16_close(bf16_bits(o)[rows], oracle.linear_int8(oq, os_, oqw, osw, rows=rows),
                          f"QKV group {name} 32768x4096x4096")
