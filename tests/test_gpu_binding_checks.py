"""The torch-facing binding refuses undersized or mismatched buffers before
any launch (so no kernel can be pointed past a tensor)."""
import pytest
import torch

import block_quantized_int8_amd as w8a8

pytestmark = pytest.mark.gpu


def z(shape, dtype):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def test_gemm_operand_sizes():
    qx, qw = z((256, 256), torch.int8), z((384, 256), torch.int8)
    sx, sw = z((2, 2), torch.float32), z((3, 2), torch.float32)
    w8a8.gemm_blockscale(qx, sx, qw, sw)
    bad = [dict(sx=z((2, 1), torch.float32)), dict(sw=z((2, 2), torch.float32)),
           dict(bias=z((383,), torch.bfloat16)), dict(out=z((256, 383), torch.bfloat16)),
           dict(qw=z((384, 128), torch.int8))]
    for b in bad:
        a = dict(qx=qx, sx=sx, qw=qw, sw=sw)
        a.update(b)
        with pytest.raises(ValueError):
            w8a8.gemm_blockscale(a["qx"], a["sx"], a["qw"], a["sw"], bias=a.get("bias"), out=a.get("out"))
    with pytest.raises(ValueError):   # post-scale: one scale per row / channel
        w8a8.gemm_postscale(qx, sx, qw, z((384,), torch.float32))
    with pytest.raises(ValueError):
        w8a8.gemm_blockscale_gated_residual(qx, sx, qw, sw, z((256, 384), torch.bfloat16), z((2, 384), torch.bfloat16),
                                            out=z((10,), torch.bfloat16))
    torch.cuda.synchronize()


def test_linear_output_and_bias_sizes():
    x, w = z((256, 256), torch.bfloat16), z((384, 256), torch.bfloat16)
    with pytest.raises(ValueError):
        w8a8.linear(x, w, out=z((256, 100), torch.bfloat16))
    with pytest.raises(ValueError):
        w8a8.linear(x, w, bias=z((100,), torch.bfloat16))
    y, path = w8a8.linear(x, w, workspace=z((8,), torch.float32))   # no qweight: fallback, no workspace needed
    torch.cuda.synchronize()
    assert path == w8a8.PATH_BF16 and y.shape == (256, 384)
