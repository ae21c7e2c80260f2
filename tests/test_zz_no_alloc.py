"""w8a8_linear_noalloc (the entry point for callers that cannot allocate)
against w8a8_linear, through the C ABI: two calls in a row, the second with
a smaller input, each equal to w8a8_linear's output bit for bit (the same
kernels on the same data; only where the workspace lives differs) and within
the bf16 tolerance of the oracle; a fallback-routed shape; and the size
limit of its fixed device array, rejected before anything is enqueued when
the INT8 path would need more, while a call the guard sends to the fallback
runs at that size."""
import ctypes

import pytest
import torch

import block_quantized_int8_amd as w8a8
import oracle
from block_quantized_int8_amd.workloads import random_bf16
from parity import assert_bf16_close, bf16_bits, to_dev_bf16

pytestmark = pytest.mark.gpu


def _noalloc(x, w, qw, sw, bias, y):
    L = w8a8.lib()
    M, K = x.shape
    N = w.shape[0]
    path = ctypes.c_int(-1)
    vp = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = L.w8a8_linear_noalloc(vp(x), 0, M, K, N, vp(w), vp(qw), vp(sw), vp(bias), vp(y),
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), ctypes.byref(path))
    return st, path.value


@pytest.mark.parametrize("case", [(1024, 2048, 768, True), (256, 256, 384, False)], ids=["first", "second_smaller"])
def test_noalloc_equals_linear_two_calls(case):
    M, K, N, with_bias = case
    x = random_bf16(400 + M, (M, K), 1.0)
    w = random_bf16(401 + K, (N, K), 0.02)
    b = random_bf16(402, (N,), 0.5) if with_bias else None
    xd, wd = to_dev_bf16(x), to_dev_bf16(w)
    bd = to_dev_bf16(b) if with_bias else None
    qw, sw = w8a8.quantize_weight(wd)
    ref, ref_path = w8a8.linear(xd, wd, qw, sw, bd)
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    st, path = _noalloc(xd, wd, qw, sw, bd, y)
    torch.cuda.synchronize()
    assert st == 0 and path == ref_path == w8a8.PATH_INT8
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
    oq, os_ = oracle.quantize_block(x)
    oqw, osw = oracle.quantize_block(w)
    assert_bf16_close(bf16_bits(y), oracle.linear_int8(oq, os_, oqw, osw, b), f"noalloc {M}x{N}x{K}")
    print(f"noalloc {M}x{N}x{K}: equal to w8a8_linear bit for bit", flush=True)


def test_noalloc_fallback_and_size_limit():
    M, K, N = 300, 256, 256
    x = random_bf16(410, (M, K), 1.0)
    w = random_bf16(411, (N, K), 0.02)
    xd, wd = to_dev_bf16(x), to_dev_bf16(w)
    qw, sw = w8a8.quantize_weight(wd)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    st, path = _noalloc(xd, wd, qw, sw, None, y)
    ref, _ = w8a8.linear(xd, wd, qw, sw)
    torch.cuda.synchronize()
    assert st == 0 and path == w8a8.PATH_BF16
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
    # M * K = 2^26 > the array: rejected (nothing enqueued, y untouched); without qw the call routes to the
    # fallback, which needs no workspace
    Mb, Kb, Nb = 16384, 4096, 128
    assert w8a8.workspace_bytes(Mb, Kb) > w8a8._lib.NOALLOC_SCRATCH_BYTES
    xb = torch.zeros((Mb, Kb), dtype=torch.bfloat16, device="cuda")
    wb = torch.zeros((Nb, Kb), dtype=torch.bfloat16, device="cuda")
    qb, sb = w8a8.quantize_weight(wb)
    yb = torch.full((Mb, Nb), 7.0, dtype=torch.bfloat16, device="cuda")
    st, path = _noalloc(xb, wb, qb, sb, None, yb)
    torch.cuda.synchronize()
    assert st == 2 and path == -1
    assert bool((yb == 7.0).all())
    st, path = _noalloc(xb, wb, None, None, None, yb)
    torch.cuda.synchronize()
    assert st == 0 and path == w8a8.PATH_BF16 and bool((yb == 0).all())
    # the same size with qw but x 2 bytes off 16-byte alignment: the guard sends
    # it to the fallback, which runs (the array's limit binds the INT8 path only)
    g = torch.Generator(device="cuda").manual_seed(412)
    xm = torch.randn(Mb * Kb + 1, generator=g, device="cuda").to(torch.bfloat16)[1:].view(Mb, Kb)
    wm = (torch.randn((Nb, Kb), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    qm, sm = w8a8.quantize_weight(wm)
    st, path = _noalloc(xm, wm, qm, sm, None, yb)
    ref, ref_path = w8a8.linear(xm, wm, qm, sm)
    torch.cuda.synchronize()
    assert st == 0 and path == ref_path == w8a8.PATH_BF16
    assert torch.equal(yb.view(torch.int16), ref.view(torch.int16))
