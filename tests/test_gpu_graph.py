"""The library under HIP graph capture.

Every entry point only enqueues kernels on the caller's stream and never
allocates, copies or synchronizes, so a whole layer step can be captured
once and replayed.  Each test captures the calls with preallocated buffers,
then replays the graph several times with new inputs written eagerly in
between, and checks every replay bit for bit against an eager call on the
same input (and one replay against the oracle).
"""
import numpy as np
import pytest
import torch

import block_quantized_int8_amd as w8a8
import oracle
from block_quantized_int8_amd.workloads import random_bf16
from parity import assert_bf16_close, bf16_bits, to_dev_bf16

pytestmark = pytest.mark.gpu


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                   # eager warm-up off the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("M,K,N,int8", [(512, 256, 384, True), (1000, 256, 384, False)])
def test_linear_step_replays(M, K, N, int8):
    w = to_dev_bf16(random_bf16(31, (N, K), 0.02))
    b = to_dev_bf16(random_bf16(32, (N,), 0.1))
    layer = w8a8.W8A8Linear(w)
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    x.copy_(to_dev_bf16(random_bf16(33, (M, K))))
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(w8a8.workspace_bytes(M, K), 1), dtype=torch.uint8, device="cuda")
    paths = []

    def step():
        _, path = w8a8.linear(x, w, layer.qweight, layer.wscale, bias=b, out=y, workspace=ws)
        paths.append(path)

    g = capture(step)
    assert paths[-1] == (w8a8.PATH_INT8 if int8 else w8a8.PATH_BF16)
    for seed in (34, 35, 36):
        xh = random_bf16(seed, (M, K))
        x.copy_(to_dev_bf16(xh))               # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got = y.clone()
        ref, _ = w8a8.linear(x, w, layer.qweight, layer.wscale, bias=b)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay with input seed {seed}"
    wh = bf16_bits(w)
    if int8:
        qx, sx = oracle.quantize_block(xh)
        qw, sw = oracle.quantize_block(wh)
        want = oracle.linear_int8(qx, sx, qw, sw, bias=bf16_bits(b))
    else:
        want = oracle.linear_bf16(xh, oracle.DTYPE_BF16, wh, bias=bf16_bits(b))
    assert_bf16_close(bf16_bits(got), want, f"graph replay {M}x{K}x{N}")


def test_producer_and_qk_replay():
    # fused GELU + quantize, INT8 Q/K and FP8 V in one graph
    M, K, H, D = 256, 512, 4, 128
    yh = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((M, K), dtype=torch.int8, device="cuda")
    s = torch.empty((M // 128, K // 128), dtype=torch.float32, device="cuda")
    kq = torch.empty((H, M, D), dtype=torch.int8, device="cuda")
    ks = torch.empty((H, M // 128), dtype=torch.float32, device="cuda")
    vq = torch.empty((1, H, M, D), dtype=torch.uint8, device="cuda")
    vs = torch.empty((1, H, M // 128), dtype=torch.float32, device="cuda")

    def work():
        w8a8.gelu_quantize_act(yh, q, s)
        w8a8.quantize_qk(yh, H, kq, ks)
        w8a8.quantize_v_fp8(yh, H, vq, vs)

    yh.copy_(to_dev_bf16(random_bf16(40, (M, K))))
    g = capture(work)
    for seed in (41, 42):
        host = random_bf16(seed, (M, K))
        yh.copy_(to_dev_bf16(host))
        g.replay()
        torch.cuda.synchronize()
        oq, os_ = oracle.gelu_quantize_block(host)
        assert np.array_equal(q.cpu().numpy(), oq) and np.array_equal(s.cpu().numpy(), os_)
        kq_o, ks_o = oracle.quantize_qk(host, 1, M, H, D, K)
        assert np.array_equal(kq.cpu().numpy(), kq_o[0]) and np.array_equal(ks.cpu().numpy(), ks_o[0])
        vq_o, vs_o = oracle.quantize_v_fp8(host, 1, M, H, D, K)
        assert np.array_equal(vq.cpu().numpy(), vq_o) and np.array_equal(vs.cpu().numpy(), vs_o)


def test_block_slice_replay():
    # a transformer-block slice in one graph: modulated RMSNorm fused into the
    # projection input's quantization, the block GEMM with the gated residual
    # update in its epilogue (in place on the residual stream h), then the
    # rotary embedding fused into the INT8 quantization of the updated stream
    # read as 2 heads of 128 (standing in for a Q projection)
    B, L, K, H, D = 2, 256, 256, 2, 128
    M = B * L
    w = to_dev_bf16(random_bf16(60, (K, K), 0.02))
    layer = w8a8.W8A8Linear(w)
    x = torch.empty((B, L, K), dtype=torch.bfloat16, device="cuda")
    h = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    sc = to_dev_bf16(random_bf16(61, (B, K), 0.3))
    sh = to_dev_bf16(random_bf16(62, (B, K), 0.3))
    gate = to_dev_bf16(random_bf16(63, (B, K), 0.5))
    from block_quantized_int8_amd.workloads import rope_tables
    cs_h, sn_h = rope_tables(L, D)
    cs, sn = torch.from_numpy(cs_h).cuda(), torch.from_numpy(sn_h).cuda()
    qx = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sx = torch.empty((M // 128, K // 128), dtype=torch.float32, device="cuda")
    kq = torch.empty((B, H, L, D), dtype=torch.int8, device="cuda")
    ks = torch.empty((B, H, L // 128), dtype=torch.float32, device="cuda")

    def work():
        w8a8.rmsnorm_modulate_quantize_act(x, sc, sh, 1e-6, qx, sx)
        w8a8.gemm_blockscale_gated_residual(qx, sx, layer.qweight, layer.wscale, h, gate, out=h)
        w8a8.rope_quantize_qk(h.view(B, L, K), H, cs, sn, kq, ks)

    def load(seed):
        xh, hh = random_bf16(seed, (M, K), 2.0), random_bf16(seed + 1, (M, K), 2.0)
        x.copy_(to_dev_bf16(xh).view(B, L, K))
        h.copy_(to_dev_bf16(hh))
        return xh, hh

    load(64)
    g = capture(work)
    for seed in (66, 68):
        xh, hh = load(seed)
        g.replay()
        torch.cuda.synchronize()
        got = (qx.clone(), sx.clone(), h.clone(), kq.clone(), ks.clone())
        load(seed)
        work()                                  # eager, same inputs
        torch.cuda.synchronize()
        for a, b in zip(got, (qx, sx, h, kq, ks)):
            assert torch.equal(a.view(torch.int8), b.view(torch.int8)), f"replay with input seed {seed}"
    # the last replay against the oracle: codes bit-exact, the updated stream
    # within the output tolerance, and its rotation + Q/K codes bit-exact
    oq, os_ = oracle.rmsnorm_modulate_quantize_block(xh, L, bf16_bits(sc), bf16_bits(sh), 1e-6)
    assert np.array_equal(got[0].cpu().numpy(), oq) and np.array_equal(got[1].cpu().numpy(), os_)
    wq, ws = oracle.quantize_block(bf16_bits(w))
    want_h = oracle.gated_residual(hh, oracle.linear_int8(oq, os_, wq, ws), bf16_bits(gate), L)
    assert_bf16_close(bf16_bits(got[2]), want_h, "graph replay: GEMM + gated residual")
    rq, rs = oracle.rope_quantize_qk(bf16_bits(got[2]), B, L, H, D, K, cs_h, sn_h)
    assert np.array_equal(got[3].cpu().numpy(), rq) and np.array_equal(got[4].cpu().numpy(), rs)
