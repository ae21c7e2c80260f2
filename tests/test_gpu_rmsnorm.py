"""Modulated RMS normalization on the GPU against the oracle, alone and fused
with the 128x128 block quantization (TurboT2VA paper, architecture-aware
inference stack, fused-kernels paragraph).

The bf16 output is compared bit for bit, the fused codes and scales bit for
bit, on ragged row counts, 128-row blocks that straddle two batch entries,
extreme magnitudes, zero rows, both eps regimes, and the full 32768 x 4096
transformer-block input (oracle on sampled 128-row blocks, plus fused ==
unfused on the whole matrix).
"""
import numpy as np
import pytest
import torch

import block_quantized_int8_amd as w8a8
import oracle
from block_quantized_int8_amd.workloads import bf16_bits_to_f32, block_hidden, f32_to_bf16_bits, random_bf16
from parity import bf16_bits, to_dev_bf16

pytestmark = pytest.mark.gpu


def dev(a):
    return to_dev_bf16(a)


def gpu_y(x, L, sc, sh, eps):
    B = x.shape[0] // L
    y = w8a8.rmsnorm_modulate_bf16(dev(x).view(B, L, -1), dev(sc), dev(sh), eps)
    torch.cuda.synchronize()
    return bf16_bits(y).reshape(x.shape)


@pytest.mark.parametrize("B,L,K,eps", [(2, 300, 512, 1e-6), (3, 77, 136, 1e-6), (1, 5, 8, 0.5), (4, 96, 4096, 1e-5)])
def test_bf16_output_bit_exact(B, L, K, eps):
    x = random_bf16(B * 1000 + L, (B * L, K), 3.0)
    sc = random_bf16(K + 1, (B, K), 0.3)
    sh = random_bf16(K + 2, (B, K), 0.3)
    assert np.array_equal(gpu_y(x, L, sc, sh, eps), oracle.rmsnorm_modulate(x, L, sc, sh, eps))


def test_extreme_magnitudes_and_zero_rows():
    B, L, K = 2, 8, 256
    xf = bf16_bits_to_f32(random_bf16(31, (B * L, K)))
    xf[0] *= np.float32(2.0 ** -100)    # tiny row: r ~ 2^100
    xf[1] *= np.float32(2.0 ** 100)     # huge row: r ~ 2^-100
    xf[2] = 0.0                         # zero row: y = shift
    xf[9, :5] = np.float32(1e30)        # a few huge values in an otherwise normal row
    x = f32_to_bf16_bits(xf)
    sc = random_bf16(32, (B, K), 0.3)
    sh = random_bf16(33, (B, K), 0.3)
    for eps in (1e-6, 1e-30):
        y = gpu_y(x, L, sc, sh, eps)
        assert np.array_equal(y, oracle.rmsnorm_modulate(x, L, sc, sh, eps)), eps
    assert np.array_equal(gpu_y(x, L, sc, sh, 1e-6)[2], sh[0])


@pytest.mark.parametrize("B,L,K", [(2, 384, 512), (4, 96, 256), (1, 128, 128), (4, 96, 1024), (2, 192, 2560),
                                   (1, 256, 384)])
def test_fused_codes_bit_exact(B, L, K):
    # L = 96, 192: some 128-row blocks hold rows of two batch entries; K % 256 == 0
    # takes the single-read kernel (1 to 10 workgroups per band), K = 128, 384 the two-read pair
    x = random_bf16(B * 7 + L, (B * L, K), 2.0)
    sc = random_bf16(K + 3, (B, K), 0.3)
    sh = random_bf16(K + 4, (B, K), 0.3)
    q, s = w8a8.rmsnorm_modulate_quantize_act(dev(x).view(B, L, K), dev(sc), dev(sh), 1e-6)
    torch.cuda.synchronize()
    oq, os_ = oracle.rmsnorm_modulate_quantize_block(x, L, sc, sh, 1e-6)
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(s.cpu().numpy(), os_)


def test_single_read_workspace_reuse_and_error_word():
    """One workspace through calls of different widths: the single-read kernel
    (K % 256 == 0) clears its counters itself on every call, so stale
    counters of an earlier, larger call do not release a band early; its error
    word stays 0; each result equals the unfused chain bit for bit."""
    ws = torch.empty(w8a8.rmsnorm_quantize_workspace_bytes(1024, 4096), dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)                       # nonzero garbage in the counters and partials
    for i, (B, L, K) in enumerate([(2, 512, 4096), (2, 512, 4096), (3, 128, 768), (1, 256, 384), (4, 256, 2048)]):
        x = dev(random_bf16(600 + i, (B * L, K), 2.0)).view(B, L, K)
        sc, sh = dev(random_bf16(610 + i, (B, K), 0.3)), dev(random_bf16(620 + i, (B, K), 0.3))
        q, s = w8a8.rmsnorm_modulate_quantize_act(x, sc, sh, 1e-6, workspace=ws)
        q2, s2 = w8a8.quantize_act(w8a8.rmsnorm_modulate_bf16(x, sc, sh, 1e-6).view(B * L, K))
        torch.cuda.synchronize()
        assert torch.equal(q, q2) and torch.equal(s, s2), (B, L, K)
        if K % 256 == 0:
            assert int(ws[:4].view(torch.int32).item()) == 0, (B, L, K)
        print(f"rms single-read reuse {B}x{L}x{K}: equal to the unfused chain", flush=True)



def test_band_larger_than_the_device_takes_two_reads():
    """The workgroups of a band wait for one another, so a width whose band
    cannot be resident at once (K = 2^20: 4096 workgroups per band, beyond
    what any single device holds) must take the two-read path: the error word
    keeps what the caller left there, and the codes and scales equal the
    oracle's bit for bit."""
    B, L, K = 1, 128, 1 << 20
    x = random_bf16(700, (B * L, K), 2.0)
    sc, sh = random_bf16(701, (B, K), 0.3), random_bf16(702, (B, K), 0.3)
    ws = torch.empty(w8a8.rmsnorm_quantize_workspace_bytes(B * L, K), dtype=torch.uint8, device="cuda")
    ws[:4].view(torch.int32).fill_(0x5A5A5A5A)
    q, s = w8a8.rmsnorm_modulate_quantize_act(dev(x).view(B, L, K), dev(sc), dev(sh), 1e-6, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 0x5A5A5A5A, "the single-read kernel ran"
    oq, os_ = oracle.rmsnorm_modulate_quantize_block(x, L, sc, sh, 1e-6)
    assert np.array_equal(q.cpu().numpy(), oq) and np.array_equal(s.cpu().numpy(), os_)


def test_single_read_on_two_streams_at_once():
    """Two single-read launches in flight together on two streams (default
    priority), each with its own workspace: K = 65536 gives 256 workgroups
    per band, within the half of the device's capacity the router allows, so
    both kernels' bands can be resident at once and neither wait gives up
    (error words 0); each result equals the unfused chain bit for bit."""
    B, L, K = 1, 512, 65536
    xs, scs, shs, wss = [], [], [], []
    for i in range(2):
        xs.append(dev(random_bf16(710 + i, (B * L, K), 2.0)).view(B, L, K))
        scs.append(dev(random_bf16(720 + i, (B, K), 0.3)))
        shs.append(dev(random_bf16(730 + i, (B, K), 0.3)))
        ws = torch.empty(w8a8.rmsnorm_quantize_workspace_bytes(B * L, K), dtype=torch.uint8, device="cuda")
        ws.fill_(0xA5)
        wss.append(ws)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [None, None]
    for i in range(2):
        with torch.cuda.stream(streams[i]):
            outs[i] = w8a8.rmsnorm_modulate_quantize_act(xs[i], scs[i], shs[i], 1e-6, workspace=wss[i])
    torch.cuda.synchronize()
    for i in range(2):
        assert int(wss[i][:4].view(torch.int32).item()) == 0, f"stream {i}: a wait gave up"
        q2, s2 = w8a8.quantize_act(w8a8.rmsnorm_modulate_bf16(xs[i], scs[i], shs[i], 1e-6).view(B * L, K))
        torch.cuda.synchronize()
        assert torch.equal(outs[i][0], q2) and torch.equal(outs[i][1], s2), i

def test_zero_modulated_block_gives_zero_scale():
    # x = 0 and shift = 0: y = 0 in the whole block -> s = 0 and q = 0
    B, L, K = 1, 128, 256
    x = random_bf16(41, (B * L, K))
    x[:, :128] = 0
    sc = random_bf16(42, (B, K), 0.3)
    sh = random_bf16(43, (B, K), 0.3)
    sh[:, :128] = 0
    q, s = w8a8.rmsnorm_modulate_quantize_act(dev(x).view(B, L, K), dev(sc), dev(sh), 1e-6)
    torch.cuda.synchronize()
    assert s[0, 0].item() == 0.0 and not q[:, :128].any().item()
    oq, os_ = oracle.rmsnorm_modulate_quantize_block(x, L, sc, sh, 1e-6)
    assert np.array_equal(q.cpu().numpy(), oq) and np.array_equal(s.cpu().numpy(), os_)


def test_transformer_block_input_full_size():
    d = block_hidden()
    x, sc, sh, L = d["x"], d["scale"], d["shift"], d["L"]
    B, K = sc.shape
    xd = dev(x).view(B, L, K)
    scd, shd = dev(sc), dev(sh)
    q, s = w8a8.rmsnorm_modulate_quantize_act(xd, scd, shd, 1e-6)
    y = w8a8.rmsnorm_modulate_bf16(xd, scd, shd, 1e-6).view(B * L, K)
    q2, s2 = w8a8.quantize_act(y)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s, s2), "fused differs from the unfused chain"
    # oracle on sampled 128-row blocks from every batch entry (at L = 8192 no
    # block spans two entries; the small cases above cover that)
    for blk in (0, L // 128 - 1, L // 128, 2 * L // 128 + 17, B * L // 128 - 1):
        rows = slice(blk * 128, blk * 128 + 128)
        b = blk * 128 // L
        oy = oracle.rmsnorm_modulate(x[rows], 128, sc[b:b + 1], sh[b:b + 1], 1e-6)
        assert np.array_equal(bf16_bits(y[rows]), oy), blk
        oq, os_ = oracle.quantize_block(oy)
        assert np.array_equal(q[rows].cpu().numpy(), oq) and np.array_equal(s[blk].cpu().numpy(), os_[0]), blk


def test_layer_forward_modulated_matches_unfused_chain():
    B, L, K, N = 2, 256, 512, 384
    x = dev(random_bf16(51, (B * L, K), 2.0)).view(B, L, K)
    sc = dev(random_bf16(52, (B, K), 0.3))
    sh = dev(random_bf16(53, (B, K), 0.3))
    layer = w8a8.W8A8Linear(dev(random_bf16(54, (N, K), 0.02)))
    fused = layer.forward_modulated(x, sc, sh, 1e-6)
    assert layer.last_path == w8a8.PATH_INT8
    chained = layer(w8a8.rmsnorm_modulate_bf16(x, sc, sh, 1e-6))
    torch.cuda.synchronize()
    assert fused.shape == (B, L, N)
    assert torch.equal(fused.view(torch.int16), chained.view(torch.int16))
