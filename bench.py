"""Benchmark of the guarded W8A8 block-quantized linear on one MI355X.

A step is one call of the guarded linear (w8a8_linear) on the
attention-projection workload: X[32768, 4096] bf16 with heavy-tailed
activations (1% of channels x20), W[4096, 4096] bf16 ~ N(0, 0.02^2), seed 2.
On this shape the guard takes the INT8 path, so a step is the dynamic
128x128 activation quantization followed by the INT8 GEMM with per-K-block
dequantization and bf16 output.  The weight is quantized once, before
timing (static weights).  Inputs are resident in HBM when timing starts.
A fixed settle phase (SETTLE_S seconds of steps) runs ahead of the --warmup
steps: from a cold start the GPU clock dips for its first dozen or so
GEMM launches, and a continuously running layer never sees that transient.

Printed: one JSON line with the whole-step throughput (value, in TOPS of
2*M*N*K per step), the per-kernel figures measured with HIP events on the
stream the kernels run on, the roofline of the dominant kernel (the GEMM,
bound by the INT8 MFMA peak), the GPU clock sampled during a run of
back-to-back GEMM launches, and the CPU oracle timed on a bounded sample of
the same workload on this host.

The other workloads of the scope table are measured beside it (not part of a
step): the 256^3 single linear, the 4096^3 square linear, the MLP pair's up
(32768 x 16384 x 4096) and down (32768 x 4096 x 16384) projections and the
two-stream step's INT8 stream (65536 x 4096 x 4096): each with its GEMM
(TOPS, fraction of peak), its activation quantization (GB/s, fraction of
HBM) and the oracle timed on one 128-row block of it; the guard's bf16
fallback (M = 4000 and 1000 x 2048 x 2048) and the two-stream step itself;
the post-scale form; the producers fused with the quantization (exact
GELU, modulated RMSNorm and LayerNorm); Q, K, V as one concatenated linear
vs three; and the INT8 quantization of a video self-attention's Q and K.
--extras adds the measurements of patterns beyond that table: V in FP8,
the rotary embedding fused into the Q/K quantizer, the gated residual update
in the GEMM epilogue and one transformer block's W8A8 work.

Modes for profiling runs: --only gemm|quantize|linear|gelu_quant|gelu|qk|v|rope|rms|ln|residual|mlp_up|mlp_down|fallback
launches just that work for --steps iterations (no oracle; fallback runs the
guarded bf16 linear on the M = 4000 guard case, then the BLAS library's bf16
linear on the same operands);
--copy-calibration runs a plain 1 GiB device copy used to scale the HBM byte
counters.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

M, N, K = 32768, 4096, 4096
PEAK_INT8_TOPS = 256 * 8192 * 2.4e9 / 1e12   # 5033.2: 256 CUs x 8192 int8 ops/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12  # 2516.6: dense bf16 MFMA
METRIC = "INT8 GEMM TOPS + % of INT8 MFMA peak; quantize GB/s (M=32768,K=N=4096)"
# algorithmic bytes of the activation quantization: read bf16 X, write int8
# qX and one fp32 scale per 128x128 block
QUANT_BYTES = M * K * 2 + M * K * 1 + (M // 128) * (K // 128) * 4
# algorithmic bytes of the GEMM: read qX, qW and both scale grids, write bf16 Y
GEMM_BYTES = M * K + N * K + (M // 128 + N // 128) * (K // 128) * 4 + M * N * 2
GEMM_OPS = 2 * M * N * K
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_i8_attnproj.json")
GEMM_SOURCE = os.path.join(ROOT, "block_quantized_int8_amd", "csrc", "gemm_i8_blockscale.hip")
QUANT_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_quantize_block_attnproj.json")
QUANT_SOURCE = os.path.join(ROOT, "block_quantized_int8_amd", "csrc", "quantize_block.hip")
CPU_SAMPLE_BLOCKS = 256     # 128-row blocks of X the oracle processes (all 32768 rows)
# MLP hidden activation (input of the fused GELU + quantize producer)
HM, HK = 32768, 16384
PRODUCER_BYTES = HM * HK * 2 + HM * HK + (HM // 128) * (HK // 128) * 4   # read bf16, write int8 + scales
GELU_BYTES = HM * HK * 2 * 2                                              # read and write bf16
# transformer-block input for the modulated-RMSNorm producer: read bf16 x,
# write int8 + block scales, read the [B, K] scale and shift
RB, RL, RK = 4, 8192, 4096
RMS_BYTES = RB * RL * RK * 3 + (RB * RL // 128) * (RK // 128) * 4 + 2 * RB * RK * 2
# gated residual update of the attention projection's output: 4 batch
# entries; the fused GEMM reads h and writes y instead of writing o, the
# update kernel reads h and o and writes y
RES_B = 4
RES_UPDATE_BYTES = M * N * 2 * 3 + RES_B * N * 2
# attention Q or K of one video self-attention: read bf16, write int8 + one scale per 128 tokens x head
AL, AH, AD = 28672, 32, 128
QK_BYTES = AL * AH * AD * 3 + AH * (AL // 128) * 4
# the same with the rotary embedding in front: plus the fp32 cos and sin
# tables [AL, AD/2] (latent grid 16 frames x 56 x 32 for the three axes)
ROPE_GRID = (16, 56, 32)
ROPE_TABLE_BYTES = AL * (AD // 2) * 4 * 2
ROPE_QK_BYTES = QK_BYTES + ROPE_TABLE_BYTES


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def code_sha(path):
    """Hash of a kernel source's code: comments removed and whitespace
    collapsed, so that editing comments does not retire measured counters."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()[:16]


def load_traffic(path=TRAFFIC_FILE, source=GEMM_SOURCE):
    """HBM bytes per launch of a kernel (the GEMM by default) from committed
    rocprofv3 counter runs, or None when absent or taken on different
    kernel code."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("code_sha") != code_sha(source):
        return None
    return t.get("bytes_per_launch")


def ensure_built():
    from block_quantized_int8_amd import build as b
    if not os.path.exists(b.OUT):
        b.build()


def make_inputs(dev):
    import numpy as np
    import torch
    from block_quantized_int8_amd.workloads import attention_projection
    d = attention_projection(M)
    x = torch.from_numpy(d["x"].view(np.int16)).to(dev).view(torch.bfloat16)
    w = torch.from_numpy(d["w"].view(np.int16)).to(dev).view(torch.bfloat16)
    return d, x, w


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def vendor_int8_context(qx, qw):
    """The ROCm BLAS library's plain INT8 GEMM (torch._int_mm: int32 out, no
    scales, no bf16 conversion) on the same operands: context for the
    roofline fraction, not part of the path.  None if torch lacks it."""
    import torch
    try:
        torch._int_mm(qx, qw.t())  # untimed first launch
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record()
        for _ in range(reps):
            torch._int_mm(qx, qw.t())
        e1.record()
        torch.cuda.synchronize()
    except (RuntimeError, AttributeError) as exc:
        log(f"vendor int8 GEMM unavailable: {exc}")
        return None
    us = e0.elapsed_time(e1) / reps * 1e3
    tops = GEMM_OPS / (us * 1e-6) / 1e12
    log(f"vendor plain int8 GEMM (torch._int_mm): {us:.1f} us = {tops:.0f} TOPS")
    return {"note": "torch._int_mm on the same int8 operands (ROCm BLAS library; int32 output, no scales): "
                    "context only", "us": round(us, 2), "tops": round(tops, 1),
            "frac_of_int8_peak": round(tops / PEAK_INT8_TOPS, 4)}


def cpu_baseline(d):
    """The oracle (untuned) on the first CPU_SAMPLE_BLOCKS row-blocks of X:
    quantize those rows and compute their full output rows."""
    import numpy as np
    import oracle
    from oracle import build as ob
    if not os.path.exists(ob.OUT):
        ob.build()
    rows = CPU_SAMPLE_BLOCKS * 128
    xs = np.ascontiguousarray(d["x"][:rows])
    t0 = time.perf_counter()
    qw, sw = oracle.quantize_block(d["w"])            # static: excluded below
    t1 = time.perf_counter()
    qx, sx = oracle.quantize_block(xs)
    t2 = time.perf_counter()
    oracle.linear_int8(qx, sx, qw, sw)
    t3 = time.perf_counter()
    secs = t3 - t1
    ops = 2 * rows * N * K
    return {"value": ops / secs / 1e12, "unit": "TOPS", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(secs, 3),
            "quantize_seconds": round(t2 - t1, 3), "gemm_seconds": round(t3 - t2, 3),
            "cpu_model": cpu_model(),
            "sample": f"first {rows} of {M} rows of X (quantize + full output rows), "
                      f"N=K={K}; weight quantization ({t1 - t0:.2f} s) excluded as static"}


def qk_buffers(dev):
    """A fused Q/K/V output [AL, 3 * AH * AD] in HBM holding the video
    self-attention's Q and K, and the head-major outputs."""
    import numpy as np
    import torch
    from block_quantized_int8_amd.workloads import attention_qk
    d = attention_qk(AL, AH, AD)
    qkv = torch.empty((AL, 3 * AH * AD), dtype=torch.bfloat16, device=dev)
    for i, name in enumerate(("q", "k")):
        qkv[:, i * AH * AD:(i + 1) * AH * AD] = torch.from_numpy(d[name].view(np.int16)).to(dev).view(torch.bfloat16)
    qkv[:, 2 * AH * AD:] = 0
    qq = torch.empty((AH, AL, AD), dtype=torch.int8, device=dev)
    sq = torch.empty((AH, AL // 128), dtype=torch.float32, device=dev)
    return qkv, qq, sq


def residual_buffers(dev):
    """Residual stream h [M, N] and gate [4, N] (4 batch entries of M/4
    tokens) for the attention projection's gated residual update, and its
    output."""
    import numpy as np
    import torch
    from block_quantized_int8_amd.workloads import random_bf16
    h = torch.from_numpy(random_bf16(93, (M, N), 2.0).view(np.int16)).to(dev).view(torch.bfloat16)
    g = torch.from_numpy(random_bf16(94, (RES_B, N), 0.5).view(np.int16)).to(dev).view(torch.bfloat16)
    return h, g, torch.empty((M, N), dtype=torch.bfloat16, device=dev)


def block_slice_ab(w8a8, dev, steps):
    """One transformer block's W8A8 work, attention excluded: modulated
    RMSNorm -> Q/K/V projection group -> split rotary embedding and INT8 Q/K
    -> output projection + gated residual -> modulated RMSNorm -> MLP up ->
    GELU -> MLP down + gated residual.  Fused: each producer in the next
    quantizer, each residual update in the GEMM epilogue; unfused: every step
    on its own through bf16 tensors.  V stands in for the attention output.
    Returns the mean time per block of each chain (us)."""
    import numpy as np
    import torch
    from block_quantized_int8_amd.workloads import random_bf16, rope_tables
    B, L, D, H, HD, F = RB, RL, RK, 32, 128, 16384
    Mb = B * L
    t = lambda bits: torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    h0 = t(random_bf16(200, (Mb, D), 2.0))
    mod = [t(random_bf16(201 + i, (B, D), 0.3)) for i in range(4)]      # scale/shift of the two norms
    gates = [t(random_bf16(205 + i, (B, D), 0.5)) for i in range(2)]
    qkv = w8a8.W8A8Linear(t(random_bf16(207, (3 * D, D), 0.02)))
    out_p = w8a8.W8A8Linear(t(random_bf16(208, (D, D), 0.02)))
    up = w8a8.W8A8Linear(t(random_bf16(209, (F, D), 0.02)))
    down = w8a8.W8A8Linear(t(random_bf16(210, (D, F), 0.02)))
    cs, sn = (torch.from_numpy(a).to(dev) for a in rope_tables(L, HD))
    h = torch.empty_like(h0)
    h1 = torch.empty_like(h0)
    qq = torch.empty((B, H, L, HD), dtype=torch.int8, device=dev)
    sq = torch.empty((B, H, L // 128), dtype=torch.float32, device=dev)
    kq, ks = torch.empty_like(qq), torch.empty_like(sq)
    qg = torch.empty((Mb, F), dtype=torch.int8, device=dev)
    sg = torch.empty((Mb // 128, F // 128), dtype=torch.float32, device=dev)

    def fused():
        y = qkv.forward_modulated(h.view(B, L, D), mod[0], mod[1]).view(B, L, 3 * D)
        w8a8.rope_quantize_qk(y[:, :, :D], H, cs, sn, qq, sq)
        w8a8.rope_quantize_qk(y[:, :, D:2 * D], H, cs, sn, kq, ks)
        out_p.forward_gated_residual(y[:, :, 2 * D:], h, gates[0], out=h1)
        u = up.forward_modulated(h1.view(B, L, D), mod[2], mod[3])
        w8a8.gelu_quantize_act(u.view(Mb, F), qg, sg)
        w8a8.gemm_blockscale_gated_residual(qg, sg, down.qweight, down.wscale, h1, gates[1], out=h)

    def unfused():
        y = qkv(w8a8.rmsnorm_modulate_bf16(h.view(B, L, D), mod[0], mod[1])).view(B, L, 3 * D)
        w8a8.quantize_qk(w8a8.rope_bf16(y[:, :, :D], H, cs, sn), H, qq, sq)
        w8a8.quantize_qk(w8a8.rope_bf16(y[:, :, D:2 * D], H, cs, sn), H, kq, ks)
        w8a8.gated_residual(h, out_p(y[:, :, 2 * D:].reshape(Mb, D)), gates[0], out=h1)
        u = up(w8a8.rmsnorm_modulate_bf16(h1.view(B, L, D), mod[2], mod[3]))
        o = down(w8a8.gelu_bf16(u))
        w8a8.gated_residual(h1, o.view(Mb, D), gates[1], out=h)

    res = {}
    for name, fn in (("fused", fused), ("unfused", unfused)):
        h.copy_(h0)
        fn()                                   # untimed first launches
        torch.cuda.synchronize()
        h.copy_(h0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        res[name] = a.elapsed_time(b) / steps * 1e3
    return res


def rope_tables_dev(dev):
    import torch
    from block_quantized_int8_amd.workloads import rope_tables
    cs, sn = rope_tables(AL, AD, grid=ROPE_GRID)
    return torch.from_numpy(cs).to(dev), torch.from_numpy(sn).to(dev)


def rms_buffers(dev):
    """A transformer block's hidden state (B = 4 x L = 8192 tokens x 4096)
    with its modulation, and the producer's outputs."""
    import numpy as np
    import torch
    from block_quantized_int8_amd.workloads import block_hidden
    t0 = time.perf_counter()
    d = block_hidden(RB, RL, RK)
    to = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    xr, sc, sh = to(d["x"]).view(RB, RL, RK), to(d["scale"]), to(d["shift"])
    log(f"block hidden state ready ({time.perf_counter() - t0:.1f} s): {tuple(xr.shape)}")
    yr = torch.empty_like(xr)
    q = torch.empty((RB * RL, RK), dtype=torch.int8, device=dev)
    s = torch.empty((RB * RL // 128, RK // 128), dtype=torch.float32, device=dev)
    return xr, sc, sh, yr, q, s


def producer_buffers(w8a8, dev):
    """The MLP hidden activation in HBM and the producer's outputs."""
    import numpy as np
    import torch
    from block_quantized_int8_amd.workloads import mlp_hidden
    t0 = time.perf_counter()
    yh = torch.from_numpy(mlp_hidden(HM, HK).view(np.int16)).to(dev).view(torch.bfloat16)
    log(f"MLP hidden activation ready ({time.perf_counter() - t0:.1f} s): {tuple(yh.shape)}")
    xh = torch.empty_like(yh)
    qh = torch.empty((HM, HK), dtype=torch.int8, device=dev)
    sh = torch.empty((HM // 128, HK // 128), dtype=torch.float32, device=dev)
    return yh, xh, qh, sh


SETTLE_S = 1.0          # seconds of steps ahead of the --warmup steps (clock settle)
CLOCK_LOOP_S = 0.3      # seconds of back-to-back GEMM launches while the clock is sampled
ORACLE_ROWS = 128       # rows (one 128-row block) of each extra workload the oracle is timed on


class ClockSampler:
    """Samples the GPU's gfx clock (MHz, the mean over the chip's XCDs) from
    the SMI library's GPU metrics every ~2 ms in a background thread."""

    def __init__(self):
        self.samples, self.error, self._h = [], None, None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            self._read()
        except Exception as exc:  # no SMI access on this host: reported, not fatal
            self.error = f"{type(exc).__name__}: {exc}"
            self._h = None

    def _read(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
        xs = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and 0 < c < 10000]
        if xs:
            return sum(xs) / len(xs)
        c = m.get("current_gfxclk")
        return float(c) if isinstance(c, (int, float)) and 0 < c < 10000 else None

    def run(self, fn):
        """Calls fn() while sampling; returns fn's result."""
        import threading
        if self._h is None:
            return fn()
        stop = threading.Event()

        def loop():
            while not stop.is_set():
                try:
                    v = self._read()
                    if v:
                        self.samples.append(v)
                except Exception as exc:
                    self.error = f"{type(exc).__name__}: {exc}"
                time.sleep(0.002)

        th = threading.Thread(target=loop, daemon=True)
        th.start()
        try:
            return fn()
        finally:
            stop.set()
            th.join()


def event_times(fns, reps, flush=None):
    """Median and mean us of each callable over `reps` rounds (one HIP event
    pair around each launch on the current stream), rounds interleaved;
    `flush` (if given) runs untimed before every launch."""
    import statistics
    import torch
    res = {k: [] for k in fns}
    for _ in range(reps):
        for k, fn in fns.items():
            if flush is not None:
                flush()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            res[k].append((a, b))
    torch.cuda.synchronize()
    out = {}
    for k, v in res.items():
        us = [a.elapsed_time(b) * 1e3 for a, b in v]
        out[k] = {"median": statistics.median(us), "mean": sum(us) / len(us)}
    return out


def gpu_normal(gen, shape, scale=1.0, outlier_frac=0.0, outlier_factor=1.0, dev="cuda"):
    """Seeded N(0, scale^2) bf16 tensor made on the GPU (fp32 draw, optional
    outlier channels scaled in fp32, one conversion to bf16), for the workloads
    that are timed only."""
    import torch
    a = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
    if scale != 1.0:
        a *= scale
    if outlier_frac:
        k = shape[-1]
        ch = torch.randperm(k, generator=gen, device=dev)[:int(round(outlier_frac * k))]
        a[:, ch] *= outlier_factor
    return a.to(torch.bfloat16)


def oracle_rows_seconds(x_rows_bf16, w_bf16):
    """Oracle time (s) for the quantization of a block of activation rows and
    their full output rows; the static weight quantization is done first and
    not counted."""
    import numpy as np
    import torch
    import oracle
    xs = np.ascontiguousarray(x_rows_bf16.view(torch.int16).cpu().numpy().view(np.uint16))
    ws = np.ascontiguousarray(w_bf16.view(torch.int16).cpu().numpy().view(np.uint16))
    qw, sw = oracle.quantize_block(ws)
    t0 = time.perf_counter()
    qx, sx = oracle.quantize_block(xs)
    oracle.linear_int8(qx, sx, qw, sw)
    return time.perf_counter() - t0


def measure_config(w8a8, name, x, w, flush, reps, with_oracle=True, note=""):
    """Activation quantization and INT8 block GEMM of one workload: us, TOPS,
    fractions of the peaks, and the oracle on one 128-row block."""
    import torch
    M, K = x.shape
    N = w.shape[0]
    qw, sw = w8a8.quantize_weight(w)
    qx, sx = w8a8.quantize_act(x)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    w8a8.gemm_blockscale(qx, sx, qw, sw, out=y)
    torch.cuda.synchronize()
    g = event_times({"gemm": lambda: w8a8.gemm_blockscale(qx, sx, qw, sw, out=y)}, reps)["gemm"]
    q = event_times({"q": lambda: w8a8.quantize_act(x, qx, sx)}, reps, flush=flush)["q"]
    ops = 2 * M * N * K
    qbytes = M * K * 3 + (M // 128) * (K // 128) * 4
    tops = ops / (g["median"] * 1e-6) / 1e12
    gbs = qbytes / (q["median"] * 1e-6) / 1e9
    out = {"shape": [M, N, K], "gemm_us": round(g["median"], 2), "gemm_tops": round(tops, 1),
           "gemm_frac_of_int8_peak": round(tops / PEAK_INT8_TOPS, 4),
           "quantize_us": round(q["median"], 2), "quantize_gbs": round(gbs, 1),
           "quantize_frac_of_hbm": round(gbs / PEAK_HBM_GBS, 4), "quantize_bytes": qbytes, "gemm_ops": ops}
    if note:
        out["note"] = note
    if with_oracle:
        import oracle
        rows = min(ORACLE_ROWS, M)
        secs = oracle_rows_seconds(x[:rows], w)
        out["oracle"] = {"rows": rows, "seconds": round(secs, 3), "cores": oracle.num_threads(),
                         "full_seconds_extrapolated": round(secs * M / rows, 2),
                         "tops": round(2 * rows * N * K / secs / 1e12, 4)}
    log(f"{name} {M}x{N}x{K}: gemm {g['median']:.1f} us = {tops:.0f} TOPS ({tops / PEAK_INT8_TOPS:.1%}); "
        f"quantize {q['median']:.1f} us = {gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS:.1%})"
        + (f"; oracle {out['oracle']['seconds']} s / {out['oracle']['rows']} rows" if with_oracle else ""))
    del qx, sx, qw, sw, y
    return out


def extras(w8a8, dev, args, x, y, qx, sx, qw, sw, flush):
    """Patterns beyond the scope table: V in FP8, the rotary embedding fused
    into the Q/K quantizer, the gated residual update in the GEMM epilogue and
    one transformer block's W8A8 work."""
    import torch
    res = {}
    hres, gres, yres = residual_buffers(dev)
    runs = {"fused": lambda: w8a8.gemm_blockscale_gated_residual(qx, sx, qw, sw, hres, gres, out=yres),
            "gemm": lambda: w8a8.gemm_blockscale(qx, sx, qw, sw, out=y),
            "update": lambda: w8a8.gated_residual(hres, y, gres, out=yres)}
    for fn in runs.values():
        fn()
    torch.cuda.synchronize()
    t = event_times(runs, args.steps, flush=flush)
    r = {k: v["median"] for k, v in t.items()}
    del hres, gres, yres
    res["gated_residual_ab"] = {
        "note": "gated residual update h + gate * o of the attention projection's output (4 batch entries of "
                "8192 tokens) in the block GEMM's epilogue vs the GEMM then the update kernel",
        "shape": [M, N, K], "batch_entries": RES_B, "fused_us": round(r["fused"], 2),
        "unfused_gemm_us": round(r["gemm"], 2), "unfused_update_us": round(r["update"], 2),
        "update_gbs": round(RES_UPDATE_BYTES / r["update"] / 1e3, 1),
        "speedup": round((r["gemm"] + r["update"]) / r["fused"], 3)}
    log(f"gated residual: fused {r['fused']:.1f} us vs GEMM {r['gemm']:.1f} + update {r['update']:.1f} us")

    qkv, qq, sq = qk_buffers(dev)
    qkv[:, 2 * AH * AD:] = qkv[:, AH * AD:2 * AH * AD]
    vq = torch.empty((AH, AL, AD), dtype=torch.uint8, device=dev)
    w8a8.quantize_v_fp8(qkv[:, 2 * AH * AD:], AH, vq, sq)
    torch.cuda.synchronize()
    v_us = event_times({"v": lambda: w8a8.quantize_v_fp8(qkv[:, 2 * AH * AD:], AH, vq, sq)}, args.steps,
                       flush=flush)["v"]["median"]
    del vq
    res["v_fp8_quantize"] = {"note": "attention V in FP8 E4M3 (s = max-abs/448 per 128 tokens x head) from the "
                                     "third column slice of the fused Q/K/V output -> head-major codes",
                             "us": round(v_us, 2), "gbs": round(QK_BYTES / v_us / 1e3, 1),
                             "frac_of_hbm": round(QK_BYTES / v_us / 1e3 / PEAK_HBM_GBS, 4),
                             "algorithmic_bytes": QK_BYTES}
    log(f"V FP8: {v_us:.1f} us")

    cs, sn = rope_tables_dev(dev)
    yrot = torch.empty((AL, AH * AD), dtype=torch.bfloat16, device=dev)
    rope_runs = {"fused": lambda: w8a8.rope_quantize_qk(qkv[:, :AH * AD], AH, cs, sn, qq, sq),
                 "rotate": lambda: w8a8.rope_bf16(qkv[:, :AH * AD], AH, cs, sn, out=yrot),
                 "quantize": lambda: w8a8.quantize_qk(yrot, AH, qq, sq)}
    for fn in rope_runs.values():
        fn()
    torch.cuda.synchronize()
    r = {k: v["median"] for k, v in event_times(rope_runs, args.steps, flush=flush).items()}
    del qkv, qq, sq, yrot, cs, sn
    res["rope_qk_ab"] = {"note": "split-halves rotary embedding fused into the INT8 Q/K quantizer vs rotation "
                                 "to bf16 then quantization, per Q or K tensor; tables fp32 [tokens, head_dim/2]",
                         "shape": {"tokens": AL, "heads": AH, "head_dim": AD, "row_stride": 3 * AH * AD,
                                   "table_grid": list(ROPE_GRID)},
                         "fused_us": round(r["fused"], 2),
                         "fused_gbs_algorithmic": round(ROPE_QK_BYTES / r["fused"] / 1e3, 1),
                         "algorithmic_bytes": ROPE_QK_BYTES, "unfused_rotate_us": round(r["rotate"], 2),
                         "unfused_quantize_us": round(r["quantize"], 2),
                         "speedup": round((r["rotate"] + r["quantize"]) / r["fused"], 3)}
    log(f"RoPE + Q/K: fused {r['fused']:.1f} us vs {r['rotate']:.1f} + {r['quantize']:.1f} us")

    blk = block_slice_ab(w8a8, dev, args.steps)
    res["block_slice_ab"] = {"note": "one transformer block's W8A8 work, attention excluded (4 x 8192 tokens x "
                                     "4096, 32 heads of 128, MLP 16384), every fusion in place vs the same steps "
                                     "through bf16 tensors",
                             "fused_us": round(blk["fused"], 1), "unfused_us": round(blk["unfused"], 1),
                             "speedup": round(blk["unfused"] / blk["fused"], 3)}
    log(f"block slice: fused {blk['fused']:.1f} us vs unfused {blk['unfused']:.1f} us")
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--only", choices=["gemm", "quantize", "linear", "gelu_quant", "gelu", "qk", "v", "rope", "rms",
                                       "ln", "residual", "mlp_up", "mlp_down", "fallback"],
                    default=None)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extras", action="store_true",
                    help="also measure the patterns beyond the scope table (FP8 V, fused RoPE, gated residual, "
                         "block slice)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the layer would shard by rows of X, with no communication). "
              "Run with --gpus 1.", file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch
    ensure_built()
    import block_quantized_int8_amd as w8a8

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_start = time.perf_counter()

    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        a.fill_(1)
        for _ in range(args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copy calibration: {args.steps} copies of {n} bytes")
        return

    if args.only == "fallback":
        # the guard's bf16 fallback on M = 4000 at 4096^2, then the BLAS
        # library's bf16 linear on the same operands (for counter comparisons)
        xf = gpu_normal(torch.Generator(device=dev).manual_seed(70), (4000, 4096), dev=dev)
        wf = gpu_normal(torch.Generator(device=dev).manual_seed(71), (4096, 4096), 0.02, dev=dev)
        lf = w8a8.W8A8Linear(wf)
        for _ in range(args.steps):
            lf(xf)
        torch.cuda.synchronize()
        assert lf.last_path == w8a8.PATH_BF16
        for _ in range(args.steps):
            torch.nn.functional.linear(xf, wf)
        torch.cuda.synchronize()
        log(f"--only fallback: {args.steps} launches of each done")
        return

    if args.only in ("mlp_up", "mlp_down"):
        gen = torch.Generator(device=dev).manual_seed(3)
        if args.only == "mlp_up":
            xm, wm = gpu_normal(gen, (32768, 4096), dev=dev), gpu_normal(gen, (16384, 4096), 0.02, dev=dev)
        else:
            xm = w8a8.gelu_bf16(gpu_normal(gen, (32768, 16384), 1.28, dev=dev))
            wm = gpu_normal(gen, (4096, 16384), 0.02, dev=dev)
        qwm, swm = w8a8.quantize_weight(wm)
        qxm, sxm = w8a8.quantize_act(xm)
        ym = torch.empty((xm.shape[0], wm.shape[0]), dtype=torch.bfloat16, device=dev)
        for _ in range(args.steps):
            w8a8.quantize_act(xm, qxm, sxm)
            w8a8.gemm_blockscale(qxm, sxm, qwm, swm, out=ym)
        torch.cuda.synchronize()
        log(f"--only {args.only}: {args.steps} quantize + GEMM launches done")
        return

    t_gen = time.perf_counter()
    d, x, w = make_inputs(dev)
    log(f"inputs ready ({time.perf_counter() - t_gen:.1f} s): X {tuple(x.shape)}, W {tuple(w.shape)}")
    layer = w8a8.W8A8Linear(w)                       # static weight quantization
    qw, sw = layer.qweight, layer.wscale
    ws = torch.empty(w8a8.workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    qx = ws[:M * K].view(torch.int8).view(M, K)
    sx_off = (M * K + 255) // 256 * 256
    sx = ws[sx_off:sx_off + (M // 128) * (K // 128) * 4].view(torch.float32).view(M // 128, K // 128)

    def step():
        _, path = w8a8.linear(x, w, qw, sw, out=y, workspace=ws)
        return path

    if args.only == "qk":
        qkv, qq, sq = qk_buffers(dev)
        for _ in range(args.steps):
            w8a8.quantize_qk(qkv[:, :AH * AD], AH, qq, sq)
        torch.cuda.synchronize()
        log(f"--only qk: {args.steps} launches done")
        return

    if args.only == "v":
        qkv, _, sq = qk_buffers(dev)
        qkv[:, 2 * AH * AD:] = qkv[:, AH * AD:2 * AH * AD]
        vq = torch.empty((AH, AL, AD), dtype=torch.uint8, device=dev)
        for _ in range(args.steps):
            w8a8.quantize_v_fp8(qkv[:, 2 * AH * AD:], AH, vq, sq)
        torch.cuda.synchronize()
        log(f"--only v: {args.steps} launches done")
        return

    if args.only == "rope":
        qkv, qq, sq = qk_buffers(dev)
        cs, sn = rope_tables_dev(dev)
        for _ in range(args.steps):
            w8a8.rope_quantize_qk(qkv[:, :AH * AD], AH, cs, sn, qq, sq)
        torch.cuda.synchronize()
        log(f"--only rope: {args.steps} launches done")
        return

    if args.only == "residual":
        hres, gres, yres = residual_buffers(dev)
        w8a8.quantize_act(x, qx, sx)
        for _ in range(args.steps):
            w8a8.gemm_blockscale_gated_residual(qx, sx, qw, sw, hres, gres, out=yres)
        torch.cuda.synchronize()
        log(f"--only residual: {args.steps} launches done")
        return

    if args.only in ("rms", "ln"):
        xr, rsc, rsh, yr, rq, rs = rms_buffers(dev)
        rws = torch.empty(w8a8.rmsnorm_quantize_workspace_bytes(RB * RL, RK), dtype=torch.uint8, device=dev)
        fn = (lambda: w8a8.rmsnorm_modulate_quantize_act(xr, rsc, rsh, 1e-6, rq, rs, workspace=rws)) \
            if args.only == "rms" else (lambda: w8a8.layernorm_modulate_quantize_act(xr, rsc, rsh, 1e-6, rq, rs))
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        log(f"--only {args.only}: {args.steps} launches done")
        return

    if args.only in ("gelu_quant", "gelu"):
        yh, xh, qh, sh = producer_buffers(w8a8, dev)
        fn = (lambda: w8a8.gelu_quantize_act(yh, qh, sh)) if args.only == "gelu_quant" else \
            (lambda: w8a8.gelu_bf16(yh, out=xh))
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        log(f"--only {args.only}: {args.steps} launches done")
        return

    if args.only:
        fn = {"linear": step,
              "quantize": lambda: w8a8.quantize_act(x, qx, sx),
              "gemm": lambda: w8a8.gemm_blockscale(qx, sx, qw, sw, out=y)}[args.only]
        step()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        log(f"--only {args.only}: {args.steps} launches done")
        return

    # ---- settle, warm-up, then the timed region: K whole steps
    assert step() == w8a8.PATH_INT8
    torch.cuda.synchronize()
    settle_steps = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(20):
            step()
        settle_steps += 20
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = e0.elapsed_time(e1) / args.steps
    log(f"step: {ms_step * 1e3:.1f} us (events), wall {wall / args.steps * 1e6:.1f} us; "
        f"settle {settle_steps} steps, warm-up {args.warmup}")

    # ---- per-kernel durations: events between the two launches of each
    # step, on the stream the kernels run on (torch's current stream)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record()
        w8a8.quantize_act(x, qx, sx)
        ev[i][1].record()
        w8a8.gemm_blockscale(qx, sx, qw, sw, out=y)
        ev[i][2].record()
    torch.cuda.synchronize()
    gemm_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps

    # the GPU clock over back-to-back GEMM launches (sampled from the SMI
    # metrics), and the GEMM's cycle efficiency at that clock
    clk = ClockSampler()
    n_clk = max(1, int(CLOCK_LOOP_S / (gemm_ms * 1e-3)))

    def clock_loop():
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n_clk):
            w8a8.gemm_blockscale(qx, sx, qw, sw, out=y)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n_clk

    clk_ms = clk.run(clock_loop)
    if clk.samples:
        mhz = sum(clk.samples) / len(clk.samples)
        clk_tops = GEMM_OPS / (clk_ms * 1e-3) / 1e12
        peak_at_clk = 256 * 8192 * mhz * 1e6 / 1e12
        clock = {"source": "SMI GPU metrics: current gfx clock, mean over the XCDs, sampled every ~2 ms during "
                           f"{n_clk} back-to-back GEMM launches",
                 "mhz_mean": round(mhz, 1), "mhz_min": round(min(clk.samples), 1),
                 "mhz_max": round(max(clk.samples), 1), "samples": len(clk.samples),
                 "gemm_us_during": round(clk_ms * 1e3, 2),
                 "gemm_frac_of_peak_at_this_clock": round(clk_tops / peak_at_clk, 4),
                 "clock_frac_of_2400mhz": round(mhz / 2400.0, 4)}
        log(f"clock during {n_clk} GEMMs: {mhz:.0f} MHz mean ({min(clk.samples):.0f}-{max(clk.samples):.0f}); "
            f"GEMM {clk_ms * 1e3:.1f} us = {clk_tops / peak_at_clk:.1%} of the peak at that clock")
    else:
        clock = {"source": "SMI GPU metrics", "mhz_mean": None, "error": clk.error,
                 "gemm_us_during": round(clk_ms * 1e3, 2)}
        log(f"clock not sampled: {clk.error}")

    # quantize with the 256 MiB last-level cache flushed before each launch
    # by READING 1 GiB (a write-based flush would leave dirty lines whose
    # write-back competes with the timed kernel)
    flush_buf = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    flush = flush_buf.amax
    quant_ms = event_times({"q": lambda: w8a8.quantize_act(x, qx, sx)}, args.steps, flush=flush)["q"]["mean"] / 1e3

    # ---- the other workloads of the scope table
    reps = max(10, args.steps // 2)
    configs = {}
    gen = torch.Generator(device=dev).manual_seed(11)
    from block_quantized_int8_amd.workloads import single_linear_256, square_4096
    d1 = single_linear_256()
    tb = lambda bits: torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    configs["single_linear_256"] = measure_config(w8a8, "single linear", tb(d1["x"]), tb(d1["w"]), flush, reps,
                                                  note="latency-bound; seeded workload bits")
    d2 = square_4096()
    x2, w2 = tb(d2["x"]), tb(d2["w"])
    configs["square_4096"] = measure_config(w8a8, "square", x2, w2, flush, reps, note="seeded workload bits")
    del d2, x2, w2
    xu, wu = gpu_normal(gen, (32768, 4096), dev=dev), gpu_normal(gen, (16384, 4096), 0.02, dev=dev)
    configs["mlp_up"] = measure_config(w8a8, "MLP up", xu, wu, flush, reps,
                                       note="GPU-seeded N(0,1) activations, N(0, 0.02^2) weights")
    del xu, wu
    xd = w8a8.gelu_bf16(gpu_normal(gen, (32768, 16384), 1.28, dev=dev))
    wd = gpu_normal(gen, (4096, 16384), 0.02, dev=dev)
    configs["mlp_down"] = measure_config(w8a8, "MLP down", xd, wd, flush, reps,
                                         note="input = exact GELU of GPU-seeded N(0, 1.28^2) (the up projection's "
                                              "spread), 128 K-blocks per output")
    del xd, wd
    xa = gpu_normal(gen, (65536, 4096), outlier_frac=0.005, outlier_factor=30.0, dev=dev)
    wa = gpu_normal(gen, (4096, 4096), 0.02, dev=dev)
    configs["two_stream_a"] = measure_config(w8a8, "two-stream A", xa, wa, flush, reps,
                                             note="GPU-seeded N(0,1), 0.5% of channels x30")
    del xa, wa
    torch.cuda.empty_cache()

    # shared-input projections: Q, K, V (3 x 4096 output channels) on X as
    # three guarded linears vs one group over the concatenated channels
    from block_quantized_int8_amd.workloads import random_bf16
    wk = torch.from_numpy(random_bf16(51, (N, K), 0.02).view(np.int16)).to(dev).view(torch.bfloat16)
    wv = torch.from_numpy(random_bf16(52, (N, K), 0.02).view(np.int16)).to(dev).view(torch.bfloat16)
    projs = [layer, w8a8.W8A8Linear(wk), w8a8.W8A8Linear(wv)]
    group = w8a8.W8A8ProjectionGroup([w, wk, wv])
    group(x)
    for p in projs:
        p(x)
    torch.cuda.synchronize()
    ga, gb, sa, sb = (torch.cuda.Event(enable_timing=True) for _ in range(4))
    ga.record()
    for _ in range(args.steps):
        group(x)
    gb.record()
    sa.record()
    for _ in range(args.steps):
        for p in projs:
            p(x)
    sb.record()
    torch.cuda.synchronize()
    qkv_group_us = ga.elapsed_time(gb) / args.steps * 1e3
    qkv_sep_us = sa.elapsed_time(sb) / args.steps * 1e3
    del group, projs, wk, wv
    log(f"QKV 32768x(3x4096)x4096: one group {qkv_group_us:.1f} us vs three linears {qkv_sep_us:.1f} us")

    # INT8 attention Q and K from the fused Q/K/V output (row stride 3 * 4096)
    qkv, qq, sq = qk_buffers(dev)
    w8a8.quantize_qk(qkv[:, :AH * AD], AH, qq, sq)   # untimed first launch (code object load)
    torch.cuda.synchronize()
    qk_t = event_times({"q": lambda: w8a8.quantize_qk(qkv[:, :AH * AD], AH, qq, sq),
                        "k": lambda: w8a8.quantize_qk(qkv[:, AH * AD:2 * AH * AD], AH, qq, sq)},
                       args.steps, flush=flush)
    qk_us = (qk_t["q"]["mean"] + qk_t["k"]["mean"]) / 2
    del qkv, qq, sq
    log(f"Q/K INT8 [{AL}, {AH}x{AD}] from a fused QKV output: {qk_us:.1f} us per tensor "
        f"({QK_BYTES / qk_us / 1e3:.0f} GB/s)")

    # the guard's bf16 fallback on the shapes that take it: M = 4000 (not a
    # multiple of 128) at 4096^2, and the two-stream workload's 1000 x 2048^2
    fb = {}
    for name, (fm, fn, fk) in (("m4000_n4096_k4096", (4000, 4096, 4096)), ("m1000_n2048_k2048", (1000, 2048, 2048))):
        xf = torch.from_numpy(random_bf16(70 + fk, (fm, fk)).view(np.int16)).to(dev).view(torch.bfloat16)
        wf = torch.from_numpy(random_bf16(71 + fk, (fn, fk), 0.02).view(np.int16)).to(dev).view(torch.bfloat16)
        lf = w8a8.W8A8Linear(wf)
        lf(xf)
        torch.cuda.synchronize()
        assert lf.last_path == w8a8.PATH_BF16
        us = event_times({"f": lambda: lf(xf)}, args.steps)["f"]["median"]
        tf = 2 * fm * fn * fk / (us * 1e-6) / 1e12
        fb[name] = {"us": round(us, 2), "tflops": round(tf, 1), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        del xf, wf, lf
    log("bf16 fallback: " + "; ".join(f"{k} {v['us']} us = {v['tflops']} TFLOP/s" for k, v in fb.items()))

    # two-stream step: A (INT8, 65536 x 4096 x 4096) and B (guarded to the
    # bf16 fallback, 1000 x 2048 x 2048) launched on two streams at once, and
    # each alone
    from block_quantized_int8_amd.workloads import two_stream
    d5 = two_stream()
    xa5, xb5 = tb(d5["x_a"]), tb(d5["x_b"])
    la5, lb5 = w8a8.W8A8Linear(tb(d5["w_a"])), w8a8.W8A8Linear(tb(d5["w_b"]))
    del d5
    sa5, sb5 = torch.cuda.Stream(), torch.cuda.Stream()
    cur = torch.cuda.current_stream()

    def two_stream_run(run_a, run_b):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(cur)
        for _ in range(args.steps):
            start = torch.cuda.Event()
            start.record(cur)
            ends = []
            for run, st5, lay, xin in ((run_a, sa5, la5, xa5), (run_b, sb5, lb5, xb5)):
                if not run:
                    continue
                st5.wait_event(start)
                with torch.cuda.stream(st5):
                    lay(xin)
                e = torch.cuda.Event()
                e.record(st5)
                ends.append(e)
            for e in ends:
                cur.wait_event(e)
        t1.record(cur)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps * 1e3

    two_stream_run(True, True)  # untimed first launches
    assert la5.last_path == w8a8.PATH_INT8 and lb5.last_path == w8a8.PATH_BF16
    ts_both, ts_a, ts_b = two_stream_run(True, True), two_stream_run(True, False), two_stream_run(False, True)
    del xa5, xb5, la5, lb5
    log(f"two-stream step: both {ts_both:.1f} us; A alone {ts_a:.1f} us, B alone {ts_b:.1f} us")

    # producer A/B on the MLP hidden activation: fused GELU + quantize vs
    # GELU then quantize, each launch after the same read flush
    yh, xh, qh, sh = producer_buffers(w8a8, dev)
    w8a8.gelu_quantize_act(yh, qh, sh)                # untimed first launches
    w8a8.gelu_bf16(yh, out=xh)
    torch.cuda.synchronize()
    pt = event_times({"fused": lambda: w8a8.gelu_quantize_act(yh, qh, sh),
                      "gelu": lambda: w8a8.gelu_bf16(yh, out=xh),
                      "quantize": lambda: w8a8.quantize_act(xh, qh, sh)}, args.steps, flush=flush)
    prod_us = {k: v["mean"] for k, v in pt.items()}
    del yh, xh, qh, sh
    log(f"producer A/B (32768x16384): fused {prod_us['fused']:.1f} us "
        f"({PRODUCER_BYTES / prod_us['fused'] / 1e3:.0f} GB/s) vs gelu {prod_us['gelu']:.1f} + "
        f"quantize {prod_us['quantize']:.1f} us")

    # producer A/B on a transformer block's input: modulated RMSNorm / LayerNorm
    # fused with the block quantization vs the normalization then the quantizer
    xr, rsc, rsh, yr, rq, rs = rms_buffers(dev)
    rws = torch.empty(w8a8.rmsnorm_quantize_workspace_bytes(RB * RL, RK), dtype=torch.uint8, device=dev)
    w8a8.rmsnorm_modulate_quantize_act(xr, rsc, rsh, 1e-6, rq, rs, workspace=rws)
    w8a8.layernorm_modulate_quantize_act(xr, rsc, rsh, 1e-6, rq, rs)
    w8a8.rmsnorm_modulate_bf16(xr, rsc, rsh, 1e-6, out=yr)
    w8a8.layernorm_modulate_bf16(xr, rsc, rsh, 1e-6, out=yr)
    torch.cuda.synchronize()
    rt = event_times({"fused": lambda: w8a8.rmsnorm_modulate_quantize_act(xr, rsc, rsh, 1e-6, rq, rs, workspace=rws),
                      "norm": lambda: w8a8.rmsnorm_modulate_bf16(xr, rsc, rsh, 1e-6, out=yr),
                      "quantize": lambda: w8a8.quantize_act(yr.view(RB * RL, RK), rq, rs),
                      "ln_fused": lambda: w8a8.layernorm_modulate_quantize_act(xr, rsc, rsh, 1e-6, rq, rs),
                      "ln_norm": lambda: w8a8.layernorm_modulate_bf16(xr, rsc, rsh, 1e-6, out=yr)},
                     args.steps, flush=flush)
    rms_us = {k: v["mean"] for k, v in rt.items()}
    assert int(rws[:4].view(torch.int32).item()) == 0, "a wait of the single-read RMS producer gave up"
    del xr, rsc, rsh, yr, rq, rs, rws
    log(f"RMSNorm producer A/B ({RB}x{RL}x{RK}): fused {rms_us['fused']:.1f} us "
        f"({RMS_BYTES / rms_us['fused'] / 1e3:.0f} GB/s algorithmic) vs norm {rms_us['norm']:.1f} + "
        f"quantize {rms_us['quantize']:.1f} us")
    log(f"LayerNorm producer A/B: fused {rms_us['ln_fused']:.1f} us vs norm {rms_us['ln_norm']:.1f} + "
        f"quantize {rms_us['quantize']:.1f} us")

    # A/B: the post-scale form (per-row / per-channel scales applied once,
    # INT32 over all of K) on the same inputs and shape
    qwp, swp = w8a8.quantize_rows(w)
    qxp = torch.empty((M, K), dtype=torch.int8, device=dev)
    sxp = torch.empty((M,), dtype=torch.float32, device=dev)
    w8a8.quantize_rows(x, qxp, sxp)
    w8a8.gemm_postscale(qxp, sxp, qwp, swp, out=y)     # untimed first launch
    torch.cuda.synchronize()
    ps_gemm_ms = event_times({"g": lambda: w8a8.gemm_postscale(qxp, sxp, qwp, swp, out=y)},
                             args.steps)["g"]["mean"] / 1e3
    ps_quant_ms = event_times({"q": lambda: w8a8.quantize_rows(x, qxp, sxp)}, args.steps, flush=flush)["q"]["mean"] / 1e3
    del qxp, qwp
    vendor = vendor_int8_context(qx, qw)

    extra = extras(w8a8, dev, args, x, y, qx, sx, qw, sw, flush) if args.extras else None
    del flush_buf

    gemm_tops = GEMM_OPS / (gemm_ms * 1e-3) / 1e12
    quant_gbs = QUANT_BYTES / (quant_ms * 1e-3) / 1e9
    value = GEMM_OPS / (ms_step * 1e-3) / 1e12
    log(f"gemm {gemm_ms * 1e3:.1f} us = {gemm_tops:.0f} TOPS ({gemm_tops / PEAK_INT8_TOPS:.1%}); "
        f"quantize {quant_ms * 1e3:.1f} us = {quant_gbs:.0f} GB/s ({quant_gbs / PEAK_HBM_GBS:.1%})")
    log(f"post-scale A/B: gemm {ps_gemm_ms * 1e3:.1f} us = {GEMM_OPS / (ps_gemm_ms * 1e-3) / 1e12:.0f} TOPS; "
        f"row quantize {ps_quant_ms * 1e3:.1f} us")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on its sample ...")
        cpu = cpu_baseline(d)
        log(f"cpu oracle: {cpu['value'] * 1e3:.2f} GOPS on {cpu['cores']} threads, {cpu['seconds']} s")

    configs["attention_projection"] = {
        "shape": [M, N, K], "gemm_us": round(gemm_ms * 1e3, 2), "gemm_tops": round(gemm_tops, 1),
        "gemm_frac_of_int8_peak": round(gemm_tops / PEAK_INT8_TOPS, 4),
        "quantize_us": round(quant_ms * 1e3, 2), "quantize_gbs": round(quant_gbs, 1),
        "quantize_frac_of_hbm": round(quant_gbs / PEAK_HBM_GBS, 4),
        "note": "the headline workload (the step); oracle: cpu_baseline"}

    traffic = load_traffic()
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "attention-projection W8A8 linear, heavy-tailed activations "
                               "(1% of K channels x20), seed 2",
                   "M": M, "N": N, "K": K, "block": 128, "path": "int8",
                   "step": "w8a8_linear = activation quantize + INT8 block-scale GEMM"},
        "gemm_tops": round(gemm_tops, 1),
        "gemm_frac_of_int8_peak": round(gemm_tops / PEAK_INT8_TOPS, 4),
        "gemm_us": round(gemm_ms * 1e3, 2),
        "quantize_gbs": round(quant_gbs, 1),
        "quantize_frac_of_hbm": round(quant_gbs / PEAK_HBM_GBS, 4),
        "quantize_us": round(quant_ms * 1e3, 2),
        "roofline": {"bound": "mfma", "kernel": "gemm_i8_blockscale",
                     "achieved": round(gemm_tops, 1), "peak": round(PEAK_INT8_TOPS, 1),
                     "unit": "TFLOP/s", "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
                     "unit_note": "int8 operations (a multiply-add counts 2) per second, 1e12, against the "
                                  "dense int8 MFMA peak",
                     "traffic": traffic,
                     "algorithmic_bytes": GEMM_BYTES, "ops_per_launch": GEMM_OPS},
        "roofline_quantize": {"bound": "hbm", "kernel": "quantize_block",
                              "achieved": round(quant_gbs, 1), "peak": PEAK_HBM_GBS,
                              "unit": "GB/s", "frac": round(quant_gbs / PEAK_HBM_GBS, 4),
                              "traffic": load_traffic(QUANT_TRAFFIC_FILE, QUANT_SOURCE),
                              "algorithmic_bytes": QUANT_BYTES},
        "clock": clock,
        "cpu_baseline": cpu,
        "configs": configs,
        "postscale_ab": {"note": "post-scale form on the same shape (not the headline path)",
                         "gemm_us": round(ps_gemm_ms * 1e3, 2),
                         "gemm_tops": round(GEMM_OPS / (ps_gemm_ms * 1e-3) / 1e12, 1),
                         "gemm_frac_of_int8_peak": round(GEMM_OPS / (ps_gemm_ms * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
                         "quantize_rows_us": round(ps_quant_ms * 1e3, 2)},
        "vendor_int8_context": vendor,
        "two_stream": {"note": "A: INT8 linear 65536x4096x4096 (0.5% channels x30); B: 1000x2048x2048 "
                               "guarded to the bf16 fallback; launched on two streams per step (not the headline)",
                       "step_us": round(ts_both, 2), "a_alone_us": round(ts_a, 2), "b_alone_us": round(ts_b, 2)},
        "fallback_bf16": {"note": "the guard's bf16 fallback (row-major bf16 MFMA GEMM) on the shapes "
                                  "that take it; peak = dense bf16 MFMA 2516.6 TFLOP/s", **fb},
        "qkv_concat_ab": {"note": "Q, K, V projections of X (3 x 4096 output channels): one "
                                  "concatenated guarded linear vs three (not part of a step)",
                          "group_us": round(qkv_group_us, 2), "separate_us": round(qkv_sep_us, 2),
                          "group_tops": round(3 * GEMM_OPS / (qkv_group_us * 1e-6) / 1e12, 1),
                          "speedup": round(qkv_sep_us / qkv_group_us, 3)},
        "qk_quantize": {"note": "INT8 Q or K of a video self-attention, sequence-major rows of a fused "
                                "Q/K/V output -> head-major codes + per-128-token scales (not part of a step)",
                        "shape": {"tokens": AL, "heads": AH, "head_dim": AD, "row_stride": 3 * AH * AD},
                        "us": round(qk_us, 2), "gbs": round(QK_BYTES / qk_us / 1e3, 1),
                        "frac_of_hbm": round(QK_BYTES / qk_us / 1e3 / PEAK_HBM_GBS, 4),
                        "algorithmic_bytes": QK_BYTES},
        "rmsnorm_producer_ab": {"note": "transformer-block input: modulated RMSNorm fused with the 128x128 "
                                        "block quantize (single read of x: band workgroups exchange fp64 row "
                                        "partials) vs the normalization then the quantizer (not part of a step)",
                                "shape": [RB, RL, RK],
                                "fused_us": round(rms_us["fused"], 2),
                                "fused_gbs_algorithmic": round(RMS_BYTES / rms_us["fused"] / 1e3, 1),
                                "fused_frac_of_hbm": round(RMS_BYTES / rms_us["fused"] / 1e3 / PEAK_HBM_GBS, 4),
                                "algorithmic_bytes": RMS_BYTES,
                                "unfused_norm_us": round(rms_us["norm"], 2),
                                "unfused_quantize_us": round(rms_us["quantize"], 2),
                                "speedup": round((rms_us["norm"] + rms_us["quantize"]) / rms_us["fused"], 3)},
        "layernorm_producer_ab": {"note": "the same input with the modulated layer normalization fused with "
                                          "the 128x128 block quantize (row statistics, then a second read of x) "
                                          "vs the normalization then the quantizer",
                                  "shape": [RB, RL, RK],
                                  "fused_us": round(rms_us["ln_fused"], 2),
                                  "fused_gbs_algorithmic": round(RMS_BYTES / rms_us["ln_fused"] / 1e3, 1),
                                  "fused_frac_of_hbm": round(RMS_BYTES / rms_us["ln_fused"] / 1e3 / PEAK_HBM_GBS, 4),
                                  "algorithmic_bytes": RMS_BYTES,
                                  "unfused_norm_us": round(rms_us["ln_norm"], 2),
                                  "unfused_quantize_us": round(rms_us["quantize"], 2),
                                  "speedup": round((rms_us["ln_norm"] + rms_us["quantize"]) / rms_us["ln_fused"], 3)},
        "producer_ab": {"note": "MLP producer: exact GELU + 128x128 block quantize of the hidden "
                                "activation, fused vs GELU then quantize (not part of a step)",
                        "shape": [HM, HK],
                        "fused_us": round(prod_us["fused"], 2),
                        "fused_gbs": round(PRODUCER_BYTES / prod_us["fused"] / 1e3, 1),
                        "fused_frac_of_hbm": round(PRODUCER_BYTES / prod_us["fused"] / 1e3 / PEAK_HBM_GBS, 4),
                        "algorithmic_bytes": PRODUCER_BYTES,
                        "unfused_gelu_us": round(prod_us["gelu"], 2),
                        "unfused_quantize_us": round(prod_us["quantize"], 2),
                        "speedup": round((prod_us["gelu"] + prod_us["quantize"]) / prod_us["fused"], 3)},
        "run_seconds": round(time.perf_counter() - t_start, 1),
    }
    if extra:
        out["extras"] = extra
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
