"""Seeded synthetic inputs for the W8A8 block-quantized linear.

This module only draws random numbers and stores them as bf16 bit patterns.
It holds none of the method's arithmetic (no quantization, no GEMM, no
rounding of results) and is shared, unchanged, by the GPU tests, the CPU
oracle's tests and the benchmark, so both sides see the same bits.

The pages give no layer widths or token counts for the video-audio model
(TurboT2VA paper, experiments: LTX-2 at 1024x1792, 121 frames, batch 1), so
these transformer-linear shapes stand in for them:

* ``single_linear_256``  M=N=K=256 (2x2 blocks on each operand), seed 0
* ``square_4096``  square 4096^3, seed 1, plus a guard case with M=4000 (same W)
* ``attention_projection``  attention-projection shape M=32768, N=K=4096 with heavy-tailed
          activations (1% of K channels scaled by 20), seed 2
* ``mlp_pair``  MLP pair: up 32768x16384x4096, then down 32768x4096x16384, seed 3
* ``two_stream``  two-stream step: A 65536x4096x4096 (INT8 path) and B 1000x2048x2048
          (guarded to the bf16 fallback), 0.5% outlier channels x30, seed 4
* ``attention_qk``  query and key of one video self-attention, sequence-major
          [28672, 32 x 128], seed 6: 28672 = 32 x 56 x 16 latent tokens of a
          1024x1792, 121-frame clip under 32x32 spatial and 8x temporal
          compression (assumed; the pages give the resolution and frame count
          only), 32 heads of 128; N(0, 1.28^2) with 1% of the key's channels
          x10 (heavy tails); ``l``/``heads``/``d`` select other (e.g. short,
          ragged audio) sequences
* ``block_hidden``  a transformer block's hidden state with its modulation,
          the input of the fused modulated-RMSNorm + quantize producer, seed 8:
          x [b*l, k] ~ N(0, 2^2) with 1% of channels x10 (massive activations),
          scale and shift [b, k] ~ N(0, 0.3^2) (per batch entry, as timestep
          modulation is); default b = 4, l = 8192, k = 4096 (32768 rows, the
          attention-projection input)
* ``mlp_hidden``  stand-in for the MLP pair's up-projection output (the input
          of the fused GELU + quantize producer), 32768 x 16384, seed 5:
          N(0, 1.28^2), the spread of the MLP pair's up projection (sqrt(4096) * 0.02)

Recipe: ``numpy.random.default_rng(seed)`` (PCG64); every tensor is drawn
with ``standard_normal(shape, dtype=float32)`` in the order listed per workload;
weights are multiplied by 0.02 and outlier channels by their factor in fp32;
each fp32 array is converted to bf16 once, round-to-nearest-even on the bits.
Outlier channels are ``rng.choice(K, round(p*K), replace=False)`` drawn after
all tensors of the workload.
"""
from __future__ import annotations

import numpy as np

WEIGHT_STD = np.float32(0.02)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Inputs are finite by construction; this is data preparation, not part of
    the method.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(rng, shape, scale=None):
    a = rng.standard_normal(shape, dtype=np.float32)
    if scale is not None:
        a *= np.float32(scale)
    return a


def _outlier_channels(rng, k: int, frac: float) -> np.ndarray:
    n = int(round(frac * k))
    return rng.choice(k, n, replace=False)


def single_linear_256():
    rng = np.random.default_rng(0)
    x = _normal(rng, (256, 256))
    w = _normal(rng, (256, 256), WEIGHT_STD)
    return {"x": f32_to_bf16_bits(x), "w": f32_to_bf16_bits(w)}


def square_4096():
    rng = np.random.default_rng(1)
    x = _normal(rng, (4096, 4096))
    w = _normal(rng, (4096, 4096), WEIGHT_STD)
    xg = _normal(rng, (4000, 4096))
    return {"x": f32_to_bf16_bits(x), "w": f32_to_bf16_bits(w), "x_guard": f32_to_bf16_bits(xg)}


def attention_projection(m: int = 32768):
    """The benchmarked shape. ``m`` may be lowered only by callers that state so."""
    rng = np.random.default_rng(2)
    x = _normal(rng, (m, 4096))
    w = _normal(rng, (4096, 4096), WEIGHT_STD)
    ch = _outlier_channels(rng, 4096, 0.01)
    x[:, ch] *= np.float32(20.0)
    return {"x": f32_to_bf16_bits(x), "w": f32_to_bf16_bits(w), "outlier_channels": np.sort(ch)}


def mlp_pair():
    rng = np.random.default_rng(3)
    x = _normal(rng, (32768, 4096))
    w_up = _normal(rng, (16384, 4096), WEIGHT_STD)
    w_down = _normal(rng, (4096, 16384), WEIGHT_STD)
    return {"x": f32_to_bf16_bits(x), "w_up": f32_to_bf16_bits(w_up),
            "w_down": f32_to_bf16_bits(w_down)}


def two_stream():
    rng = np.random.default_rng(4)
    xa = _normal(rng, (65536, 4096))
    wa = _normal(rng, (4096, 4096), WEIGHT_STD)
    xb = _normal(rng, (1000, 2048))
    wb = _normal(rng, (2048, 2048), WEIGHT_STD)
    cha = _outlier_channels(rng, 4096, 0.005)
    chb = _outlier_channels(rng, 2048, 0.005)
    xa[:, cha] *= np.float32(30.0)
    xb[:, chb] *= np.float32(30.0)
    return {"x_a": f32_to_bf16_bits(xa), "w_a": f32_to_bf16_bits(wa),
            "x_b": f32_to_bf16_bits(xb), "w_b": f32_to_bf16_bits(wb),
            "outlier_channels_a": np.sort(cha), "outlier_channels_b": np.sort(chb)}


def random_bf16(seed: int, shape, scale: float = 1.0) -> np.ndarray:
    """Generic seeded N(0, scale^2) tensor as bf16 bits, for parity cases."""
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(_normal(rng, shape, scale))


def sample_rows(seed: int, m: int, extra: int = 1024, block: int = 128) -> np.ndarray:
    """Deterministic row sample: every row of the first, middle and last
    128-row block plus ``extra`` seeded rows, sorted and unique."""
    nb = max(1, m // block)
    rows = []
    for b in sorted({0, nb // 2, nb - 1}):
        rows.extend(range(b * block, min(m, (b + 1) * block)))
    rng = np.random.default_rng(seed)
    rows.extend(rng.integers(0, m, size=extra).tolist())
    return np.unique(np.asarray(rows, dtype=np.int64))


def mlp_hidden(m: int = 32768, n: int = 16384, seed: int = 5) -> np.ndarray:
    """bf16 [m, n] ~ N(0, 1.28^2): the MLP's hidden pre-activation (``m`` or
    ``n`` may be lowered only by callers that state so)."""
    rng = np.random.default_rng(seed)
    a = _normal(rng, (m, n), 1.28)
    out = np.empty((m, n), np.uint16)
    for r in range(0, m, 2048):  # bounded temporaries; same bits as one call
        out[r:r + 2048] = f32_to_bf16_bits(a[r:r + 2048])
    return out


def attention_qk(l: int = 28672, heads: int = 32, d: int = 128, seed: int = 6):
    """{"q", "k"}: bf16 [l, heads * d] each, sequence-major."""
    rng = np.random.default_rng(seed)
    q = _normal(rng, (l, heads * d), 1.28)
    k = _normal(rng, (l, heads * d), 1.28)
    ch = _outlier_channels(rng, heads * d, 0.01)
    k[:, ch] *= np.float32(10.0)
    return {"q": f32_to_bf16_bits(q), "k": f32_to_bf16_bits(k)}


def block_hidden(b: int = 4, l: int = 8192, k: int = 4096, seed: int = 8):
    """{"x": bf16 [b*l, k], "scale": bf16 [b, k], "shift": bf16 [b, k], "L": l}."""
    rng = np.random.default_rng(seed)
    x = _normal(rng, (b * l, k), 2.0)
    scale = _normal(rng, (b, k), 0.3)
    shift = _normal(rng, (b, k), 0.3)
    ch = _outlier_channels(rng, k, 0.01)
    x[:, ch] *= np.float32(10.0)
    out = np.empty((b * l, k), np.uint16)
    for r in range(0, b * l, 2048):  # bounded temporaries; same bits as one call
        out[r:r + 2048] = f32_to_bf16_bits(x[r:r + 2048])
    return {"x": out, "scale": f32_to_bf16_bits(scale), "shift": f32_to_bf16_bits(shift), "L": l}


def rope_tables(l: int, d: int, grid=None, base: float = 10000.0):
    """(cos, sin): fp32 [l, d/2] tables of rotary angles, one row per token.

    Inputs of the rotary embedding, not part of it: angle(p, i) = p *
    base^(-i / n) for pair i of a group of n pairs, in fp64, then cos and sin
    rounded once to fp32.  With ``grid = (f, h, w)`` (f*h*w = l tokens in
    frame, row, column order) the d/2 pairs are split into three groups
    (the first takes the remainder) driven by the token's frame, row and
    column index, as video transformers place tokens; else one group driven
    by the position l.  No random numbers are drawn.
    """
    half = d // 2
    pos = np.arange(l, dtype=np.float64)
    if grid is None:
        groups = [(pos, half)]
    else:
        f, h, w = grid
        if f * h * w != l:
            raise ValueError("grid does not cover l tokens")
        n_hw = half // 3
        groups = [(pos // (h * w), half - 2 * n_hw), ((pos // w) % h, n_hw), (pos % w, n_hw)]
    ang = np.concatenate([p[:, None] * base ** (-np.arange(n, dtype=np.float64) / n)[None, :] for p, n in groups],
                         axis=1)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
