"""A second, independent oracle for tiny inputs, in numpy and plain Python.

TEST INFRASTRUCTURE ONLY, like the C oracle beside it: the CPU tests run
both on the same small seeded inputs and require identical codes, scales,
partials and bf16 outputs, so that a slip in either one (an index, an
operand order, a rounding step) shows up as a disagreement.  It shares no
code with the C oracle or with the GPU library; it is written straight from
the definitions:

* block quantization (TurboDiffusion news article, bjdmk.com.cn, section on
  sparsity, distillation and full-pipeline quantization and the inference
  list: 128x128 blocks for weights and, at the same granularity, for
  activations; TurboT2VA paper, architecture-aware inference stack, W8A8
  paragraph: scale = max-abs / 127, INT8 codes);
* the block-scaled product: exact integer sums inside each 128-deep K-block,
  each scaled by its two block scales, summed in fp64 and rounded once to
  bf16 (nearest, ties to even);
* the bf16 fallback and the guard (TurboT2VA paper, guard paragraph);
* the post-scale form (TurboT2VA paper, W8A8 paragraph: per-row and
  per-output-channel max(max-abs, 1e-4) / 127, integer sum over all of K,
  scales and bias once at the end);
* INT8 attention Q/K (TurboT2VA paper, sparse-attention paragraph): the
  block rule over 128 tokens x the head dimension, per batch and head; V in
  FP8 E4M3 over the same blocks (same paragraph: FP8 values);
* the modulated RMS and layer normalizations, the split-halves rotary
  embedding and the gated residual update (TurboT2VA paper, fused-kernels
  paragraph).

Everything is O(M*N*K) Python-level numpy on small arrays: use it on
inputs of a few hundred rows at most.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 128
EPS = np.float32(1e-4)


# ---------------------------------------------------------------- bf16 bits

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values (a bf16 is the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _round_half_even(v: float) -> float:
    f = math.floor(v)
    d = v - f  # exact: v and f are within one unit of each other
    if d > 0.5 or (d == 0.5 and f % 2 == 1):
        f += 1
    return float(f)


def f64_to_bf16_bits(v: float) -> int:
    """Round one finite float64 to bf16 (nearest, ties to even), directly
    rather than through fp32 (which could round twice)."""
    if v == 0.0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    _, e = math.frexp(a)           # a = m * 2^e with 0.5 <= m < 1
    # bf16 keeps 8 significant bits; below 2^-126 the spacing stays 2^-133
    ulp_exp = max(e - 8, -133)
    r = _round_half_even(math.ldexp(a, -ulp_exp))   # exact scaling by a power of two
    val = math.ldexp(r, ulp_exp)
    bits = int(np.array([val], dtype=np.float32).view(np.uint32)[0] >> 16)
    return sign | bits


def f64_to_bf16_array(a: np.ndarray) -> np.ndarray:
    flat = [f64_to_bf16_bits(float(v)) for v in np.asarray(a, dtype=np.float64).ravel()]
    return np.array(flat, dtype=np.uint16).reshape(np.shape(a))


# ------------------------------------------------------------- quantization

def _codes(x32: np.ndarray, s: np.float32) -> np.ndarray:
    """q = rint(fl32(x / s)), ties to even, clamped to [-127, 127]; s = 0 -> 0."""
    if s == 0:
        return np.zeros(x32.shape, np.int8)
    quo = (x32 / s).astype(np.float32)          # IEEE fp32 division, one rounding
    return np.clip(np.rint(quo), -127, 127).astype(np.int8)


def quantize_block(x_bits: np.ndarray):
    """128x128 block quantization of a bf16 matrix -> (q int8, s fp32 [R/128, C/128])."""
    x32 = bf16_to_f64(x_bits).astype(np.float32)    # exact
    R, C = x32.shape
    q = np.zeros((R, C), np.int8)
    s = np.zeros((R // BLOCK, C // BLOCK), np.float32)
    for i in range(R // BLOCK):
        for j in range(C // BLOCK):
            blk = x32[i * BLOCK:(i + 1) * BLOCK, j * BLOCK:(j + 1) * BLOCK]
            a = np.float32(np.max(np.abs(blk)))
            sc = np.float32(a / np.float32(127.0))
            s[i, j] = sc
            q[i * BLOCK:(i + 1) * BLOCK, j * BLOCK:(j + 1) * BLOCK] = _codes(blk, sc)
    return q, s


def kblock_partials(qx: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """P[m, n, kb] = sum over the K-block of qx[m, k] * qw[n, k], exact (int64)."""
    M, K = qx.shape
    kbs = K // BLOCK
    a = qx.astype(np.int64).reshape(M, kbs, BLOCK)
    b = qw.astype(np.int64).reshape(qw.shape[0], kbs, BLOCK)
    return np.einsum("mkb,nkb->mnk", a, b)


def linear_int8(qx, sx, qw, sw, bias=None) -> np.ndarray:
    """bf16( sum_kb P * sx[m/128, kb] * sw[n/128, kb] (+ bias) ), fp64 sums in K-block order."""
    P = kblock_partials(qx, qw).astype(np.float64)
    M, N, kbs = P.shape
    sxd = np.asarray(sx, np.float32).astype(np.float64)
    swd = np.asarray(sw, np.float32).astype(np.float64)
    rowblk = np.arange(M) // BLOCK
    colblk = np.arange(N) // BLOCK
    acc = np.zeros((M, N), np.float64)
    for kb in range(kbs):
        acc = acc + P[:, :, kb] * sxd[rowblk, kb][:, None] * swd[colblk, kb][None, :]
    if bias is not None:
        acc = acc + bf16_to_f64(bias)[None, :]
    return f64_to_bf16_array(acc)


def linear_bf16(x_bits, w_bits, bias=None) -> np.ndarray:
    """The fallback on bf16 input: bf16( sum_k x * w (+ bias) ) with fp64 sums."""
    acc = bf16_to_f64(x_bits) @ bf16_to_f64(w_bits).T
    if bias is not None:
        acc = acc + bf16_to_f64(bias)[None, :]
    return f64_to_bf16_array(acc)


def route(is_bf16: bool, M: int, K: int, N: int, has_qweight: bool) -> int:
    """0 (INT8 path) iff bf16 input, M, K, N multiples of 128 and a quantized weight; else 1."""
    ok = is_bf16 and has_qweight and M > 0 and K > 0 and N > 0 and M % BLOCK == 0 \
        and K % BLOCK == 0 and N % BLOCK == 0
    return 0 if ok else 1


# ------------------------------------------------------------ post-scale form

def quantize_rows(x_bits: np.ndarray):
    """Per-row s = fl32(max(max-abs, 1e-4) / 127), q = rint(fl32(x / s))."""
    x32 = bf16_to_f64(x_bits).astype(np.float32)
    q = np.zeros(x32.shape, np.int8)
    s = np.zeros(x32.shape[0], np.float32)
    for i in range(x32.shape[0]):
        a = np.float32(max(np.float32(np.max(np.abs(x32[i]))), np.float32(EPS)))
        s[i] = np.float32(a / np.float32(127.0))
        q[i] = _codes(x32[i], s[i])
    return q, s


def linear_postscale(qx, sx, qw, sw, bias=None) -> np.ndarray:
    """bf16( (sum_k qx * qw) * sx[m] * sw[n] (+ bias) ): integer sum over all of K."""
    acc = (qx.astype(np.int64) @ qw.astype(np.int64).T).astype(np.float64)
    acc = acc * np.asarray(sx, np.float32).astype(np.float64)[:, None] \
        * np.asarray(sw, np.float32).astype(np.float64)[None, :]
    if bias is not None:
        acc = acc + bf16_to_f64(bias)[None, :]
    return f64_to_bf16_array(acc)


# ---------------------------------------------------------- attention Q / K

def quantize_qk(x_bits: np.ndarray, B: int, L: int, H: int, D: int, ld: int):
    """Rows b*L + l of width ld hold token l of batch b, head h at columns
    h*D .. h*D + D-1.  Each (b, h) is cut into blocks of 128 tokens (the last
    may be shorter), each quantized by the block rule over tokens x D.
    -> (q int8 [B, H, L, D], s fp32 [B, H, ceil(L/128)])."""
    x = np.asarray(x_bits, np.uint16).reshape(B * L, ld)
    nblk = -(-L // BLOCK)
    q = np.zeros((B, H, L, D), np.int8)
    s = np.zeros((B, H, nblk), np.float32)
    for b in range(B):
        for h in range(H):
            head = bf16_to_f64(x[b * L:(b + 1) * L, h * D:(h + 1) * D]).astype(np.float32)
            for j in range(nblk):
                blk = head[j * BLOCK:min((j + 1) * BLOCK, L)]
                a = np.float32(np.max(np.abs(blk)))
                sc = np.float32(a / np.float32(127.0))
                s[b, h, j] = sc
                q[b, h, j * BLOCK:j * BLOCK + blk.shape[0]] = _codes(blk, sc)
    return q, s


# ------------------------------------------------------------ attention V, FP8

def _e4m3_table():
    """(value, code) of every finite non-negative E4M3 code, by its definition."""
    out = []
    for c in range(0x7F):            # 0x7F is NaN
        e, m = c >> 3, c & 7
        v = math.ldexp(m, -9) if e == 0 else math.ldexp(8 + m, e - 10)
        out.append((v, c))
    return out


_E4M3 = _e4m3_table()


def e4m3_code(v: float) -> int:
    """Nearest finite E4M3 code by search over all codes, ties to the even
    code; NaN (0x7F) beyond 464, where the next step up (480, not a finite
    code) is nearer than 448 (at 464 itself the tie goes to 448's even code)."""
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    if a > 464.0:
        return sign | 0x7F
    best = min(_E4M3, key=lambda vc: (abs(vc[0] - a), vc[1] & 1))
    return sign | best[1]


def quantize_v_fp8(x_bits: np.ndarray, B: int, L: int, H: int, D: int, ld: int):
    """Per (b, h) and block of 128 tokens x D: s = fl32(max|x| / 448), codes
    E4M3(fl32(x / s)); head-major [B, H, L, D] codes and [B, H, blocks] scales."""
    x = np.asarray(x_bits, np.uint16).reshape(B * L, ld)
    nblk = -(-L // BLOCK)
    q = np.zeros((B, H, L, D), np.uint8)
    s = np.zeros((B, H, nblk), np.float32)
    for b in range(B):
        for h in range(H):
            head = bf16_to_f64(x[b * L:(b + 1) * L, h * D:(h + 1) * D]).astype(np.float32)
            for j in range(nblk):
                blk = head[j * BLOCK:min((j + 1) * BLOCK, L)]
                a = np.float32(np.max(np.abs(blk)))
                sc = np.float32(a / np.float32(448.0))
                s[b, h, j] = sc
                if a == 0:
                    continue
                quo = (blk / sc).astype(np.float32)
                q[b, h, j * BLOCK:j * BLOCK + blk.shape[0]] = np.vectorize(lambda v: e4m3_code(float(v)))(quo)
    return q, s


# ------------------------------------------------ modulated RMS normalization

def rmsnorm_modulate(x_bits: np.ndarray, L: int, scale_bits: np.ndarray, shift_bits: np.ndarray,
                     eps: float = 1e-6) -> np.ndarray:
    """Row i = b*L + l: r = fl32(1 / sqrt(sum_k x^2 / K + eps)) with the sum
    taken exactly (math.fsum) and the rest in fp64; then per element, each
    step one fp32 rounding: bf16(((x * r) * (1 + scale[b])) + shift[b])."""
    x = bf16_to_f64(x_bits)
    sc = bf16_to_f64(scale_bits).astype(np.float32)
    sh = bf16_to_f64(shift_bits).astype(np.float32)
    R, K = x.shape
    y = np.zeros((R, K), np.uint16)
    for i in range(R):
        b = i // L
        S = math.fsum(float(v) * float(v) for v in x[i])
        r = np.float32(1.0 / math.sqrt(S / K + eps))
        for k in range(K):
            t = np.float32(np.float32(x[i, k]) * r)
            u = np.float32(t * np.float32(np.float32(1.0) + sc[b, k]))
            v = np.float32(u + sh[b, k])
            y[i, k] = f64_to_bf16_bits(float(v))
    return y


def layernorm_modulate(x_bits: np.ndarray, L: int, scale_bits: np.ndarray, shift_bits: np.ndarray,
                       eps: float = 1e-6) -> np.ndarray:
    """Row i = b*L + l: the mean (exact sum, math.fsum) and the variance of
    the deviations from it in fp64, m = fl32(mean), r = fl32(1 / sqrt(var +
    eps)); then per element, each step one fp32 rounding:
    bf16((((x - m) * r) * (1 + scale[b])) + shift[b])."""
    x = bf16_to_f64(x_bits)
    sc = bf16_to_f64(scale_bits).astype(np.float32)
    sh = bf16_to_f64(shift_bits).astype(np.float32)
    R, K = x.shape
    y = np.zeros((R, K), np.uint16)
    for i in range(R):
        b = i // L
        mu = math.fsum(float(v) for v in x[i]) / K
        var = math.fsum((float(v) - mu) ** 2 for v in x[i]) / K
        m = np.float32(mu)
        r = np.float32(1.0 / math.sqrt(var + eps))
        for k in range(K):
            c = np.float32(np.float32(x[i, k]) - m)
            t = np.float32(c * r)
            u = np.float32(t * np.float32(np.float32(1.0) + sc[b, k]))
            v = np.float32(u + sh[b, k])
            y[i, k] = f64_to_bf16_bits(float(v))
    return y


# ------------------------------------------------------ split rotary embedding

def rope(x_bits: np.ndarray, B: int, L: int, H: int, D: int, ld: int, cos_t: np.ndarray, sin_t: np.ndarray):
    """Pairs (d, d + D/2) of each head rotated by the token's table angle,
    each product and sum one fp32 rounding, the result rounded to bf16."""
    x = bf16_to_f64(np.asarray(x_bits, np.uint16).reshape(B * L, ld)).astype(np.float32)
    half = D // 2
    y = np.zeros((B * L, H * D), np.uint16)
    for row in range(B * L):
        l = row % L
        c = np.asarray(cos_t, np.float32)[l]
        s = np.asarray(sin_t, np.float32)[l]
        for h in range(H):
            x1 = x[row, h * D:h * D + half]
            x2 = x[row, h * D + half:h * D + D]
            lo = (x1 * c).astype(np.float32) - (x2 * s).astype(np.float32)
            hi = (x2 * c).astype(np.float32) + (x1 * s).astype(np.float32)
            y[row, h * D:h * D + half] = f64_to_bf16_array(lo.astype(np.float32).astype(np.float64))
            y[row, h * D + half:h * D + D] = f64_to_bf16_array(hi.astype(np.float32).astype(np.float64))
    return y


# ------------------------------------------------------- gated residual update

def gated_residual(h_bits: np.ndarray, o_bits: np.ndarray, gate_bits: np.ndarray, L: int) -> np.ndarray:
    """Row i: bf16(fl32(h + fl32(gate[i // L] * o))), each fl32 one numpy fp32
    operation, then one rounding to bf16."""
    h = bf16_to_f64(h_bits).astype(np.float32)
    o = bf16_to_f64(o_bits).astype(np.float32)
    g = bf16_to_f64(gate_bits).astype(np.float32)
    R, N = h.shape
    y = np.zeros((R, N), np.uint16)
    for i in range(R):
        p = (g[i // L] * o[i]).astype(np.float32)
        s = (h[i] + p).astype(np.float32)
        y[i] = f64_to_bf16_array(s.astype(np.float64))
    return y
