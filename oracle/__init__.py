"""CPU oracle for the guarded W8A8 block-quantized linear (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are its only users.  The GPU library never
imports, links or calls it, and it shares no code with it.  The arithmetic
lives in ``oracle.c`` (plain C, see its header for the passages it follows);
this module only marshals numpy arrays.

bf16 tensors are passed as ``uint16`` bit patterns, quantized tensors as
``int8``, scales as ``float32``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

DTYPE_BF16, DTYPE_FP16, DTYPE_FP32 = 0, 1, 2
PATH_INT8, PATH_BF16 = 0, 1
BLOCK = 128

_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                               "or python oracle/build.py")
        _lib = load(_LIB_PATH)
    return _lib


def load(path):
    """ctypes handle of an oracle build at ``path`` with every signature set
    (the mutation tests load deliberately broken copies this way)."""
    L = ctypes.CDLL(path)
    L.oracle_quantize_block.argtypes = [_P, _I64, _I64, _P, _P]
    L.oracle_kblock_partials.argtypes = [_P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I64, _P]
    L.oracle_linear_int8_rows.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P, _P]
    L.oracle_linear_bf16_rows.argtypes = [_P, ctypes.c_int, _P, _P, _I64, _I64, _I64, _P, _I64, _P]
    L.oracle_route.argtypes = [ctypes.c_int, _I64, _I64, _I64, ctypes.c_int]
    L.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
    L.oracle_f64_to_bf16.restype = ctypes.c_uint16
    L.oracle_fp16_to_f64.argtypes = [ctypes.c_uint16]
    L.oracle_fp16_to_f64.restype = ctypes.c_double
    L.oracle_gelu_bf16.argtypes = [_P, _I64, _P]
    L.oracle_quantize_rows.argtypes = [_P, _I64, _I64, _P, _P]
    L.oracle_linear_postscale_rows.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P]
    L.oracle_quantize_qk.argtypes = [_P, _I64, _I64, _I64, _I64, _I64, _P, _P]
    L.oracle_rmsnorm_modulate.argtypes = [_P, _I64, _I64, _I64, _P, _P, ctypes.c_double, _P, _P]
    L.oracle_rope.argtypes = [_P, _I64, _I64, _I64, _I64, _I64, _P, _P, _P]
    L.oracle_gated_residual.argtypes = [_P, _P, _P, _I64, _I64, _I64, _P]
    L.oracle_layernorm_modulate.argtypes = [_P, _I64, _I64, _I64, _P, _P, ctypes.c_double, _P, _P]
    L.oracle_quantize_v_fp8.argtypes = [_P, _I64, _I64, _I64, _I64, _I64, _P, _P]
    L.oracle_f32_to_e4m3.argtypes = [ctypes.c_float]
    L.oracle_f32_to_e4m3.restype = ctypes.c_uint8
    L.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
    L.oracle_e4m3_to_f64.restype = ctypes.c_double
    for f in ("oracle_quantize_block", "oracle_kblock_partials", "oracle_linear_int8_rows",
              "oracle_linear_bf16_rows", "oracle_route", "oracle_gelu_bf16",
              "oracle_num_threads", "oracle_quantize_rows", "oracle_linear_postscale_rows",
              "oracle_quantize_qk", "oracle_rmsnorm_modulate", "oracle_rope",
              "oracle_gated_residual", "oracle_layernorm_modulate", "oracle_quantize_v_fp8"):
        getattr(L, f).restype = ctypes.c_int
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return lib().oracle_num_threads()


def quantize_block(x_bf16: np.ndarray):
    """128x128 block-absmax INT8 quantization -> (q int8 [R,C], s fp32 [R/128, C/128])."""
    x = _c(x_bf16, np.uint16)
    r, c = x.shape
    q = np.empty((r, c), np.int8)
    s = np.empty((max(r // BLOCK, 1), max(c // BLOCK, 1)), np.float32)
    _check(lib().oracle_quantize_block(_ptr(x), r, c, _ptr(q), _ptr(s)), "quantize_block")
    return q, s


def kblock_partials(qx, qw, m0=0, mt=None, n0=0, nt=None):
    """int32 per-K-block partial sums, shape [mt, nt, K/128]."""
    qx = _c(qx, np.int8)
    qw = _c(qw, np.int8)
    M, K = qx.shape
    N = qw.shape[0]
    mt = M - m0 if mt is None else mt
    nt = N - n0 if nt is None else nt
    out = np.empty((mt, nt, K // BLOCK), np.int32)
    _check(lib().oracle_kblock_partials(_ptr(qx), _ptr(qw), M, N, K, m0, mt, n0, nt, _ptr(out)),
           "kblock_partials")
    return out


def linear_int8(qx, sx, qw, sw, bias=None, rows=None, want_f64=False):
    """Dequantized bf16 output for the given rows (all rows if None)."""
    qx = _c(qx, np.int8)
    qw = _c(qw, np.int8)
    sx = _c(sx, np.float32)
    sw = _c(sw, np.float32)
    b = None if bias is None else _c(bias, np.uint16)
    M, K = qx.shape
    N = qw.shape[0]
    r = None if rows is None else _c(rows, np.int64)
    nr = M if r is None else r.shape[0]
    y = np.empty((nr, N), np.uint16)
    y64 = np.empty((nr, N), np.float64) if want_f64 else None
    _check(lib().oracle_linear_int8_rows(_ptr(qx), _ptr(sx), _ptr(qw), _ptr(sw), _ptr(b), M, N, K,
                                         _ptr(r), nr, _ptr(y), _ptr(y64)), "linear_int8")
    return (y, y64) if want_f64 else y


def linear_bf16(x, x_dtype, w_bf16, bias=None, rows=None):
    """bf16 fallback linear; x is uint16 bits (bf16/fp16) or float32."""
    xd = {DTYPE_BF16: np.uint16, DTYPE_FP16: np.uint16, DTYPE_FP32: np.float32}[x_dtype]
    x = _c(x, xd)
    w = _c(w_bf16, np.uint16)
    b = None if bias is None else _c(bias, np.uint16)
    M, K = x.shape
    N = w.shape[0]
    r = None if rows is None else _c(rows, np.int64)
    nr = M if r is None else r.shape[0]
    y = np.empty((nr, N), np.uint16)
    _check(lib().oracle_linear_bf16_rows(_ptr(x), x_dtype, _ptr(w), _ptr(b), M, N, K, _ptr(r), nr,
                                         _ptr(y)), "linear_bf16")
    return y


def route(x_dtype, M, K, N, has_qweight):
    return lib().oracle_route(x_dtype, M, K, N, int(bool(has_qweight)))


def f64_to_bf16(v: float) -> int:
    return int(lib().oracle_f64_to_bf16(float(v)))


def fp16_to_f64(h: int) -> float:
    return float(lib().oracle_fp16_to_f64(int(h)))


def gelu_bf16(x_bf16):
    x = _c(x_bf16, np.uint16)
    y = np.empty_like(x)
    _check(lib().oracle_gelu_bf16(_ptr(x), x.size, _ptr(y)), "gelu_bf16")
    return y


def quantize_qk(x_bf16: np.ndarray, B: int, L: int, H: int, D: int, ld: int):
    """Attention Q or K: x holds B*L rows of ``ld`` bf16 values, element
    (b, l, h, d) at row b*L + l, column h*D + d -> (q int8 [B, H, L, D],
    s fp32 [B, H, ceil(L/128)])."""
    x = _c(x_bf16, np.uint16)
    if x.size != B * L * ld:
        raise ValueError("x must hold B*L rows of ld values")
    nblk = -(-L // 128)
    q = np.empty((B, H, L, D), np.int8)
    s = np.empty((B, H, nblk), np.float32)
    _check(lib().oracle_quantize_qk(_ptr(x), B, L, H, D, ld, _ptr(q), _ptr(s)), "quantize_qk")
    return q, s


def gelu_quantize_block(y_bf16: np.ndarray):
    """The fused producer's result: GELU rounded to bf16, then the 128x128
    block quantization of that bf16 matrix -> (q int8, s fp32)."""
    return quantize_block(gelu_bf16(y_bf16))


def quantize_rows(x_bf16: np.ndarray):
    """Row-wise INT8 quantization with the 1e-4 floor -> (q int8 [R,C], s fp32 [R])."""
    x = _c(x_bf16, np.uint16)
    r, c = x.shape
    q = np.empty((r, c), np.int8)
    s = np.empty((r,), np.float32)
    _check(lib().oracle_quantize_rows(_ptr(x), r, c, _ptr(q), _ptr(s)), "quantize_rows")
    return q, s


def linear_postscale(qx, sx, qw, sw, bias=None, rows=None):
    """Post-scale output: exact integer sum over K, scales and bias once."""
    qx = _c(qx, np.int8)
    qw = _c(qw, np.int8)
    sx = _c(sx, np.float32)
    sw = _c(sw, np.float32)
    b = None if bias is None else _c(bias, np.uint16)
    M, K = qx.shape
    N = qw.shape[0]
    r = None if rows is None else _c(rows, np.int64)
    nr = M if r is None else r.shape[0]
    y = np.empty((nr, N), np.uint16)
    _check(lib().oracle_linear_postscale_rows(_ptr(qx), _ptr(sx), _ptr(qw), _ptr(sw), _ptr(b), M, N, K,
                                              _ptr(r), nr, _ptr(y)), "linear_postscale")
    return y


def rmsnorm_modulate(x_bf16: np.ndarray, L: int, scale_bf16: np.ndarray, shift_bf16: np.ndarray,
                     eps: float = 1e-6, want_r: bool = False):
    """Modulated RMS normalization of x [B*L, K] (bf16 bits) with per-batch
    scale and shift [B, K] -> y bf16 bits [B*L, K] (and r fp32 [B*L])."""
    x = _c(x_bf16, np.uint16)
    sc = _c(scale_bf16, np.uint16)
    sh = _c(shift_bf16, np.uint16)
    R, K = x.shape
    if R % L:
        raise ValueError("rows must be a multiple of L")
    B = R // L
    if sc.shape != (B, K) or sh.shape != (B, K):
        raise ValueError("scale and shift must be [B, K]")
    y = np.empty((R, K), np.uint16)
    r = np.empty((R,), np.float32)
    _check(lib().oracle_rmsnorm_modulate(_ptr(x), B, L, K, _ptr(sc), _ptr(sh), float(eps), _ptr(y), _ptr(r)),
           "rmsnorm_modulate")
    return (y, r) if want_r else y


def rmsnorm_modulate_quantize_block(x_bf16, L, scale_bf16, shift_bf16, eps=1e-6):
    """The fused producer's result: the modulated RMS normalization rounded to
    bf16, then the 128x128 block quantization of that matrix -> (q, s)."""
    return quantize_block(rmsnorm_modulate(x_bf16, L, scale_bf16, shift_bf16, eps))


def layernorm_modulate(x_bf16: np.ndarray, L: int, scale_bf16: np.ndarray, shift_bf16: np.ndarray,
                       eps: float = 1e-6, want_stats: bool = False):
    """Modulated layer normalization of x [B*L, K] (bf16 bits) with per-batch
    scale and shift [B, K] -> y bf16 bits [B*L, K] (and fp32 (mean, r) [B*L, 2])."""
    x = _c(x_bf16, np.uint16)
    sc = _c(scale_bf16, np.uint16)
    sh = _c(shift_bf16, np.uint16)
    R, K = x.shape
    if R % L:
        raise ValueError("rows must be a multiple of L")
    B = R // L
    if sc.shape != (B, K) or sh.shape != (B, K):
        raise ValueError("scale and shift must be [B, K]")
    y = np.empty((R, K), np.uint16)
    st = np.empty((R, 2), np.float32)
    _check(lib().oracle_layernorm_modulate(_ptr(x), B, L, K, _ptr(sc), _ptr(sh), float(eps), _ptr(y), _ptr(st)),
           "layernorm_modulate")
    return (y, st) if want_stats else y


def layernorm_modulate_quantize_block(x_bf16, L, scale_bf16, shift_bf16, eps=1e-6):
    """The fused producer's result: the modulated layer normalization rounded
    to bf16, then the 128x128 block quantization of that matrix -> (q, s)."""
    return quantize_block(layernorm_modulate(x_bf16, L, scale_bf16, shift_bf16, eps))


def rope(x_bf16: np.ndarray, B: int, L: int, H: int, D: int, ld: int, cos_t: np.ndarray, sin_t: np.ndarray):
    """Split-halves rotary embedding of sequence-major Q or K (rows of ``ld``
    bf16, element (b, l, h, d) at row b*L + l, column h*D + d) with fp32
    tables [L, D/2] -> bf16 [B*L, H*D] (contiguous, sequence-major)."""
    x = _c(x_bf16, np.uint16)
    c = _c(cos_t, np.float32)
    s = _c(sin_t, np.float32)
    if x.size != B * L * ld or c.shape != (L, D // 2) or s.shape != (L, D // 2):
        raise ValueError("shapes: x [B*L, ld], tables [L, D/2]")
    y = np.empty((B * L, H * D), np.uint16)
    _check(lib().oracle_rope(_ptr(x), B, L, H, D, ld, _ptr(c), _ptr(s), _ptr(y)), "rope")
    return y


def rope_quantize_qk(x_bf16, B, L, H, D, ld, cos_t, sin_t):
    """The fused Q/K producer's result: the rotary embedding rounded to bf16,
    then quantize_qk of that (contiguous) result -> (q [B, H, L, D], s)."""
    return quantize_qk(rope(x_bf16, B, L, H, D, ld, cos_t, sin_t), B, L, H, D, H * D)


def gated_residual(h_bf16: np.ndarray, o_bf16: np.ndarray, gate_bf16: np.ndarray, L: int):
    """y = bf16(h + gate[i // L] * o) for rows i of h and o [B*L, N]; gate [B, N]."""
    h = _c(h_bf16, np.uint16)
    o = _c(o_bf16, np.uint16)
    g = _c(gate_bf16, np.uint16)
    R, N = h.shape
    if o.shape != (R, N) or R % L or g.shape != (R // L, N):
        raise ValueError("shapes: h, o [B*L, N], gate [B, N]")
    y = np.empty((R, N), np.uint16)
    _check(lib().oracle_gated_residual(_ptr(h), _ptr(o), _ptr(g), R // L, L, N, _ptr(y)), "gated_residual")
    return y


def f32_to_e4m3(v: float) -> int:
    """One finite float -> its FP8 E4M3 code (nearest, ties to even; beyond 448: NaN)."""
    return int(lib().oracle_f32_to_e4m3(float(v)))


def e4m3_to_f64(code: int) -> float:
    return float(lib().oracle_e4m3_to_f64(int(code)))


def quantize_v_fp8(x_bf16: np.ndarray, B: int, L: int, H: int, D: int, ld: int):
    """Attention V in FP8: rows b*L + l of width ld, head h at columns h*D ..;
    per (b, h) and 128-token block s = fl32(max|x| / 448), codes E4M3(fl32(x / s))
    -> (q uint8 [B, H, L, D], s fp32 [B, H, ceil(L/128)])."""
    x = _c(x_bf16, np.uint16)
    if x.size != B * L * ld:
        raise ValueError("x must hold B*L rows of ld values")
    nblk = -(-L // 128)
    q = np.empty((B, H, L, D), np.uint8)
    s = np.empty((B, H, nblk), np.float32)
    _check(lib().oracle_quantize_v_fp8(_ptr(x), B, L, H, D, ld, _ptr(q), _ptr(s)), "quantize_v_fp8")
    return q, s
