"""Guarded W8A8 block-quantized INT8 linear for AMD MI355X (gfx950).

Thin torch-facing wrappers over the C ABI of libw8a8.so (include/w8a8.h).
torch provides device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  Function names follow the
C entry points:

* ``quantize_weight(w)``   -> (qw int8 [N,K], sw fp32 [N/128, K/128])  (static)
* ``quantize_act(x)``      -> (qx int8 [M,K], sx fp32 [M/128, K/128])  (dynamic)
* ``gemm_blockscale(qx, sx, qw, sw, bias)`` -> Y bf16 [M, N]
* ``linear(x, w, qw, sw, bias)``            -> (Y bf16 [..., N], path)  guarded
* ``route(dtype, M, K, N, has_qweight)``    -> path (host only)
* ``debug_kblock_partials(qx, qw, m0, mt, n0, nt)`` -> int32 [mt, nt, K/128]
* ``W8A8Linear``: a linear layer that quantizes its weight once at
  construction and keeps the bf16 copy for the fallback.

Post-scale form (per-row / per-output-channel scales, scales applied once):
``quantize_rows``, ``gemm_postscale``, ``linear_postscale`` and
``W8A8Linear(..., scaling="postscale")``.

Producer fused with the quantization: ``gelu_bf16(x)`` (exact GELU, bf16 in
and out), ``gelu_quantize_act(y)`` (block quantization of bf16(GELU(y))
without writing it) and ``W8A8Linear.forward_gelu(y)`` = layer(GELU(y));
likewise ``rmsnorm_modulate_*`` / ``layernorm_modulate_*`` and
``W8A8Linear.forward_modulated(x, scale, shift, norm=...)``.

Projections sharing one input (Q/K/V, or cross-attention K/V):
``W8A8ProjectionGroup`` runs them as one guarded linear over the
concatenated output channels and returns one view per projection;
``quantize_qk(x, heads)`` turns such a Q or K view (sequence-major) into
head-major INT8 codes with one scale per 128 tokens of each head;
``rope_bf16(x, heads, cos, sin)`` applies the split-halves rotary embedding
and ``rope_quantize_qk(x, heads, cos, sin)`` fuses it into that quantizer;
``quantize_v_fp8(x, heads)`` gives V the same treatment in FP8 E4M3.

Consumer fused with the GEMM: ``gated_residual(h, o, gate)`` (h + gate * o),
``gemm_blockscale_gated_residual`` (the update in the block GEMM's epilogue)
and ``W8A8Linear.forward_gated_residual(x, h, gate)``.
"""
from __future__ import annotations

import ctypes
import os

import torch

from ._lib import (BLOCK, BLOCK_MAX_K, DTYPE_BF16, DTYPE_FP16, DTYPE_FP32, EXPORTS, PATH_BF16, PATH_INT8,
                   POSTSCALE_MAX_K, W8A8Error, check, lib)

__all__ = ["quantize_weight", "quantize_act", "gemm_blockscale", "linear", "route",
           "workspace_bytes", "debug_kblock_partials", "W8A8Linear", "W8A8ProjectionGroup",
           "W8A8Error", "lib",
           "quantize_rows", "gemm_postscale", "linear_postscale", "postscale_workspace_bytes",
           "POSTSCALE_MAX_K", "gelu_bf16", "gelu_quantize_act", "quantize_qk",
           "rmsnorm_modulate_bf16", "rmsnorm_modulate_quantize_act", "rmsnorm_quantize_workspace_bytes",
           "layernorm_modulate_bf16",
           "layernorm_modulate_quantize_act", "rope_bf16", "rope_quantize_qk", "quantize_v_fp8",
           "gated_residual", "gemm_blockscale_gated_residual", "linear_gelu", "linear_modulated",
           "producer_workspace_bytes", "force_fallback",
           "PATH_INT8", "PATH_BF16", "DTYPE_BF16", "DTYPE_FP16", "DTYPE_FP32", "BLOCK", "EXPORTS"]

_DTYPES = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_FP16, torch.float32: DTYPE_FP32}


def force_fallback() -> bool:
    """True when the environment sets W8A8_FORCE_FALLBACK=1 (a test switch):
    the guarded entry points are then called without the quantized weight,
    so the library's router sends every call to the bf16 fallback."""
    return os.environ.get("W8A8_FORCE_FALLBACK", "") == "1"


def _need_cuda(name, t, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def route(dtype, M: int, K: int, N: int, has_qweight: bool) -> int:
    """The guard (host only). ``dtype`` is a torch dtype or a DTYPE_* code."""
    code = _DTYPES.get(dtype, dtype) if isinstance(dtype, torch.dtype) else dtype
    if isinstance(dtype, torch.dtype) and dtype not in _DTYPES:
        code = 99
    return lib().w8a8_route(int(code), int(M), int(K), int(N), int(bool(has_qweight)))


def workspace_bytes(M: int, K: int) -> int:
    return int(lib().w8a8_linear_workspace_bytes(int(M), int(K)))


def _quantize(fn, name, x, q, s):
    _need_cuda(name, x, torch.bfloat16)
    if x.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    R, C = x.shape
    sshape = (max(R // BLOCK, 1), max(C // BLOCK, 1))
    if q is None:
        q = torch.empty((R, C), dtype=torch.int8, device=x.device)
    if s is None:
        s = torch.empty(sshape, dtype=torch.float32, device=x.device)
    _need_cuda("q", q, torch.int8)
    _need_cuda("s", s, torch.float32)
    if q.numel() != R * C or s.numel() != sshape[0] * sshape[1]:
        raise ValueError("output buffers have the wrong size")
    check(fn.__name__, fn(_ptr(x), R, C, _ptr(q), _ptr(s), _stream(x.device)))
    return q, s


def quantize_weight(w: torch.Tensor, q=None, s=None):
    """Static 128x128 block INT8 quantization of a bf16 weight [N, K]."""
    return _quantize(lib().w8a8_quantize_weight, "w", w, q, s)


def quantize_act(x: torch.Tensor, q=None, s=None):
    """Dynamic 128x128 block INT8 quantization of bf16 activations [M, K]
    (into ``q``/``s`` when given)."""
    return _quantize(lib().w8a8_quantize_act, "x", x, q, s)


def gelu_bf16(x: torch.Tensor, out=None):
    """Exact GELU, x * Phi(x), of a bf16 tensor of any shape, rounded once
    to bf16 (``out`` may be ``x`` itself)."""
    _need_cuda("x", x, torch.bfloat16)
    if out is None:
        out = torch.empty_like(x)
    _need_cuda("out", out, torch.bfloat16)
    if out.numel() != x.numel():
        raise ValueError("out must have as many elements as x")
    check("w8a8_gelu_bf16", lib().w8a8_gelu_bf16(_ptr(x), x.numel(), _ptr(out), _stream(x.device)))
    return out


def gelu_quantize_act(y: torch.Tensor, q=None, s=None):
    """Block quantization of bf16(GELU(y)) for bf16 y [M, K], fused: the
    GELU result is never written -> (q int8 [M, K], s fp32 [M/128, K/128])."""
    return _quantize(lib().w8a8_gelu_quantize_act, "y", y, q, s)


def _modulation_args(x, scale, shift):
    """x bf16 [B, L, K] (or [L, K] with B = 1), scale and shift bf16 [B, K]."""
    _need_cuda("x", x, torch.bfloat16)
    x3 = x.unsqueeze(0) if x.dim() == 2 else x
    if x3.dim() != 3:
        raise ValueError("x must be [B, L, K] or [L, K]")
    B, L, K = x3.shape
    for name, t in (("scale", scale), ("shift", shift)):
        _need_cuda(name, t, torch.bfloat16)
        if t.numel() != B * K:
            raise ValueError(f"{name} must hold B*K = {B * K} values ([B, K])")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not x3.is_contiguous():
        x3 = x3.contiguous()
    return x3, B, L, K


def rmsnorm_modulate_bf16(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor, eps: float = 1e-6,
                          out=None):
    """Modulated RMS normalization of bf16 x [B, L, K] with per-batch scale and
    shift [B, K]: bf16(x * r * (1 + scale) + shift), r = 1/sqrt(mean(x^2) + eps)."""
    x3, B, L, K = _modulation_args(x, scale, shift)
    if out is None:
        out = torch.empty_like(x)
    _need_cuda("out", out, torch.bfloat16)
    if out.numel() != x3.numel() or not out.is_contiguous():
        raise ValueError("out must be contiguous with as many elements as x")
    r = torch.empty(B * L, dtype=torch.float32, device=x.device)   # the entry point's workspace
    check("w8a8_rmsnorm_modulate_bf16",
          lib().w8a8_rmsnorm_modulate_bf16(_ptr(x3), B, L, K, _ptr(scale), _ptr(shift), float(eps), _ptr(r),
                                           _ptr(out), _stream(x.device)))
    return out


def rmsnorm_quantize_workspace_bytes(M: int, K: int) -> int:
    return int(lib().w8a8_rmsnorm_quantize_workspace_bytes(M, K))


def rmsnorm_modulate_quantize_act(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor, eps: float = 1e-6,
                                  q=None, s=None, workspace=None):
    """Block quantization of the modulated RMS normalization of x [B, L, K],
    fused (the bf16 result is never written) -> (q int8 [B*L, K],
    s fp32 [B*L/128, K/128]).  `workspace` (uint8, device, optional) is the
    entry point's scratch memory, allocated here when not given."""
    x3, B, L, K = _modulation_args(x, scale, shift)
    M = B * L
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if s is None:
        s = torch.empty((max(M // BLOCK, 1), max(K // BLOCK, 1)), dtype=torch.float32, device=x.device)
    _need_cuda("q", q, torch.int8)
    _need_cuda("s", s, torch.float32)
    if q.numel() != M * K or s.numel() < (M // BLOCK) * (K // BLOCK):
        raise ValueError("output buffers have the wrong size")
    need = rmsnorm_quantize_workspace_bytes(M, K)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _need_cuda("workspace", workspace, torch.uint8)
    check("w8a8_rmsnorm_modulate_quantize_act",
          lib().w8a8_rmsnorm_modulate_quantize_act(_ptr(x3), B, L, K, _ptr(scale), _ptr(shift), float(eps),
                                                   _ptr(workspace), workspace.numel(), _ptr(q), _ptr(s),
                                                   _stream(x.device)))
    return q, s


def layernorm_modulate_bf16(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor, eps: float = 1e-6,
                            out=None):
    """Modulated layer normalization of bf16 x [B, L, K] with per-batch scale
    and shift [B, K]: bf16((x - mean) * r * (1 + scale) + shift),
    r = 1/sqrt(var + eps), no affine weight."""
    x3, B, L, K = _modulation_args(x, scale, shift)
    if out is None:
        out = torch.empty_like(x)
    _need_cuda("out", out, torch.bfloat16)
    if out.numel() != x3.numel() or not out.is_contiguous():
        raise ValueError("out must be contiguous with as many elements as x")
    st = torch.empty(2 * B * L, dtype=torch.float32, device=x.device)  # the entry point's workspace
    check("w8a8_layernorm_modulate_bf16",
          lib().w8a8_layernorm_modulate_bf16(_ptr(x3), B, L, K, _ptr(scale), _ptr(shift), float(eps), _ptr(st),
                                             _ptr(out), _stream(x.device)))
    return out


def layernorm_modulate_quantize_act(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor, eps: float = 1e-6,
                                    q=None, s=None):
    """Block quantization of the modulated layer normalization of x
    [B, L, K], fused (the bf16 result is never written) -> (q int8 [B*L, K],
    s fp32 [B*L/128, K/128])."""
    x3, B, L, K = _modulation_args(x, scale, shift)
    M = B * L
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if s is None:
        s = torch.empty((max(M // BLOCK, 1), max(K // BLOCK, 1)), dtype=torch.float32, device=x.device)
    _need_cuda("q", q, torch.int8)
    _need_cuda("s", s, torch.float32)
    if q.numel() != M * K or s.numel() < (M // BLOCK) * (K // BLOCK):
        raise ValueError("output buffers have the wrong size")
    st = torch.empty(2 * M, dtype=torch.float32, device=x.device)     # the entry point's workspace
    check("w8a8_layernorm_modulate_quantize_act",
          lib().w8a8_layernorm_modulate_quantize_act(_ptr(x3), B, L, K, _ptr(scale), _ptr(shift), float(eps),
                                                     _ptr(st), _ptr(q), _ptr(s), _stream(x.device)))
    return q, s


def _qk_view(x, heads):
    if not isinstance(x, torch.Tensor) or not x.is_cuda or x.dtype != torch.bfloat16:
        raise ValueError("x must be a bf16 CUDA (HIP) tensor")
    x3 = x.unsqueeze(0) if x.dim() == 2 else x
    if x3.dim() != 3:
        raise ValueError("x must be [B, L, H*D] or [L, H*D]")
    B, L, HD = x3.shape
    if HD % heads:
        raise ValueError("the last dimension must be heads * D")
    D, ld = HD // heads, x3.stride(1)
    if x3.stride(2) != 1 or (B > 1 and x3.stride(0) != L * ld):
        raise ValueError("rows of x must be evenly strided with unit-stride columns")
    return x3, B, L, D, ld


def _rope_tables(cos, sin, L, D):
    for name, t in (("cos", cos), ("sin", sin)):
        _need_cuda(name, t, torch.float32)
        if tuple(t.shape) != (L, D // 2) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous fp32 [L, D/2] table")


def rope_bf16(x: torch.Tensor, heads: int, cos: torch.Tensor, sin: torch.Tensor, out=None):
    """Split-halves rotary embedding of Q or K: ``x`` bf16 [B, L, H*D] or
    [L, H*D] as for ``quantize_qk``, ``cos``/``sin`` fp32 [L, D/2] -> bf16
    of x's shape (contiguous)."""
    x3, B, L, D, ld = _qk_view(x, heads)
    _rope_tables(cos, sin, L, D)
    if out is None:
        out = torch.empty((B, L, heads * D), dtype=torch.bfloat16, device=x.device)
    _need_cuda("out", out, torch.bfloat16)
    if out.numel() != B * L * heads * D or not out.is_contiguous():
        raise ValueError("out must be contiguous with B*L*H*D elements")
    check("w8a8_rope_bf16", lib().w8a8_rope_bf16(_ptr(x3), B, L, heads, D, ld, _ptr(cos), _ptr(sin), _ptr(out),
                                                 _stream(x.device)))
    return out.view(x.shape) if x.dim() == 2 else out.view(B, L, heads * D)


def rope_quantize_qk(x: torch.Tensor, heads: int, cos: torch.Tensor, sin: torch.Tensor, q=None, s=None):
    """``quantize_qk(rope_bf16(x, heads, cos, sin), heads)`` in one pass: the
    rotated bf16 values are quantized without being written."""
    x3, B, L, D, ld = _qk_view(x, heads)
    _rope_tables(cos, sin, L, D)
    nblk = -(-L // BLOCK)
    if q is None:
        q = torch.empty((B, heads, L, D), dtype=torch.int8, device=x.device)
    if s is None:
        s = torch.empty((B, heads, nblk), dtype=torch.float32, device=x.device)
    _need_cuda("q", q, torch.int8)
    _need_cuda("s", s, torch.float32)
    if q.numel() != B * heads * L * D or s.numel() != B * heads * nblk:
        raise ValueError("output buffers have the wrong size")
    check("w8a8_rope_quantize_qk", lib().w8a8_rope_quantize_qk(_ptr(x3), B, L, heads, D, ld, _ptr(cos), _ptr(sin),
                                                               _ptr(q), _ptr(s), _stream(x.device)))
    return (q, s) if x.dim() == 3 else (q[0], s[0])


def quantize_qk(x: torch.Tensor, heads: int, q=None, s=None):
    """INT8 attention Q or K: ``x`` is bf16 [B, L, H*D] or [L, H*D],
    sequence-major, with unit stride in the last dimension (a column slice
    of a wider row is fine) -> (q int8 [B, H, L, D], s fp32 [B, H, ceil(L/128)]),
    one scale per block of 128 tokens of each head (H = ``heads``)."""
    x3, B, L, D, ld = _qk_view(x, heads)
    nblk = -(-L // BLOCK)
    if q is None:
        q = torch.empty((B, heads, L, D), dtype=torch.int8, device=x.device)
    if s is None:
        s = torch.empty((B, heads, nblk), dtype=torch.float32, device=x.device)
    _need_cuda("q", q, torch.int8)
    _need_cuda("s", s, torch.float32)
    if q.numel() != B * heads * L * D or s.numel() != B * heads * nblk:
        raise ValueError("output buffers have the wrong size")
    check("w8a8_quantize_qk", lib().w8a8_quantize_qk(_ptr(x3), B, L, heads, D, ld, _ptr(q), _ptr(s),
                                                     _stream(x.device)))
    return (q, s) if x.dim() == 3 else (q[0], s[0])


def _residual_args(h, gate, M, N):
    _need_cuda("h", h, torch.bfloat16)
    _need_cuda("gate", gate, torch.bfloat16)
    if h.numel() != M * N or not h.is_contiguous():
        raise ValueError("h must be contiguous with the output's M x N elements")
    if gate.dim() != 2 or gate.shape[1] != N or not gate.is_contiguous() or M % gate.shape[0]:
        raise ValueError("gate must be a contiguous [B, N] tensor with B dividing the rows")
    return M // gate.shape[0]


def gated_residual(h: torch.Tensor, o: torch.Tensor, gate: torch.Tensor, out=None):
    """Gated residual update y = bf16(h + gate[b] * o): h and o bf16
    [..., N] with B*L rows, gate bf16 [B, N] (row i takes gate row i // L).
    ``out`` may be ``h`` or ``o`` (in place)."""
    _need_cuda("o", o, torch.bfloat16)
    N = o.shape[-1]
    M = o.numel() // N
    if not o.is_contiguous():
        raise ValueError("o must be contiguous")
    L = _residual_args(h, gate, M, N)
    if out is None:
        out = torch.empty_like(o)
    _need_cuda("out", out, torch.bfloat16)
    if out.numel() != M * N:
        raise ValueError("out must have as many elements as o")
    check("w8a8_gated_residual", lib().w8a8_gated_residual(_ptr(h), _ptr(o), _ptr(gate), M // L, L, N, _ptr(out),
                                                           _stream(o.device)))
    return out


def gemm_blockscale_gated_residual(qx, sx, qw, sw, h, gate, bias=None, out=None):
    """``gated_residual(h, gemm_blockscale(qx, sx, qw, sw, bias), gate)`` with
    the update in the GEMM's epilogue; ``out`` may be ``h`` (in place)."""
    M, N, K, out = _gemm_operands(qx, sx, qw, sw, bias, out, True)
    L = _residual_args(h, gate, M, N)
    check("w8a8_gemm_blockscale_gated_residual",
          lib().w8a8_gemm_blockscale_gated_residual(_ptr(qx), _ptr(sx), _ptr(qw), _ptr(sw), _ptr(bias), M, N, K,
                                                    _ptr(h), _ptr(gate), L, _ptr(out), _stream(qx.device)))
    return out


def _gemm_operands(qx, sx, qw, sw, bias, out, block_scales: bool):
    """Check the quantized operands, bias and output of a GEMM call (sizes
    included, so that no kernel can be pointed past a buffer) -> (M, N, K, out)."""
    _need_cuda("qx", qx, torch.int8)
    _need_cuda("qw", qw, torch.int8)
    _need_cuda("sx", sx, torch.float32)
    _need_cuda("sw", sw, torch.float32)
    if qx.dim() != 2 or qw.dim() != 2:
        raise ValueError("qx and qw must be 2-D")
    M, K = qx.shape
    N = qw.shape[0]
    if qw.shape[1] != K:
        raise ValueError("qx and qw disagree on K")
    want_sx, want_sw = ((-(-M // BLOCK)) * (-(-K // BLOCK)), (-(-N // BLOCK)) * (-(-K // BLOCK))) if block_scales \
        else (M, N)
    if sx.numel() != want_sx or sw.numel() != want_sw:
        raise ValueError("scale grids do not match the operands")
    if bias is not None:
        _need_cuda("bias", bias, torch.bfloat16)
        if bias.numel() != N:
            raise ValueError("bias must have N elements")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=qx.device)
    _need_cuda("out", out, torch.bfloat16)
    if out.numel() != M * N:
        raise ValueError("out must have M x N elements")
    return M, N, K, out


def quantize_v_fp8(x: torch.Tensor, heads: int, q=None, s=None):
    """Attention V in FP8 E4M3: ``x`` as for ``quantize_qk`` -> (q uint8
    [B, H, L, D] holding E4M3 bit patterns, s fp32 [B, H, ceil(L/128)]),
    one scale (max-abs / 448) per block of 128 tokens of each head."""
    x3, B, L, D, ld = _qk_view(x, heads)
    nblk = -(-L // BLOCK)
    if q is None:
        q = torch.empty((B, heads, L, D), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((B, heads, nblk), dtype=torch.float32, device=x.device)
    _need_cuda("q", q, torch.uint8)
    _need_cuda("s", s, torch.float32)
    if q.numel() != B * heads * L * D or s.numel() != B * heads * nblk:
        raise ValueError("output buffers have the wrong size")
    check("w8a8_quantize_v_fp8", lib().w8a8_quantize_v_fp8(_ptr(x3), B, L, heads, D, ld, _ptr(q), _ptr(s),
                                                           _stream(x.device)))
    return (q, s) if x.dim() == 3 else (q[0], s[0])


def gemm_blockscale(qx, sx, qw, sw, bias=None, out=None):
    """INT8 GEMM with per-K-block dequantization -> bf16 [M, N]."""
    M, N, K, out = _gemm_operands(qx, sx, qw, sw, bias, out, True)
    check("w8a8_gemm_blockscale",
          lib().w8a8_gemm_blockscale(_ptr(qx), _ptr(sx), _ptr(qw), _ptr(sw), _ptr(bias), M, N, K,
                                     _ptr(out), _stream(qx.device)))
    return out


def _guarded(fn_name, ws_bytes, x, w, qw, sw, bias, out, workspace):
    if not isinstance(x, torch.Tensor) or x.dtype not in _DTYPES:
        raise ValueError("x must be a bf16, fp16 or fp32 tensor")
    _need_cuda("w", w, torch.bfloat16)
    N, K = w.shape
    if x.shape[-1] != K:
        raise ValueError("x and w disagree on K")
    lead = x.shape[:-1]
    x2 = x.reshape(-1, K)
    if not x2.is_contiguous():
        x2 = x2.contiguous()
    _need_cuda("x", x2)
    M = x2.shape[0]
    if (qw is None) != (sw is None):
        raise ValueError("qw and sw go together")
    if force_fallback():
        qw = sw = None
    if qw is not None:
        _need_cuda("qw", qw, torch.int8)
        _need_cuda("sw", sw, torch.float32)
    if bias is not None:
        _need_cuda("bias", bias, torch.bfloat16)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need_cuda("out", out, torch.bfloat16)
    if out.numel() != M * N:
        raise ValueError("out must have M x N elements")
    if bias is not None and bias.numel() != N:
        raise ValueError("bias must have N elements")
    need = ws_bytes(M, K) if qw is not None else 0
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if need:
        _need_cuda("workspace", workspace)
    path = ctypes.c_int(-1)
    check(fn_name,
          getattr(lib(), fn_name)(_ptr(x2), _DTYPES[x.dtype], M, K, N, _ptr(w), _ptr(qw), _ptr(sw),
                                  _ptr(bias), _ptr(out), _ptr(workspace) if need else None,
                                  need, _stream(x.device), ctypes.byref(path)))
    return out.reshape(*lead, N), path.value


def linear(x, w, qw=None, sw=None, bias=None, out=None, workspace=None):
    """Guarded W8A8 linear: Y = x @ w.T (+ bias) in bf16; returns (Y, path).

    x may be bf16, fp16 or fp32 with any leading dims (flattened to M rows).
    The INT8 path needs bf16 x, M, K, N multiples of 128 and (qw, sw);
    everything else runs the bf16 fallback on ``w``.
    """
    return _guarded("w8a8_linear", workspace_bytes, x, w, qw, sw, bias, out, workspace)


def quantize_rows(x: torch.Tensor, q=None, s=None):
    """Row-wise INT8 quantization with the 1e-4 floor -> (q int8 [R,K], s fp32 [R])."""
    _need_cuda("x", x, torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    R, C = x.shape
    if q is None:
        q = torch.empty((R, C), dtype=torch.int8, device=x.device)
    if s is None:
        s = torch.empty((R,), dtype=torch.float32, device=x.device)
    _need_cuda("q", q, torch.int8)
    _need_cuda("s", s, torch.float32)
    if q.numel() != R * C or s.numel() != R:
        raise ValueError("output buffers have the wrong size")
    check("w8a8_quantize_rows", lib().w8a8_quantize_rows(_ptr(x), R, C, _ptr(q), _ptr(s), _stream(x.device)))
    return q, s


def gemm_postscale(qx, sx, qw, sw, bias=None, out=None):
    """Post-scale INT8 GEMM (int32 over all of K, scales once) -> bf16 [M, N]."""
    M, N, K, out = _gemm_operands(qx, sx, qw, sw, bias, out, False)
    check("w8a8_gemm_postscale",
          lib().w8a8_gemm_postscale(_ptr(qx), _ptr(sx), _ptr(qw), _ptr(sw), _ptr(bias), M, N, K,
                                    _ptr(out), _stream(qx.device)))
    return out


def postscale_workspace_bytes(M: int, K: int) -> int:
    return int(lib().w8a8_linear_postscale_workspace_bytes(int(M), int(K)))


def linear_postscale(x, w, qw=None, sw=None, bias=None, out=None, workspace=None):
    """Guarded post-scale W8A8 linear (qw, sw from ``quantize_rows``)."""
    return _guarded("w8a8_linear_postscale", postscale_workspace_bytes, x, w, qw, sw, bias, out,
                    workspace)


def debug_kblock_partials(qx, qw, m0: int, mt: int, n0: int, nt: int):
    """Exact int32 per-K-block partial sums of a 128-aligned output window."""
    _need_cuda("qx", qx, torch.int8)
    _need_cuda("qw", qw, torch.int8)
    M, K = qx.shape
    N = qw.shape[0]
    out = torch.empty((mt, nt, K // BLOCK), dtype=torch.int32, device=qx.device)
    check("w8a8_debug_kblock_partials",
          lib().w8a8_debug_kblock_partials(_ptr(qx), _ptr(qw), M, N, K, m0, mt, n0, nt, _ptr(out),
                                           _stream(qx.device)))
    return out


def producer_workspace_bytes(M: int, K: int) -> int:
    return int(lib().w8a8_linear_producer_workspace_bytes(M, K))


def _producer_common(w, qw, sw, bias, M, K, out, workspace, device):
    _need_cuda("w", w, torch.bfloat16)
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("the input and w disagree on K")
    if (qw is None) != (sw is None):
        raise ValueError("qw and sw go together")
    if force_fallback():
        qw = sw = None
    if qw is not None:
        _need_cuda("qw", qw, torch.int8)
        _need_cuda("sw", sw, torch.float32)
    if bias is not None:
        _need_cuda("bias", bias, torch.bfloat16)
        if bias.numel() != N:
            raise ValueError("bias must have N elements")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=device)
    _need_cuda("out", out, torch.bfloat16)
    if out.numel() != M * N:
        raise ValueError("out must have M x N elements")
    need = producer_workspace_bytes(M, K)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    _need_cuda("workspace", workspace)
    return N, qw, sw, out, workspace, need


def linear_gelu(u, w, qw=None, sw=None, bias=None, out=None, workspace=None):
    """Guarded ``GELU(u) @ w.T (+ bias)`` for bf16 u [..., K]: the library
    fuses the exact GELU into the INT8 path's activation quantization, or
    runs GELU then the bf16 fallback; returns (Y bf16 [..., N], path)."""
    _need_cuda("u", u, torch.bfloat16)
    K = w.shape[1]
    if u.shape[-1] != K:
        raise ValueError(f"last dimension of u must be {K}")
    u2 = u.reshape(-1, K)
    if not u2.is_contiguous():
        u2 = u2.contiguous()
    M = u2.shape[0]
    N, qw, sw, out, workspace, need = _producer_common(w, qw, sw, bias, M, K, out, workspace, u.device)
    path = ctypes.c_int(-1)
    check("w8a8_linear_gelu",
          lib().w8a8_linear_gelu(_ptr(u2), M, K, N, _ptr(w), _ptr(qw), _ptr(sw), _ptr(bias), _ptr(out),
                                 _ptr(workspace), need, _stream(u.device), ctypes.byref(path)))
    return out.reshape(*u.shape[:-1], N), path.value


def linear_modulated(x, scale, shift, w, qw=None, sw=None, bias=None, eps: float = 1e-6, norm: str = "rms",
                     out=None, workspace=None):
    """Guarded ``norm_modulate(x, scale, shift, eps) @ w.T (+ bias)`` for bf16
    x [B, L, K] (or [L, K]) with scale, shift [B, K] (``norm``: "rms" or
    "layer"): the normalization is fused into the INT8 path's activation
    quantization, or runs alone before the bf16 fallback; returns
    (Y bf16 [..., N], path)."""
    if norm not in ("rms", "layer"):
        raise ValueError("norm must be 'rms' or 'layer'")
    x3, B, L, K = _modulation_args(x, scale, shift)
    M = B * L
    N, qw, sw, out, workspace, need = _producer_common(w, qw, sw, bias, M, K, out, workspace, x.device)
    fn = "w8a8_linear_rmsnorm_modulate" if norm == "rms" else "w8a8_linear_layernorm_modulate"
    path = ctypes.c_int(-1)
    check(fn, getattr(lib(), fn)(_ptr(x3), B, L, K, _ptr(scale), _ptr(shift), float(eps), N, _ptr(w), _ptr(qw),
                                 _ptr(sw), _ptr(bias), _ptr(out), _ptr(workspace), need, _stream(x.device),
                                 ctypes.byref(path)))
    return out.view(*x.shape[:-1], N), path.value


class W8A8Linear(torch.nn.Module):
    """Linear layer on the guarded W8A8 path.

    The bf16 weight [N, K] is kept (the fallback needs it) and quantized once
    here: per 128x128 block (``scaling="block"``, the default) or per output
    channel (``scaling="postscale"``).  ``forward`` quantizes the activations
    on every call (or falls back) and returns bf16.

    The quantized activations go to a workspace cached on the layer and
    reused by every call, so calls of one layer object on several streams
    must not overlap: order them, or give each stream its own layer.
    """

    def __init__(self, weight: torch.Tensor, bias: torch.Tensor | None = None, scaling: str = "block"):
        super().__init__()
        _need_cuda("weight", weight, torch.bfloat16)
        if scaling not in ("block", "postscale"):
            raise ValueError("scaling is 'block' or 'postscale'")
        self.weight = weight
        self.bias = bias
        self.scaling = scaling
        N, K = weight.shape
        self.qweight, self.wscale = None, None
        if N % BLOCK == 0 and K % BLOCK == 0:
            if scaling == "block":
                self.qweight, self.wscale = quantize_weight(weight)
            elif K <= POSTSCALE_MAX_K:
                self.qweight, self.wscale = quantize_rows(weight)
        self._workspace = None
        self._pworkspace = None
        self.last_path = None

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        K = self.weight.shape[1]
        M = x.numel() // K if K else 0
        ws_fn = workspace_bytes if self.scaling == "block" else postscale_workspace_bytes
        need = ws_fn(M, K) if self.qweight is not None else 0
        if need and (self._workspace is None or self._workspace.numel() < need
                     or self._workspace.device != x.device):
            self._workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        fn = linear if self.scaling == "block" else linear_postscale
        y, self.last_path = fn(x, self.weight, self.qweight, self.wscale, self.bias,
                               workspace=self._workspace)
        return y

    def _producer_workspace(self, M, K, device):
        need = producer_workspace_bytes(M, K)
        if self._pworkspace is None or self._pworkspace.numel() < need or self._pworkspace.device != device:
            self._pworkspace = torch.empty(need, dtype=torch.uint8, device=device)
        return self._pworkspace

    def _block_weights(self):
        # the producer entries implement the block form only
        return (self.qweight, self.wscale) if self.scaling == "block" else (None, None)

    def forward_gelu(self, y: torch.Tensor) -> torch.Tensor:
        """``self(GELU(y))`` for a bf16 ``y`` [..., K]: the second linear of an
        MLP, one guarded library call (w8a8_linear_gelu) that fuses the
        activation into the input quantization on the INT8 path."""
        if self.scaling != "block":
            return self.forward(gelu_bf16(y))
        K = self.weight.shape[1]
        qw, sw = self._block_weights()
        out, self.last_path = linear_gelu(y, self.weight, qw, sw, self.bias,
                                          workspace=self._producer_workspace(y.numel() // K if K else 0, K,
                                                                             y.device))
        return out

    def forward_modulated(self, x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor,
                          eps: float = 1e-6, norm: str = "rms") -> torch.Tensor:
        """``self(rmsnorm_modulate_bf16(x, scale, shift, eps))`` for bf16 x
        [B, L, K] (``norm="layer"``: ``layernorm_modulate_bf16``): one guarded
        library call that fuses the normalization into the input quantization
        on the INT8 path."""
        if norm not in ("rms", "layer"):
            raise ValueError("norm must be 'rms' or 'layer'")
        if self.scaling != "block":
            alone = rmsnorm_modulate_bf16 if norm == "rms" else layernorm_modulate_bf16
            return self.forward(alone(x, scale, shift, eps))
        K = self.weight.shape[1]
        qw, sw = self._block_weights()
        ws = self._producer_workspace(x.numel() // K if K else 0, K, x.device)
        out, self.last_path = linear_modulated(x, scale, shift, self.weight, qw, sw, self.bias, eps, norm,
                                               workspace=ws)
        return out

    def forward_gated_residual(self, x: torch.Tensor, h: torch.Tensor, gate: torch.Tensor,
                               out=None) -> torch.Tensor:
        """``gated_residual(h, self(x), gate)``: h bf16 with the output's shape,
        gate bf16 [B, N]; on the INT8 block path the update runs in the GEMM's
        epilogue, so the layer's output never reaches memory.  ``out`` must
        not overlap h."""
        if self.scaling != "block":
            return gated_residual(h, self.forward(x), gate, out)
        N, K = self.weight.shape
        x2 = x.reshape(-1, K)
        if not x2.is_contiguous():
            x2 = x2.contiguous()
        if x2.dtype not in _DTYPES:
            raise ValueError("x must be a bf16, fp16 or fp32 tensor")
        _need_cuda("x", x2)
        M = x2.shape[0]
        L = _residual_args(h, gate, M, N)
        if out is None:
            out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
        _need_cuda("out", out, torch.bfloat16)
        if out.numel() != M * N:
            raise ValueError("out must have the output's M x N elements")
        qw, sw = (None, None) if force_fallback() else (self.qweight, self.wscale)
        need = workspace_bytes(M, K) if qw is not None else 0
        if need and (self._workspace is None or self._workspace.numel() < need
                     or self._workspace.device != x.device):
            self._workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        path = ctypes.c_int(-1)
        check("w8a8_linear_gated_residual",
              lib().w8a8_linear_gated_residual(_ptr(x2), _DTYPES[x2.dtype], M, K, N, _ptr(self.weight),
                                               _ptr(qw), _ptr(sw), _ptr(self.bias), _ptr(h),
                                               _ptr(gate), L, _ptr(out), _ptr(self._workspace) if need else None,
                                               need, _stream(x.device), ctypes.byref(path)))
        self.last_path = path.value
        return out.reshape(*x.shape[:-1], N)


class W8A8ProjectionGroup(torch.nn.Module):
    """Linear projections that share one input, run as a single guarded linear.

    The TurboT2VA paper (architecture-aware inference stack, guard paragraph)
    concatenates the query, key and value projections of a shared input, and
    the key and value projections of cross-attention, so that the activation
    is quantized once and one GEMM runs.  Here the weights [N_i, K] are
    concatenated along the output channels into one ``W8A8Linear``;
    ``forward(x)`` returns one bf16 view [..., N_i] per projection into the
    single output [..., sum N_i] (column slices, row stride sum N_i).

    Guard: the INT8 path additionally needs every N_i to be a multiple of
    128, so that the concatenated weight's 128x128 blocks (or its output
    channels, in the post-scale form) are exactly the projections' own and
    each view equals that projection run alone, bit for bit.  Otherwise the
    group runs the bf16 fallback on the retained concatenated bf16 weight.
    """

    def __init__(self, weights, biases=None, scaling: str = "block"):
        super().__init__()
        weights = list(weights)
        if not weights:
            raise ValueError("at least one projection")
        for i, w in enumerate(weights):
            _need_cuda(f"weights[{i}]", w, torch.bfloat16)
            if w.dim() != 2 or w.shape[1] != weights[0].shape[1]:
                raise ValueError("every weight is [N_i, K] with one common K")
        if biases is not None and len(biases) != len(weights):
            raise ValueError("one bias (or None) per projection")
        self.splits = [int(w.shape[0]) for w in weights]
        bias = None
        if biases is not None and any(b is not None for b in biases):
            bias = torch.cat([b if b is not None else torch.zeros(n, dtype=torch.bfloat16, device=w.device)
                              for b, n, w in zip(biases, self.splits, weights)])
        self.linear = W8A8Linear(torch.cat(weights, 0), bias, scaling=scaling)
        if any(n % BLOCK for n in self.splits):
            # blocks would straddle two projections: keep the bf16 path only
            self.linear.qweight, self.linear.wscale = None, None

    @property
    def last_path(self):
        return self.linear.last_path

    def forward(self, x: torch.Tensor):
        return tuple(torch.split(self.linear(x), self.splits, dim=-1))
