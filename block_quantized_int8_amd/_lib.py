"""ctypes binding of libw8a8.so (the C ABI in include/w8a8.h).

Argument marshalling only: every computation happens in the library's HIP
kernels.  Loading fails loudly when the library is not built; there is no
CPU fallback anywhere in this package.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libw8a8.so")

W8A8_OK, W8A8_ERR_INVALID_ARG, W8A8_ERR_UNSUPPORTED, W8A8_ERR_HIP = 0, 1, 2, 3
DTYPE_BF16, DTYPE_FP16, DTYPE_FP32 = 0, 1, 2
PATH_INT8, PATH_BF16 = 0, 1
BLOCK = 128

# every symbol include/w8a8.h declares
EXPORTS = (
    "w8a8_quantize_weight", "w8a8_quantize_act", "w8a8_gemm_blockscale",
    "w8a8_linear_workspace_bytes", "w8a8_linear", "w8a8_route",
    "w8a8_debug_kblock_partials", "w8a8_status_string", "w8a8_last_hip_error",
    "w8a8_quantize_rows", "w8a8_gemm_postscale", "w8a8_linear_postscale_workspace_bytes",
    "w8a8_linear_postscale", "w8a8_gelu_bf16", "w8a8_gelu_quantize_act", "w8a8_quantize_qk",
    "w8a8_rmsnorm_modulate_bf16", "w8a8_rmsnorm_modulate_quantize_act", "w8a8_rope_bf16",
    "w8a8_rope_quantize_qk", "w8a8_gated_residual", "w8a8_gemm_blockscale_gated_residual",
    "w8a8_linear_gated_residual", "w8a8_layernorm_modulate_bf16", "w8a8_layernorm_modulate_quantize_act",
    "w8a8_quantize_v_fp8", "w8a8_linear_producer_workspace_bytes", "w8a8_linear_gelu",
    "w8a8_linear_rmsnorm_modulate", "w8a8_linear_layernorm_modulate", "w8a8_linear_noalloc",
    "w8a8_rmsnorm_quantize_workspace_bytes",
)
POSTSCALE_MAX_K = 133120
BLOCK_MAX_K = 4194304
GELU_QUANT_MAX_K = 8388480
NOALLOC_SCRATCH_BYTES = 33554432 + 65536

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_lib = None


class W8A8Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        name = lib().w8a8_status_string(status).decode()
        extra = f" (hipError {lib().w8a8_last_hip_error()})" if status == W8A8_ERR_HIP else ""
        super().__init__(f"{fn} failed: {name}{extra}")
        self.status = status


def lib():
    """Load libw8a8.so (built in-tree by build.py); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() or "
                           "python block_quantized_int8_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    L.w8a8_quantize_weight.argtypes = [_P, _I64, _I64, _P, _P, _P]
    L.w8a8_quantize_act.argtypes = [_P, _I64, _I64, _P, _P, _P]
    L.w8a8_gemm_blockscale.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P]
    L.w8a8_linear_workspace_bytes.argtypes = [_I64, _I64]
    L.w8a8_linear_workspace_bytes.restype = ctypes.c_size_t
    L.w8a8_linear.argtypes = [_P, ctypes.c_int, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P,
                              ctypes.c_size_t, _P, ctypes.POINTER(ctypes.c_int)]
    L.w8a8_route.argtypes = [ctypes.c_int, _I64, _I64, _I64, ctypes.c_int]
    L.w8a8_debug_kblock_partials.argtypes = [_P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                             _P, _P]
    L.w8a8_quantize_rows.argtypes = [_P, _I64, _I64, _P, _P, _P]
    L.w8a8_gemm_postscale.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P]
    L.w8a8_linear_postscale_workspace_bytes.argtypes = [_I64, _I64]
    L.w8a8_linear_postscale_workspace_bytes.restype = ctypes.c_size_t
    L.w8a8_linear_postscale.argtypes = L.w8a8_linear.argtypes
    L.w8a8_gelu_bf16.argtypes = [_P, _I64, _P, _P]
    L.w8a8_gelu_quantize_act.argtypes = [_P, _I64, _I64, _P, _P, _P]
    L.w8a8_quantize_qk.argtypes = [_P, _I64, _I64, _I64, _I64, _I64, _P, _P, _P]
    L.w8a8_quantize_v_fp8.argtypes = [_P, _I64, _I64, _I64, _I64, _I64, _P, _P, _P]
    L.w8a8_rope_bf16.argtypes = [_P, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P]
    L.w8a8_rope_quantize_qk.argtypes = [_P, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P]
    L.w8a8_gated_residual.argtypes = [_P, _P, _P, _I64, _I64, _I64, _P, _P]
    L.w8a8_gemm_blockscale_gated_residual.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _I64, _P, _P]
    L.w8a8_linear_gated_residual.argtypes = [_P, ctypes.c_int, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _I64,
                                             _P, _P, ctypes.c_size_t, _P, ctypes.POINTER(ctypes.c_int)]
    L.w8a8_layernorm_modulate_bf16.argtypes = [_P, _I64, _I64, _I64, _P, _P, ctypes.c_double, _P, _P, _P]
    L.w8a8_layernorm_modulate_quantize_act.argtypes = [_P, _I64, _I64, _I64, _P, _P, ctypes.c_double, _P, _P,
                                                       _P, _P]
    L.w8a8_rmsnorm_modulate_bf16.argtypes = [_P, _I64, _I64, _I64, _P, _P, ctypes.c_double, _P, _P, _P]
    L.w8a8_rmsnorm_modulate_quantize_act.argtypes = [_P, _I64, _I64, _I64, _P, _P, ctypes.c_double, _P,
                                                     ctypes.c_size_t, _P, _P, _P]
    L.w8a8_rmsnorm_quantize_workspace_bytes.argtypes = [_I64, _I64]
    L.w8a8_rmsnorm_quantize_workspace_bytes.restype = ctypes.c_size_t
    L.w8a8_linear_producer_workspace_bytes.argtypes = [_I64, _I64]
    L.w8a8_linear_producer_workspace_bytes.restype = ctypes.c_size_t
    L.w8a8_linear_gelu.argtypes = [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P,
                                   ctypes.POINTER(ctypes.c_int)]
    L.w8a8_linear_rmsnorm_modulate.argtypes = [_P, _I64, _I64, _I64, _P, _P, ctypes.c_double, _I64, _P, _P, _P, _P,
                                               _P, _P, ctypes.c_size_t, _P, ctypes.POINTER(ctypes.c_int)]
    L.w8a8_linear_layernorm_modulate.argtypes = L.w8a8_linear_rmsnorm_modulate.argtypes
    L.w8a8_linear_noalloc.argtypes = [_P, ctypes.c_int, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P,
                                      ctypes.POINTER(ctypes.c_int)]
    L.w8a8_status_string.argtypes = [ctypes.c_int]
    L.w8a8_status_string.restype = ctypes.c_char_p
    L.w8a8_last_hip_error.argtypes = []
    for f in ("w8a8_quantize_weight", "w8a8_quantize_act", "w8a8_gemm_blockscale", "w8a8_linear",
              "w8a8_route", "w8a8_debug_kblock_partials", "w8a8_last_hip_error",
              "w8a8_quantize_rows", "w8a8_gemm_postscale", "w8a8_linear_postscale",
              "w8a8_gelu_bf16", "w8a8_gelu_quantize_act", "w8a8_quantize_qk", "w8a8_rope_bf16",
              "w8a8_rope_quantize_qk", "w8a8_rmsnorm_modulate_bf16", "w8a8_rmsnorm_modulate_quantize_act",
              "w8a8_gated_residual", "w8a8_gemm_blockscale_gated_residual", "w8a8_linear_gated_residual",
              "w8a8_layernorm_modulate_bf16", "w8a8_layernorm_modulate_quantize_act", "w8a8_quantize_v_fp8",
              "w8a8_linear_gelu", "w8a8_linear_rmsnorm_modulate", "w8a8_linear_layernorm_modulate",
              "w8a8_linear_noalloc"):
        getattr(L, f).restype = ctypes.c_int
    _lib = L
    return L


def check(fn: str, status: int) -> None:
    if status != W8A8_OK:
        raise W8A8Error(fn, status)
