"""Host-side checks of libw8a8.so that need no GPU.

The library loads, exports every entry point include/w8a8.h declares, its
guard matches the pages' rule on the golden table, and argument errors that
are decided before any device access come back as status codes.  No call
here reaches a kernel or a device query.
"""
import ctypes
import os
import re

import pytest

from conftest import ROOT, load_golden


@pytest.fixture(scope="module")
def L():
    from block_quantized_int8_amd import _lib
    from block_quantized_int8_amd import build as b
    if not os.path.exists(b.OUT):
        b.build()
    return _lib.lib()


def _declared():
    src = open(os.path.join(ROOT, "include", "w8a8.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(w8a8_\w+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    from block_quantized_int8_amd import _lib
    declared = _declared()
    assert len(declared) >= 9
    assert sorted(_lib.EXPORTS) == declared
    for name in declared:
        assert hasattr(L, name), name


def test_package_exports_every_wrapper():
    # every public function and class of the binding is in __all__, and
    # every name in __all__ exists
    import block_quantized_int8_amd as m
    assert all(hasattr(m, n) for n in m.__all__)
    public = [n for n, v in vars(m).items() if not n.startswith("_") and callable(v)
              and getattr(v, "__module__", "") == m.__name__]
    assert sorted(n for n in public if n not in m.__all__) == []


def test_route_golden(L):
    g = load_golden("route_cases.json")
    for dt, M, K, N, hq, want, note in g["cases"]:
        assert L.w8a8_route(dt, M, K, N, hq) == want, note


def test_route_matches_oracle_exhaustive_small(L):
    import oracle
    for dt in (0, 1, 2, 5):
        for M in (1, 127, 128, 256, 4000):
            for K in (128, 130, 4096):
                for N in (64, 128, 2048):
                    for hq in (0, 1):
                        assert L.w8a8_route(dt, M, K, N, hq) == oracle.route(dt, M, K, N, hq)


def test_status_strings(L):
    assert L.w8a8_status_string(0) == b"W8A8_OK"
    assert L.w8a8_status_string(1) == b"W8A8_ERR_INVALID_ARG"
    assert L.w8a8_status_string(2) == b"W8A8_ERR_UNSUPPORTED"
    assert L.w8a8_status_string(3) == b"W8A8_ERR_HIP"
    assert L.w8a8_status_string(42) == b"W8A8_UNKNOWN_STATUS"
    assert L.w8a8_last_hip_error() == 0


def test_workspace_bytes(L):
    assert L.w8a8_linear_workspace_bytes(256, 256) == 65536 + 256
    assert L.w8a8_linear_workspace_bytes(32768, 4096) == 32768 * 4096 + 32768 // 128 * 32 * 4
    assert L.w8a8_linear_workspace_bytes(4000, 4096) == 0
    assert L.w8a8_linear_workspace_bytes(128, 0) == 0


def test_host_decided_errors(L):
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails validation first
    null = None
    # null or non-positive arguments
    assert L.w8a8_quantize_weight(null, 128, 128, fake, fake, null) == 1
    assert L.w8a8_quantize_act(fake, 0, 128, fake, fake, null) == 1
    # strict quantizers: shapes that are not multiples of 128
    assert L.w8a8_quantize_act(fake, 130, 128, fake, fake, null) == 2
    assert L.w8a8_quantize_weight(fake, 128, 4000, fake, fake, null) == 2
    # misaligned pointer on a strict entry point
    assert L.w8a8_quantize_act(ctypes.c_void_p(0x1002), 128, 128, fake, fake, null) == 2
    assert L.w8a8_gemm_blockscale(fake, fake, fake, fake, null, 4000, 128, 128, fake, null) == 2
    assert L.w8a8_gemm_blockscale(null, fake, fake, fake, null, 128, 128, 128, fake, null) == 1
    # K beyond the block GEMM's 32-bit tile addressing
    from block_quantized_int8_amd._lib import BLOCK_MAX_K
    assert L.w8a8_gemm_blockscale(fake, fake, fake, fake, null, 128, 128, BLOCK_MAX_K + 128, fake, null) == 2
    assert L.w8a8_debug_kblock_partials(fake, fake, 128, 128, BLOCK_MAX_K + 128, 0, 128, 0, 128, fake, null) == 2
    # linear: missing weight copy, unknown dtype, half a quantized weight
    path = ctypes.c_int(-7)
    assert L.w8a8_linear(fake, 0, 128, 128, 128, null, null, null, null, fake, null, 0, null,
                         ctypes.byref(path)) == 1
    assert L.w8a8_linear(fake, 9, 128, 128, 128, fake, null, null, null, fake, null, 0, null,
                         ctypes.byref(path)) == 1
    assert L.w8a8_linear(fake, 0, 128, 128, 128, fake, fake, null, null, fake, null, 0, null,
                         ctypes.byref(path)) == 1
    assert path.value == -7  # untouched on early errors
    # partials window checks
    assert L.w8a8_debug_kblock_partials(fake, fake, 256, 256, 256, 128, 256, 0, 128, fake, null) == 1
    assert L.w8a8_debug_kblock_partials(fake, fake, 256, 256, 256, 64, 128, 0, 128, fake, null) == 2


def test_host_decided_errors_producer_and_qk(L):
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails validation first
    null = None
    # GELU: negative size; n = 0 is a no-op that accepts null pointers
    assert L.w8a8_gelu_bf16(fake, -1, fake, null) == 1
    assert L.w8a8_gelu_bf16(null, 0, null, null) == 0
    assert L.w8a8_gelu_bf16(ctypes.c_void_p(0x1001), 8, fake, null) == 2
    # fused GELU + quantize: strict like quantize_act, K bounded
    assert L.w8a8_gelu_quantize_act(fake, 100, 128, fake, fake, null) == 2
    assert L.w8a8_gelu_quantize_act(fake, 128, 8388608, fake, fake, null) == 2
    assert L.w8a8_gelu_quantize_act(null, 128, 128, fake, fake, null) == 1
    # Q/K: head dim, row stride, alignment
    assert L.w8a8_quantize_qk(fake, 1, 100, 2, 96, 192, fake, fake, null) == 2
    assert L.w8a8_quantize_qk(fake, 1, 100, 2, 64, 100, fake, fake, null) == 1
    assert L.w8a8_quantize_qk(fake, 1, 100, 2, 64, 132, fake, fake, null) == 2
    assert L.w8a8_quantize_qk(fake, 1, 0, 2, 64, 128, fake, fake, null) == 1
    assert L.w8a8_quantize_qk(ctypes.c_void_p(0x1008), 1, 100, 2, 64, 128, fake, fake, null) == 2


def test_host_decided_errors_rmsnorm(L):
    fake = ctypes.c_void_p(0x1000)  # never dereferenced
    null = None
    # eps must be finite and positive; sizes positive; K a multiple of 8
    assert L.w8a8_rmsnorm_modulate_bf16(fake, 2, 64, 256, fake, fake, 0.0, fake, fake, null) == 1
    assert L.w8a8_rmsnorm_modulate_bf16(fake, 2, 64, 256, fake, fake, float("nan"), fake, fake, null) == 1
    assert L.w8a8_rmsnorm_modulate_bf16(fake, 2, 0, 256, fake, fake, 1e-6, fake, fake, null) == 1
    assert L.w8a8_rmsnorm_modulate_bf16(fake, 2, 64, 252, fake, fake, 1e-6, fake, fake, null) == 2
    assert L.w8a8_rmsnorm_modulate_bf16(fake, 2, 64, 256, fake, fake, 1e-6, null, fake, null) == 1
    # fused: B*L and K multiples of 128, a 16-byte aligned workspace of the stated size
    big = 1 << 30
    assert L.w8a8_rmsnorm_modulate_quantize_act(fake, 2, 100, 256, fake, fake, 1e-6, fake, big, fake, fake,
                                                null) == 2
    assert L.w8a8_rmsnorm_modulate_quantize_act(fake, 2, 128, 192, fake, fake, 1e-6, fake, big, fake, fake,
                                                null) == 2
    assert L.w8a8_rmsnorm_modulate_quantize_act(ctypes.c_void_p(0x1008), 2, 128, 256, fake, fake, 1e-6, fake, big,
                                                fake, fake, null) == 2
    assert L.w8a8_rmsnorm_modulate_quantize_act(fake, 2, 128, 256, fake, fake, 1e-6, ctypes.c_void_p(0x1008), big,
                                                fake, fake, null) == 2
    need = L.w8a8_rmsnorm_quantize_workspace_bytes(256, 256)
    assert L.w8a8_rmsnorm_modulate_quantize_act(fake, 2, 128, 256, fake, fake, 1e-6, fake, need - 1, fake, fake,
                                                null) == 1
    assert L.w8a8_rmsnorm_modulate_quantize_act(fake, 2, 128, 256, fake, fake, 1e-6, null, big, fake, fake,
                                                null) == 1


def test_rmsnorm_quantize_workspace_bytes(L):
    """Single-read widths (K % 256 == 0): a 256-byte control line, one 256-byte
    counter line per 128-row band and 8 bytes per row per 256 columns; other
    widths: the control line and 4 bytes of r per row."""
    f = L.w8a8_rmsnorm_quantize_workspace_bytes
    assert f(0, 256) == 0 and f(256, 0) == 0
    assert f(32768, 4096) == 256 * (1 + 256) + 32768 * 16 * 8
    assert f(256, 256) == 256 * 3 + 256 * 8
    assert f(256, 384) == 256 + 1024
    assert f(128, 128) == 256 + 512


def test_host_decided_errors_rope(L):
    fake = ctypes.c_void_p(0x1000)  # never dereferenced
    null = None
    # head dimension 64 or 128, row stride >= H*D and a multiple of 8, 16-byte aligned tables
    assert L.w8a8_rope_bf16(fake, 1, 256, 2, 96, 192, fake, fake, fake, null) == 2
    assert L.w8a8_rope_bf16(fake, 1, 256, 2, 128, 255, fake, fake, fake, null) == 1
    assert L.w8a8_rope_bf16(fake, 1, 256, 2, 128, 260, fake, fake, fake, null) == 2
    assert L.w8a8_rope_bf16(fake, 1, 256, 2, 128, 256, ctypes.c_void_p(0x1004), fake, fake, null) == 2
    assert L.w8a8_rope_bf16(fake, 1, 256, 2, 128, 256, fake, null, fake, null) == 1
    assert L.w8a8_rope_quantize_qk(fake, 1, 0, 2, 128, 256, fake, fake, fake, fake, null) == 1
    assert L.w8a8_rope_quantize_qk(fake, 1, 256, 2, 128, 256, fake, fake, null, fake, null) == 1
    # the fused entry's row stride limit (32-bit buffer offsets)
    big = 4194304 + 8
    assert L.w8a8_rope_quantize_qk(fake, 1, 256, 2, 128, big, fake, fake, fake, fake, null) == 2
    # host memory is refused before any launch
    assert L.w8a8_rope_quantize_qk(fake, 1, 256, 2, 128, 256, fake, fake, fake, fake, null) == 1


def test_host_decided_errors_gated_residual(L):
    fake = ctypes.c_void_p(0x100000)  # never dereferenced
    far = ctypes.c_void_p(0x4000000)
    null = None
    assert L.w8a8_gated_residual(fake, fake, fake, 2, 64, 252, far, null) == 2           # N % 8
    assert L.w8a8_gated_residual(fake, fake, fake, 2, 0, 256, far, null) == 1
    assert L.w8a8_gated_residual(fake, fake, fake, 2, 64, 256, ctypes.c_void_p(0x100010), null) == 1  # overlaps h
    assert L.w8a8_gated_residual(fake, fake, fake, 2, 64, 256, far, null) == 1           # host memory
    assert L.w8a8_gemm_blockscale_gated_residual(fake, fake, fake, fake, null, 256, 256, 256, fake, fake, 3, far,
                                                 null) == 1                              # L must divide M
    assert L.w8a8_gemm_blockscale_gated_residual(fake, fake, fake, fake, null, 256, 256, 200, fake, fake, 128, far,
                                                 null) == 2
    path = ctypes.c_int(-7)
    assert L.w8a8_linear_gated_residual(fake, 0, 256, 256, 256, fake, fake, fake, null, fake, fake, 128, fake,
                                        fake, 1 << 20, null, ctypes.byref(path)) == 1   # y == h
    assert path.value == -7
