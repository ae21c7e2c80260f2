// Exercises the host side of libw8a8 (include/w8a8.h) with AddressSanitizer
// and UndefinedBehaviorSanitizer on the host code (tests/test_sanitizers.py):
// the guard over a grid, the workspace sizes, the status strings and every
// argument error that is decided before any device work.  It links the
// library's API source with stand-in launchers that abort if reached, so it
// also proves that none of these calls gets as far as a kernel launch.
#include <cstdio>
#include <cstdlib>

#include "w8a8.h"
#include "w8a8_internal.h"

[[noreturn]] static void reached(const char *what) {
    std::fprintf(stderr, "unexpected launch: %s\n", what);
    std::abort();
}

namespace w8a8 {
hipError_t launch_quantize_block(const uint16_t *, int64_t, int64_t, int8_t *, float *, hipStream_t) { reached("quantize_block"); }
hipError_t launch_gemm_i8_blockscale(const int8_t *, const float *, const int8_t *, const float *, const uint16_t *,
                                     int64_t, int64_t, int64_t, uint16_t *, hipStream_t) { reached("gemm_i8_blockscale"); }
hipError_t launch_kblock_partials(const int8_t *, const int8_t *, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                                  int64_t, int32_t *, hipStream_t) { reached("kblock_partials"); }
hipError_t launch_quantize_rows(const uint16_t *, int64_t, int64_t, int8_t *, float *, hipStream_t) { reached("quantize_rows"); }
hipError_t launch_gemm_i8_postscale(const int8_t *, const float *, const int8_t *, const float *, const uint16_t *,
                                    int64_t, int64_t, int64_t, uint16_t *, hipStream_t) { reached("gemm_i8_postscale"); }
hipError_t launch_gelu_bf16(const uint16_t *, int64_t, uint16_t *, hipStream_t) { reached("gelu_bf16"); }
hipError_t launch_gelu_quantize_block(const uint16_t *, int64_t, int64_t, int8_t *, float *, hipStream_t) { reached("gelu_quantize"); }
hipError_t launch_quantize_qk(const uint16_t *, int64_t, int64_t, int64_t, int64_t, int64_t, int8_t *, float *,
                              hipStream_t) { reached("quantize_qk"); }
hipError_t launch_rope_quantize_qk(const uint16_t *, int64_t, int64_t, int64_t, int64_t, int64_t, const float *,
                                   const float *, int8_t *, float *, hipStream_t) { reached("rope_quantize_qk"); }
hipError_t launch_rope_bf16(const uint16_t *, int64_t, int64_t, int64_t, int64_t, int64_t, const float *, const float *,
                            uint16_t *, hipStream_t) { reached("rope_bf16"); }
hipError_t launch_gemm_i8_blockscale_residual(const int8_t *, const float *, const int8_t *, const float *,
                                              const uint16_t *, int64_t, int64_t, int64_t, const uint16_t *,
                                              const uint16_t *, int64_t, uint16_t *, hipStream_t) { reached("gemm_residual"); }
hipError_t launch_gated_residual(const uint16_t *, const uint16_t *, const uint16_t *, int64_t, int64_t, int64_t,
                                 uint16_t *, hipStream_t) { reached("gated_residual"); }
hipError_t launch_gemm_bf16_tiled(const uint16_t *, const uint16_t *, const uint16_t *, int64_t, int64_t, int64_t,
                                  uint16_t *, hipStream_t) { reached("gemm_bf16_tiled"); }
hipError_t launch_gemm_bf16(const void *, int, const uint16_t *, const uint16_t *, int64_t, int64_t, int64_t, uint16_t *,
                            hipStream_t) { reached("gemm_bf16"); }
hipError_t launch_rms_rows(const uint16_t *, int64_t, int64_t, double, float *, hipStream_t) { reached("rms_rows"); }
hipError_t launch_modulate_bf16(const uint16_t *, const float *, bool, int64_t, int64_t, int64_t, const uint16_t *,
                                const uint16_t *, uint16_t *, hipStream_t) { reached("modulate_bf16"); }
hipError_t launch_modulate_quantize(const uint16_t *, const float *, bool, int64_t, int64_t, int64_t,
                                    const uint16_t *, const uint16_t *, int8_t *, float *, hipStream_t) {
    reached("modulate_quantize");
}
hipError_t launch_quantize_v_fp8(const uint16_t *, int64_t, int64_t, int64_t, int64_t, int64_t, uint8_t *, float *,
                                 hipStream_t) { reached("quantize_v_fp8"); }
hipError_t launch_ln_rows(const uint16_t *, int64_t, int64_t, double, float *, hipStream_t) { reached("ln_rows"); }
hipError_t launch_rms_band_quantize(const uint16_t *, int64_t, int64_t, int64_t, double, const uint16_t *,
                                    const uint16_t *, void *, int8_t *, float *, hipStream_t) {
    reached("rms_band_quantize");
}
bool rms_band_fits(int64_t) { reached("rms_band_fits (a device query)"); }
}  // namespace w8a8

#define CHECK(cond)                                                                    \
    do {                                                                               \
        if (!(cond)) {                                                                 \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__);     \
            return 1;                                                                  \
        }                                                                              \
    } while (0)

int main() {
    // the guard: INT8 iff bf16, M, K, N multiples of 128 and a quantized weight
    const long long dims[] = {-128, 0, 1, 127, 128, 130, 256, 4000, 4096};
    for (int dt = -1; dt <= 3; ++dt)
        for (long long m : dims)
            for (long long k : dims)
                for (long long n : dims)
                    for (int hq = 0; hq <= 1; ++hq) {
                        const int r = w8a8_route(dt, m, k, n, hq);
                        const bool bad = m <= 0 || k <= 0 || n <= 0 || dt < 0 || dt > 2;
                        const bool int8 = !bad && dt == W8A8_DTYPE_BF16 && m % 128 == 0 && k % 128 == 0 &&
                                          n % 128 == 0 && hq;
                        CHECK(r == (bad ? -1 : int8 ? W8A8_PATH_INT8 : W8A8_PATH_BF16));
                    }
    // workspace sizes: 0 when the INT8 path cannot be taken, else 256-byte rounded pieces
    CHECK(w8a8_linear_workspace_bytes(0, 128) == 0 && w8a8_linear_workspace_bytes(128, 100) == 0);
    CHECK(w8a8_linear_workspace_bytes(128, 128) == 16384 + 256);
    CHECK(w8a8_linear_postscale_workspace_bytes(256, 128) == 32768 + 1024);
    CHECK(w8a8_linear_workspace_bytes((1LL << 40), 1LL << 20) > 0);
    for (int st = -1; st <= 5; ++st) CHECK(w8a8_status_string(st) != nullptr);

    // argument errors decided on the host (fake, never dereferenced, aligned addresses)
    void *p = reinterpret_cast<void *>(0x10000);
    int8_t *q8 = static_cast<int8_t *>(p);
    float *f = static_cast<float *>(p);
    int path = -7;
    CHECK(w8a8_quantize_act(nullptr, 128, 128, q8, f, nullptr) == W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_quantize_act(p, 100, 128, q8, f, nullptr) == W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_quantize_weight(p, 128, -128, q8, f, nullptr) == W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_quantize_weight(static_cast<char *>(p) + 2, 128, 128, q8, f, nullptr) == W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_gemm_blockscale(q8, f, q8, f, nullptr, 128, 130, 128, p, nullptr) == W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_gemm_blockscale(q8, nullptr, q8, f, nullptr, 128, 128, 128, p, nullptr) == W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_gemm_blockscale(q8, f, q8, f, nullptr, 128, 128, W8A8_BLOCK_MAX_K + 128, p, nullptr) ==
          W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_debug_kblock_partials(q8, q8, 128, 128, W8A8_BLOCK_MAX_K + 128, 0, 128, 0, 128,
                                     static_cast<int32_t *>(p), nullptr) == W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_linear(p, 7, 128, 128, 128, p, q8, f, nullptr, p, p, 1 << 20, nullptr, &path) == W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_linear(p, 0, 128, 128, 128, p, q8, nullptr, nullptr, p, p, 1 << 20, nullptr, &path) ==
          W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_linear(p, 0, 0, 128, 128, p, nullptr, nullptr, nullptr, p, nullptr, 0, nullptr, &path) ==
          W8A8_ERR_INVALID_ARG);
    CHECK(path == -7);  // untouched on an argument error
    CHECK(w8a8_linear_postscale(nullptr, 0, 128, 128, 128, p, q8, f, nullptr, p, p, 0, nullptr, nullptr) ==
          W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_debug_kblock_partials(q8, q8, 256, 256, 256, 128, 256, 0, 128, static_cast<int32_t *>(p), nullptr) ==
          W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_debug_kblock_partials(q8, q8, 256, 256, 256, 64, 128, 0, 128, static_cast<int32_t *>(p), nullptr) ==
          W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_quantize_rows(p, 128, 12, q8, f, nullptr) == W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_gemm_postscale(q8, f, q8, f, nullptr, 128, 128, W8A8_POSTSCALE_MAX_K + 128, p, nullptr) ==
          W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_gelu_bf16(p, 0, p, nullptr) == W8A8_OK);
    CHECK(w8a8_gelu_bf16(p, -1, p, nullptr) == W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_gelu_bf16(static_cast<char *>(p) + 1, 8, p, nullptr) == W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_gelu_quantize_act(p, 128, W8A8_GELU_QUANT_MAX_K + 128, q8, f, nullptr) == W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_quantize_qk(p, 1, 256, 2, 96, 192, q8, f, nullptr) == W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_quantize_qk(p, 1, 256, 2, 128, 255, q8, f, nullptr) == W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_quantize_qk(p, 1LL << 40, 256, 1LL << 20, 128, 1LL << 27, q8, f, nullptr) == W8A8_ERR_UNSUPPORTED);
    // FP8 V: as for Q/K
    CHECK(w8a8_quantize_v_fp8(p, 1, 256, 2, 96, 192, reinterpret_cast<uint8_t *>(q8), f, nullptr) ==
          W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_quantize_v_fp8(p, 1, 256, 2, 128, 255, reinterpret_cast<uint8_t *>(q8), f, nullptr) ==
          W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_quantize_v_fp8(p, 1, 256, 2, 128, 256, nullptr, f, nullptr) == W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_quantize_v_fp8(p, 1, 256, 2, 128, 256, reinterpret_cast<uint8_t *>(q8), f, nullptr) ==
          W8A8_ERR_INVALID_ARG);                                                                   // host memory
    // rotary embedding: head dimension, stride, table alignment, sizes, missing outputs
    CHECK(w8a8_rope_bf16(p, 1, 256, 2, 96, 192, f, f, p, nullptr) == W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_rope_bf16(p, 1, 256, 2, 128, 255, f, f, p, nullptr) == W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_rope_bf16(p, 1, 256, 2, 128, 260, f, f, p, nullptr) == W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_rope_bf16(p, 1, 256, 2, 128, 256, f + 1, f, p, nullptr) == W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_rope_bf16(p, 1, 256, 2, 128, 256, f, nullptr, p, nullptr) == W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_rope_bf16(p, 1, 256, 2, 128, 256, f, f, nullptr, nullptr) == W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_rope_bf16(p, 1, 256, 1LL << 40, 128, 1LL << 47, f, f, p, nullptr) == W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_rope_bf16(p, 1, 256, 2, 128, 256, f, f, p, nullptr) == W8A8_ERR_INVALID_ARG);  // host memory
    CHECK(w8a8_rope_quantize_qk(p, 0, 256, 2, 128, 256, f, f, q8, f, nullptr) == W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_rope_quantize_qk(p, 1, 256, 2, 64, 128, f, f, nullptr, f, nullptr) == W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_rope_quantize_qk(p, 1, 256, 2, 128, W8A8_ROPE_MAX_LD + 8, f, f, q8, f, nullptr) == W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_rope_quantize_qk(p, 1LL << 40, 256, 1LL << 20, 128, 1LL << 27, f, f, q8, f, nullptr) ==
          W8A8_ERR_UNSUPPORTED);
    // gated residual: L dividing the rows, N a multiple of 8, partial overlap, aliasing
    char *pc = static_cast<char *>(p);
    CHECK(w8a8_gated_residual(p, p, p, 2, 64, 256, p, nullptr) == W8A8_ERR_INVALID_ARG);        // host memory
    CHECK(w8a8_gated_residual(p, p, p, 2, 0, 256, p, nullptr) == W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_gated_residual(p, p, p, 2, 64, 252, p, nullptr) == W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_gated_residual(p, p, p, 2, 64, 256, pc + 16, nullptr) == W8A8_ERR_INVALID_ARG);  // overlaps h
    CHECK(w8a8_gated_residual(p, pc + (1 << 20), pc + 8, 2, 64, 256, pc + (2 << 20), nullptr) == W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_gemm_blockscale_gated_residual(q8, f, q8, f, nullptr, 256, 256, 256, p, p, 3, p, nullptr) ==
          W8A8_ERR_INVALID_ARG);                                                                  // 3 does not divide M
    CHECK(w8a8_gemm_blockscale_gated_residual(q8, f, q8, f, nullptr, 256, 256, 200, p, p, 128, pc + (1 << 20),
                                              nullptr) == W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_gemm_blockscale_gated_residual(q8, f, q8, f, nullptr, 256, 256, 256, nullptr, p, 128, p, nullptr) ==
          W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_linear_gated_residual(p, 0, 256, 256, 256, p, q8, f, nullptr, p, p, 128, p, p, 1 << 20, nullptr,
                                     &path) == W8A8_ERR_INVALID_ARG);                             // y == h
    CHECK(w8a8_linear_gated_residual(p, 0, 256, 256, 256, p, q8, f, nullptr, p, p, 128, pc + (1 << 20), p, 1 << 20,
                                     nullptr, &path) == W8A8_ERR_INVALID_ARG);                    // host memory
    CHECK(path == -7);
    // modulated layer normalization: the statistics workspace holds (m, r) pairs, 8-byte aligned
    CHECK(w8a8_layernorm_modulate_bf16(p, 2, 64, 256, p, p, 0.0, f, p, nullptr) == W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_layernorm_modulate_bf16(p, 2, 64, 256, p, p, 1e-6, f + 1, p, nullptr) == W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_layernorm_modulate_bf16(p, 2, 64, 256, p, p, 1e-6, f, nullptr, nullptr) == W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_layernorm_modulate_quantize_act(p, 2, 100, 256, p, p, 1e-6, f, q8, f, nullptr) ==
          W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_layernorm_modulate_quantize_act(p, 2, 128, 256, p, p, 1e-6, f, q8, f, nullptr) ==
          W8A8_ERR_INVALID_ARG);                                                                  // host memory
    // modulated RMS normalization: eps, sizes, alignment, the fused path's block shape
    CHECK(w8a8_rmsnorm_modulate_bf16(p, 2, 64, 256, p, p, 0.0, f, p, nullptr) == W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_rmsnorm_modulate_bf16(p, 2, 64, 256, p, p, -1e-6, f, p, nullptr) == W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_rmsnorm_modulate_bf16(p, 2, 64, 256, p, p, __builtin_inf(), f, p, nullptr) == W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_rmsnorm_modulate_bf16(p, 2, 64, 252, p, p, 1e-6, f, p, nullptr) == W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_rmsnorm_modulate_bf16(p, 0, 64, 256, p, p, 1e-6, f, p, nullptr) == W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_rmsnorm_modulate_bf16(p, 2, 64, 256, static_cast<char *>(p) + 8, p, 1e-6, f, p, nullptr) ==
          W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_rmsnorm_modulate_bf16(p, 1LL << 20, 1LL << 12, 256, p, p, 1e-6, f, p, nullptr) == W8A8_ERR_UNSUPPORTED);
    const size_t rws = w8a8_rmsnorm_quantize_workspace_bytes(256, 256);
    CHECK(rws == 256 * 3 + 256 * 8 && w8a8_rmsnorm_quantize_workspace_bytes(-1, 256) == 0);
    CHECK(w8a8_rmsnorm_modulate_quantize_act(p, 2, 100, 256, p, p, 1e-6, p, rws, q8, f, nullptr) ==
          W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_rmsnorm_modulate_quantize_act(p, 2, 128, 200, p, p, 1e-6, p, rws, q8, f, nullptr) ==
          W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_rmsnorm_modulate_quantize_act(p, 2, 128, 256, p, p, 1e-6, p, rws, nullptr, f, nullptr) ==
          W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_rmsnorm_modulate_quantize_act(p, 2, 128, 256, p, p, 1e-6, p, rws - 1, q8, f, nullptr) ==
          W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_rmsnorm_modulate_quantize_act(p, 2, 128, 256, p, p, 1e-6, nullptr, rws, q8, f, nullptr) ==
          W8A8_ERR_INVALID_ARG);
    // the path is decided before the workspace: a misaligned x takes the fallback, so a missing
    // workspace is not an error there (the call stops at the host-pointer check instead)
    CHECK(w8a8_linear(pc + 2, 0, 128, 128, 128, p, q8, f, nullptr, p, nullptr, 0, nullptr, &path) ==
          W8A8_ERR_INVALID_ARG);
    CHECK(path == -7);
    // producer linears: workspace size, missing workspace, sizes, the normalization's own rules
    const size_t pws = w8a8_linear_producer_workspace_bytes(256, 256);
    CHECK(pws == 256 * 256 * 2 + 256 * 8 && w8a8_linear_producer_workspace_bytes(0, 256) == 0);
    CHECK(w8a8_linear_producer_workspace_bytes(4000, 4096) == (size_t)4000 * 4096 * 2 + 32000);
    CHECK(w8a8_linear_gelu(p, 256, 256, 256, p, q8, f, nullptr, p, p, pws - 1, nullptr, &path) == W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_linear_gelu(p, 256, 256, 256, p, q8, nullptr, nullptr, p, p, pws, nullptr, &path) ==
          W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_linear_gelu(pc + 1, 256, 256, 256, p, q8, f, nullptr, p, p, pws, nullptr, &path) == W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_linear_gelu(p, 256, 256, 256, p, q8, f, nullptr, p, p, pws, nullptr, &path) ==
          W8A8_ERR_INVALID_ARG);                                                                  // host memory
    CHECK(w8a8_linear_rmsnorm_modulate(p, 2, 128, 256, p, p, 0.0, 256, p, q8, f, nullptr, p, p, pws, nullptr, &path) ==
          W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_linear_rmsnorm_modulate(p, 2, 128, 252, p, p, 1e-6, 256, p, q8, f, nullptr, p, p, 1 << 20, nullptr,
                                       &path) == W8A8_ERR_UNSUPPORTED);
    CHECK(w8a8_linear_layernorm_modulate(p, 2, 128, 256, p, p, 1e-6, 256, p, q8, f, nullptr, p, nullptr, 1 << 20,
                                         nullptr, &path) == W8A8_ERR_INVALID_ARG);
    CHECK(w8a8_linear_layernorm_modulate(p, 2, 128, 256, p, p, 1e-6, 256, p, q8, f, nullptr, p, p, 1 << 20, nullptr,
                                         &path) == W8A8_ERR_INVALID_ARG);                         // host memory
    CHECK(path == -7);
    std::printf("host sanitizer driver: ok\n");
    return 0;
}
