// Internal declarations shared by the HIP sources of libw8a8 (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

constexpr int kBlock = 128;  // quantization block edge (rows and K columns)

// Launchers: enqueue on `stream`, return the launch status.  Shapes and
// alignment are validated by the caller (w8a8_api.cpp).
hipError_t launch_quantize_block(const uint16_t *x, int64_t rows, int64_t cols, int8_t *q, float *s,
                                 hipStream_t stream);

hipError_t launch_gemm_i8_blockscale(const int8_t *qx, const float *sx, const int8_t *qw,
                                     const float *sw, const uint16_t *bias, int64_t M, int64_t N,
                                     int64_t K, uint16_t *y, hipStream_t stream);

hipError_t launch_kblock_partials(const int8_t *qx, const int8_t *qw, int64_t M, int64_t N,
                                  int64_t K, int64_t m0, int64_t mt, int64_t n0, int64_t nt,
                                  int32_t *partials, hipStream_t stream);

// Post-scale form: per-row scales sx[M], per-output-channel scales sw[N].
hipError_t launch_quantize_rows(const uint16_t *x, int64_t rows, int64_t cols, int8_t *q, float *s,
                                hipStream_t stream);
hipError_t launch_gemm_i8_postscale(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw,
                                    const uint16_t *bias, int64_t M, int64_t N, int64_t K, uint16_t *y,
                                    hipStream_t stream);

// Exact GELU (bf16 -> bf16), alone and fused with the 128x128 block quantization.
hipError_t launch_gelu_bf16(const uint16_t *x, int64_t n, uint16_t *y, hipStream_t stream);
hipError_t launch_gelu_quantize_block(const uint16_t *y, int64_t rows, int64_t cols, int8_t *q, float *s,
                                      hipStream_t stream);

// Attention Q/K: sequence-major bf16 -> head-major int8 + per-128-token scales; D is 64 or 128.
hipError_t launch_gemm_i8_blockscale_residual(const int8_t *qx, const float *sx, const int8_t *qw,
                                              const float *sw, const uint16_t *bias, int64_t M, int64_t N,
                                              int64_t K, const uint16_t *h, const uint16_t *gate, int64_t L,
                                              uint16_t *y, hipStream_t stream);
hipError_t launch_gated_residual(const uint16_t *h, const uint16_t *o, const uint16_t *gate, int64_t B, int64_t L,
                                 int64_t N, uint16_t *y, hipStream_t stream);
hipError_t launch_quantize_v_fp8(const uint16_t *x, int64_t B, int64_t L, int64_t H, int64_t D, int64_t ld,
                                 uint8_t *q, float *s, hipStream_t stream);
hipError_t launch_quantize_qk(const uint16_t *x, int64_t B, int64_t L, int64_t H, int64_t D, int64_t ld,
                              int8_t *q, float *s, hipStream_t stream);
hipError_t launch_rope_quantize_qk(const uint16_t *x, int64_t B, int64_t L, int64_t H, int64_t D, int64_t ld,
                                   const float *cos_t, const float *sin_t, int8_t *q, float *s,
                                   hipStream_t stream);
hipError_t launch_rope_bf16(const uint16_t *x, int64_t B, int64_t L, int64_t H, int64_t D, int64_t ld,
                            const float *cos_t, const float *sin_t, uint16_t *y, hipStream_t stream);

// Modulated RMS normalization: r [rows] (fp32), y bf16, and y fused with the
// 128x128 block quantization (rows and K multiples of 128, rows < 2^31).
hipError_t launch_rms_rows(const uint16_t *x, int64_t rows, int64_t K, double eps, float *r, hipStream_t stream);
hipError_t launch_ln_rows(const uint16_t *x, int64_t rows, int64_t K, double eps, float *stats, hipStream_t stream);
// stats: the RMS form's r per row (center = false) or the layer form's (m, r) per row (center = true)
hipError_t launch_modulate_bf16(const uint16_t *x, const float *stats, bool center, int64_t rows, int64_t L,
                                int64_t K, const uint16_t *scale, const uint16_t *shift, uint16_t *y,
                                hipStream_t stream);
hipError_t launch_modulate_quantize(const uint16_t *x, const float *stats, bool center, int64_t rows, int64_t L,
                                    int64_t K, const uint16_t *scale, const uint16_t *shift, int8_t *q, float *s,
                                    hipStream_t stream);
// RMS form, single read of x (K % 256 == 0, K < 2^26, rows and K multiples of
// 128; taken only where rms_band_fits(K)).  Workspace, 16-byte aligned: a
// control line (word 0: nonzero if a wait between workgroups gave up), one
// line per 128-row band holding its arrival counter, then the fp64 row
// partials [rows / 128][K / 256][128].
constexpr size_t kBandCtrlLine = 256;
constexpr int64_t kBandCols = 256;
inline size_t rms_band_workspace_bytes(int64_t rows, int64_t K) {
    return kBandCtrlLine * (size_t)(1 + rows / kBlock) + (size_t)rows * (size_t)(K / kBandCols) * sizeof(double);
}
hipError_t launch_rms_band_quantize(const uint16_t *x, int64_t rows, int64_t L, int64_t K, double eps,
                                    const uint16_t *scale, const uint16_t *shift, void *workspace, int8_t *q,
                                    float *s, hipStream_t stream);
// True when the current device can hold all K / 256 workgroups of a band
// at once with half of its resident capacity for the band kernel to spare
// (the band's workgroups wait for one another); false if the query fails.
bool rms_band_fits(int64_t K);

// bf16 fallback on the 256x256-tile kernel: x, w, y 16-byte aligned, K % 64 == 0,
// K <= 2^21, N % 128 == 0, any M >= 1; bias 8-byte aligned or null.
hipError_t launch_gemm_bf16_tiled(const uint16_t *x, const uint16_t *w, const uint16_t *bias, int64_t M,
                                  int64_t N, int64_t K, uint16_t *y, hipStream_t stream);

// Records a failed HIP call in the per-thread slot of w8a8_last_hip_error
// and returns W8A8_ERR_HIP.
int hip_failure(hipError_t e);

// The body of w8a8_linear (guard, checks, launches) with the caller's
// workspace; shared by the entry points that bring the workspace differently.
// A call that takes the INT8 path with a workspace smaller than it needs
// returns small_workspace_status (W8A8_ERR_INVALID_ARG for a caller's
// workspace, W8A8_ERR_UNSUPPORTED for the library's fixed array).
int guarded_linear(const void *x, int x_dtype, int64_t M, int64_t K, int64_t N, const void *w_bf16, const int8_t *qw,
                   const float *sw, const void *bias_bf16, void *y_bf16, void *workspace, size_t workspace_bytes,
                   hipStream_t stream, int *path_out, int small_workspace_status);

// x_dtype: 0 bf16, 1 fp16, 2 fp32 (the W8A8_DTYPE_* codes).
hipError_t launch_gemm_bf16(const void *x, int x_dtype, const uint16_t *w, const uint16_t *bias,
                            int64_t M, int64_t N, int64_t K, uint16_t *y, hipStream_t stream);

}  // namespace w8a8
