// C ABI of libw8a8: argument checks, the guard (router) and kernel launches.
// Every entry point is declared and documented in include/w8a8.h.
#include "w8a8.h"

#include <hip/hip_runtime.h>

#include <cmath>

#include "w8a8_internal.h"

namespace {
thread_local int g_last_hip_error = 0;
}  // namespace

int w8a8::hip_failure(hipError_t e) {
    g_last_hip_error = (int)e;
    return W8A8_ERR_HIP;
}

namespace {

int hip_status(hipError_t e) { return e == hipSuccess ? W8A8_OK : w8a8::hip_failure(e); }

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// True iff HIP knows p as device (or managed) memory.  Rejecting anything
// else up front keeps a host pointer from ever reaching a kernel.
bool is_device_ptr(const void *p) {
    if (!p) return false;
    hipPointerAttribute_t attr;
    hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();  // clear the sticky error this query may leave
        return false;
    }
    return attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged;
}

bool valid_dtype(int d) { return d == W8A8_DTYPE_BF16 || d == W8A8_DTYPE_FP16 || d == W8A8_DTYPE_FP32; }

bool mult128(int64_t v) { return v > 0 && v % W8A8_BLOCK == 0; }

size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

int quantize_strict(const void *x, int64_t R, int64_t C, int8_t *q, float *s, hipStream_t stream) {
    if (!x || !q || !s || R <= 0 || C <= 0) return W8A8_ERR_INVALID_ARG;
    if (!mult128(R) || !mult128(C)) return W8A8_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4)) return W8A8_ERR_UNSUPPORTED;
    if (!is_device_ptr(x) || !is_device_ptr(q) || !is_device_ptr(s)) return W8A8_ERR_INVALID_ARG;
    return hip_status(w8a8::launch_quantize_block(static_cast<const uint16_t *>(x), R, C, q, s, stream));
}

// Shared checks of the two modulated-RMSNorm entry points (x, scale, shift,
// r: device pointers; eps > 0 and finite).
int rmsnorm_args(const void *x, int64_t B, int64_t L, int64_t K, const void *scale, const void *shift, double eps,
                 const float *r_ws) {
    if (!x || !scale || !shift || !r_ws || B <= 0 || L <= 0 || K <= 0 || !(eps > 0.0) || !std::isfinite(eps))
        return W8A8_ERR_INVALID_ARG;
    if (B > INT64_MAX / L || B * L > INT32_MAX) return W8A8_ERR_UNSUPPORTED;
    if (K % 8 || !aligned(x, 16) || !aligned(scale, 16) || !aligned(shift, 16) || !aligned(r_ws, 4))
        return W8A8_ERR_UNSUPPORTED;
    return W8A8_OK;
}

// Final path of a guarded linear before its workspace is looked at: the
// route (dtype, shapes, quantized weight), the GEMM's K limit, then the
// alignment the INT8 kernels need on x, y, qw (16 bytes), sw (sw_align) and
// bias (8); any miss takes the bf16 fallback.  y may be null when the caller
// checks it separately.
int guarded_path(int x_dtype, int64_t M, int64_t K, int64_t N, const void *x, const void *y, const int8_t *qw,
                 const float *sw, uintptr_t sw_align, const void *bias, int64_t max_k) {
    int path = w8a8_route(x_dtype, M, K, N, qw != nullptr);
    if (path == W8A8_PATH_INT8 && K > max_k) path = W8A8_PATH_BF16;
    if (path == W8A8_PATH_INT8 && (!aligned(x, 16) || (y && !aligned(y, 16)) || !aligned(qw, 16) ||
                                   !aligned(sw, sw_align) || !aligned(bias, 8)))
        path = W8A8_PATH_BF16;
    return path;
}

// Workspace checks of a call that takes the INT8 path: present and large
// enough (else small_status), device memory (else W8A8_ERR_INVALID_ARG); a
// workspace that is not 16-byte aligned sends the call to the fallback
// instead.
int int8_workspace(int &path, const int8_t *qw, const float *sw, void *workspace, size_t workspace_bytes,
                   size_t need, int small_status = W8A8_ERR_INVALID_ARG) {
    if (path != W8A8_PATH_INT8) return W8A8_OK;
    if (!workspace || workspace_bytes < need) return small_status;
    if (!is_device_ptr(qw) || !is_device_ptr(sw) || !is_device_ptr(workspace)) return W8A8_ERR_INVALID_ARG;
    if (!aligned(workspace, 16)) path = W8A8_PATH_BF16;
    return W8A8_OK;
}

}  // namespace

extern "C" {

int w8a8_route(int x_dtype, int64_t M, int64_t K, int64_t N, int has_qweight) {
    if (M <= 0 || K <= 0 || N <= 0 || !valid_dtype(x_dtype)) return -1;
    if (x_dtype == W8A8_DTYPE_BF16 && M % W8A8_BLOCK == 0 && K % W8A8_BLOCK == 0 &&
        N % W8A8_BLOCK == 0 && has_qweight)
        return W8A8_PATH_INT8;
    return W8A8_PATH_BF16;
}

int w8a8_quantize_weight(const void *w_bf16, int64_t N, int64_t K, int8_t *qw, float *sw,
                         hipStream_t stream) {
    return quantize_strict(w_bf16, N, K, qw, sw, stream);
}

int w8a8_quantize_act(const void *x_bf16, int64_t M, int64_t K, int8_t *qx, float *sx,
                      hipStream_t stream) {
    return quantize_strict(x_bf16, M, K, qx, sx, stream);
}

int w8a8_gemm_blockscale(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw,
                         const void *bias_bf16, int64_t M, int64_t N, int64_t K, void *y_bf16,
                         hipStream_t stream) {
    if (!qx || !sx || !qw || !sw || !y_bf16 || M <= 0 || N <= 0 || K <= 0) return W8A8_ERR_INVALID_ARG;
    if (!mult128(M) || !mult128(N) || !mult128(K) || K > W8A8_BLOCK_MAX_K) return W8A8_ERR_UNSUPPORTED;
    if (!aligned(qx, 16) || !aligned(qw, 16) || !aligned(y_bf16, 16) || !aligned(sx, 4) ||
        !aligned(sw, 4) || !aligned(bias_bf16, 8))
        return W8A8_ERR_UNSUPPORTED;
    if (!is_device_ptr(qx) || !is_device_ptr(sx) || !is_device_ptr(qw) || !is_device_ptr(sw) ||
        !is_device_ptr(y_bf16) || (bias_bf16 && !is_device_ptr(bias_bf16)))
        return W8A8_ERR_INVALID_ARG;
    return hip_status(w8a8::launch_gemm_i8_blockscale(qx, sx, qw, sw,
                                                      static_cast<const uint16_t *>(bias_bf16), M, N,
                                                      K, static_cast<uint16_t *>(y_bf16), stream));
}

size_t w8a8_linear_workspace_bytes(int64_t M, int64_t K) {
    if (!mult128(M) || !mult128(K)) return 0;
    const size_t q = round256((size_t)M * (size_t)K);
    const size_t s = round256((size_t)(M / W8A8_BLOCK) * (size_t)(K / W8A8_BLOCK) * sizeof(float));
    return q + s;
}

int w8a8_linear(const void *x, int x_dtype, int64_t M, int64_t K, int64_t N, const void *w_bf16,
                const int8_t *qw, const float *sw, const void *bias_bf16, void *y_bf16,
                void *workspace, size_t workspace_bytes, hipStream_t stream, int *path_out) {
    return w8a8::guarded_linear(x, x_dtype, M, K, N, w_bf16, qw, sw, bias_bf16, y_bf16, workspace, workspace_bytes,
                                stream, path_out, W8A8_ERR_INVALID_ARG);
}

}  // extern "C"

namespace w8a8 {

int guarded_linear(const void *x, int x_dtype, int64_t M, int64_t K, int64_t N, const void *w_bf16, const int8_t *qw,
                   const float *sw, const void *bias_bf16, void *y_bf16, void *workspace, size_t workspace_bytes,
                   hipStream_t stream, int *path_out, int small_workspace_status) {
    if (!x || !w_bf16 || !y_bf16 || M <= 0 || K <= 0 || N <= 0 || !valid_dtype(x_dtype))
        return W8A8_ERR_INVALID_ARG;
    if ((qw == nullptr) != (sw == nullptr)) return W8A8_ERR_INVALID_ARG;
    if (!is_device_ptr(x) || !is_device_ptr(w_bf16) || !is_device_ptr(y_bf16) ||
        (bias_bf16 && !is_device_ptr(bias_bf16)))
        return W8A8_ERR_INVALID_ARG;

    // the INT8 kernels use 16-byte loads/stores: misaligned operands fall back
    int path = guarded_path(x_dtype, M, K, N, x, y_bf16, qw, sw, 4, bias_bf16, W8A8_BLOCK_MAX_K);
    const int ws_status = int8_workspace(path, qw, sw, workspace, workspace_bytes, w8a8_linear_workspace_bytes(M, K),
                                         small_workspace_status);
    if (ws_status != W8A8_OK) return ws_status;
    if (path_out) *path_out = path;

    if (path == W8A8_PATH_INT8) {
        int8_t *qx = static_cast<int8_t *>(workspace);
        float *sx = reinterpret_cast<float *>(static_cast<char *>(workspace) + round256((size_t)M * (size_t)K));
        hipError_t e = w8a8::launch_quantize_block(static_cast<const uint16_t *>(x), M, K, qx, sx, stream);
        if (e != hipSuccess) return hip_status(e);
        return hip_status(w8a8::launch_gemm_i8_blockscale(qx, sx, qw, sw,
                                                          static_cast<const uint16_t *>(bias_bf16), M,
                                                          N, K, static_cast<uint16_t *>(y_bf16), stream));
    }
    return hip_status(w8a8::launch_gemm_bf16(x, x_dtype, static_cast<const uint16_t *>(w_bf16),
                                             static_cast<const uint16_t *>(bias_bf16), M, N, K,
                                             static_cast<uint16_t *>(y_bf16), stream));
}

}  // namespace w8a8

extern "C" {

// Two equally sized ranges that overlap without coinciding (exact aliasing
// is the in-place case some entries allow).
static bool partial_overlap(const void *a, const void *b, size_t bytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x != y && (x < y ? y - x : x - y) < bytes;
}

static int residual_args(const void *h, const void *gate, int64_t M, int64_t N, int64_t L, const void *y) {
    if (!h || !gate || L <= 0 || M % L) return W8A8_ERR_INVALID_ARG;
    if (partial_overlap(y, h, (size_t)M * (size_t)N * 2)) return W8A8_ERR_INVALID_ARG;
    if (N % 8 || !aligned(h, 16) || !aligned(gate, 16) || !aligned(y, 16)) return W8A8_ERR_UNSUPPORTED;
    return W8A8_OK;
}

int w8a8_gated_residual(const void *h_bf16, const void *o_bf16, const void *gate_bf16, int64_t B, int64_t L,
                        int64_t N, void *y_bf16, hipStream_t stream) {
    if (!o_bf16 || !y_bf16 || B <= 0 || L <= 0 || N <= 0) return W8A8_ERR_INVALID_ARG;
    if (B > INT64_MAX / L || B * L > INT64_MAX / N / 2) return W8A8_ERR_UNSUPPORTED;
    const int st = residual_args(h_bf16, gate_bf16, B * L, N, L, y_bf16);
    if (st != W8A8_OK) return st;
    if (partial_overlap(y_bf16, o_bf16, (size_t)(B * L) * (size_t)N * 2)) return W8A8_ERR_INVALID_ARG;
    if (!aligned(o_bf16, 16)) return W8A8_ERR_UNSUPPORTED;
    if (!is_device_ptr(h_bf16) || !is_device_ptr(o_bf16) || !is_device_ptr(gate_bf16) || !is_device_ptr(y_bf16))
        return W8A8_ERR_INVALID_ARG;
    return hip_status(w8a8::launch_gated_residual(static_cast<const uint16_t *>(h_bf16),
                                                  static_cast<const uint16_t *>(o_bf16),
                                                  static_cast<const uint16_t *>(gate_bf16), B, L, N,
                                                  static_cast<uint16_t *>(y_bf16), stream));
}

int w8a8_gemm_blockscale_gated_residual(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw,
                                        const void *bias_bf16, int64_t M, int64_t N, int64_t K,
                                        const void *h_bf16, const void *gate_bf16, int64_t L, void *y_bf16,
                                        hipStream_t stream) {
    if (!qx || !sx || !qw || !sw || !y_bf16 || M <= 0 || N <= 0 || K <= 0) return W8A8_ERR_INVALID_ARG;
    const int st = residual_args(h_bf16, gate_bf16, M, N, L, y_bf16);
    if (st != W8A8_OK) return st;
    if (!mult128(M) || !mult128(N) || !mult128(K) || K > W8A8_BLOCK_MAX_K || M > INT32_MAX)
        return W8A8_ERR_UNSUPPORTED;
    if (!aligned(qx, 16) || !aligned(qw, 16) || !aligned(sx, 4) || !aligned(sw, 4) || !aligned(bias_bf16, 8))
        return W8A8_ERR_UNSUPPORTED;
    if (!is_device_ptr(qx) || !is_device_ptr(sx) || !is_device_ptr(qw) || !is_device_ptr(sw) ||
        !is_device_ptr(y_bf16) || !is_device_ptr(h_bf16) || !is_device_ptr(gate_bf16) ||
        (bias_bf16 && !is_device_ptr(bias_bf16)))
        return W8A8_ERR_INVALID_ARG;
    return hip_status(w8a8::launch_gemm_i8_blockscale_residual(
        qx, sx, qw, sw, static_cast<const uint16_t *>(bias_bf16), M, N, K, static_cast<const uint16_t *>(h_bf16),
        static_cast<const uint16_t *>(gate_bf16), L, static_cast<uint16_t *>(y_bf16), stream));
}

int w8a8_linear_gated_residual(const void *x, int x_dtype, int64_t M, int64_t K, int64_t N, const void *w_bf16,
                               const int8_t *qw, const float *sw, const void *bias_bf16, const void *h_bf16,
                               const void *gate_bf16, int64_t L, void *y_bf16, void *workspace,
                               size_t workspace_bytes, hipStream_t stream, int *path_out) {
    if (!x || !w_bf16 || !y_bf16 || M <= 0 || K <= 0 || N <= 0 || !valid_dtype(x_dtype))
        return W8A8_ERR_INVALID_ARG;
    if ((qw == nullptr) != (sw == nullptr)) return W8A8_ERR_INVALID_ARG;
    const int st = residual_args(h_bf16, gate_bf16, M, N, L, y_bf16);
    if (st != W8A8_OK) return st;
    if (h_bf16 == y_bf16) return W8A8_ERR_INVALID_ARG;  // the fallback writes o into y before the update
    if (!is_device_ptr(x) || !is_device_ptr(w_bf16) || !is_device_ptr(y_bf16) || !is_device_ptr(h_bf16) ||
        !is_device_ptr(gate_bf16) || (bias_bf16 && !is_device_ptr(bias_bf16)))
        return W8A8_ERR_INVALID_ARG;

    int path = guarded_path(x_dtype, M, K, N, x, nullptr, qw, sw, 4, bias_bf16, W8A8_BLOCK_MAX_K);
    if (path == W8A8_PATH_INT8 && M > INT32_MAX) path = W8A8_PATH_BF16;
    const int ws_status = int8_workspace(path, qw, sw, workspace, workspace_bytes, w8a8_linear_workspace_bytes(M, K));
    if (ws_status != W8A8_OK) return ws_status;
    if (path_out) *path_out = path;

    if (path == W8A8_PATH_INT8) {
        int8_t *qx = static_cast<int8_t *>(workspace);
        float *sx = reinterpret_cast<float *>(static_cast<char *>(workspace) + round256((size_t)M * (size_t)K));
        hipError_t e = w8a8::launch_quantize_block(static_cast<const uint16_t *>(x), M, K, qx, sx, stream);
        if (e != hipSuccess) return hip_status(e);
        return hip_status(w8a8::launch_gemm_i8_blockscale_residual(
            qx, sx, qw, sw, static_cast<const uint16_t *>(bias_bf16), M, N, K,
            static_cast<const uint16_t *>(h_bf16), static_cast<const uint16_t *>(gate_bf16), L,
            static_cast<uint16_t *>(y_bf16), stream));
    }
    hipError_t e = w8a8::launch_gemm_bf16(x, x_dtype, static_cast<const uint16_t *>(w_bf16),
                                          static_cast<const uint16_t *>(bias_bf16), M, N, K,
                                          static_cast<uint16_t *>(y_bf16), stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(w8a8::launch_gated_residual(static_cast<const uint16_t *>(h_bf16),
                                                  static_cast<const uint16_t *>(y_bf16),
                                                  static_cast<const uint16_t *>(gate_bf16), M / L, L, N,
                                                  static_cast<uint16_t *>(y_bf16), stream));
}

int w8a8_debug_kblock_partials(const int8_t *qx, const int8_t *qw, int64_t M, int64_t N, int64_t K,
                               int64_t m0, int64_t mt, int64_t n0, int64_t nt, int32_t *partials,
                               hipStream_t stream) {
    if (!qx || !qw || !partials || M <= 0 || N <= 0 || K <= 0) return W8A8_ERR_INVALID_ARG;
    if (m0 < 0 || n0 < 0 || mt <= 0 || nt <= 0 || m0 + mt > M || n0 + nt > N) return W8A8_ERR_INVALID_ARG;
    if (!mult128(M) || !mult128(N) || !mult128(K) || K > W8A8_BLOCK_MAX_K || m0 % W8A8_BLOCK ||
        n0 % W8A8_BLOCK || mt % W8A8_BLOCK || nt % W8A8_BLOCK)
        return W8A8_ERR_UNSUPPORTED;
    if (!aligned(qx, 16) || !aligned(qw, 16) || !aligned(partials, 4)) return W8A8_ERR_UNSUPPORTED;
    if (!is_device_ptr(qx) || !is_device_ptr(qw) || !is_device_ptr(partials)) return W8A8_ERR_INVALID_ARG;
    return hip_status(w8a8::launch_kblock_partials(qx, qw, M, N, K, m0, mt, n0, nt, partials, stream));
}

int w8a8_quantize_rows(const void *x_bf16, int64_t R, int64_t K, int8_t *q, float *s, hipStream_t stream) {
    if (!x_bf16 || !q || !s || R <= 0 || K <= 0) return W8A8_ERR_INVALID_ARG;
    if (K % 8 || !aligned(x_bf16, 16) || !aligned(q, 16) || !aligned(s, 4)) return W8A8_ERR_UNSUPPORTED;
    if (!is_device_ptr(x_bf16) || !is_device_ptr(q) || !is_device_ptr(s)) return W8A8_ERR_INVALID_ARG;
    return hip_status(w8a8::launch_quantize_rows(static_cast<const uint16_t *>(x_bf16), R, K, q, s, stream));
}

int w8a8_gemm_postscale(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw,
                        const void *bias_bf16, int64_t M, int64_t N, int64_t K, void *y_bf16,
                        hipStream_t stream) {
    if (!qx || !sx || !qw || !sw || !y_bf16 || M <= 0 || N <= 0 || K <= 0) return W8A8_ERR_INVALID_ARG;
    if (!mult128(M) || !mult128(N) || !mult128(K) || K > W8A8_POSTSCALE_MAX_K) return W8A8_ERR_UNSUPPORTED;
    if (!aligned(qx, 16) || !aligned(qw, 16) || !aligned(y_bf16, 16) || !aligned(sx, 4) ||
        !aligned(sw, 16) || !aligned(bias_bf16, 8))
        return W8A8_ERR_UNSUPPORTED;
    if (!is_device_ptr(qx) || !is_device_ptr(sx) || !is_device_ptr(qw) || !is_device_ptr(sw) ||
        !is_device_ptr(y_bf16) || (bias_bf16 && !is_device_ptr(bias_bf16)))
        return W8A8_ERR_INVALID_ARG;
    return hip_status(w8a8::launch_gemm_i8_postscale(qx, sx, qw, sw, static_cast<const uint16_t *>(bias_bf16), M,
                                                     N, K, static_cast<uint16_t *>(y_bf16), stream));
}

size_t w8a8_linear_postscale_workspace_bytes(int64_t M, int64_t K) {
    if (!mult128(M) || !mult128(K)) return 0;
    return round256((size_t)M * (size_t)K) + round256((size_t)M * sizeof(float));
}

int w8a8_linear_postscale(const void *x, int x_dtype, int64_t M, int64_t K, int64_t N, const void *w_bf16,
                          const int8_t *qw, const float *sw, const void *bias_bf16, void *y_bf16,
                          void *workspace, size_t workspace_bytes, hipStream_t stream, int *path_out) {
    if (!x || !w_bf16 || !y_bf16 || M <= 0 || K <= 0 || N <= 0 || !valid_dtype(x_dtype))
        return W8A8_ERR_INVALID_ARG;
    if ((qw == nullptr) != (sw == nullptr)) return W8A8_ERR_INVALID_ARG;
    if (!is_device_ptr(x) || !is_device_ptr(w_bf16) || !is_device_ptr(y_bf16) ||
        (bias_bf16 && !is_device_ptr(bias_bf16)))
        return W8A8_ERR_INVALID_ARG;
    int path = guarded_path(x_dtype, M, K, N, x, y_bf16, qw, sw, 16, bias_bf16, W8A8_POSTSCALE_MAX_K);
    const int ws_status =
        int8_workspace(path, qw, sw, workspace, workspace_bytes, w8a8_linear_postscale_workspace_bytes(M, K));
    if (ws_status != W8A8_OK) return ws_status;
    if (path_out) *path_out = path;
    if (path == W8A8_PATH_INT8) {
        int8_t *qx = static_cast<int8_t *>(workspace);
        float *sx = reinterpret_cast<float *>(static_cast<char *>(workspace) + round256((size_t)M * (size_t)K));
        hipError_t e = w8a8::launch_quantize_rows(static_cast<const uint16_t *>(x), M, K, qx, sx, stream);
        if (e != hipSuccess) return hip_status(e);
        return hip_status(w8a8::launch_gemm_i8_postscale(qx, sx, qw, sw, static_cast<const uint16_t *>(bias_bf16),
                                                         M, N, K, static_cast<uint16_t *>(y_bf16), stream));
    }
    return hip_status(w8a8::launch_gemm_bf16(x, x_dtype, static_cast<const uint16_t *>(w_bf16),
                                             static_cast<const uint16_t *>(bias_bf16), M, N, K,
                                             static_cast<uint16_t *>(y_bf16), stream));
}

int w8a8_gelu_bf16(const void *x_bf16, int64_t n, void *y_bf16, hipStream_t stream) {
    if (n < 0) return W8A8_ERR_INVALID_ARG;
    if (n == 0) return W8A8_OK;
    if (!x_bf16 || !y_bf16) return W8A8_ERR_INVALID_ARG;
    if (!aligned(x_bf16, 2) || !aligned(y_bf16, 2)) return W8A8_ERR_UNSUPPORTED;
    if (!is_device_ptr(x_bf16) || !is_device_ptr(y_bf16)) return W8A8_ERR_INVALID_ARG;
    return hip_status(w8a8::launch_gelu_bf16(static_cast<const uint16_t *>(x_bf16), n,
                                             static_cast<uint16_t *>(y_bf16), stream));
}

int w8a8_gelu_quantize_act(const void *y_bf16, int64_t M, int64_t K, int8_t *qx, float *sx,
                           hipStream_t stream) {
    if (!y_bf16 || !qx || !sx || M <= 0 || K <= 0) return W8A8_ERR_INVALID_ARG;
    if (!mult128(M) || !mult128(K) || K > W8A8_GELU_QUANT_MAX_K) return W8A8_ERR_UNSUPPORTED;
    if (!aligned(y_bf16, 16) || !aligned(qx, 16) || !aligned(sx, 4)) return W8A8_ERR_UNSUPPORTED;
    if (!is_device_ptr(y_bf16) || !is_device_ptr(qx) || !is_device_ptr(sx)) return W8A8_ERR_INVALID_ARG;
    return hip_status(w8a8::launch_gelu_quantize_block(static_cast<const uint16_t *>(y_bf16), M, K, qx, sx,
                                                       stream));
}

int w8a8_quantize_qk(const void *x_bf16, int64_t B, int64_t L, int64_t H, int64_t D, int64_t ld, int8_t *q,
                     float *s, hipStream_t stream) {
    if (!x_bf16 || !q || !s || B <= 0 || L <= 0 || H <= 0 || D <= 0 || ld < H * D) return W8A8_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return W8A8_ERR_UNSUPPORTED;
    if (ld % 8 || !aligned(x_bf16, 16) || !aligned(q, 16) || !aligned(s, 4)) return W8A8_ERR_UNSUPPORTED;
    const int64_t nblk = (L + W8A8_BLOCK - 1) / W8A8_BLOCK;
    if (B > INT32_MAX / H || B * H > INT32_MAX / nblk) return W8A8_ERR_UNSUPPORTED;
    if (!is_device_ptr(x_bf16) || !is_device_ptr(q) || !is_device_ptr(s)) return W8A8_ERR_INVALID_ARG;
    return hip_status(w8a8::launch_quantize_qk(static_cast<const uint16_t *>(x_bf16), B, L, H, D, ld, q, s, stream));
}

int w8a8_quantize_v_fp8(const void *x_bf16, int64_t B, int64_t L, int64_t H, int64_t D, int64_t ld, uint8_t *q,
                        float *s, hipStream_t stream) {
    if (!x_bf16 || !q || !s || B <= 0 || L <= 0 || H <= 0 || D <= 0) return W8A8_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return W8A8_ERR_UNSUPPORTED;
    if (H > INT32_MAX / D) return W8A8_ERR_UNSUPPORTED;
    if (ld < H * D) return W8A8_ERR_INVALID_ARG;
    if (ld % 8 || !aligned(x_bf16, 16) || !aligned(q, 16) || !aligned(s, 4)) return W8A8_ERR_UNSUPPORTED;
    const int64_t nblk = (L + W8A8_BLOCK - 1) / W8A8_BLOCK;
    if (B > INT32_MAX / H || B * H > INT32_MAX / nblk) return W8A8_ERR_UNSUPPORTED;
    if (!is_device_ptr(x_bf16) || !is_device_ptr(q) || !is_device_ptr(s)) return W8A8_ERR_INVALID_ARG;
    return hip_status(
        w8a8::launch_quantize_v_fp8(static_cast<const uint16_t *>(x_bf16), B, L, H, D, ld, q, s, stream));
}

static int rope_args(const void *x, int64_t B, int64_t L, int64_t H, int64_t D, int64_t ld, const float *cos_t,
                     const float *sin_t) {
    if (!x || !cos_t || !sin_t || B <= 0 || L <= 0 || H <= 0 || D <= 0) return W8A8_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return W8A8_ERR_UNSUPPORTED;
    if (H > INT32_MAX / D) return W8A8_ERR_UNSUPPORTED;
    if (ld < H * D) return W8A8_ERR_INVALID_ARG;
    if (ld % 8 || !aligned(x, 16) || !aligned(cos_t, 16) || !aligned(sin_t, 16)) return W8A8_ERR_UNSUPPORTED;
    return W8A8_OK;
}

int w8a8_rope_bf16(const void *x_bf16, int64_t B, int64_t L, int64_t H, int64_t D, int64_t ld, const float *cos_t,
                   const float *sin_t, void *y_bf16, hipStream_t stream) {
    if (!y_bf16) return W8A8_ERR_INVALID_ARG;
    const int st = rope_args(x_bf16, B, L, H, D, ld, cos_t, sin_t);
    if (st != W8A8_OK) return st;
    if (B > INT64_MAX / L || B * L > INT64_MAX / (H * D)) return W8A8_ERR_UNSUPPORTED;
    if (!aligned(y_bf16, 16)) return W8A8_ERR_UNSUPPORTED;
    if (!is_device_ptr(x_bf16) || !is_device_ptr(cos_t) || !is_device_ptr(sin_t) || !is_device_ptr(y_bf16))
        return W8A8_ERR_INVALID_ARG;
    return hip_status(w8a8::launch_rope_bf16(static_cast<const uint16_t *>(x_bf16), B, L, H, D, ld, cos_t, sin_t,
                                             static_cast<uint16_t *>(y_bf16), stream));
}

int w8a8_rope_quantize_qk(const void *x_bf16, int64_t B, int64_t L, int64_t H, int64_t D, int64_t ld,
                          const float *cos_t, const float *sin_t, int8_t *q, float *s, hipStream_t stream) {
    if (!q || !s) return W8A8_ERR_INVALID_ARG;
    const int st = rope_args(x_bf16, B, L, H, D, ld, cos_t, sin_t);
    if (st != W8A8_OK) return st;
    if (!aligned(q, 16) || !aligned(s, 4) || ld > W8A8_ROPE_MAX_LD) return W8A8_ERR_UNSUPPORTED;
    const int64_t nblk = (L + W8A8_BLOCK - 1) / W8A8_BLOCK;
    if (B > INT32_MAX / H || B * H > INT32_MAX / nblk) return W8A8_ERR_UNSUPPORTED;
    if (!is_device_ptr(x_bf16) || !is_device_ptr(cos_t) || !is_device_ptr(sin_t) || !is_device_ptr(q) ||
        !is_device_ptr(s))
        return W8A8_ERR_INVALID_ARG;
    return hip_status(w8a8::launch_rope_quantize_qk(static_cast<const uint16_t *>(x_bf16), B, L, H, D, ld, cos_t,
                                                    sin_t, q, s, stream));
}

int w8a8_rmsnorm_modulate_bf16(const void *x_bf16, int64_t B, int64_t L, int64_t K, const void *scale_bf16,
                               const void *shift_bf16, double eps, float *r_ws, void *y_bf16, hipStream_t stream) {
    const int st = rmsnorm_args(x_bf16, B, L, K, scale_bf16, shift_bf16, eps, r_ws);
    if (st != W8A8_OK) return st;
    if (!y_bf16) return W8A8_ERR_INVALID_ARG;
    if (!aligned(y_bf16, 16)) return W8A8_ERR_UNSUPPORTED;
    if (!is_device_ptr(x_bf16) || !is_device_ptr(scale_bf16) || !is_device_ptr(shift_bf16) || !is_device_ptr(r_ws) ||
        !is_device_ptr(y_bf16))
        return W8A8_ERR_INVALID_ARG;
    const uint16_t *x = static_cast<const uint16_t *>(x_bf16);
    hipError_t e = w8a8::launch_rms_rows(x, B * L, K, eps, r_ws, stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(w8a8::launch_modulate_bf16(x, r_ws, false, B * L, L, K,
                                                 static_cast<const uint16_t *>(scale_bf16),
                                                 static_cast<const uint16_t *>(shift_bf16),
                                                 static_cast<uint16_t *>(y_bf16), stream));
}

// Bytes of the control line (word 0: the wait error word) that starts the
// workspace of the fused RMS producer.
static constexpr size_t kRmsCtrl = 256;

// The fused RMS producer can read x once (the band kernel) when K % 256 == 0;
// it does so when a band's workgroups also fit on the current device at once
// (rms_band_fits), else it runs the row-statistics kernel and the two-read
// quantizer, with r after the control line.  The workspace is sized by K
// alone, for the single-read layout where K allows it, which is the larger.
static bool rms_single_read(int64_t K) { return K % 256 == 0 && K < ((int64_t)1 << 26); }

size_t w8a8_rmsnorm_quantize_workspace_bytes(int64_t M, int64_t K) {
    if (M <= 0 || K <= 0) return 0;
    if (rms_single_read(K)) return round256(w8a8::rms_band_workspace_bytes(M, K));
    return kRmsCtrl + round256((size_t)M * sizeof(float));
}

// Fused RMS producer into qx/sx with `ws` (device, 16-byte aligned, large enough).
static hipError_t rms_quantize(const uint16_t *x, int64_t M, int64_t L, int64_t K, double eps, const uint16_t *scale,
                               const uint16_t *shift, void *ws, int8_t *qx, float *sx, hipStream_t stream) {
    if (rms_single_read(K) && w8a8::rms_band_fits(K))
        return w8a8::launch_rms_band_quantize(x, M, L, K, eps, scale, shift, ws, qx, sx, stream);
    float *r = reinterpret_cast<float *>(static_cast<char *>(ws) + kRmsCtrl);
    const hipError_t e = w8a8::launch_rms_rows(x, M, K, eps, r, stream);
    if (e != hipSuccess) return e;
    return w8a8::launch_modulate_quantize(x, r, false, M, L, K, scale, shift, qx, sx, stream);
}

int w8a8_rmsnorm_modulate_quantize_act(const void *x_bf16, int64_t B, int64_t L, int64_t K, const void *scale_bf16,
                                       const void *shift_bf16, double eps, void *workspace, size_t workspace_bytes,
                                       int8_t *qx, float *sx, hipStream_t stream) {
    const int st = rmsnorm_args(x_bf16, B, L, K, scale_bf16, shift_bf16, eps, static_cast<const float *>(workspace));
    if (st != W8A8_OK) return st;
    if (!qx || !sx) return W8A8_ERR_INVALID_ARG;
    if (!mult128(B * L) || !mult128(K) || !aligned(qx, 16) || !aligned(sx, 4) || !aligned(workspace, 16))
        return W8A8_ERR_UNSUPPORTED;
    if (workspace_bytes < w8a8_rmsnorm_quantize_workspace_bytes(B * L, K)) return W8A8_ERR_INVALID_ARG;
    if (!is_device_ptr(x_bf16) || !is_device_ptr(scale_bf16) || !is_device_ptr(shift_bf16) ||
        !is_device_ptr(workspace) || !is_device_ptr(qx) || !is_device_ptr(sx))
        return W8A8_ERR_INVALID_ARG;
    return hip_status(rms_quantize(static_cast<const uint16_t *>(x_bf16), B * L, L, K, eps,
                                   static_cast<const uint16_t *>(scale_bf16),
                                   static_cast<const uint16_t *>(shift_bf16), workspace, qx, sx, stream));
}

int w8a8_layernorm_modulate_bf16(const void *x_bf16, int64_t B, int64_t L, int64_t K, const void *scale_bf16,
                                 const void *shift_bf16, double eps, float *stats_ws, void *y_bf16,
                                 hipStream_t stream) {
    const int st = rmsnorm_args(x_bf16, B, L, K, scale_bf16, shift_bf16, eps, stats_ws);
    if (st != W8A8_OK) return st;
    if (!y_bf16) return W8A8_ERR_INVALID_ARG;
    if (!aligned(y_bf16, 16) || !aligned(stats_ws, 8)) return W8A8_ERR_UNSUPPORTED;
    if (!is_device_ptr(x_bf16) || !is_device_ptr(scale_bf16) || !is_device_ptr(shift_bf16) ||
        !is_device_ptr(stats_ws) || !is_device_ptr(y_bf16))
        return W8A8_ERR_INVALID_ARG;
    const uint16_t *x = static_cast<const uint16_t *>(x_bf16);
    hipError_t e = w8a8::launch_ln_rows(x, B * L, K, eps, stats_ws, stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(w8a8::launch_modulate_bf16(x, stats_ws, true, B * L, L, K,
                                                 static_cast<const uint16_t *>(scale_bf16),
                                                 static_cast<const uint16_t *>(shift_bf16),
                                                 static_cast<uint16_t *>(y_bf16), stream));
}

int w8a8_layernorm_modulate_quantize_act(const void *x_bf16, int64_t B, int64_t L, int64_t K,
                                         const void *scale_bf16, const void *shift_bf16, double eps,
                                         float *stats_ws, int8_t *qx, float *sx, hipStream_t stream) {
    const int st = rmsnorm_args(x_bf16, B, L, K, scale_bf16, shift_bf16, eps, stats_ws);
    if (st != W8A8_OK) return st;
    if (!qx || !sx) return W8A8_ERR_INVALID_ARG;
    if (!mult128(B * L) || !mult128(K) || !aligned(qx, 16) || !aligned(sx, 4) || !aligned(stats_ws, 8))
        return W8A8_ERR_UNSUPPORTED;
    if (!is_device_ptr(x_bf16) || !is_device_ptr(scale_bf16) || !is_device_ptr(shift_bf16) ||
        !is_device_ptr(stats_ws) || !is_device_ptr(qx) || !is_device_ptr(sx))
        return W8A8_ERR_INVALID_ARG;
    const uint16_t *x = static_cast<const uint16_t *>(x_bf16);
    hipError_t e = w8a8::launch_ln_rows(x, B * L, K, eps, stats_ws, stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(w8a8::launch_modulate_quantize(x, stats_ws, true, B * L, L, K,
                                                     static_cast<const uint16_t *>(scale_bf16),
                                                     static_cast<const uint16_t *>(shift_bf16), qx, sx, stream));
}

size_t w8a8_linear_producer_workspace_bytes(int64_t M, int64_t K) {
    if (M <= 0 || K <= 0) return 0;
    const size_t stats = round256((size_t)M * 2 * sizeof(float));
    const size_t rms = w8a8_rmsnorm_quantize_workspace_bytes(M, K);
    const size_t fallback = round256((size_t)M * (size_t)K * 2) + stats;
    const size_t int8 = w8a8_linear_workspace_bytes(M, K) + (rms > stats ? rms : stats);
    return fallback > int8 ? fallback : int8;
}

// Workspace of the producer linears: on the INT8 path qx and sx (as in
// w8a8_linear) then the per-row statistics (for the RMS form, the fused
// producer's whole workspace); on the fallback the producer's bf16 output
// [M, K] then the statistics.
static float *producer_stats(void *workspace, int path, int64_t M, int64_t K) {
    const size_t off = path == W8A8_PATH_INT8 ? w8a8_linear_workspace_bytes(M, K) : round256((size_t)M * (size_t)K * 2);
    return reinterpret_cast<float *>(static_cast<char *>(workspace) + off);
}

int w8a8_linear_gelu(const void *u_bf16, int64_t M, int64_t K, int64_t N, const void *w_bf16, const int8_t *qw,
                     const float *sw, const void *bias_bf16, void *y_bf16, void *workspace, size_t workspace_bytes,
                     hipStream_t stream, int *path_out) {
    if (!u_bf16 || !w_bf16 || !y_bf16 || M <= 0 || K <= 0 || N <= 0) return W8A8_ERR_INVALID_ARG;
    if ((qw == nullptr) != (sw == nullptr)) return W8A8_ERR_INVALID_ARG;
    if (M > INT64_MAX / K) return W8A8_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < w8a8_linear_producer_workspace_bytes(M, K)) return W8A8_ERR_INVALID_ARG;
    if (!aligned(u_bf16, 2) || !aligned(workspace, 16)) return W8A8_ERR_UNSUPPORTED;
    if (!is_device_ptr(u_bf16) || !is_device_ptr(w_bf16) || !is_device_ptr(y_bf16) || !is_device_ptr(workspace) ||
        (bias_bf16 && !is_device_ptr(bias_bf16)))
        return W8A8_ERR_INVALID_ARG;
    const int64_t max_k = W8A8_GELU_QUANT_MAX_K < W8A8_BLOCK_MAX_K ? W8A8_GELU_QUANT_MAX_K : W8A8_BLOCK_MAX_K;
    int path = guarded_path(W8A8_DTYPE_BF16, M, K, N, u_bf16, y_bf16, qw, sw, 4, bias_bf16, max_k);
    if (path == W8A8_PATH_INT8 && (!is_device_ptr(qw) || !is_device_ptr(sw))) return W8A8_ERR_INVALID_ARG;
    if (path_out) *path_out = path;
    const uint16_t *u = static_cast<const uint16_t *>(u_bf16);
    const uint16_t *bias = static_cast<const uint16_t *>(bias_bf16);
    uint16_t *y = static_cast<uint16_t *>(y_bf16);
    if (path == W8A8_PATH_INT8) {
        int8_t *qx = static_cast<int8_t *>(workspace);
        float *sx = reinterpret_cast<float *>(static_cast<char *>(workspace) + round256((size_t)M * (size_t)K));
        hipError_t e = w8a8::launch_gelu_quantize_block(u, M, K, qx, sx, stream);
        if (e != hipSuccess) return hip_status(e);
        return hip_status(w8a8::launch_gemm_i8_blockscale(qx, sx, qw, sw, bias, M, N, K, y, stream));
    }
    uint16_t *g = static_cast<uint16_t *>(workspace);
    hipError_t e = w8a8::launch_gelu_bf16(u, M * K, g, stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(w8a8::launch_gemm_bf16(g, W8A8_DTYPE_BF16, static_cast<const uint16_t *>(w_bf16), bias, M, N,
                                             K, y, stream));
}

// The two modulated-normalization linears share everything but the
// statistic kernel and the centring.
static int linear_modulated(bool layer, const void *x_bf16, int64_t B, int64_t L, int64_t K, const void *scale_bf16,
                            const void *shift_bf16, double eps, int64_t N, const void *w_bf16, const int8_t *qw,
                            const float *sw, const void *bias_bf16, void *y_bf16, void *workspace,
                            size_t workspace_bytes, hipStream_t stream, int *path_out) {
    if (!w_bf16 || !y_bf16 || N <= 0 || !workspace) return W8A8_ERR_INVALID_ARG;
    if ((qw == nullptr) != (sw == nullptr)) return W8A8_ERR_INVALID_ARG;
    // the statistics pointer only has to be non-null and aligned here; the real one follows the path
    const int st = rmsnorm_args(x_bf16, B, L, K, scale_bf16, shift_bf16, eps, static_cast<const float *>(workspace));
    if (st != W8A8_OK) return st;
    const int64_t M = B * L;
    if (workspace_bytes < w8a8_linear_producer_workspace_bytes(M, K)) return W8A8_ERR_INVALID_ARG;
    if (!aligned(workspace, 16)) return W8A8_ERR_UNSUPPORTED;
    if (!is_device_ptr(x_bf16) || !is_device_ptr(scale_bf16) || !is_device_ptr(shift_bf16) || !is_device_ptr(w_bf16) ||
        !is_device_ptr(y_bf16) || !is_device_ptr(workspace) || (bias_bf16 && !is_device_ptr(bias_bf16)))
        return W8A8_ERR_INVALID_ARG;
    int path = guarded_path(W8A8_DTYPE_BF16, M, K, N, x_bf16, y_bf16, qw, sw, 4, bias_bf16, W8A8_BLOCK_MAX_K);
    if (path == W8A8_PATH_INT8 && (!is_device_ptr(qw) || !is_device_ptr(sw))) return W8A8_ERR_INVALID_ARG;
    if (path_out) *path_out = path;
    const uint16_t *x = static_cast<const uint16_t *>(x_bf16);
    const uint16_t *scale = static_cast<const uint16_t *>(scale_bf16), *shift = static_cast<const uint16_t *>(shift_bf16);
    const uint16_t *bias = static_cast<const uint16_t *>(bias_bf16);
    uint16_t *y = static_cast<uint16_t *>(y_bf16);
    float *stats = producer_stats(workspace, path, M, K);
    hipError_t e;
    if (path == W8A8_PATH_INT8) {
        int8_t *qx = static_cast<int8_t *>(workspace);
        float *sx = reinterpret_cast<float *>(static_cast<char *>(workspace) + round256((size_t)M * (size_t)K));
        if (layer) {
            e = w8a8::launch_ln_rows(x, M, K, eps, stats, stream);
            if (e == hipSuccess) e = w8a8::launch_modulate_quantize(x, stats, true, M, L, K, scale, shift, qx, sx, stream);
        } else {
            e = rms_quantize(x, M, L, K, eps, scale, shift, stats, qx, sx, stream);
        }
        if (e != hipSuccess) return hip_status(e);
        return hip_status(w8a8::launch_gemm_i8_blockscale(qx, sx, qw, sw, bias, M, N, K, y, stream));
    }
    e = layer ? w8a8::launch_ln_rows(x, M, K, eps, stats, stream) : w8a8::launch_rms_rows(x, M, K, eps, stats, stream);
    if (e != hipSuccess) return hip_status(e);
    uint16_t *g = static_cast<uint16_t *>(workspace);
    e = w8a8::launch_modulate_bf16(x, stats, layer, M, L, K, scale, shift, g, stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(w8a8::launch_gemm_bf16(g, W8A8_DTYPE_BF16, static_cast<const uint16_t *>(w_bf16), bias, M, N,
                                             K, y, stream));
}

int w8a8_linear_rmsnorm_modulate(const void *x_bf16, int64_t B, int64_t L, int64_t K, const void *scale_bf16,
                                 const void *shift_bf16, double eps, int64_t N, const void *w_bf16, const int8_t *qw,
                                 const float *sw, const void *bias_bf16, void *y_bf16, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream, int *path_out) {
    return linear_modulated(false, x_bf16, B, L, K, scale_bf16, shift_bf16, eps, N, w_bf16, qw, sw, bias_bf16, y_bf16,
                            workspace, workspace_bytes, stream, path_out);
}

int w8a8_linear_layernorm_modulate(const void *x_bf16, int64_t B, int64_t L, int64_t K, const void *scale_bf16,
                                   const void *shift_bf16, double eps, int64_t N, const void *w_bf16,
                                   const int8_t *qw, const float *sw, const void *bias_bf16, void *y_bf16,
                                   void *workspace, size_t workspace_bytes, hipStream_t stream, int *path_out) {
    return linear_modulated(true, x_bf16, B, L, K, scale_bf16, shift_bf16, eps, N, w_bf16, qw, sw, bias_bf16, y_bf16,
                            workspace, workspace_bytes, stream, path_out);
}

const char *w8a8_status_string(int status) {
    switch (status) {
    case W8A8_OK: return "W8A8_OK";
    case W8A8_ERR_INVALID_ARG: return "W8A8_ERR_INVALID_ARG";
    case W8A8_ERR_UNSUPPORTED: return "W8A8_ERR_UNSUPPORTED";
    case W8A8_ERR_HIP: return "W8A8_ERR_HIP";
    default: return "W8A8_UNKNOWN_STATUS";
    }
}

int w8a8_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
