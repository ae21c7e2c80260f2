/*
 * Runs every function of the C oracle on small and ragged inputs, plus its
 * argument errors, in a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py): any out-of-bounds
 * access, overflow or other undefined behaviour in the oracle aborts.
 * Buffers are allocated at their exact sizes so that an overrun is caught.
 */
#include <stdint.h>
#include <math.h>
#include <stdio.h>
#include <string.h>
#include <stdlib.h>

int oracle_quantize_block(const uint16_t *x, int64_t rows, int64_t cols, int8_t *q, float *s);
int oracle_kblock_partials(const int8_t *qx, const int8_t *qw, int64_t M, int64_t N, int64_t K, int64_t m0,
                           int64_t mt, int64_t n0, int64_t nt, int32_t *out);
int oracle_linear_int8_rows(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw,
                            const uint16_t *bias, int64_t M, int64_t N, int64_t K, const int64_t *rows,
                            int64_t nrows, uint16_t *y, double *y_f64);
int oracle_linear_bf16_rows(const void *x, int x_dtype, const uint16_t *w, const uint16_t *bias, int64_t M,
                            int64_t N, int64_t K, const int64_t *rows, int64_t nrows, uint16_t *y);
int oracle_quantize_rows(const uint16_t *x, int64_t rows, int64_t cols, int8_t *q, float *s);
int oracle_linear_postscale_rows(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw,
                                 const uint16_t *bias, int64_t M, int64_t N, int64_t K, const int64_t *rows,
                                 int64_t nrows, uint16_t *y);
int oracle_quantize_qk(const uint16_t *x, int64_t B, int64_t L, int64_t H, int64_t D, int64_t ld, int8_t *q,
                       float *s);
int oracle_route(int x_dtype, int64_t M, int64_t K, int64_t N, int has_qweight);
int oracle_quantize_v_fp8(const uint16_t *x, int64_t B, int64_t L, int64_t H, int64_t D, int64_t ld, uint8_t *q,
                          float *s);
uint8_t oracle_f32_to_e4m3(float v);
double oracle_e4m3_to_f64(uint8_t c);
int oracle_layernorm_modulate(const uint16_t *x, int64_t B, int64_t L, int64_t K, const uint16_t *scale,
                              const uint16_t *shift, double eps, uint16_t *y, float *stats_out);
int oracle_gated_residual(const uint16_t *h, const uint16_t *o, const uint16_t *gate, int64_t B, int64_t L,
                          int64_t N, uint16_t *y);
int oracle_rope(const uint16_t *x, int64_t B, int64_t L, int64_t H, int64_t D, int64_t ld, const float *cos_t,
                const float *sin_t, uint16_t *y);
int oracle_rmsnorm_modulate(const uint16_t *x, int64_t B, int64_t L, int64_t K, const uint16_t *scale,
                            const uint16_t *shift, double eps, uint16_t *y, float *r_out);
int oracle_gelu_bf16(const uint16_t *x, int64_t n, uint16_t *y);
uint16_t oracle_f64_to_bf16(double v);
double oracle_fp16_to_f64(uint16_t h);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) { /* xorshift64*: input bits only, no method arithmetic */
    state ^= state >> 12; state ^= state << 25; state ^= state >> 27;
    return (uint32_t)((state * 0x2545F4914F6CDD1Dull) >> 32);
}
/* finite bf16 bit patterns of moderate magnitude, both signs */
static uint16_t rand_bf16(void) { return (uint16_t)(((next_u32() & 1u) << 15) | (0x3000u + (next_u32() % 0x1800u))); }
static void *xmalloc(size_t n) { void *p = malloc(n ? n : 1); if (!p) abort(); return p; }
static uint16_t *bf16_buf(int64_t n) {
    uint16_t *p = xmalloc((size_t)n * sizeof(uint16_t));
    for (int64_t i = 0; i < n; ++i) p[i] = rand_bf16();
    return p;
}
#define CHECK(cond) do { if (!(cond)) { fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); return 1; } } while (0)

int main(void) {
    const int64_t M = 256, N = 384, K = 256;
    uint16_t *x = bf16_buf(M * K), *w = bf16_buf(N * K), *b = bf16_buf(N);
    for (int64_t r = 0; r < 128; ++r) for (int64_t c = 128; c < 256; ++c) x[r * K + c] = 0; /* a zero block */
    int8_t *qx = xmalloc(M * K), *qw = xmalloc(N * K);
    float *sx = xmalloc(sizeof(float) * (M / 128) * (K / 128)), *sw = xmalloc(sizeof(float) * (N / 128) * (K / 128));
    CHECK(oracle_quantize_block(x, M, K, qx, sx) == 0);
    CHECK(oracle_quantize_block(w, N, K, qw, sw) == 0);
    for (int64_t i = 0; i < M * K; ++i) CHECK(qx[i] >= -127 && qx[i] <= 127);
    CHECK(oracle_quantize_block(x, 100, K, qx, sx) != 0);              /* not a multiple of 128 */

    int32_t *p = xmalloc(sizeof(int32_t) * 128 * 256 * (K / 128));
    CHECK(oracle_kblock_partials(qx, qw, M, N, K, 128, 128, 128, 256, p) == 0);
    CHECK(oracle_kblock_partials(qx, qw, M, N, K, 200, 128, 0, 128, p) != 0);  /* window past M */

    int64_t rows[3] = {0, 129, 255};
    uint16_t *y = xmalloc(sizeof(uint16_t) * 3 * N);
    double *y64 = xmalloc(sizeof(double) * 3 * N);
    CHECK(oracle_linear_int8_rows(qx, sx, qw, sw, b, M, N, K, rows, 3, y, y64) == 0);
    uint16_t *yall = xmalloc(sizeof(uint16_t) * M * N);
    CHECK(oracle_linear_int8_rows(qx, sx, qw, sw, NULL, M, N, K, NULL, 0, yall, NULL) == 0);
    int64_t bad_row = M;
    CHECK(oracle_linear_int8_rows(qx, sx, qw, sw, NULL, M, N, K, &bad_row, 1, y, NULL) != 0);

    /* fallback on odd shapes, all three input types */
    const int64_t fm = 77, fk = 130, fn = 45;
    uint16_t *fx = bf16_buf(fm * fk), *fw = bf16_buf(fn * fk), *fy = xmalloc(sizeof(uint16_t) * fm * fn);
    float *fx32 = xmalloc(sizeof(float) * fm * fk);
    for (int64_t i = 0; i < fm * fk; ++i) fx32[i] = (float)((int)(next_u32() % 2001) - 1000) / 256.0f;
    CHECK(oracle_linear_bf16_rows(fx, 0, fw, b, fm, fn, fk, NULL, 0, fy) == 0);
    CHECK(oracle_linear_bf16_rows(fx, 1, fw, NULL, fm, fn, fk, NULL, 0, fy) == 0);
    CHECK(oracle_linear_bf16_rows(fx32, 2, fw, NULL, fm, fn, fk, NULL, 0, fy) == 0);
    CHECK(oracle_linear_bf16_rows(fx, 3, fw, NULL, fm, fn, fk, NULL, 0, fy) != 0);

    /* post-scale form */
    float *rsx = xmalloc(sizeof(float) * M), *rsw = xmalloc(sizeof(float) * N);
    CHECK(oracle_quantize_rows(x, M, K, qx, rsx) == 0);
    CHECK(oracle_quantize_rows(w, N, K, qw, rsw) == 0);
    CHECK(oracle_linear_postscale_rows(qx, rsx, qw, rsw, b, M, N, K, rows, 3, y) == 0);

    /* attention Q/K: ragged token count, padded rows */
    const int64_t B = 2, L = 200, H = 3, D = 64, ld = H * D + 16, nblk = (L + 127) / 128;
    uint16_t *qkx = bf16_buf(B * L * ld);
    int8_t *qq = xmalloc(B * H * L * D);
    float *qs = xmalloc(sizeof(float) * B * H * nblk);
    CHECK(oracle_quantize_qk(qkx, B, L, H, D, ld, qq, qs) == 0);
    CHECK(oracle_quantize_qk(qkx, B, L, H, D, H * D - 1, qq, qs) != 0);

    /* V in FP8 on the same padded rows; every code decoded and every bf16 pattern encoded */
    uint8_t *vq = xmalloc(B * H * L * D);
    CHECK(oracle_quantize_v_fp8(qkx, B, L, H, D, ld, vq, qs) == 0);
    CHECK(oracle_quantize_v_fp8(qkx, B, L, H, D, H * D - 1, vq, qs) != 0);
    for (int c = 0; c < 256; ++c) (void)oracle_e4m3_to_f64((uint8_t)c);
    for (int i = 0; i < 65536; ++i) {
        uint32_t u = (uint32_t)i << 16;
        float f;
        memcpy(&f, &u, 4);
        if (isfinite(f)) (void)oracle_f32_to_e4m3(f);
    }
    free(vq);

    /* split rotary embedding on the same padded rows */
    float *rc = xmalloc(sizeof(float) * L * (D / 2)), *rs = xmalloc(sizeof(float) * L * (D / 2));
    for (int64_t i = 0; i < L * (D / 2); ++i) {
        rc[i] = (float)((int)(next_u32() % 2001) - 1000) / 1000.0f;
        rs[i] = (float)((int)(next_u32() % 2001) - 1000) / 1000.0f;
    }
    uint16_t *ry = xmalloc(sizeof(uint16_t) * B * L * H * D);
    CHECK(oracle_rope(qkx, B, L, H, D, ld, rc, rs, ry) == 0);
    CHECK(oracle_rope(qkx, B, L, H, D - 1, ld, rc, rs, ry) != 0);      /* odd head dimension */
    CHECK(oracle_rope(qkx, B, L, H, D, H * D - 1, rc, rs, ry) != 0);

    /* gated residual update, out of place and in place */
    uint16_t *gh = bf16_buf(4 * 3 * 40), *go = bf16_buf(4 * 3 * 40), *gg = bf16_buf(4 * 40),
             *gy = xmalloc(sizeof(uint16_t) * 4 * 3 * 40);
    CHECK(oracle_gated_residual(gh, go, gg, 4, 3, 40, gy) == 0);
    CHECK(oracle_gated_residual(gh, go, gg, 4, 3, 40, gh) == 0);
    CHECK(oracle_gated_residual(gh, go, gg, 4, 0, 40, gy) != 0);
    free(gh); free(go); free(gg); free(gy);

    /* modulated RMS normalization, with its r */
    uint16_t *nsc = bf16_buf(2 * K), *nsh = bf16_buf(2 * K), *ny = xmalloc(sizeof(uint16_t) * M * K);
    float *nr = xmalloc(sizeof(float) * M);
    CHECK(oracle_rmsnorm_modulate(x, 2, M / 2, K, nsc, nsh, 1e-6, ny, nr) == 0);
    CHECK(oracle_rmsnorm_modulate(x, 2, M / 2, K, nsc, nsh, 1e-6, ny, NULL) == 0);
    /* modulated layer normalization, with and without its statistics */
    float *nst = xmalloc(sizeof(float) * 2 * M);
    CHECK(oracle_layernorm_modulate(x, 2, M / 2, K, nsc, nsh, 1e-6, ny, nst) == 0);
    CHECK(oracle_layernorm_modulate(x, 2, M / 2, K, nsc, nsh, 1e-6, ny, NULL) == 0);
    CHECK(oracle_layernorm_modulate(x, 2, M / 2, K, nsc, nsh, 0.0, ny, NULL) != 0);
    free(nst);

    /* GELU over every bf16 pattern (NaN/Inf included: defined output, no UB) */
    uint16_t *gin = xmalloc(sizeof(uint16_t) * 65536), *gout = xmalloc(sizeof(uint16_t) * 65536);
    for (int i = 0; i < 65536; ++i) gin[i] = (uint16_t)i;
    CHECK(oracle_gelu_bf16(gin, 65536, gout) == 0);

    /* guard and conversions */
    for (int dt = -1; dt <= 3; ++dt)
        for (int64_t mm = -128; mm <= 256; mm += 64) CHECK(oracle_route(dt, mm, 128, 256, 1) >= -1);
    for (int i = 0; i < 65536; ++i) (void)oracle_fp16_to_f64((uint16_t)i);
    const double edge[] = {0.0, -0.0, 1e-45, 3.4e38, -3.5e38, 1e300, -1e-300, 1.0 + 1.0 / 256};
    for (unsigned i = 0; i < sizeof edge / sizeof edge[0]; ++i) (void)oracle_f64_to_bf16(edge[i]);

    free(x); free(w); free(b); free(qx); free(qw); free(sx); free(sw); free(p); free(y); free(y64); free(yall);
    free(fx); free(fw); free(fy); free(fx32); free(rsx); free(rsw); free(qkx); free(qq); free(qs); free(gin); free(gout);
    free(rc); free(rs); free(ry); free(nsc); free(nsh); free(ny); free(nr);
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
