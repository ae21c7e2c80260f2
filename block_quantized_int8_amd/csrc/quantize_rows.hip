// Row-wise INT8 quantization with an epsilon floor, for the post-scale W8A8
// form (TurboT2VA paper, architecture-aware inference stack, W8A8 paragraph:
// per-row activation scales and per-output-channel weight scales, both
// max(max-abs, 1e-4) / 127, INT8 codes):
//   s_i = fl32(max(max_k |x_ik|, eps) / 127),  q_ik = rint(fl32(x_ik / s_i)).
//
// One wavefront per row, four rows per workgroup; no LDS and no barrier.
// Rows of up to 16384 elements stay in registers: each lane holds kChunks
// chunks of 8 bf16 (the smallest power of two that covers the row, all
// loaded back to back, nontemporal: X is not needed again), so X is read
// once; longer rows take a second pass over the row for the codes.  The absmax is taken on the magnitude bits and
// reduced with lane shuffles.  Division and rounding: quant_math.h; the
// floor keeps s >= 2^-21, far above the range that needs a prescale, and
// the scheme was checked against correctly rounded division for every bf16
// x with the floor's scale as well as for every unfloored one.  |x/s| never
// exceeds 127, so no clamp is active.
#include "quant_math.h"
#include "w8a8_internal.h"

namespace w8a8 {
namespace {

constexpr int kWavesPerGroup = 4;
constexpr int kMaxChunks = 32;  // per lane: 32 x 8 bf16 -> rows up to 16384 in registers

__device__ __forceinline__ float row_scale(uint32_t m) {
    for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
    const float a = fmaxf(__uint_as_float(m << 16), 1e-4f);
    return a / 127.0f;  // IEEE division, correctly rounded
}

// kChunks > 0: the row in registers, kChunks chunks per lane (kFull: the row
// is exactly kChunks * 64 chunks, no bounds test); kChunks == 0: two passes.
template <int kChunks, bool kFull>
__global__ __launch_bounds__(64 * kWavesPerGroup) void quantize_rows_kernel(const uint16_t *__restrict__ x,
                                                                             int64_t rows, int64_t cols,
                                                                             int8_t *__restrict__ q,
                                                                             float *__restrict__ s) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
    if (row >= rows) return;  // whole wavefront leaves together
    const int64_t chunks = cols / 8;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(x + row * cols);
    u32x2 *dst = reinterpret_cast<u32x2 *>(q + row * cols);

    if constexpr (kChunks > 0) {
        u32x4 v[kChunks];
        uint32_t m = 0;
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            const int64_t ch = (int64_t)c * 64 + lane;
            v[c] = (kFull || ch < chunks) ? __builtin_nontemporal_load(&src[ch]) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int c = 0; c < kChunks; ++c) m = max(m, chunk_absmax_bits(v[c]));
        const float sc = row_scale(m), r = 1.0f / sc;
        if (lane == 0) s[row] = sc;
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            const int64_t ch = (int64_t)c * 64 + lane;
            if (kFull || ch < chunks) dst[ch] = code_chunk<false>(v[c], 1.0f, sc, r);
        }
    } else {
        uint32_t m = 0;
        for (int64_t ch = lane; ch < chunks; ch += 64) m = max(m, chunk_absmax_bits(src[ch]));
        const float sc = row_scale(m), r = 1.0f / sc;
        if (lane == 0) s[row] = sc;
        for (int64_t ch = lane; ch < chunks; ch += 64) dst[ch] = code_chunk<false>(src[ch], 1.0f, sc, r);
    }
}

template <int kChunks>
void launch_rows(unsigned groups, const uint16_t *x, int64_t rows, int64_t cols, int8_t *q, float *s,
                 hipStream_t stream) {
    if (cols / 8 == (int64_t)kChunks * 64)
        quantize_rows_kernel<kChunks, true><<<groups, 64 * kWavesPerGroup, 0, stream>>>(x, rows, cols, q, s);
    else
        quantize_rows_kernel<kChunks, false><<<groups, 64 * kWavesPerGroup, 0, stream>>>(x, rows, cols, q, s);
}

}  // namespace

hipError_t launch_quantize_rows(const uint16_t *x, int64_t rows, int64_t cols, int8_t *q, float *s,
                                hipStream_t stream) {
    const int64_t groups = (rows + kWavesPerGroup - 1) / kWavesPerGroup;
    if (groups <= 0) return hipSuccess;
    if (groups > 0x7FFFFFFF) return hipErrorInvalidValue;
    const unsigned g = (unsigned)groups;
    const int64_t per_lane = (cols / 8 + 63) / 64;  // chunks per lane
    if (per_lane <= 1)
        launch_rows<1>(g, x, rows, cols, q, s, stream);
    else if (per_lane <= 2)
        launch_rows<2>(g, x, rows, cols, q, s, stream);
    else if (per_lane <= 4)
        launch_rows<4>(g, x, rows, cols, q, s, stream);
    else if (per_lane <= 8)
        launch_rows<8>(g, x, rows, cols, q, s, stream);
    else if (per_lane <= 16)
        launch_rows<16>(g, x, rows, cols, q, s, stream);
    else if (per_lane <= kMaxChunks)
        launch_rows<kMaxChunks>(g, x, rows, cols, q, s, stream);
    else
        quantize_rows_kernel<0, false><<<g, 64 * kWavesPerGroup, 0, stream>>>(x, rows, cols, q, s);
    return hipGetLastError();
}

}  // namespace w8a8
