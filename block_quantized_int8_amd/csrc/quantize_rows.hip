// Row-wise INT8 quantization with an epsilon floor, for the post-scale W8A8
// form (TurboT2VA paper, architecture-aware inference stack, W8A8 paragraph:
// per-row activation scales and per-output-channel weight scales, both
// max(max-abs, 1e-4) / 127, INT8 codes):
//   s_i = fl32(max(max_k |x_ik|, eps) / 127),  q_ik = rint(fl32(x_ik / s_i)).
//
// One wavefront per row, four rows per workgroup; no LDS and no barrier.
// Rows of up to 8192 elements stay in registers (each lane holds up to 16
// chunks of 8 bf16, loaded back to back), so X is read once; longer rows take
// a second pass over the row for the codes.  The absmax is taken on the
// magnitude bits and reduced with lane shuffles.  Division and rounding use
// the same exact scheme as the block quantizer (per-row reciprocal, one FMA
// correction, ties-to-even by adding 1.5*2^23): the floor keeps s >= 2^-21,
// and the scheme was checked against correctly rounded division for every
// bf16 x with the floor's scale as well as for every unfloored one.  |x/s|
// never exceeds 127, so no clamp is active.
#include "w8a8_internal.h"

namespace w8a8 {
namespace {

constexpr int kWavesPerGroup = 4;
constexpr int kMaxChunks = 16;  // per lane: 16 x 8 bf16 -> rows up to 8192 in registers
constexpr float kRoundMagic = 12582912.0f;  // 1.5 * 2^23

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t code_byte(float x, float s, float r) {
    const float q0 = x * r;
    const float e = __builtin_fmaf(-q0, s, x);
    const float q1 = __builtin_fmaf(e, r, q0);
    return __float_as_uint(q1 + kRoundMagic) & 0xFFu;
}

__device__ __forceinline__ u32x2 code_chunk(const u32x4 v, float s, float r) {
    u32x2 out;
    out.x = code_byte(__uint_as_float(v.x << 16), s, r) | (code_byte(__uint_as_float(v.x & 0xFFFF0000u), s, r) << 8) |
            (code_byte(__uint_as_float(v.y << 16), s, r) << 16) |
            (code_byte(__uint_as_float(v.y & 0xFFFF0000u), s, r) << 24);
    out.y = code_byte(__uint_as_float(v.z << 16), s, r) | (code_byte(__uint_as_float(v.z & 0xFFFF0000u), s, r) << 8) |
            (code_byte(__uint_as_float(v.w << 16), s, r) << 16) |
            (code_byte(__uint_as_float(v.w & 0xFFFF0000u), s, r) << 24);
    return out;
}

__device__ __forceinline__ uint32_t mag_max(const u32x4 v) {
    uint32_t m = max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu);
    m = max(m, max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu));
    m = max(m, max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu));
    return max(m, max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu));
}

__device__ __forceinline__ float row_scale(uint32_t m) {
    for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
    const float a = fmaxf(__uint_as_float(m << 16), 1e-4f);
    return a / 127.0f;  // IEEE division, correctly rounded
}

template <bool kInRegisters>
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

    if constexpr (kInRegisters) {
        u32x4 v[kMaxChunks];
        uint32_t m = 0;
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) {
            const int64_t ch = (int64_t)c * 64 + lane;
            v[c] = ch < chunks ? src[ch] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) m = max(m, mag_max(v[c]));
        const float sc = row_scale(m), r = 1.0f / sc;
        if (lane == 0) s[row] = sc;
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) {
            const int64_t ch = (int64_t)c * 64 + lane;
            if (ch < chunks) dst[ch] = code_chunk(v[c], sc, r);
        }
    } else {
        uint32_t m = 0;
        for (int64_t ch = lane; ch < chunks; ch += 64) m = max(m, mag_max(src[ch]));
        const float sc = row_scale(m), r = 1.0f / sc;
        if (lane == 0) s[row] = sc;
        for (int64_t ch = lane; ch < chunks; ch += 64) dst[ch] = code_chunk(src[ch], sc, r);
    }
}

}  // namespace

hipError_t launch_quantize_rows(const uint16_t *x, int64_t rows, int64_t cols, int8_t *q, float *s,
                                hipStream_t stream) {
    const int64_t groups = (rows + kWavesPerGroup - 1) / kWavesPerGroup;
    if (groups <= 0) return hipSuccess;
    if (groups > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (cols / 8 <= (int64_t)kMaxChunks * 64)
        quantize_rows_kernel<true><<<dim3((unsigned)groups), dim3(64 * kWavesPerGroup), 0, stream>>>(x, rows, cols, q, s);
    else
        quantize_rows_kernel<false><<<dim3((unsigned)groups), dim3(64 * kWavesPerGroup), 0, stream>>>(x, rows, cols, q, s);
    return hipGetLastError();
}

}  // namespace w8a8
