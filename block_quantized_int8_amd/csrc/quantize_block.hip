// Block-absmax INT8 quantization of a bf16 matrix, one workgroup per
// 128x128 block, for gfx950.
//
// Rule (TurboDiffusion news article, bjdmk.com.cn: 128x128 block-wise INT8
// for linear weights and, at the same granularity, activations; TurboT2VA
// paper, inference stack, W8A8 paragraph: scale = max-abs / 127):
//   a = max |x| over the block, s = fl32(a / 127),
//   q = rint(fl32(x / s)) ties-to-even, in [-127, 127]; a = 0 -> s = 0, q = 0.
//
// Memory-bound: one HBM read of the bf16 block (32 KiB) and one write of the
// int8 block (16 KiB) plus one fp32 scale.  Each of the 256 threads holds 64
// values (8 x 16-byte loads, all issued before any use) so the block is
// never re-read (nontemporal loads: x is not needed again, and keeping it
// out of the last-level cache leaves room there for the codes, which the
// GEMM reads next); the absmax is taken on the magnitude bits (for non-negative
// floats the bit order is the value order), reduced across the wavefront
// with lane shuffles and across the 4 wavefronts through LDS.
//
// Division and rounding: see quant_math.h.
#include "quant_math.h"
#include "w8a8_internal.h"

namespace w8a8 {
namespace {

constexpr int kThreads = 256;
constexpr int kChunksPerRow = kBlock * 2 / 16;                 // 16-byte chunks per block row: 16
constexpr int kRowsPerPass = kThreads / kChunksPerRow;         // 16
constexpr int kPasses = kBlock / kRowsPerPass;                 // 8

template <bool kScaled>
__device__ __forceinline__ void emit_codes(const u32x4 (&v)[kPasses], int8_t *dst, int64_t cols,
                                           float f, float ss, float r) {
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        *reinterpret_cast<u32x2 *>(dst + (int64_t)p * kRowsPerPass * cols) = code_chunk<kScaled>(v[p], f, ss, r);
    }
}

__global__ __launch_bounds__(kThreads) void quantize_block_kernel(const uint16_t *__restrict__ x,
                                                                  int64_t cols, int64_t col_blocks,
                                                                  int8_t *__restrict__ q,
                                                                  float *__restrict__ s) {
    __shared__ uint32_t red[kThreads / 64];
    const int64_t tile = blockIdx.x;
    const int64_t rb = tile / col_blocks, cb = tile - rb * col_blocks;
    const int t = threadIdx.x;
    const int chunk = t % kChunksPerRow, r0 = t / kChunksPerRow;
    const int64_t row = rb * kBlock + r0;
    const int64_t col = cb * kBlock + chunk * 8;

    const uint16_t *src = x + row * cols + col;
    u32x4 v[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
        v[p] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(src + (int64_t)p * kRowsPerPass * cols));

    // absmax on the 15 magnitude bits of each bf16, two lanes of 16 bits at once
    uint32_t mhi = 0, mlo = 0;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        const uint32_t w[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            mlo = max(mlo, w[i] & 0x7FFFu);
            mhi = max(mhi, (w[i] >> 16) & 0x7FFFu);
        }
    }
    uint32_t m = max(mlo, mhi);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    m = max(max(red[0], red[1]), max(red[2], red[3]));

    const float a = __uint_as_float(m << 16);
    const float sc = a / 127.0f;  // IEEE division, correctly rounded
    if (t == 0) s[tile] = sc;

    int8_t *dst = q + row * cols + col;
    if (m == 0) {
#pragma unroll
        for (int p = 0; p < kPasses; ++p)
            *reinterpret_cast<u32x2 *>(dst + (int64_t)p * kRowsPerPass * cols) = u32x2{0u, 0u};
        return;
    }
    if (sc < kTinyScale) {
        const float f = kPrescale, ss = sc * f, r = 1.0f / ss;
        emit_codes<true>(v, dst, cols, f, ss, r);
    } else {
        const float r = 1.0f / sc;
        emit_codes<false>(v, dst, cols, 1.0f, sc, r);
    }
}

}  // namespace

hipError_t launch_quantize_block(const uint16_t *x, int64_t rows, int64_t cols, int8_t *q, float *s,
                                 hipStream_t stream) {
    const int64_t col_blocks = cols / kBlock;
    const int64_t tiles = (rows / kBlock) * col_blocks;
    if (tiles <= 0) return hipSuccess;
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    quantize_block_kernel<<<dim3((unsigned)tiles), dim3(kThreads), 0, stream>>>(x, cols, col_blocks,
                                                                              q, s);
    return hipGetLastError();
}

}  // namespace w8a8
