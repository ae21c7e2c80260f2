// INT8 block quantization of attention queries or keys, rearranged from
// sequence-major to head-major on the way, for gfx950.
//
// The TurboT2VA paper's sparse-attention adapter (architecture-aware
// inference stack, sparse-attention paragraph) turns the sequence-major
// query, key and value tensors into the layout of the sparse kernel and
// quantizes query and key to INT8.  Here: input element (b, l, h, d) is
// x[(b*L + l)*ld + h*D + d] (for example a column slice of a fused Q/K/V
// projection's output, ld being its row stride); each (b, h) is cut into
// blocks of 128 consecutive tokens (the last one may be shorter) and every
// block gets the library's block rule over its tokens x D head dims:
// a = max |x|, s = fl32(a/127), q = rint(fl32(x/s)) ties to even (a = 0 ->
// s = 0, q = 0).  Codes go to q[((b*H + h)*L + l)*D + d] (head-major
// [B, H, L, D]), scales to s[(b*H + h)*ceil(L/128) + block].
//
// One 256-thread workgroup per block, launched token block by token block
// (all heads of a block, then the next block): each token row of D bf16 values is
// D/8 16-byte chunks, so a pass covers 256/(D/8) rows and the 128 rows take
// 128*D/2048 passes, every load issued before the first use (nontemporal:
// the projection output is not re-read, so it need not displace anything
// in the last-level cache).  Rows past L
// are neither read nor written.  Memory-bound, like the 128x128 quantizer.
//
// Also here: the split-halves rotary embedding that precedes this
// quantization in attention, alone (bf16 out) and fused into the quantizer.
#include "quant_math.h"
#include "w8a8_internal.h"

namespace w8a8 {
namespace {

constexpr int kThreads = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void quantize_qk_kernel(const uint16_t *__restrict__ x, int64_t L,
                                                              int64_t H, int64_t ld, int64_t nblk,
                                                              int8_t *__restrict__ q, float *__restrict__ s) {
    constexpr int kChunksPerRow = D / 8;
    constexpr int kRowsPerPass = kThreads / kChunksPerRow;
    constexpr int kPasses = kBlock / kRowsPerPass;
    __shared__ uint32_t red[kThreads / 64];
    // consecutive workgroups take the heads of one token block, so that
    // together they read whole rows of x
    const int64_t bblk = blockIdx.x / H, h = blockIdx.x - bblk * H;
    const int64_t b = bblk / nblk, blk = bblk - b * nblk;
    const int64_t bh = b * H + h, task = bh * nblk + blk;
    const int t = threadIdx.x;
    const int chunk = t % kChunksPerRow, r0 = t / kChunksPerRow;
    const int64_t l0 = blk * kBlock + r0;

    const uint16_t *src = x + (b * L + l0) * ld + h * D + chunk * 8;
    u32x4 v[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
        v[p] = l0 + p * kRowsPerPass < L
                   ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + (int64_t)p * kRowsPerPass * ld))
                   : u32x4{0u, 0u, 0u, 0u};

    uint32_t m = 0;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) m = max(m, chunk_absmax_bits(v[p]));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    m = __builtin_amdgcn_readfirstlane(max(max(red[0], red[1]), max(red[2], red[3])));  // uniform

    const float sc = __uint_as_float(m << 16) / 127.0f;  // IEEE division, correctly rounded
    if (t == 0) s[task] = sc;
    // an all-zero block (every value +-0) gets codes 0 from divisor 1
    const bool scaled = m != 0 && sc < kTinyScale;
    const float f = scaled ? kPrescale : 1.0f;
    const float ss = m == 0 ? 1.0f : sc * f;
    const float r = 1.0f / ss;
    int8_t *dst = q + (bh * L + l0) * D + chunk * 8;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        if (l0 + p * kRowsPerPass < L)
            *reinterpret_cast<u32x2 *>(dst + (int64_t)p * kRowsPerPass * D) =
                scaled ? code_chunk<true>(v[p], f, ss, r) : code_chunk<false>(v[p], 1.0f, ss, r);
    }
}

// ----------------------------------------------------------------------------
// Split-halves rotary embedding (TurboT2VA paper, architecture-aware inference
// stack, fused-kernels paragraph: split rotary embeddings): element d < D/2 of
// a head pairs with d + D/2 and both turn by the token's angle, cos and sin
// from fp32 tables [L, D/2] shared by every batch entry and head:
//   y(d)       = bf16(fl32(fl32(x(d) * c) - fl32(x(d + D/2) * s)))
//   y(d + D/2) = bf16(fl32(fl32(x(d + D/2) * c) + fl32(x(d) * s)))
// (the library is built without floating-point contraction, so each product
// and sum is one fp32 rounding; bf16 to nearest even).  A thread owns one
// 16-byte chunk of the lower half and the matching chunk of the upper half,
// so a pair never crosses lanes and each table chunk is loaded once per row.

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t bf16_bits(float v) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v);  // round to nearest even
}

// One word (two bf16) of each half, with the angles of those two pairs.
__device__ __forceinline__ void rope_word(uint32_t a, uint32_t b, float c0, float c1, float s0, float s1,
                                          uint32_t &ya, uint32_t &yb) {
    const float a0 = lo_bf16(a), a1 = hi_bf16(a), b0 = lo_bf16(b), b1 = hi_bf16(b);
    const float ya0 = a0 * c0 - b0 * s0, ya1 = a1 * c1 - b1 * s1;
    const float yb0 = b0 * c0 + a0 * s0, yb1 = b1 * c1 + a1 * s1;
    ya = bf16_bits(ya0) | (bf16_bits(ya1) << 16);
    yb = bf16_bits(yb0) | (bf16_bits(yb1) << 16);
}

// Eight pairs: chunk a of the lower half, chunk b of the upper half.
__device__ __forceinline__ void rope_chunk(u32x4 &a, u32x4 &b, f32x4 c01, f32x4 c23, f32x4 s01, f32x4 s23) {
    uint32_t ya[4], yb[4];
    rope_word(a.x, b.x, c01.x, c01.y, s01.x, s01.y, ya[0], yb[0]);
    rope_word(a.y, b.y, c01.z, c01.w, s01.z, s01.w, ya[1], yb[1]);
    rope_word(a.z, b.z, c23.x, c23.y, s23.x, s23.y, ya[2], yb[2]);
    rope_word(a.w, b.w, c23.z, c23.w, s23.z, s23.w, ya[3], yb[3]);
    a = u32x4{ya[0], ya[1], ya[2], ya[3]};
    b = u32x4{yb[0], yb[1], yb[2], yb[3]};
}

// Rotary embedding fused with the Q/K block quantizer: the same tasks and
// outputs as quantize_qk_kernel, the block rule applied to the rotated bf16
// values, which never reach HBM.  Thread t covers pair chunk t % (D/16) of
// rows t / (D/16) + k * 256/(D/16).  The tables are read with ordinary loads:
// every head of a token block reads the same rows, from cache.
template <int D>
__global__ __launch_bounds__(kThreads) void rope_quantize_qk_kernel(const uint16_t *__restrict__ x, int64_t L,
                                                                   int64_t H, int64_t ld, int64_t nblk,
                                                                   const float *__restrict__ cos_t,
                                                                   const float *__restrict__ sin_t,
                                                                   int8_t *__restrict__ q, float *__restrict__ s) {
    constexpr int kHalf = D / 2;
    constexpr int kPairChunks = D / 16;
    constexpr int kRowsPerPass = kThreads / kPairChunks;
    constexpr int kPasses = kBlock / kRowsPerPass;
    __shared__ uint32_t red[kThreads / 64];
    const int64_t bblk = blockIdx.x / H, h = blockIdx.x - bblk * H;
    const int64_t b = bblk / nblk, blk = bblk - b * nblk;
    const int64_t bh = b * H + h, task = bh * nblk + blk;
    const int t = threadIdx.x;
    const int pc = t % kPairChunks, r0 = t / kPairChunks;
    const int64_t l0 = blk * kBlock + r0;

    const uint16_t *src = x + (b * L + l0) * ld + h * D + pc * 8;
    const float *cs = cos_t + l0 * kHalf + pc * 8, *sn = sin_t + l0 * kHalf + pc * 8;
    u32x4 va[kPasses], vb[kPasses];
    f32x4 c[kPasses][2], sv[kPasses][2];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        const bool in = l0 + p * kRowsPerPass < L;
        const u32x4 *ra = reinterpret_cast<const u32x4 *>(src + (int64_t)p * kRowsPerPass * ld);
        const f32x4 *rc = reinterpret_cast<const f32x4 *>(cs + (int64_t)p * kRowsPerPass * kHalf);
        const f32x4 *rs = reinterpret_cast<const f32x4 *>(sn + (int64_t)p * kRowsPerPass * kHalf);
        va[p] = in ? __builtin_nontemporal_load(ra) : u32x4{0u, 0u, 0u, 0u};
        vb[p] = in ? __builtin_nontemporal_load(ra + kHalf / 8) : u32x4{0u, 0u, 0u, 0u};
        c[p][0] = in ? rc[0] : f32x4{0.f, 0.f, 0.f, 0.f};
        c[p][1] = in ? rc[1] : f32x4{0.f, 0.f, 0.f, 0.f};
        sv[p][0] = in ? rs[0] : f32x4{0.f, 0.f, 0.f, 0.f};
        sv[p][1] = in ? rs[1] : f32x4{0.f, 0.f, 0.f, 0.f};
    }

    uint32_t m = 0;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        rope_chunk(va[p], vb[p], c[p][0], c[p][1], sv[p][0], sv[p][1]);
        m = max(m, max(chunk_absmax_bits(va[p]), chunk_absmax_bits(vb[p])));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    m = __builtin_amdgcn_readfirstlane(max(max(red[0], red[1]), max(red[2], red[3])));  // uniform

    const float sc = __uint_as_float(m << 16) / 127.0f;  // IEEE division, correctly rounded
    if (t == 0) s[task] = sc;
    const bool scaled = m != 0 && sc < kTinyScale;
    const float f = scaled ? kPrescale : 1.0f;
    const float ss = m == 0 ? 1.0f : sc * f;
    const float r = 1.0f / ss;
    int8_t *dst = q + (bh * L + l0) * D + pc * 8;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        if (l0 + p * kRowsPerPass < L) {
            int8_t *row = dst + (int64_t)p * kRowsPerPass * D;
            *reinterpret_cast<u32x2 *>(row) =
                scaled ? code_chunk<true>(va[p], f, ss, r) : code_chunk<false>(va[p], 1.0f, ss, r);
            *reinterpret_cast<u32x2 *>(row + kHalf) =
                scaled ? code_chunk<true>(vb[p], f, ss, r) : code_chunk<false>(vb[p], 1.0f, ss, r);
        }
    }
}

// The rotary embedding alone: bf16 y [B*L, H*D] (contiguous, sequence-major)
// from x rows of stride ld.  Thread g owns pair chunk g % (D/16) of head
// (g / (D/16)) % H of row g / (H*D/16).
template <int D>
__global__ __launch_bounds__(kThreads) void rope_bf16_kernel(const uint16_t *__restrict__ x, int64_t L, int64_t H,
                                                            int64_t ld, int64_t items,
                                                            const float *__restrict__ cos_t,
                                                            const float *__restrict__ sin_t,
                                                            uint16_t *__restrict__ y) {
    constexpr int kHalf = D / 2;
    constexpr int kPairChunks = D / 16;
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (g >= items) return;
    const int64_t hp = g / kPairChunks;
    const int pc = (int)(g - hp * kPairChunks);
    const int64_t row = hp / H, h = hp - row * H;
    const int64_t l = row % L;
    const u32x4 *ra = reinterpret_cast<const u32x4 *>(x + row * ld + h * D + pc * 8);
    const f32x4 *rc = reinterpret_cast<const f32x4 *>(cos_t + l * kHalf + pc * 8);
    const f32x4 *rs = reinterpret_cast<const f32x4 *>(sin_t + l * kHalf + pc * 8);
    u32x4 a = __builtin_nontemporal_load(ra), b = __builtin_nontemporal_load(ra + kHalf / 8);
    rope_chunk(a, b, rc[0], rc[1], rs[0], rs[1]);
    u32x4 *out = reinterpret_cast<u32x4 *>(y + row * H * D + h * D + pc * 8);
    out[0] = a;
    out[kHalf / 8] = b;
}

}  // namespace

hipError_t launch_rope_quantize_qk(const uint16_t *x, int64_t B, int64_t L, int64_t H, int64_t D, int64_t ld,
                                   const float *cos_t, const float *sin_t, int8_t *q, float *s,
                                   hipStream_t stream) {
    const int64_t nblk = (L + kBlock - 1) / kBlock;
    const int64_t tasks = B * H * nblk;
    if (tasks <= 0) return hipSuccess;
    if (tasks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)tasks), block(kThreads);
    if (D == 64)
        rope_quantize_qk_kernel<64><<<grid, block, 0, stream>>>(x, L, H, ld, nblk, cos_t, sin_t, q, s);
    else if (D == 128)
        rope_quantize_qk_kernel<128><<<grid, block, 0, stream>>>(x, L, H, ld, nblk, cos_t, sin_t, q, s);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_rope_bf16(const uint16_t *x, int64_t B, int64_t L, int64_t H, int64_t D, int64_t ld,
                            const float *cos_t, const float *sin_t, uint16_t *y, hipStream_t stream) {
    const int64_t items = B * L * H * (D / 16);
    if (items <= 0) return hipSuccess;
    const int64_t blocks = (items + kThreads - 1) / kThreads;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks), block(kThreads);
    if (D == 64)
        rope_bf16_kernel<64><<<grid, block, 0, stream>>>(x, L, H, ld, items, cos_t, sin_t, y);
    else if (D == 128)
        rope_bf16_kernel<128><<<grid, block, 0, stream>>>(x, L, H, ld, items, cos_t, sin_t, y);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_quantize_qk(const uint16_t *x, int64_t B, int64_t L, int64_t H, int64_t D, int64_t ld,
                              int8_t *q, float *s, hipStream_t stream) {
    const int64_t nblk = (L + kBlock - 1) / kBlock;
    const int64_t tasks = B * H * nblk;
    if (tasks <= 0) return hipSuccess;
    if (tasks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)tasks), block(kThreads);
    if (D == 64)
        quantize_qk_kernel<64><<<grid, block, 0, stream>>>(x, L, H, ld, nblk, q, s);
    else if (D == 128)
        quantize_qk_kernel<128><<<grid, block, 0, stream>>>(x, L, H, ld, nblk, q, s);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace w8a8
