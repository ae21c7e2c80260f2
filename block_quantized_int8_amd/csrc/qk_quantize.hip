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

}  // namespace

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
