// INT8 block quantization of attention queries or keys, rearranged from
// sequence-major to head-major on the way, for gfx950.
//
// Source: TurboT2VA paper, architecture-aware inference stack, sparse-attention
// paragraph (the attention's Q and K enter its kernel as INT8, in that
// kernel's layout rather than token-major).  Here: input element (b, l, h, d) is
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
#include "w8a8.h"
#include "w8a8_internal.h"

namespace w8a8 {
namespace {

constexpr int kThreads = 256;
constexpr int kXcds = 8;  // accelerator complex dies of gfx950, each with its own L2

// ---- FP8 values (the same blocks and layout, codes in FP8 E4M3)
//
// The sparse attention takes V in FP8 beside the INT8 Q and K (TurboT2VA
// paper, sparse-attention paragraph).  Per block s = fl32(a / 448) and
// code = E4M3(fl32(x / s)), the OCP format (bias 7, largest finite 448),
// nearest with ties to even: v_cvt_pk_fp8_f32 rounds an fp32 value that way.
// The quotient comes from quant_math.h's corrected reciprocal product
// (checked on the CPU for every pair of bf16 values 0 <= x <= a with
// s = fl32(a / 448), prescaled below 2^-60: it is not always the correctly
// rounded fp32 quotient, but its E4M3 code always equals that quotient's).
// A block's max-abs element can give a quotient a hair above 448; it is
// clamped to 448, which is also where E4M3 rounding takes anything below 464.
constexpr float kFp8Max = 448.0f;

__device__ __forceinline__ float quotient(float x, float ss, float r) {
    const float q0 = x * r;
    const float e = __builtin_fmaf(-q0, ss, x);
    return __builtin_fmaf(e, r, q0);
}

// Four E4M3 codes from two words of packed bf16 (elements 0-3, little endian).
template <bool kScaled>
__device__ __forceinline__ uint32_t fp8_word(uint32_t lo, uint32_t hi, float f, float ss, float r) {
    float v[4] = {__uint_as_float(lo << 16), __uint_as_float(lo & 0xFFFF0000u), __uint_as_float(hi << 16),
                  __uint_as_float(hi & 0xFFFF0000u)};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (kScaled) v[i] *= f;
        // the corrected product turns x = -0 into +0; E4M3 keeps the sign of a zero quotient
        v[i] = __builtin_copysignf(__builtin_fminf(__builtin_fmaxf(quotient(v[i], ss, r), -kFp8Max), kFp8Max), v[i]);
    }
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w, true);
}

template <bool kScaled>
__device__ __forceinline__ u32x2 fp8_chunk(u32x4 w, float f, float ss, float r) {
    return u32x2{fp8_word<kScaled>(w.x, w.y, f, ss, r), fp8_word<kScaled>(w.z, w.w, f, ss, r)};
}

// INT8 codes (the Q/K rule) or E4M3 codes (V) of one chunk.
template <bool kFp8, bool kScaled>
__device__ __forceinline__ u32x2 block_codes(u32x4 w, float f, float ss, float r) {
    if constexpr (kFp8)
        return fp8_chunk<kScaled>(w, f, ss, r);
    else
        return code_chunk<kScaled>(w, f, ss, r);
}

template <int D, bool kFp8>
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

    const float sc = __uint_as_float(m << 16) / (kFp8 ? kFp8Max : 127.0f);  // IEEE division, correctly rounded
    if (t == 0) s[task] = sc;
    // an all-zero block (every value +-0) gets codes 0 from divisor 1 (INT8),
    // or is written as zeros (E4M3 would keep the sign of a -0)
    const bool scaled = m != 0 && sc < kTinyScale;
    const float f = scaled ? kPrescale : 1.0f;
    const float ss = m == 0 ? 1.0f : sc * f;
    const float r = 1.0f / ss;
    int8_t *dst = q + (bh * L + l0) * D + chunk * 8;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        if (l0 + p * kRowsPerPass < L)
            *reinterpret_cast<u32x2 *>(dst + (int64_t)p * kRowsPerPass * D) =
                (kFp8 && m == 0) ? u32x2{0u, 0u}
                : scaled         ? block_codes<kFp8, true>(v[p], f, ss, r)
                                 : block_codes<kFp8, false>(v[p], 1.0f, ss, r);
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
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> one word of two bf16 (round to nearest even), lo first.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// One word (two bf16) of each half, with the angles of those two pairs.
__device__ __forceinline__ void rope_word(uint32_t a, uint32_t b, float c0, float c1, float s0, float s1,
                                          uint32_t &ya, uint32_t &yb) {
    const float a0 = lo_bf16(a), a1 = hi_bf16(a), b0 = lo_bf16(b), b1 = hi_bf16(b);
    const float ya0 = a0 * c0 - b0 * s0, ya1 = a1 * c1 - b1 * s1;
    const float yb0 = b0 * c0 + a0 * s0, yb1 = b1 * c1 + a1 * s1;
    ya = pack_bf16(ya0, ya1);
    yb = pack_bf16(yb0, yb1);
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

// Rotary embedding fused with the Q/K block quantizer: the outputs of
// quantize_qk_kernel, the block rule applied to the rotated bf16 values,
// which never reach HBM.
//
// A workgroup takes one token block and four heads, one wavefront per
// (token block, head): the wave holds the head's 128 x D block in registers
// (a lane owns a 16-byte chunk of the lower half and the matching chunk of
// the upper half of D/16 ... rows), so the max-abs reduction is wave-local.
// The block's cos and sin rows (128 x D/2 fp32 each, 64 KiB at D = 128) are
// copied once into LDS by direct buffer-to-LDS loads and shared by the four
// heads.  All loads go through buffer descriptors spanning the block: rows
// past L read as zero and their code stores are dropped by the range check,
// so the ragged last block needs no per-row tests (its LDS rows past L are
// cleared so that stale LDS contents never meet those zeros).  Workgroups
// are dealt to the 8 XCDs in turn (workgroup i runs on XCD i % 8); all head
// groups of a token block go to one XCD, whose L2 then fetches that block's
// table rows once.
constexpr int kRopeWaves = 4;
constexpr int kRopeThreads = kRopeWaves * 64;
constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit dwords
constexpr int kNontemporal = 2;         // cache-policy operand: the projection output is not re-read

typedef __attribute__((address_space(3))) void *lds_ptr_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const void *origin, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(origin), (short)0, (int)bytes, kRsrcFlags);
}

template <int D>
struct RopeGeo {
    static constexpr int kHalf = D / 2;
    static constexpr int kLanesPerRow = D / 16;              // lanes per token row
    static constexpr int kRowsPerPass = 64 / kLanesPerRow;   // rows per wave instruction
    static constexpr int kPasses = kBlock / kRowsPerPass;    // 16 (D = 128) or 8 (D = 64)
    static constexpr int kTableBytes = kBlock * kHalf * 4;   // one of cos, sin for a block
    static constexpr int kDmaPerWave = kTableBytes / 1024 / kRopeWaves;
};

// Codes of the wave's block, pass by pass (kScaled: the 2^64 prescale).
template <int D, bool kScaled>
__device__ __forceinline__ void rope_emit(const u32x4 (&va)[RopeGeo<D>::kPasses],
                                          const u32x4 (&vb)[RopeGeo<D>::kPasses], __amdgpu_buffer_rsrc_t out,
                                          int qoff, float f, float ss, float r) {
    using G = RopeGeo<D>;
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
        __builtin_amdgcn_raw_buffer_store_b64(code_chunk<kScaled>(va[p], f, ss, r), out, qoff,
                                              p * G::kRowsPerPass * D, 0);
        __builtin_amdgcn_raw_buffer_store_b64(code_chunk<kScaled>(vb[p], f, ss, r), out, qoff + G::kHalf,
                                              p * G::kRowsPerPass * D, 0);
        __builtin_amdgcn_sched_barrier(0);  // one pass at a time: few live temporaries
    }
}

// Launch requirement (checked by the caller): (128 * ld) * 2 bytes < 2^31.
template <int D>
__global__ __launch_bounds__(kRopeThreads) void rope_quantize_qk_kernel(
    const uint16_t *__restrict__ x, int64_t L, int64_t H, int64_t ld, int64_t nblk, int64_t token_blocks,
    int64_t head_groups, const float *__restrict__ cos_t, const float *__restrict__ sin_t, int8_t *__restrict__ q,
    float *__restrict__ s) {
    using G = RopeGeo<D>;
    __shared__ f32x4 tab[2 * G::kTableBytes / 16];  // cos rows, then sin rows
    const int64_t xcd = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
    const int64_t hg = j % head_groups, bblk = (j / head_groups) * kXcds + xcd;
    if (bblk >= token_blocks) return;  // uniform over the workgroup
    const int64_t b = bblk / nblk, blk = bblk - b * nblk;
    const int64_t row0 = blk * kBlock;
    const int rows = (int)min((int64_t)kBlock, L - row0);
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);

    // the block's table rows -> LDS, 1 KiB per wave instruction, lane-linear
    {
        const __amdgpu_buffer_rsrc_t rc = span_rsrc(cos_t + row0 * G::kHalf, (int64_t)rows * G::kHalf * 4);
        const __amdgpu_buffer_rsrc_t rs = span_rsrc(sin_t + row0 * G::kHalf, (int64_t)rows * G::kHalf * 4);
        char *base = reinterpret_cast<char *>(tab);
#pragma unroll
        for (int i = 0; i < G::kDmaPerWave; ++i) {
            const int ci = wave + kRopeWaves * i;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (lds_ptr_t)(base + ci * 1024), 16, lane * 16, ci * 1024, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(base + G::kTableBytes + ci * 1024), 16,
                                                     lane * 16, ci * 1024, 0, 0);
        }
        if (rows < kBlock) {  // clear the rows past L (the copy above skips them)
            for (int i = rows * G::kHalf / 4 + t; i < kBlock * G::kHalf / 4; i += kRopeThreads) {
                tab[i] = f32x4{0.f, 0.f, 0.f, 0.f};
                tab[G::kTableBytes / 16 + i] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }

    // this wave's head: all of its block's chunks loaded before the barrier
    const int64_t h = hg * kRopeWaves + wave;
    const bool live = h < H;
    const int r_in = lane / G::kLanesPerRow, pc = lane % G::kLanesPerRow;
    const __amdgpu_buffer_rsrc_t xr =
        live ? span_rsrc(x + (b * L + row0) * ld, ((int64_t)(rows - 1) * ld + H * D) * 2) : span_rsrc(x, 0);
    const int xoff = (r_in * (int)ld + pc * 8) * 2;
    u32x4 va[G::kPasses], vb[G::kPasses];
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
        const int so = (int)(((int64_t)p * G::kRowsPerPass * ld + (live ? h : 0) * D) * 2);
        va[p] = __builtin_amdgcn_raw_buffer_load_b128(xr, xoff, so, kNontemporal);
        vb[p] = __builtin_amdgcn_raw_buffer_load_b128(xr, xoff + G::kHalf * 2, so, kNontemporal);
    }
    __syncthreads();  // the table is in LDS
    if (!live) return;

    const f32x4 *tc = tab + (r_in * G::kHalf + pc * 8) / 4;
    const f32x4 *ts = tc + G::kTableBytes / 16;
    uint32_t m = 0;
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
        const int o = p * G::kRowsPerPass * G::kHalf / 4;
        rope_chunk(va[p], vb[p], tc[o], tc[o + 1], ts[o], ts[o + 1]);
        asm volatile("" : "+v"(va[p]), "+v"(vb[p]));  // keep the block packed as bf16, 8 words a lane-chunk
        m = max(m, max(chunk_absmax_bits(va[p]), chunk_absmax_bits(vb[p])));
        if (p & 1) __builtin_amdgcn_sched_barrier(0);  // table reads two passes at a time
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
    m = __builtin_amdgcn_readfirstlane(m);  // equal in every lane: make it scalar

    const float sc = __uint_as_float(m << 16) / 127.0f;  // IEEE division, correctly rounded
    const int64_t bh = b * H + h;
    if (lane == 0) s[bh * nblk + blk] = sc;
    // an all-zero block (every value +-0) gets codes 0 from divisor 1
    const bool scaled = m != 0 && sc < kTinyScale;
    const float f = scaled ? kPrescale : 1.0f;
    const float ss = m == 0 ? 1.0f : sc * f;
    const __amdgpu_buffer_rsrc_t out = span_rsrc(q + (bh * L + row0) * D, (int64_t)rows * D);
    const int qoff = r_in * D + pc * 8;
    if (__builtin_expect(scaled, 0))
        rope_emit<D, true>(va, vb, out, qoff, f, ss, 1.0f / ss);
    else
        rope_emit<D, false>(va, vb, out, qoff, 1.0f, ss, 1.0f / ss);
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
    const int64_t token_blocks = B * nblk;
    if (token_blocks <= 0 || H <= 0) return hipSuccess;
    if (ld > W8A8_ROPE_MAX_LD) return hipErrorInvalidValue;
    // token blocks rounded up to a multiple of the XCD count, times the head groups
    const int64_t head_groups = (H + kRopeWaves - 1) / kRopeWaves;
    const int64_t groups = (token_blocks + kXcds - 1) / kXcds;
    if (groups > 0x7FFFFFFF / kXcds / head_groups) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(groups * kXcds * head_groups)), block(kRopeThreads);
    if (D == 64)
        rope_quantize_qk_kernel<64><<<grid, block, 0, stream>>>(x, L, H, ld, nblk, token_blocks, head_groups, cos_t,
                                                                sin_t, q, s);
    else if (D == 128)
        rope_quantize_qk_kernel<128><<<grid, block, 0, stream>>>(x, L, H, ld, nblk, token_blocks, head_groups,
                                                                 cos_t, sin_t, q, s);
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
        quantize_qk_kernel<64, false><<<grid, block, 0, stream>>>(x, L, H, ld, nblk, q, s);
    else if (D == 128)
        quantize_qk_kernel<128, false><<<grid, block, 0, stream>>>(x, L, H, ld, nblk, q, s);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_quantize_v_fp8(const uint16_t *x, int64_t B, int64_t L, int64_t H, int64_t D, int64_t ld,
                                 uint8_t *q, float *s, hipStream_t stream) {
    const int64_t nblk = (L + kBlock - 1) / kBlock;
    const int64_t tasks = B * H * nblk;
    if (tasks <= 0) return hipSuccess;
    if (tasks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)tasks), block(kThreads);
    int8_t *qb = reinterpret_cast<int8_t *>(q);
    if (D == 64)
        quantize_qk_kernel<64, true><<<grid, block, 0, stream>>>(x, L, H, ld, nblk, qb, s);
    else if (D == 128)
        quantize_qk_kernel<128, true><<<grid, block, 0, stream>>>(x, L, H, ld, nblk, qb, s);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace w8a8
