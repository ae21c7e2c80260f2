// Exact GELU on bf16 values, alone and fused with the 128x128 block INT8
// quantization of its result, for gfx950.
//
// GELU(x) = x * Phi(x), Phi the standard normal CDF (the erf-exact GELU of
// Hendrycks and Gimpel), evaluated to fp64 accuracy and rounded once to bf16
// (nearest, ties to even).  It is the producer between the two linears of an
// MLP; fusing it with the activation quantization of the second linear is the
// kind of producer/quantize fusion the TurboT2VA paper applies to its
// memory-bound elementwise work (architecture-aware inference stack, fused
// kernels paragraph) and avoids writing and re-reading the bf16 activation.
// The quantization rule is the block rule of the library (TurboDiffusion news
// article, bjdmk.com.cn, 128x128 blocks for activations; TurboT2VA paper,
// W8A8 paragraph, scale = max-abs / 127).
//
// The map bf16 -> bf16 has only 2^16 inputs, so each workgroup first builds
// the whole map as a 128 KiB table in LDS and every element then costs one
// LDS read.  Table entries by magnitude:
//   |x| < 2^-10        x/2 rounded to bf16 (the x^2/sqrt(2 pi) term is below
//                      half a bf16 ulp of x/2; ties exist only where x/2 is
//                      subnormal, where fp64 evaluation cannot see the term);
//   2^-10 <= |x| < 16  t = |x| Phi(-|x|) = |x| erfc(|x|/sqrt 2) / 2 in fp64,
//                      GELU(-|x|) = -t and GELU(|x|) = |x| - t;
//   |x| >= 16          GELU(x) = x for x > 0 (Phi(x) = 1 in fp64) and -0 for
//                      x < 0 (|GELU(x)| < 2^-150, below the bf16 subnormals).
// Inputs must be finite (an infinity or NaN maps to x or -0).
//
// The fused kernel gives each wavefront a whole 128x128 tile: every lane
// holds 256 values (32 x 16-byte loads, issued together), so the tile's
// absmax needs only lane shuffles and no workgroup barrier; the quantization
// itself (correctly rounded division via one reciprocal and Markstein's
// correction, ties-to-even via the 1.5*2^23 add) is the one of the plain
// quantizer and gives identical codes and scales for the same bf16 input.
#include <math.h>

#include "quant_math.h"
#include "w8a8_internal.h"

namespace w8a8 {
namespace {

// One workgroup per CU: the table fills 128 KiB of LDS.  The fused kernel
// keeps a whole tile per lane (128 VGPRs of data), so 3 waves per SIMD.
constexpr int kGeluThreads = 1024;
constexpr int kQuantThreads = 768;
constexpr int kQuantWaves = kQuantThreads / 64;
constexpr uint32_t kTableMagLo = 117u << 7;     // |x| = 2^-10
constexpr uint32_t kTableMagHi = 131u << 7;     // |x| = 16

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// fp64 -> bf16 bits, rounded to nearest even, for finite |v| < 2^128.
__device__ uint32_t bf16_from_f64(double v) {
    const uint32_t sign = signbit(v) ? 0x8000u : 0u;
    const double a = fabs(v);
    if (a == 0.0) return sign;
    if (a < 0x1p-126) return sign | (uint32_t)rint(a * 0x1p133);  // subnormal quantum 2^-133
    const int e = ilogb(a);
    const uint32_t n = (uint32_t)rint(ldexp(a, 7 - e));           // in [128, 256]
    return sign | ((uint32_t)(e + 127) << 7) + (n - 128u);        // n = 256 carries into the exponent
}

// bf16 bits of x/2 (x given as bf16 bits), rounded to nearest even.
__device__ __forceinline__ uint32_t half_bf16(uint32_t u) {
    const uint32_t b = __float_as_uint(__uint_as_float(u << 16) * 0.5f);  // exact in fp32
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Every thread of the workgroup fills its share of the 2^16-entry table.
__device__ void build_gelu_table(uint16_t *table) {
    for (uint32_t u = threadIdx.x; u < 0x8000u; u += blockDim.x) {
        uint32_t pos, neg;
        if (u < kTableMagLo) {
            pos = half_bf16(u);
            neg = half_bf16(u | 0x8000u);
        } else if (u < kTableMagHi) {
            const double x = (double)__uint_as_float(u << 16);
            const double t = 0.5 * x * erfc(x * 0.70710678118654752440);
            pos = bf16_from_f64(x - t);
            neg = bf16_from_f64(-t);
        } else {
            pos = u;
            neg = 0x8000u;
        }
        table[u] = (uint16_t)pos;
        table[u | 0x8000u] = (uint16_t)neg;
    }
}

__device__ __forceinline__ uint32_t gelu_word(uint32_t w, const uint16_t *table) {
    return (uint32_t)table[w & 0xFFFFu] | ((uint32_t)table[w >> 16] << 16);
}

__device__ __forceinline__ u32x4 gelu_chunk(u32x4 v, const uint16_t *table) {
    return u32x4{gelu_word(v.x, table), gelu_word(v.y, table), gelu_word(v.z, table),
                 gelu_word(v.w, table)};
}

// ----------------------------------------------------------------- GELU only

// y may equal x (in place): every element is read and written by one thread.
template <bool kVec>
__global__ __launch_bounds__(kGeluThreads) void gelu_bf16_kernel(const uint16_t *x, int64_t n, uint16_t *y) {
    __shared__ uint16_t table[1 << 16];
    build_gelu_table(table);
    __syncthreads();
    const int64_t gtid = (int64_t)blockIdx.x * kGeluThreads + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kGeluThreads;
    if (kVec) {
        constexpr int kUnroll = 4;
        const int64_t chunks = n / 8;
        const u32x4 *src = reinterpret_cast<const u32x4 *>(x);
        u32x4 *dst = reinterpret_cast<u32x4 *>(y);
        int64_t i = gtid;
        for (; i + (kUnroll - 1) * stride < chunks; i += kUnroll * stride) {
            u32x4 v[kUnroll];
#pragma unroll
            for (int j = 0; j < kUnroll; ++j) v[j] = src[i + j * stride];
#pragma unroll
            for (int j = 0; j < kUnroll; ++j) dst[i + j * stride] = gelu_chunk(v[j], table);
        }
        for (; i < chunks; i += stride) dst[i] = gelu_chunk(src[i], table);
        const int64_t tail = chunks * 8 + gtid;
        if (tail < n) y[tail] = table[x[tail]];
    } else {
        for (int64_t i = gtid; i < n; i += stride) y[i] = table[x[i]];
    }
}

// ------------------------------------------------------- GELU + quantization

constexpr int kTileLoads = 32;  // 16-byte chunks per lane: 128 rows x 16 chunks / 64 lanes

// Buffer descriptors span one tile (rows 128i.., columns 128j..) so that the
// per-lane offset is 32-bit and each row group's offset is a scalar.
constexpr int kRsrcFlags = 0x00020000;
// cache-policy operand of the buffer loads: nontemporal (the input is read
// once; kept out of the last-level cache, it leaves room there for the codes
// that the next GEMM reads; 10% faster after a cold cache)
constexpr int kNontemporal = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void *origin, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(origin), (short)0, (int)bytes, kRsrcFlags);
}

__device__ __forceinline__ void load_tile(u32x4 (&v)[kTileLoads], __amdgpu_buffer_rsrc_t in, int voff,
                                          int64_t cols) {
#pragma unroll
    for (int p = 0; p < kTileLoads; ++p)
        v[p] = __builtin_amdgcn_raw_buffer_load_b128(in, voff * 2, (int)(p * 4 * cols * 2), kNontemporal);
}

// Emit the tile's codes with a rolling prefetch: as soon as chunk p's codes
// are stored its registers load chunk p of the wave's next tile, so the next
// tile's reads overlap this tile's quantization.  `scaled` (wave-uniform)
// selects the 2^64 prescale used for scales below 2^-60.
__device__ __forceinline__ void emit_tile_prefetch(u32x4 (&v)[kTileLoads], __amdgpu_buffer_rsrc_t out,
                                                   int voff, int64_t cols, bool scaled, float f, float ss,
                                                   float r, __amdgpu_buffer_rsrc_t next) {
#pragma unroll
    for (int p = 0; p < kTileLoads; ++p) {
        u32x4 w = v[p];
        asm volatile("" : "+v"(w));  // unpack here, chunk by chunk
        const u32x2 c = __builtin_expect(scaled, 0) ? code_chunk<true>(w, f, ss, r) : code_chunk<false>(w, 1.0f, ss, r);
        __builtin_amdgcn_raw_buffer_store_b64(c, out, voff, (int)(p * 4 * cols), 0);
        v[p] = __builtin_amdgcn_raw_buffer_load_b128(next, voff * 2, (int)(p * 4 * cols * 2), kNontemporal);
        __builtin_amdgcn_sched_barrier(0);  // keep the loads behind their chunk's stores
    }
}

// Launch requirement (checked by the caller): 128 * cols * 2 bytes < 2^31.
// Waves own tiles wave, wave + W, wave + 2W, ... (W = waves in the grid).
__global__ __launch_bounds__(kQuantThreads) void gelu_quantize_kernel(const uint16_t *__restrict__ yin,
                                                                     int64_t cols, int64_t col_blocks,
                                                                     int64_t tiles, int8_t *__restrict__ q,
                                                                     float *__restrict__ s) {
    __shared__ uint16_t table[1 << 16];
    build_gelu_table(table);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int r_in = lane >> 4;         // row within each group of 4 rows
    const int c_in = (lane & 15) * 8;   // first of this lane's 8 columns
    const int voff = r_in * (int)cols + c_in;          // elements from the tile origin
    const int64_t span = 127 * cols + kBlock;          // elements from the origin to the tile's end
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar tile index
    const int64_t step = (int64_t)gridDim.x * kQuantWaves;
    auto origin_of = [&](int64_t t) {
        const int64_t rb = t / col_blocks;
        return rb * kBlock * cols + (t - rb * col_blocks) * kBlock;
    };
    // a tile past the end gets an empty descriptor: its loads read nothing and return 0
    auto in_rsrc = [&](int64_t t) {
        return t < tiles ? tile_rsrc(yin + origin_of(t), span * 2) : tile_rsrc(yin, 0);
    };
    int64_t tile = (int64_t)blockIdx.x * kQuantWaves + wave;
    u32x4 v[kTileLoads];
    load_tile(v, in_rsrc(tile), voff, cols);
    for (; tile < tiles; tile += step) {
        // table lookups two chunks at a time: the scheduler would otherwise
        // hoist all 256 address computations and run out of registers
        u16x2 m2 = {0, 0};
#pragma unroll
        for (int p = 0; p < kTileLoads; ++p) {
            v[p] = gelu_chunk(v[p], table);
            asm volatile("" : "+v"(v[p]));  // keep only the packed words live
            const uint32_t w[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
            if (p & 1) __builtin_amdgcn_sched_barrier(0);
        }
        uint32_t m = max((uint32_t)m2.x, (uint32_t)m2.y);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
        m = __builtin_amdgcn_readfirstlane(m);  // equal in every lane: make it scalar
        const float a = __uint_as_float(m << 16);
        const float sc = a / 127.0f;  // IEEE division, correctly rounded
        if (lane == 0) s[tile] = sc;
        // an all-zero tile (every value +-0) gets codes 0 from divisor 1
        const bool scaled = m != 0 && sc < kTinyScale;
        const float f = scaled ? kPrescale : 1.0f;
        const float ss = m == 0 ? 1.0f : sc * f;
        emit_tile_prefetch(v, tile_rsrc(q + origin_of(tile), span), voff, cols, scaled, f, ss, 1.0f / ss,
                           in_rsrc(tile + step));
    }
}

int cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}

}  // namespace

hipError_t launch_gelu_bf16(const uint16_t *x, int64_t n, uint16_t *y, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int cus = cu_count();
    if (cus <= 0) return hipErrorInvalidDevice;
    const int64_t need = (n + kGeluThreads * 8 - 1) / (kGeluThreads * 8);
    const unsigned grid = (unsigned)(need < cus ? need : cus);
    const bool vec = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15u) == 0;
    if (vec)
        gelu_bf16_kernel<true><<<grid, kGeluThreads, 0, stream>>>(x, n, y);
    else
        gelu_bf16_kernel<false><<<grid, kGeluThreads, 0, stream>>>(x, n, y);
    return hipGetLastError();
}

hipError_t launch_gelu_quantize_block(const uint16_t *y, int64_t rows, int64_t cols, int8_t *q,
                                      float *s, hipStream_t stream) {
    const int64_t col_blocks = cols / kBlock;
    const int64_t tiles = (rows / kBlock) * col_blocks;
    if (tiles <= 0) return hipSuccess;
    const int cus = cu_count();
    if (cus <= 0) return hipErrorInvalidDevice;
    const int64_t need = (tiles + kQuantWaves - 1) / kQuantWaves;
    const unsigned grid = (unsigned)(need < cus ? need : cus);
    gelu_quantize_kernel<<<grid, kQuantThreads, 0, stream>>>(y, cols, col_blocks, tiles, q, s);
    return hipGetLastError();
}

}  // namespace w8a8
