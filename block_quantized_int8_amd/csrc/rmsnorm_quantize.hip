// Modulated RMS and layer normalization, alone and fused with the 128x128
// block INT8 quantization of their result, for gfx950.
//
// The producer in front of a transformer block's linears: normalization
// combined with timestep-dependent scale and shift (TurboT2VA paper,
// architecture-aware inference stack, fused-kernels paragraph, which fuses
// such memory-bound patterns); fused here with the activation quantization of
// the next linear (the block rule: TurboDiffusion news article, bjdmk.com.cn,
// 128x128 blocks for activations; TurboT2VA paper, W8A8 paragraph, scale =
// max-abs / 127).  For row i = b*L + l of x [B*L, K]:
//
//   r_i  = fl32( 1 / sqrt(sum_k x_ik^2 / K + eps) )    (fp64, rounded once)
//   y_ik = bf16( fl32(fl32(fl32(x_ik * r_i) * fl32(1 + scale[b,k])) + shift[b,k]) )
//
// every fl32 one IEEE fp32 operation (the library is built without
// floating-point contraction), the bf16 rounding to nearest even.  The sum of
// squares is taken in fp64 in this kernel's order (lane partials, then a
// butterfly); a different order can move it by a few fp64 ulps, which changes
// the fp32 r only when r lies within ~2^-50 of an fp32 rounding boundary.
//
// The layer form (the fused-kernels paragraph also replaces LayerNorm):
//   m_i = fl32(mean_k x_ik),  r_i = fl32( 1 / sqrt(var_k x_ik + eps) )  (fp64)
//   y_ik = bf16( fl32(fl32(fl32(fl32(x_ik - m_i) * r_i) * fl32(1 + scale[b,k])) + shift[b,k]) )
// with the variance taken over the deviations from the fp64 mean (two passes
// over the row in ln_rows, from registers for the common widths; the
// modulate kernels read (m, r) pairs).
//
// Kernels: rms_rows / ln_rows (one wavefront per row, 16-byte loads, fp64
// partial sums) write r [B*L] / (m, r) pairs; modulate_bf16 (one wavefront per
// row) writes y; modulate_quantize (one workgroup per 128x128 block, the block
// quantizer's structure) computes y in registers and emits its codes and
// scale, so the bf16 y never reaches HBM.  That pair reads x twice (the second
// time with nontemporal loads: it is x's last use) and writes one byte per
// element.  rms_band_quantize (RMS form, K a multiple of 256) reads x once:
// the workgroups of a 128-row band each hold a 256-column slice in
// registers and exchange fp64 row partials through the workspace (its own
// section below).  The layer form keeps the two-read pair: it would need two
// exchanges (the mean, then the deviations), which cost more than the
// second read saves.
#include <math.h>

#include <atomic>

#include "quant_math.h"
#include "w8a8_internal.h"

namespace w8a8 {
namespace {

constexpr int kRowWaves = 4;                        // rows (wavefronts) per workgroup
constexpr int kBlkThreads = 256;
constexpr int kChunksPerRow = kBlock * 2 / 16;      // 16-byte chunks per 128-column block row: 16
constexpr int kRowsPerPass = kBlkThreads / kChunksPerRow;  // 16
constexpr int kPasses = kBlock / kRowsPerPass;      // 8

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> one word of two bf16 (lo first), each rounded to nearest
// even: one packed conversion.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// kCenter: the layer normalization's (x - m) * r; else the RMS form x * r.
template <bool kCenter>
__device__ __forceinline__ float modulate(float x, float m, float r, float s, float h) {
    const float c = kCenter ? x - m : x;
    const float t = c * r;
    const float one_s = 1.0f + s;
    const float u = t * one_s;
    return u + h;
}

// Two packed bf16 (x, scale, shift words) -> two packed bf16 of y.
template <bool kCenter>
__device__ __forceinline__ uint32_t modulate_word(uint32_t xw, uint32_t sw, uint32_t hw, float m, float r) {
    const float y0 = modulate<kCenter>(lo_bf16(xw), m, r, lo_bf16(sw), lo_bf16(hw));
    const float y1 = modulate<kCenter>(hi_bf16(xw), m, r, hi_bf16(sw), hi_bf16(hw));
    return pack_bf16x2(y0, y1);
}

template <bool kCenter>
__device__ __forceinline__ u32x4 modulate_chunk(u32x4 x, u32x4 s, u32x4 h, float m, float r) {
    return u32x4{modulate_word<kCenter>(x.x, s.x, h.x, m, r), modulate_word<kCenter>(x.y, s.y, h.y, m, r),
                 modulate_word<kCenter>(x.z, s.z, h.z, m, r), modulate_word<kCenter>(x.w, s.w, h.w, m, r)};
}

// A row's statistics: RMS form r[row]; layer form (m, r) at stats[2 row].
template <bool kCenter>
__device__ __forceinline__ void row_stats(const float *__restrict__ st, int64_t row, float &m, float &r) {
    if (kCenter) {
        m = st[2 * row];
        r = st[2 * row + 1];
    } else {
        m = 0.0f;
        r = st[row];
    }
}

__device__ __forceinline__ double sq_chunk(u32x4 w) {
    double a = 0.0;
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const double l = (double)lo_bf16(v[i]), h = (double)hi_bf16(v[i]);
        a += l * l;
        a += h * h;
    }
    return a;
}

__global__ __launch_bounds__(64 * kRowWaves) void rms_rows_kernel(const uint16_t *__restrict__ x, int64_t rows,
                                                                  int64_t K, double eps, float *__restrict__ r) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowWaves + (threadIdx.x >> 6);
    if (row >= rows) return;  // whole wavefront leaves together
    const u32x4 *src = reinterpret_cast<const u32x4 *>(x + row * K);
    const int64_t chunks = K / 8;
    double acc = 0.0;
    int64_t c = lane;
    for (; c + 3 * 64 < chunks; c += 4 * 64) {  // four loads in flight per lane
        const u32x4 a = src[c], b = src[c + 64], d = src[c + 128], e = src[c + 192];
        acc += sq_chunk(a);
        acc += sq_chunk(b);
        acc += sq_chunk(d);
        acc += sq_chunk(e);
    }
    for (; c < chunks; c += 64) acc += sq_chunk(src[c]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0) r[row] = (float)(1.0 / sqrt(acc / (double)K + eps));
}

// Layer form: per row m = fl32(mean) and r = fl32(1 / sqrt(var + eps)), the
// mean and the variance (of the deviations from that mean) in fp64, two
// passes over the row (the second from cache).
__device__ __forceinline__ double sum_chunk(u32x4 w) {
    double a = 0.0;
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a += (double)lo_bf16(v[i]);
        a += (double)hi_bf16(v[i]);
    }
    return a;
}

__device__ __forceinline__ double dev_chunk(u32x4 w, double mu) {
    double a = 0.0;
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const double l = (double)lo_bf16(v[i]) - mu, h = (double)hi_bf16(v[i]) - mu;
        a += l * l;
        a += h * h;
    }
    return a;
}

__global__ __launch_bounds__(64 * kRowWaves) void ln_rows_kernel(const uint16_t *__restrict__ x, int64_t rows,
                                                                 int64_t K, double eps, float *__restrict__ st) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowWaves + (threadIdx.x >> 6);
    if (row >= rows) return;  // whole wavefront leaves together
    const u32x4 *src = reinterpret_cast<const u32x4 *>(x + row * K);
    const int64_t chunks = K / 8;
    double acc = 0.0;
    int64_t c = lane;
    for (; c + 3 * 64 < chunks; c += 4 * 64) {  // four loads in flight per lane
        const u32x4 a = src[c], b = src[c + 64], d = src[c + 128], e = src[c + 192];
        acc += sum_chunk(a);
        acc += sum_chunk(b);
        acc += sum_chunk(d);
        acc += sum_chunk(e);
    }
    for (; c < chunks; c += 64) acc += sum_chunk(src[c]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    const double mu = acc / (double)K;
    double var = 0.0;
    c = lane;
    for (; c + 3 * 64 < chunks; c += 4 * 64) {
        const u32x4 a = src[c], b = src[c + 64], d = src[c + 128], e = src[c + 192];
        var += dev_chunk(a, mu);
        var += dev_chunk(b, mu);
        var += dev_chunk(d, mu);
        var += dev_chunk(e, mu);
    }
    for (; c < chunks; c += 64) var += dev_chunk(src[c], mu);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) var += __shfl_xor(var, o, 64);
    if (lane == 0) {
        st[2 * row] = (float)mu;
        st[2 * row + 1] = (float)(1.0 / sqrt(var / (double)K + eps));
    }
}

// ln_rows for rows of kNc * 512 values (kNc 16-byte chunks per lane): the
// row stays in registers between the two passes, so x is read once.
template <int kNc>
__global__ __launch_bounds__(64 * kRowWaves) void ln_rows_reg_kernel(const uint16_t *__restrict__ x, int64_t rows,
                                                                     double eps, float *__restrict__ st) {
    constexpr int64_t K = kNc * 512;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowWaves + (threadIdx.x >> 6);
    if (row >= rows) return;  // whole wavefront leaves together
    const u32x4 *src = reinterpret_cast<const u32x4 *>(x + row * K);
    u32x4 v[kNc];
#pragma unroll
    for (int i = 0; i < kNc; ++i) v[i] = src[lane + 64 * i];
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < kNc; ++i) acc += sum_chunk(v[i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    const double mu = acc / (double)K;
    double var = 0.0;
#pragma unroll
    for (int i = 0; i < kNc; ++i) {
        asm volatile("" : "+v"(v[i]));  // convert again rather than keep 8 doubles per chunk live
        var += dev_chunk(v[i], mu);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) var += __shfl_xor(var, o, 64);
    if (lane == 0) {
        st[2 * row] = (float)mu;
        st[2 * row + 1] = (float)(1.0 / sqrt(var / (double)K + eps));
    }
}

// y for one row per wavefront.
template <bool kCenter>
__global__ __launch_bounds__(64 * kRowWaves) void modulate_bf16_kernel(const uint16_t *__restrict__ x,
                                                                       const float *__restrict__ r, int64_t rows,
                                                                       int64_t L, int64_t K,
                                                                       const uint16_t *__restrict__ scale,
                                                                       const uint16_t *__restrict__ shift,
                                                                       uint16_t *__restrict__ y) {
    const int lane = threadIdx.x & 63;
    // last rows first, as in modulate_quantize_kernel
    const int64_t row = rows - 1 - ((int64_t)blockIdx.x * kRowWaves + (threadIdx.x >> 6));
    if (row < 0) return;
    const int64_t b = row / L;
    float mm, rr;
    row_stats<kCenter>(r, row, mm, rr);
    const u32x4 *src = reinterpret_cast<const u32x4 *>(x + row * K);
    const u32x4 *sc = reinterpret_cast<const u32x4 *>(scale + b * K);
    const u32x4 *sh = reinterpret_cast<const u32x4 *>(shift + b * K);
    u32x4 *dst = reinterpret_cast<u32x4 *>(y + row * K);
    const int64_t chunks = K / 8;
    for (int64_t c = lane; c < chunks; c += 64) dst[c] = modulate_chunk<kCenter>(src[c], sc[c], sh[c], mm, rr);
}

// One workgroup per 128x128 block of y: each thread holds 64 values (8
// chunks of 8, rows r0 + 16p), computes them from x, its rows' r and their
// batch entries' scale and shift, then quantizes them as the block quantizer
// does (absmax on the magnitude bits, wavefront shuffles, LDS across the 4
// wavefronts, one correctly rounded division per element).
template <bool kCenter>
__global__ __launch_bounds__(kBlkThreads) void modulate_quantize_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ r, uint32_t L, int64_t K, int64_t col_blocks,
    const uint16_t *__restrict__ scale, const uint16_t *__restrict__ shift, int8_t *__restrict__ q,
    float *__restrict__ s) {
    __shared__ uint32_t red[kBlkThreads / 64];
    // last rows first: the row-norm pass has just streamed x through the
    // last-level cache, whose most recent lines are the last rows
    const int64_t tile = (int64_t)gridDim.x - 1 - blockIdx.x;
    const int64_t rb = tile / col_blocks, cb = tile - rb * col_blocks;
    const int t = threadIdx.x;
    const int chunk = t % kChunksPerRow, r0 = t / kChunksPerRow;
    const int64_t row0 = rb * kBlock + r0;
    const int64_t col = cb * kBlock + chunk * 8;

    u32x4 v[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
        v[p] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(x + (row0 + (int64_t)p * kRowsPerPass) * K + col));
    uint32_t m = 0;
    // rows < 2^31 (checked by the caller), so 32-bit division suffices
    const uint32_t b_first = (uint32_t)(rb * kBlock) / L, b_last = (uint32_t)(rb * kBlock + kBlock - 1) / L;
    if (b_first == b_last) {
        // the whole block belongs to one batch entry: one scale/shift chunk per thread
        const u32x4 sc = *reinterpret_cast<const u32x4 *>(scale + (int64_t)b_first * K + col);
        const u32x4 sh = *reinterpret_cast<const u32x4 *>(shift + (int64_t)b_first * K + col);
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
            float mm, rr;
            row_stats<kCenter>(r, row0 + (int64_t)p * kRowsPerPass, mm, rr);
            v[p] = modulate_chunk<kCenter>(v[p], sc, sh, mm, rr);
            m = max(m, chunk_absmax_bits(v[p]));
        }
    } else {
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
            const int64_t row = row0 + (int64_t)p * kRowsPerPass;
            const uint32_t b = (uint32_t)row / L;
            const u32x4 sc = *reinterpret_cast<const u32x4 *>(scale + (int64_t)b * K + col);
            const u32x4 sh = *reinterpret_cast<const u32x4 *>(shift + (int64_t)b * K + col);
            float mm, rr;
            row_stats<kCenter>(r, row, mm, rr);
            v[p] = modulate_chunk<kCenter>(v[p], sc, sh, mm, rr);
            m = max(m, chunk_absmax_bits(v[p]));
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    m = max(max(red[0], red[1]), max(red[2], red[3]));

    const float a = __uint_as_float(m << 16);
    const float sc = a / 127.0f;  // IEEE division, correctly rounded
    if (t == 0) s[tile] = sc;
    int8_t *dst = q + row0 * K + col;
    if (m == 0) {
#pragma unroll
        for (int p = 0; p < kPasses; ++p)
            *reinterpret_cast<u32x2 *>(dst + (int64_t)p * kRowsPerPass * K) = u32x2{0u, 0u};
        return;
    }
    if (sc < kTinyScale) {
        const float f = kPrescale, ss = sc * f, rcp = 1.0f / ss;
#pragma unroll
        for (int p = 0; p < kPasses; ++p)
            *reinterpret_cast<u32x2 *>(dst + (int64_t)p * kRowsPerPass * K) = code_chunk<true>(v[p], f, ss, rcp);
    } else {
        const float rcp = 1.0f / sc;
#pragma unroll
        for (int p = 0; p < kPasses; ++p)
            *reinterpret_cast<u32x2 *>(dst + (int64_t)p * kRowsPerPass * K) = code_chunk<false>(v[p], 1.0f, sc, rcp);
    }
}


// ---------------------------------------------------------------------------
// Single-read RMS form of the fused producer (K a multiple of 256).
//
// One workgroup per item (128-row band, 256-column part): P = K / 256 items
// per band, item = blockIdx.x, band = item / P.  The workgroup loads its
// 128 x 256 slice of x once into registers (16 chunks of 8 bf16 per
// thread), and
//   1. sums the squares of its slice per row in fp64 (per thread and row,
//      then the 16 chunk partials of a row in a fixed order through LDS) and
//      stores the 128 row partials at partials[band][part][row] with
//      device-coherent stores;
//   2. waits for its stores, then adds 1 to the band's arrival counter and
//      waits until the counter reaches P (all partials of the band visible);
//   3. sums the P partials of each row in part order (every workgroup of the
//      band does the same sum, so all see the same r), forms r, and
//      modulates and quantizes its slice from registers as
//      modulate_quantize_kernel does.
// So x is read once; the exchange costs 8 bytes per row per part written and
// P times that read (1/32 of x's bytes at P = 16).  The row sums are fp64 sums
// of exact squares in this kernel's order (see the file header for the
// effect of order).
//
// Progress: a workgroup waits only for the other items of its band, which
// are the P consecutive workgroup ids around it.  Workgroups are dispatched
// in id order, and an item of an older band never waits on a younger one, so
// every older band completes and frees its slots; a band whose items are not
// all resident can only be the youngest one dispatched, and it becomes whole
// once the slots ahead of it free up.  The wait is still bounded: after
// kSpinLimit polls the workgroup sets the workspace's error word and goes on
// (its codes are then wrong), so no schedule can hang the device.
//
// Workspace (16-byte aligned): [0, 256) control (word 0: error word, 0 when
// every wait completed), then one 256-byte line per band holding its
// arrival counter (counters never share a cache line), then the fp64
// partials [bands][P][128].  zero_counters_kernel clears the control word
// and the counters before every launch (no memset, so the pair can be
// captured in a graph and replayed).

constexpr int kBandBlocks = kBandCols / kBlock;      // 128-column blocks per item: 2
constexpr int kSpinLimit = 1 << 20;                  // polls before a wait gives up (~1 s)
constexpr size_t kCtrlLine = kBandCtrlLine;          // bytes per counter line

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// (1 + scale) and shift of 8 consecutive columns, as fp32.
struct ColMod {
    float one_s[8], h[8];
};

__device__ __forceinline__ ColMod load_colmod(const uint16_t *scale, const uint16_t *shift) {
    const u32x4 sc = *reinterpret_cast<const u32x4 *>(scale);
    const u32x4 sh = *reinterpret_cast<const u32x4 *>(shift);
    const uint32_t a[4] = {sc.x, sc.y, sc.z, sc.w}, b[4] = {sh.x, sh.y, sh.z, sh.w};
    ColMod m;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m.one_s[2 * i] = 1.0f + lo_bf16(a[i]);
        m.one_s[2 * i + 1] = 1.0f + hi_bf16(a[i]);
        m.h[2 * i] = lo_bf16(b[i]);
        m.h[2 * i + 1] = hi_bf16(b[i]);
    }
    return m;
}

// y = bf16(((x * r) * (1 + s)) + h) for one chunk, each step one fp32 operation.
__device__ __forceinline__ u32x4 rms_modulate_chunk(u32x4 x, const ColMod &md, float r) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float y0 = lo_bf16(w[i]) * r * md.one_s[2 * i] + md.h[2 * i];
        const float y1 = hi_bf16(w[i]) * r * md.one_s[2 * i + 1] + md.h[2 * i + 1];
        o[i] = pack_bf16x2(y0, y1);
    }
    return u32x4{o[0], o[1], o[2], o[3]};
}

// Running max of the 15-bit magnitudes of a chunk (packed 16-bit max).
__device__ __forceinline__ u16x2 absmax_acc(u16x2 acc, u32x4 w) {
    const u16x2 a = __builtin_bit_cast(u16x2, w.x & 0x7FFF7FFFu), b = __builtin_bit_cast(u16x2, w.y & 0x7FFF7FFFu);
    const u16x2 c = __builtin_bit_cast(u16x2, w.z & 0x7FFF7FFFu), d = __builtin_bit_cast(u16x2, w.w & 0x7FFF7FFFu);
    return __builtin_elementwise_max(__builtin_elementwise_max(acc, __builtin_elementwise_max(a, b)),
                                     __builtin_elementwise_max(c, d));
}

// Sum of squares of a chunk: each square of a bf16 value is exact in fp64,
// so the fused multiply-add rounds exactly as the separate product and sum.
__device__ __forceinline__ double sq_sum_chunk(u32x4 w) {
    double a = 0.0;
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const double l = (double)lo_bf16(v[i]), h = (double)hi_bf16(v[i]);
        a = __builtin_fma(l, l, a);
        a = __builtin_fma(h, h, a);
    }
    return a;
}

// Device-coherent loads through a buffer resource (cache policy sc1): plain
// loads to the compiler, so many are in flight at once; offsets past
// `bytes` read 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

__global__ void zero_counters_kernel(uint32_t *ctrl, int64_t lines) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < lines) ctrl[i * (kCtrlLine / 4)] = 0u;
}

__global__ __launch_bounds__(kBlkThreads) __attribute__((amdgpu_waves_per_eu(3, 3))) void rms_band_quantize_kernel(
    const uint16_t *__restrict__ x, int64_t K, uint32_t P, uint32_t L, double eps,
    const uint16_t *__restrict__ scale, const uint16_t *__restrict__ shift, uint32_t *ctrl, double *partials,
    int8_t *__restrict__ q, float *__restrict__ s) {
    __shared__ double red64[kBlock][kChunksPerRow + 1];
    __shared__ float s_r[kBlock];
    __shared__ uint32_t red[kBlkThreads / 64][kBandBlocks];
    const int t = threadIdx.x;
    const int64_t item = blockIdx.x;
    const int64_t band = item / P, part = item - band * P;
    const int chunk = t % kChunksPerRow, r0 = t / kChunksPerRow;
    const int64_t row0 = band * kBlock + r0;
    const int64_t col0 = part * kBandCols + chunk * 8;
    // uniform base of the slice + one 32-bit per-thread offset (r0 K + 8 chunk < 2^31: K < 2^26)
    const uint32_t voff = (uint32_t)r0 * (uint32_t)K + (uint32_t)chunk * 8u;
    const uint16_t *xb = x + band * kBlock * K + part * kBandCols;

    u32x4 v[kBandBlocks][kPasses];
#pragma unroll
    for (int j = 0; j < kBandBlocks; ++j)
#pragma unroll
        for (int p = 0; p < kPasses; ++p)
            v[j][p] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(xb + (int64_t)kRowsPerPass * p * K + j * kBlock + voff));

    // 1. row partials of this slice
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        double a = 0.0;
#pragma unroll
        for (int j = 0; j < kBandBlocks; ++j) {
            a += sq_sum_chunk(v[j][p]);
            asm volatile("" : "+v"(v[j][p]));  // the later pass unpacks again instead of keeping floats live
        }
        red64[r0 + kRowsPerPass * p][chunk] = a;
    }
    __syncthreads();
    double *band_partials = partials + band * (int64_t)P * kBlock;
    if (t < kBlock) {
        double a = 0.0;
#pragma unroll
        for (int c = 0; c < kChunksPerRow; ++c) a += red64[t][c];
        __hip_atomic_store(band_partials + part * kBlock + t, a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // 2. arrive once the stores are complete; wait for the band
    uint32_t *cnt = ctrl + (1 + band) * (kCtrlLine / 4);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t == 0) {
        __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int spins = 0;
        while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < P) {
            if (++spins > kSpinLimit) {
                __hip_atomic_store(ctrl, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    __syncthreads();

    // 3. r of the band's rows, then modulate + quantize from registers
    if (t < kBlock) {
        const __amdgpu_buffer_rsrc_t rs = coherent_rsrc(band_partials, P * (uint32_t)kBlock * 8u);
        double sum = 0.0;
#pragma unroll 8
        for (uint32_t pp = 0; pp < P; ++pp)
            sum += __builtin_bit_cast(double,
                                      __builtin_amdgcn_raw_buffer_load_b64(rs, (pp * kBlock + (uint32_t)t) * 8u, 0, 16));
        s_r[t] = (float)(1.0 / sqrt(sum / (double)K + eps));
    }
    __syncthreads();

    const uint32_t b_first = (uint32_t)(band * kBlock) / L, b_last = (uint32_t)(band * kBlock + kBlock - 1) / L;
#pragma unroll
    for (int j = 0; j < kBandBlocks; ++j) {
        u16x2 mx = u16x2{0, 0};
        if (b_first == b_last) {
            const ColMod md = load_colmod(scale + (int64_t)b_first * K + col0 + j * kBlock,
                                          shift + (int64_t)b_first * K + col0 + j * kBlock);
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                v[j][p] = rms_modulate_chunk(v[j][p], md, s_r[r0 + kRowsPerPass * p]);
                mx = absmax_acc(mx, v[j][p]);
                __builtin_amdgcn_sched_barrier(0);  // one row at a time keeps the register count down
            }
        } else {
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                const uint32_t b = (uint32_t)(row0 + kRowsPerPass * p) / L;
                const ColMod md =
                    load_colmod(scale + (int64_t)b * K + col0 + j * kBlock, shift + (int64_t)b * K + col0 + j * kBlock);
                v[j][p] = rms_modulate_chunk(v[j][p], md, s_r[r0 + kRowsPerPass * p]);
                mx = absmax_acc(mx, v[j][p]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        uint32_t m = max((uint32_t)mx.x, (uint32_t)mx.y);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
        if ((t & 63) == 0) red[t >> 6][j] = m;
    }
    __syncthreads();
    const int64_t col_blocks = K / kBlock;
#pragma unroll
    for (int j = 0; j < kBandBlocks; ++j) {
        const uint32_t m = max(max(red[0][j], red[1][j]), max(red[2][j], red[3][j]));
        const float a = __uint_as_float(m << 16);
        const float sc = a / 127.0f;  // IEEE division, correctly rounded
        if (t == 0) s[band * col_blocks + part * kBandBlocks + j] = sc;
        int8_t *qb = q + band * kBlock * K + part * kBandCols + j * kBlock;
        if (m == 0) {
#pragma unroll
            for (int p = 0; p < kPasses; ++p)
                *reinterpret_cast<u32x2 *>(qb + (int64_t)p * kRowsPerPass * K + voff) = u32x2{0u, 0u};
        } else if (sc < kTinyScale) {
            const float f = kPrescale, ss = sc * f, rcp = 1.0f / ss;
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                *reinterpret_cast<u32x2 *>(qb + (int64_t)p * kRowsPerPass * K + voff) = code_chunk<true>(v[j][p], f, ss, rcp);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            const float rcp = 1.0f / sc;
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                *reinterpret_cast<u32x2 *>(qb + (int64_t)p * kRowsPerPass * K + voff) =
                    code_chunk<false>(v[j][p], 1.0f, sc, rcp);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
}

}  // namespace

hipError_t launch_rms_rows(const uint16_t *x, int64_t rows, int64_t K, double eps, float *r, hipStream_t stream) {
    const int64_t groups = (rows + kRowWaves - 1) / kRowWaves;
    if (groups <= 0) return hipSuccess;
    if (groups > 0x7FFFFFFF) return hipErrorInvalidValue;
    rms_rows_kernel<<<dim3((unsigned)groups), dim3(64 * kRowWaves), 0, stream>>>(x, rows, K, eps, r);
    return hipGetLastError();
}

hipError_t launch_ln_rows(const uint16_t *x, int64_t rows, int64_t K, double eps, float *stats, hipStream_t stream) {
    const int64_t groups = (rows + kRowWaves - 1) / kRowWaves;
    if (groups <= 0) return hipSuccess;
    if (groups > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)groups), block(64 * kRowWaves);
    switch (K) {  // rows that fit in registers: one read of x
    case 1024: ln_rows_reg_kernel<2><<<grid, block, 0, stream>>>(x, rows, eps, stats); break;
    case 2048: ln_rows_reg_kernel<4><<<grid, block, 0, stream>>>(x, rows, eps, stats); break;
    case 3072: ln_rows_reg_kernel<6><<<grid, block, 0, stream>>>(x, rows, eps, stats); break;
    case 4096: ln_rows_reg_kernel<8><<<grid, block, 0, stream>>>(x, rows, eps, stats); break;
    case 5120: ln_rows_reg_kernel<10><<<grid, block, 0, stream>>>(x, rows, eps, stats); break;
    case 6144: ln_rows_reg_kernel<12><<<grid, block, 0, stream>>>(x, rows, eps, stats); break;
    case 8192: ln_rows_reg_kernel<16><<<grid, block, 0, stream>>>(x, rows, eps, stats); break;
    default: ln_rows_kernel<<<grid, block, 0, stream>>>(x, rows, K, eps, stats); break;
    }
    return hipGetLastError();
}

hipError_t launch_modulate_bf16(const uint16_t *x, const float *stats, bool center, int64_t rows, int64_t L,
                                int64_t K, const uint16_t *scale, const uint16_t *shift, uint16_t *y,
                                hipStream_t stream) {
    const int64_t groups = (rows + kRowWaves - 1) / kRowWaves;
    if (groups <= 0) return hipSuccess;
    if (groups > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (center)
        modulate_bf16_kernel<true><<<dim3((unsigned)groups), dim3(64 * kRowWaves), 0, stream>>>(x, stats, rows, L, K,
                                                                                                scale, shift, y);
    else
        modulate_bf16_kernel<false><<<dim3((unsigned)groups), dim3(64 * kRowWaves), 0, stream>>>(x, stats, rows, L,
                                                                                                 K, scale, shift, y);
    return hipGetLastError();
}

hipError_t launch_modulate_quantize(const uint16_t *x, const float *stats, bool center, int64_t rows, int64_t L,
                                    int64_t K, const uint16_t *scale, const uint16_t *shift, int8_t *q, float *s,
                                    hipStream_t stream) {
    const int64_t col_blocks = K / kBlock;
    const int64_t tiles = (rows / kBlock) * col_blocks;
    if (tiles <= 0) return hipSuccess;
    if (tiles > 0x7FFFFFFF || rows > 0x7FFFFFFF || L > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (center)
        modulate_quantize_kernel<true><<<dim3((unsigned)tiles), dim3(kBlkThreads), 0, stream>>>(
            x, stats, (uint32_t)L, K, col_blocks, scale, shift, q, s);
    else
        modulate_quantize_kernel<false><<<dim3((unsigned)tiles), dim3(kBlkThreads), 0, stream>>>(
            x, stats, (uint32_t)L, K, col_blocks, scale, shift, q, s);
    return hipGetLastError();
}


// The band's K / 256 workgroups wait for one another, so a band can only
// complete once all of them are resident; a band larger than the device holds
// at once would end only through the bounded wait (error word set, codes
// wrong).  The single-read form is therefore taken only when a band needs at
// most half of the device's resident capacity for this kernel (its occupancy
// per CU times the CU count, queried once per device), which leaves room for
// other work on the device or a CU mask.  A failed query answers false.
bool rms_band_fits(int64_t K) {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> capacity[kMaxDevices];  // 0: not queried yet, -1: none
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return false;
    }
    int cap = capacity[dev].load(std::memory_order_relaxed);
    if (cap == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, rms_band_quantize_kernel, kBlkThreads, 0) !=
                hipSuccess) {
            (void)hipGetLastError();
            return false;
        }
        cap = cus > 0 && per_cu > 0 ? cus * per_cu : -1;
        capacity[dev].store(cap, std::memory_order_relaxed);
    }
    return K > 0 && K / kBandCols <= cap / 2;
}

hipError_t launch_rms_band_quantize(const uint16_t *x, int64_t rows, int64_t L, int64_t K, double eps,
                                    const uint16_t *scale, const uint16_t *shift, void *workspace, int8_t *q,
                                    float *s, hipStream_t stream) {
    const int64_t bands = rows / kBlock, P = K / kBandCols;
    const int64_t items = bands * P;
    if (items <= 0) return hipSuccess;
    if (items > 0x7FFFFFFF || rows > 0x7FFFFFFF || L > 0x7FFFFFFF || K >= (int64_t)1 << 26) return hipErrorInvalidValue;
    uint32_t *ctrl = static_cast<uint32_t *>(workspace);
    double *partials = reinterpret_cast<double *>(static_cast<char *>(workspace) + kCtrlLine * (size_t)(1 + bands));
    const int64_t lines = 1 + bands;
    zero_counters_kernel<<<dim3((unsigned)((lines + 255) / 256)), dim3(256), 0, stream>>>(ctrl, lines);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    rms_band_quantize_kernel<<<dim3((unsigned)items), dim3(kBlkThreads), 0, stream>>>(
        x, K, (uint32_t)P, (uint32_t)L, eps, scale, shift, ctrl, partials, q, s);
    return hipGetLastError();
}

}  // namespace w8a8
