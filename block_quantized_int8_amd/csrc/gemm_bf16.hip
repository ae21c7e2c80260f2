// bf16 fallback linear on gfx950 matrix cores: the guard's "otherwise" path.
//
//   Y[m, n] = bf16( sum_k bf16(x[m, k]) * w[n, k] (+ bias[n]) ), fp32 sums,
//
// for any M, N, K >= 1, with the layer's bf16 weight (TurboT2VA paper,
// architecture-aware inference stack, guard paragraph: a call the INT8 path
// cannot take is computed in bf16 instead).  fp16 and fp32
// inputs are rounded to bf16 (nearest even) as they are loaded.
//
// One workgroup (4 wavefronts) per 128x128 output tile, 64-deep K steps
// staged through double-buffered LDS (128-byte rows, XOR-swizzled 16-byte
// chunks, as in the INT8 kernel).  v_mfma_f32_32x32x16_bf16 accumulates in
// fp32 across all of K.  Out-of-range rows and K positions are loaded as
// zeros; stores are predicated per element.  kVec selects 16-byte loads
// (bf16 input, K % 8 == 0, 16-byte aligned operands); otherwise elements are
// loaded one by one (per operand: the weight's loads are vectorized
// whenever K % 8 == 0 and it is 16-byte aligned).
//
// This general kernel serves the calls the faster two cannot.  bf16 input
// with K a multiple of 64, N a multiple of 128, 16-byte aligned operands and
// at least 256 output tiles of 256x256 (any M, e.g. a token count that is
// not a multiple of 128) goes to the 256x256-tile kernel of the INT8 path in
// its bf16 mode (launch_gemm_bf16_tiled); other bf16 problems with K a
// multiple of 64, N a multiple of 8 and aligned operands go to the
// pipelined 64x128-tile kernel below (gemm_bf16_pipe_kernel).
#include "w8a8_internal.h"

namespace w8a8 {
namespace {

constexpr int kTile = 128;
constexpr int kStepK = 64;   // bf16 elements per K step (128 bytes per row)
constexpr int kThreads = 256;
constexpr int kLdsTile = kTile * kStepK * 2;  // bytes per operand per stage

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);  // round to nearest even
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> one word of two bf16 (lo first), one packed conversion.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

template <int kDtype>
__device__ __forceinline__ uint16_t load_as_bf16(const void *p, int64_t idx) {
    if constexpr (kDtype == 0) {
        return static_cast<const uint16_t *>(p)[idx];
    } else if constexpr (kDtype == 1) {
        return f32_to_bf16_bits((float)static_cast<const _Float16 *>(p)[idx]);
    } else {
        return f32_to_bf16_bits(static_cast<const float *>(p)[idx]);
    }
}

// One 16-byte chunk (8 consecutive k) of row `row` starting at column k0,
// zero outside [0, rows) x [0, K).
template <int kDtype, bool kVec>
__device__ __forceinline__ u32x4 load_chunk(const void *base, int64_t row, int64_t rows, int64_t k0,
                                            int64_t K) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row >= rows || k0 >= K) return v;
    if constexpr (kVec) {
        return *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(base) + row * K + k0);
    } else {
        uint16_t e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = (k0 + i < K) ? load_as_bf16<kDtype>(base, row * K + k0 + i) : 0;
        v.x = e[0] | ((uint32_t)e[1] << 16);
        v.y = e[2] | ((uint32_t)e[3] << 16);
        v.z = e[4] | ((uint32_t)e[5] << 16);
        v.w = e[6] | ((uint32_t)e[7] << 16);
        return v;
    }
}

template <int kDtype, bool kVecX, bool kVecW>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(const void *__restrict__ x,
                                                             const uint16_t *__restrict__ w,
                                                             const uint16_t *__restrict__ bias,
                                                             uint16_t *__restrict__ y, int64_t M,
                                                             int64_t N, int64_t K, int tiles_n) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kLdsTile];
    const int t = blockIdx.x;
    const int mb = t / tiles_n, nb = t - mb * tiles_n;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;

    int crow[4], cch[4], l_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + i * kThreads;
        crow[i] = c >> 3;
        cch[i] = c & 7;
        l_off[i] = swz(crow[i], cch[i]);
    }
    const int64_t m_base = (int64_t)mb * kTile, n_base = (int64_t)nb * kTile;

    u32x4 rx[4], rw[4];
    auto load_tiles = [&](int64_t ks) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t k0 = ks * kStepK + cch[i] * 8;
            rx[i] = load_chunk<kDtype, kVecX>(x, m_base + crow[i], M, k0, K);
            rw[i] = load_chunk<0, kVecW>(w, n_base + crow[i], N, k0, K);
        }
    };
    auto store_tiles = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<u32x4 *>(&lds[buf][0][l_off[i]]) = rx[i];
            *reinterpret_cast<u32x4 *>(&lds[buf][1][l_off[i]]) = rw[i];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int64_t KS = (K + kStepK - 1) / kStepK;
    load_tiles(0);
    store_tiles(0);
    __syncthreads();

    const int frag_row = lane & 31, frag_half = lane >> 5;
    for (int64_t ks = 0; ks < KS; ++ks) {
        const int buf = (int)(ks & 1);
        if (ks + 1 < KS) load_tiles(ks + 1);
        bf16x8 fx[2][4], fw[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int row = wm * 64 + j * 32 + frag_row;
                fx[j][kk] = *reinterpret_cast<const bf16x8 *>(&lds[buf][0][swz(row, kk * 2 + frag_half)]);
            }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int row = wn * 64 + i * 32 + frag_row;
                fw[i][kk] = *reinterpret_cast<const bf16x8 *>(&lds[buf][1][swz(row, kk * 2 + frag_half)]);
            }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[i][kk], fx[j][kk], acc[i][j], 0, 0, 0);
        if (ks + 1 < KS) store_tiles(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t m = m_base + wm * 64 + j * 32 + frag_row;
            if (m >= M) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = n_base + wn * 64 + i * 32 + q * 8 + frag_half * 4;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (n + e < N) {
                        float v = acc[i][j][q * 4 + e];
                        if (bias) v += __uint_as_float((uint32_t)bias[n + e] << 16);
                        y[m * N + n + e] = f32_to_bf16_bits(v);
                    }
                }
            }
        }
}

// ---- pipelined kernel for bf16 problems too small for 256x256 tiles
//
// 64 (m) x 128 (n) output tile per workgroup of 4 wavefronts (32 x 64 each,
// two independent accumulator chains per wavefront), 64-deep K steps.  With
// few tiles per CU every K step is short, so load latency, not the matrix
// cores, sets the pace; operands therefore go global -> LDS directly
// (buffer_load_dwordx4 ... lds, range-checked: rows past M or N read as
// zeros) into a ring of kStages stages, kStages - 1 steps ahead of the MFMAs;
// the range check covers the scalar offset as well (checked on gfx950), so
// the row-group offset may sit there.
// LDS rows are 128 bytes with the INT8 kernel's chunk swizzle, so each MFMA
// fragment is one conflict-free 16-byte read.
constexpr int kPM = 64, kPN = 128;
constexpr int kPThreads = 256;
constexpr int kPRowBytes = 128;                            // 64 bf16 of K per LDS row
constexpr int kPStageBytes = (kPM + kPN) * kPRowBytes;     // 24 KiB
constexpr int kPXLoads = kPM / 8 / 4, kPWLoads = kPN / 8 / 4;  // 8-row DMA instructions per wave per step
constexpr int kPLoads = kPXLoads + kPWLoads;
constexpr int kPipeStages = 3;  // 72 KiB: two workgroups per CU (6 stages, one per CU, was slower)

__device__ __forceinline__ int pswz(int row, int chunk) { return chunk ^ (row & 7) ^ ((row >> 3) & 1); }

// s_waitcnt with only a vector-memory count (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt and lgkmcnt at their no-wait maxima)
template <int kVm>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(kVm >= 0 && kVm < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((kVm & 15) | (7 << 4) | (15 << 8) | ((kVm >> 4) << 14));
}

template <int kStages>
__global__ __launch_bounds__(kPThreads) void gemm_bf16_pipe_kernel(const uint16_t *__restrict__ x,
                                                                   const uint16_t *__restrict__ w,
                                                                   const uint16_t *__restrict__ bias,
                                                                   uint16_t *__restrict__ y, int64_t M, int64_t N,
                                                                   int64_t K, int tiles_n) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * kPStageBytes];
    typedef __attribute__((address_space(3))) void *lds_ptr_t;
    const int t = blockIdx.x;
    const int mb = t / tiles_n, nb = t - mb * tiles_n;
    const int64_t m0 = (int64_t)mb * kPM, n0 = (int64_t)nb * kPN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wm = wave & 1, wn = wave >> 1;
    const int64_t row_bytes = K * 2;
    const int KS = (int)(K / 64);

    // operand tiles as buffers: loads past the last row of X or W return zeros
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(x + m0 * K), (short)0, (int)(min((int64_t)kPM, M - m0) * row_bytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(w + n0 * K), (short)0, (int)(min((int64_t)kPN, N - n0) * row_bytes), 0x00020000);
    // one DMA instruction fills 8 rows (1 KiB, lane-linear in LDS); lane l
    // writes slot l%8 of row l/8, which holds global chunk pswz(row, l%8);
    // the slot pattern depends on bit 3 of the row, i.e. on the parity of
    // the 8-row group
    uint32_t voff[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
        voff[b] = (uint32_t)((lane >> 3) * row_bytes) + (uint32_t)(pswz((lane >> 3) + 8 * b, lane & 7) * 16);
    auto issue = [&](int step) {
        uint8_t *st = lds + (step % kStages) * kPStageBytes;
#pragma unroll
        for (int i = 0; i < kPXLoads; ++i) {
            const int g = wave * kPXLoads + i;  // 8-row group of X
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(st + g * 1024), 16, voff[g & 1],
                                                     (int)(g * 8 * row_bytes + step * kPRowBytes), 0, 0);
        }
#pragma unroll
        for (int i = 0; i < kPWLoads; ++i) {
            const int g = wave * kPWLoads + i;  // 8-row group of W
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)(st + kPM * kPRowBytes + g * 1024), 16,
                                                     voff[g & 1], (int)(g * 8 * row_bytes + step * kPRowBytes),
                                                     0, 0);
        }
    };

    const int frow = lane & 31, fhalf = lane >> 5;
    int fofs[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) fofs[kk] = frow * kPRowBytes + (pswz(frow, kk * 2 + fhalf) << 4);
    const int xo = wm * 32 * kPRowBytes, wo = kPM * kPRowBytes + wn * 64 * kPRowBytes;

    f32x16 acc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
        if (s < KS) issue(s);
    for (int k = 0; k < KS; ++k) {
        // this wave's loads of step k are done once at most the later
        // in-flight steps' loads remain; the barrier then covers every
        // wave's loads and every wave's reads of the stage refilled next
        if (k + kStages - 2 < KS)
            wait_vmcnt<kPLoads * (kStages - 2)>();
        else
            wait_vmcnt<0>();
        // a bare s_barrier: __syncthreads' release fence would also wait
        // for the younger steps' loads and undo the pipelining (every
        // fragment read of a step is consumed by its MFMAs within the step,
        // so no LDS read is outstanding here)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (k + kStages - 1 < KS) issue(k + kStages - 1);
        const uint8_t *st = lds + (k % kStages) * kPStageBytes;
        bf16x8 fx[4], fw[2][4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            fx[kk] = *reinterpret_cast<const bf16x8 *>(st + xo + fofs[kk]);
            fw[0][kk] = *reinterpret_cast<const bf16x8 *>(st + wo + fofs[kk]);
            fw[1][kk] = *reinterpret_cast<const bf16x8 *>(st + wo + 32 * kPRowBytes + fofs[kk]);
        }
        __builtin_amdgcn_sched_barrier(0);  // all 12 reads in flight before the first MFMA waits
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int i = 0; i < 2; ++i)
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[i][kk], fx[kk], acc[i], 0, 0, 0);
    }

    // lane: output row m = m0 + 32 wm + frow; register group q of sub-tile i
    // holds columns n .. n+3, n = n0 + 64 wn + 32 i + 8 q + 4 fhalf
    const int64_t m = m0 + wm * 32 + frow;
    if (m >= M) return;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t n = n0 + wn * 64 + i * 32 + q * 8 + fhalf * 4;
            if (n >= N) continue;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] = acc[i][q * 4 + e];
                if (bias) v[e] += __uint_as_float((uint32_t)bias[n + e] << 16);
            }
            u32x2 out;
            out.x = pack_bf16x2(v[0], v[1]);
            out.y = pack_bf16x2(v[2], v[3]);
            *reinterpret_cast<u32x2 *>(y + m * N + n) = out;
        }
}

template <int kDtype, bool kVecX, bool kVecW>
hipError_t launch_typed(const void *x, const uint16_t *w, const uint16_t *bias, int64_t M, int64_t N,
                        int64_t K, uint16_t *y, hipStream_t stream) {
    const int64_t tm = (M + kTile - 1) / kTile, tn = (N + kTile - 1) / kTile;
    if (tm * tn > 0x7FFFFFFF) return hipErrorInvalidValue;
    gemm_bf16_kernel<kDtype, kVecX, kVecW><<<dim3((unsigned)(tm * tn)), dim3(kThreads), 0, stream>>>(
        x, w, bias, y, M, N, K, (int)tn);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const void *x, int x_dtype, const uint16_t *w, const uint16_t *bias,
                            int64_t M, int64_t N, int64_t K, uint16_t *y, hipStream_t stream) {
    // bf16 input with K a multiple of 64 and N of 128 (any M), large enough to
    // give every CU a 256x256 tile: the 256x256-tile kernel of the INT8 path in
    // its bf16 mode (smaller problems keep the 4x more numerous 128x128 tiles)
    const bool a16 = ((uintptr_t)x % 16 == 0) && ((uintptr_t)w % 16 == 0) && ((uintptr_t)y % 16 == 0);
    const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
    if (x_dtype == 0 && K % 64 == 0 && K <= (1 << 21) && N % 128 == 0 && a16 && (uintptr_t)bias % 8 == 0 &&
        big_tiles >= 256)
        return launch_gemm_bf16_tiled(static_cast<const uint16_t *>(x), w, bias, M, N, K, y, stream);
    // other bf16 problems with K a multiple of 64 and N of 8: the pipelined
    // 64x128-tile kernel
    if (x_dtype == 0 && K % 64 == 0 && K <= (1 << 21) && N % 8 == 0 && a16) {
        const int64_t tm = (M + kPM - 1) / kPM, tn = (N + kPN - 1) / kPN;
        if (tm * tn > 0x7FFFFFFF) return hipErrorInvalidValue;
        gemm_bf16_pipe_kernel<kPipeStages><<<dim3((unsigned)(tm * tn)), dim3(kPThreads), 0, stream>>>(
            static_cast<const uint16_t *>(x), w, bias, y, M, N, K, (int)tn);
        return hipGetLastError();
    }
    const bool vec_w = (K % 8 == 0) && ((uintptr_t)w % 16 == 0);
    const bool vec_x = (x_dtype == 0) && vec_w && ((uintptr_t)x % 16 == 0);
    if (vec_x) return launch_typed<0, true, true>(x, w, bias, M, N, K, y, stream);
    switch (x_dtype) {
    case 0:
        return vec_w ? launch_typed<0, false, true>(x, w, bias, M, N, K, y, stream)
                     : launch_typed<0, false, false>(x, w, bias, M, N, K, y, stream);
    case 1:
        return vec_w ? launch_typed<1, false, true>(x, w, bias, M, N, K, y, stream)
                     : launch_typed<1, false, false>(x, w, bias, M, N, K, y, stream);
    default:
        return vec_w ? launch_typed<2, false, true>(x, w, bias, M, N, K, y, stream)
                     : launch_typed<2, false, false>(x, w, bias, M, N, K, y, stream);
    }
}

}  // namespace w8a8
