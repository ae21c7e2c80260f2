// INT8 GEMM with 128x128 block scales on gfx950 matrix cores.
//
//   Y[m, n] = bf16( sum_kb float(P[m, n, kb]) * (sx[m/128, kb] * sw[n/128, kb])
//                   (+ bias[n]) ),
//   P[m, n, kb] = exact int32 sum_{k in K-block kb} qx[m, k] * qw[n, k].
//
// The block form applies the scales once per 128-deep K-block (TurboDiffusion
// news article, bjdmk.com.cn, inference list: INT8 weights and activations
// at 128x128 block granularity on INT8 matrix units; TurboT2VA paper,
// inference stack, W8A8 paragraph, which names this repeated scaling along
// the reduction as the block form's cost and applies bias in the epilogue).
//
// Structure: one workgroup (4 wavefronts) per 128x128 output tile; one
// K-block (128 deep) per main-loop iteration.  Both operands are K-contiguous
// ("NT"), so every MFMA operand fragment is one 16-byte LDS read.  Tiles of
// qx and qw (16 KiB each) are double-buffered in LDS; the next K-block's
// global loads are issued before the current one's MFMAs.  LDS rows are 128
// bytes with the 16-byte chunk index XOR-swizzled by (row & 7), so the 8
// lanes that read one chunk column of 8 consecutive rows hit distinct banks.
//
// v_mfma_i32_32x32x32_i8 produces the exact int32 sum of one 32-deep slice;
// four of them (accumulating in int32, the first with a zero C operand) give
// P for one K-block.  P is converted to fp32 and fused into the fp32
// accumulator with one FMA by the combined block scale (a scalar per
// (m-block, n-block, K-block), identical across the tile).
//
// The weight fragment is the MFMA "A" operand and the activation fragment
// the "B" operand, so each lane ends up holding 4 consecutive output columns
// n of one row m per register group: the epilogue writes 8-byte bf16 quads.
//
// kPartials = true is the test epilogue: the same main loop stores P itself.
#include "w8a8_internal.h"

namespace w8a8 {
namespace {

constexpr int kTile = 128;   // output tile edge (M and N)
constexpr int kThreads = 256;
constexpr int kLdsTile = kTile * kBlock;  // bytes per operand tile per stage

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int swz(int row, int chunk) {
    return row * kBlock + ((chunk ^ (row & 7)) << 4);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const __bf16 a = (__bf16)lo, b = (__bf16)hi;  // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

template <bool kPartials>
__global__ __launch_bounds__(kThreads) void gemm_i8_bs_kernel(
    const int8_t *__restrict__ qx, const float *__restrict__ sx, const int8_t *__restrict__ qw,
    const float *__restrict__ sw, const uint16_t *__restrict__ bias, uint16_t *__restrict__ y,
    int64_t N, int64_t K, int tiles_m, int tiles_n, int mb0, int nb0, int32_t *__restrict__ partials,
    int64_t part_nt) {
    __shared__ __attribute__((aligned(16))) int8_t lds[2][2][kLdsTile];

    // Tile order: groups of 8 m-tiles sweep all n-tiles, m fastest inside a
    // group, so concurrently resident workgroups share operand panels.
    const int t = blockIdx.x;
    constexpr int kGroup = 8;
    const int group_size = kGroup * tiles_n;
    const int g = t / group_size;
    const int first_m = g * kGroup;
    const int gm = min(tiles_m - first_m, kGroup);
    const int in_group = t - g * group_size;
    const int mb = mb0 + first_m + in_group % gm;
    const int nb = nb0 + in_group / gm;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;  // wave's 64x64 quadrant (m, n)
    const int64_t KB = K / kBlock;

    // global -> LDS copy assignment: 1024 16-byte chunks per operand tile
    const int8_t *gx = qx + (int64_t)mb * kTile * K;
    const int8_t *gw = qw + (int64_t)nb * kTile * K;
    int64_t g_off[4];
    int l_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + i * kThreads;
        const int row = c >> 3, ch = c & 7;
        g_off[i] = (int64_t)row * K + ch * 16;
        l_off[i] = swz(row, ch);
    }

    i32x4 rx[4], rw[4];
    auto load_tiles = [&](int64_t kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rx[i] = *reinterpret_cast<const i32x4 *>(gx + g_off[i] + kb * kBlock);
            rw[i] = *reinterpret_cast<const i32x4 *>(gw + g_off[i] + kb * kBlock);
        }
    };
    auto store_tiles = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<i32x4 *>(&lds[buf][0][l_off[i]]) = rx[i];
            *reinterpret_cast<i32x4 *>(&lds[buf][1][l_off[i]]) = rw[i];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const float *sxr = kPartials ? nullptr : sx + (int64_t)mb * KB;
    const float *swr = kPartials ? nullptr : sw + (int64_t)nb * KB;

    load_tiles(0);
    store_tiles(0);
    __syncthreads();

    const int frag_row = lane & 31, frag_half = lane >> 5;
    for (int64_t kb = 0; kb < KB; ++kb) {
        const int buf = (int)(kb & 1);
        if (kb + 1 < KB) load_tiles(kb + 1);

        i32x4 fx[2][4], fw[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int row = wm * 64 + j * 32 + frag_row;
                fx[j][kk] = *reinterpret_cast<const i32x4 *>(&lds[buf][0][swz(row, kk * 2 + frag_half)]);
            }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int row = wn * 64 + i * 32 + frag_row;
                fw[i][kk] = *reinterpret_cast<const i32x4 *>(&lds[buf][1][swz(row, kk * 2 + frag_half)]);
            }

        float scale = 0.0f;
        if constexpr (!kPartials) scale = sxr[kb] * swr[kb];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                i32x16 p = {0};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    p = __builtin_amdgcn_mfma_i32_32x32x32_i8(fw[i][kk], fx[j][kk], p, 0, 0, 0);
                if constexpr (kPartials) {
                    const int64_t m = (int64_t)(mb - mb0) * kTile + wm * 64 + j * 32 + frag_row;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int64_t n = (int64_t)(nb - nb0) * kTile + wn * 64 + i * 32 +
                                          (r >> 2) * 8 + frag_half * 4 + (r & 3);
                        partials[(m * part_nt + n) * KB + kb] = p[r];
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[i][j][r] = __builtin_fmaf((float)p[r], scale, acc[i][j][r]);
                }
            }

        if (kb + 1 < KB) store_tiles(buf ^ 1);
        __syncthreads();
    }

    if constexpr (!kPartials) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int64_t m = (int64_t)mb * kTile + wm * 64 + j * 32 + frag_row;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t n = (int64_t)nb * kTile + wn * 64 + i * 32 + q * 8 + frag_half * 4;
                    float v0 = acc[i][j][q * 4 + 0], v1 = acc[i][j][q * 4 + 1];
                    float v2 = acc[i][j][q * 4 + 2], v3 = acc[i][j][q * 4 + 3];
                    if (bias) {
                        const u32x2 b = *reinterpret_cast<const u32x2 *>(bias + n);
                        v0 += bf16_to_f32((uint16_t)(b.x & 0xFFFF));
                        v1 += bf16_to_f32((uint16_t)(b.x >> 16));
                        v2 += bf16_to_f32((uint16_t)(b.y & 0xFFFF));
                        v3 += bf16_to_f32((uint16_t)(b.y >> 16));
                    }
                    u32x2 out;
                    out.x = pack_bf16x2(v0, v1);
                    out.y = pack_bf16x2(v2, v3);
                    *reinterpret_cast<u32x2 *>(y + m * N + n) = out;
                }
            }
    }
}

}  // namespace

hipError_t launch_gemm_i8_blockscale(const int8_t *qx, const float *sx, const int8_t *qw,
                                     const float *sw, const uint16_t *bias, int64_t M, int64_t N,
                                     int64_t K, uint16_t *y, hipStream_t stream) {
    const int64_t tm = M / kTile, tn = N / kTile;
    if (tm <= 0 || tn <= 0 || K < kBlock) return hipSuccess;
    if (tm * tn > 0x7FFFFFFF || tm > 0x7FFFFFFF || tn > 0x7FFFFFFF) return hipErrorInvalidValue;
    gemm_i8_bs_kernel<false><<<dim3((unsigned)(tm * tn)), dim3(kThreads), 0, stream>>>(
        qx, sx, qw, sw, bias, y, N, K, (int)tm, (int)tn, 0, 0, nullptr, 0);
    return hipGetLastError();
}

hipError_t launch_kblock_partials(const int8_t *qx, const int8_t *qw, int64_t M, int64_t N,
                                  int64_t K, int64_t m0, int64_t mt, int64_t n0, int64_t nt,
                                  int32_t *partials, hipStream_t stream) {
    (void)M;
    const int64_t tm = mt / kTile, tn = nt / kTile;
    if (tm <= 0 || tn <= 0) return hipSuccess;
    if (tm * tn > 0x7FFFFFFF) return hipErrorInvalidValue;
    // the partials epilogue reads no scale, bias or output
    gemm_i8_bs_kernel<true><<<dim3((unsigned)(tm * tn)), dim3(kThreads), 0, stream>>>(
        qx, nullptr, qw, nullptr, nullptr, nullptr, N, K, (int)tm, (int)tn, (int)(m0 / kTile),
        (int)(n0 / kTile), partials, nt);
    return hipGetLastError();
}

}  // namespace w8a8
