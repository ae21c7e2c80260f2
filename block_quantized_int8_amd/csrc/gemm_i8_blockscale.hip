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
// Work decomposition
//   * one workgroup (8 wavefronts, 2 per SIMD) per 256x256 output tile; one
//     128-deep K-block per main-loop iteration;
//   * each wavefront owns a 128 (n) x 64 (m) sub-tile = 4 x 2 MFMA tiles of
//     32x32, which lies inside a single 128x128 scale block of Y, so the
//     combined scale sx*sw is one scalar per wavefront and K-block;
//   * v_mfma_i32_32x32x32_i8 gives the exact int32 sum of a 32-deep slice;
//     four of them (the first with a zero C operand) give P for one K-block,
//     which is converted to fp32 and fused into the fp32 accumulator with one
//     FMA by that scale.  The fp32 accumulators (128 per lane) must stay in
//     VGPRs because this per-K-block dequantization runs on the VALU; that is
//     what caps the wavefront tile at 128x64.
//
// Data movement
//   * both operands are K-contiguous (Y = X W^T, "NT"): every MFMA operand
//     fragment is one 16-byte LDS read (lane l: row l%32, k-half l/32);
//   * operand tiles go from global memory straight into LDS with
//     buffer_load_dwordx4 ... lds (no VGPR staging), double-buffered: 2 stages x
//     (256 + 256) rows x 128 bytes = 128 KiB.  The next K-block's loads are
//     in flight while the current one is multiplied;
//   * LDS rows are 128 bytes with the 16-byte chunk index XOR-swizzled (see
//     swz_slot); the direct loads write 1 KiB lane-linearly, so each lane
//     fetches the global chunk that belongs at its LDS slot;
//   * workgroups are dispatched round-robin over the 8 XCDs; the tile index
//     is remapped so each XCD works on a contiguous range of tiles, ordered
//     in groups of 8 m-tiles sweeping n, so tiles resident on one XCD share
//     operand panels in its L2.
//
// Edges: N and K are multiples of 128 (K-blocks of 128 bytes), M of 128 in
// the INT8 modes and arbitrary in the bf16 mode, none necessarily of 256;
// rows past the end of a partial tile read as zeros (buffer range check),
// wavefronts whose sub-tile lies outside the output skip their work, and
// output rows past M are not stored.
//
// Within a wavefront the K-block loop is software-pipelined: the 32 VALU ops
// that dequantize the finished partial of sub-tile s-1 run between the MFMAs
// of sub-tile s, one MFMA behind (quarters 0-2 after MFMAs 1-3 of sub-tile s,
// quarter 3 just before the first MFMA of sub-tile s+1, which reuses those
// registers), so the VALU never waits for sub-tile s-1's last MFMA and the
// matrix core and the VALU work at the same time; a scheduling fence after
// every MFMA and its VALU ops holds that order.  Starting each dequantization
// right behind the sub-tile's last MFMA instead was 2-3% slower.
//
// The weight fragment is the MFMA "A" operand and the activation fragment
// the "B" operand, so each lane holds 4 consecutive output columns n of one
// row m per register group.  The output goes through LDS (free after the
// main loop) so that Y is written in whole 256-byte row segments, with
// nontemporal stores: this kernel never reads Y back, and lines of it left
// dirty in the last-level cache would be written back to HBM during the next
// kernel (in a layer sequence, the next activation quantization), which then
// ran 25% slower.
//
// The partials mode is the test epilogue: the same main loop stores P itself.
//
// kBf16 mode runs the guard's bf16 fallback through the same machinery when
// x is bf16 and K a multiple of 64: a 128-byte LDS row then holds 64 bf16
// values, and the fragment of v_mfma_f32_32x32x16_bf16 for k-slice kk (lane l:
// row l%32, elements 16kk + 8(l/32) .. +7) occupies exactly the bytes of the
// INT8 fragment, so loads, swizzle and fragment reads are unchanged; the
// MFMAs accumulate straight into the fp32 accumulators (no per-K-block
// work).  M may be ragged: rows past M read as zeros and are not stored.
#include "w8a8_internal.h"

namespace w8a8 {
namespace {

constexpr int kTileM = 256, kTileN = 256;
constexpr int kThreads = 512;
constexpr int kWaveM = 64, kWaveN = 128;
constexpr int kStage = (kTileM + kTileN) * kBlock;  // bytes per pipeline stage
constexpr int kGroupM = 8;

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void *lds_ptr_t;
// buffer descriptor word 3 for raw (untyped) dword buffer access on gfx9 parts
constexpr int kRsrcWord3 = 0x00020000;

// LDS slot of 16-byte chunk `chunk` in operand row `row`: XOR with (row & 7)
// and bit 3 of the row, so both 8 consecutive rows (32 banks x 4 bytes) and
// 16 consecutive rows (64 banks, even/odd rows in opposite 128-byte halves)
// read one chunk column without bank conflicts.  Self-inverse in `chunk`.
__device__ __forceinline__ int swz_slot(int row, int chunk) { return chunk ^ (row & 7) ^ ((row >> 3) & 1); }

// Two floats -> one word of two bf16 (lo first), each rounded to nearest
// even: one packed conversion.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Sizes of one launch.  The tensors are separate __restrict__ kernel
// arguments so the compiler can prove the scale grids read-only and fetch
// them with scalar loads (a vector load would be ordered behind the
// in-flight operand prefetch in the same vmcnt queue).
struct Problem {
    int64_t N, K;
    int64_t m_begin, m_end, n_begin, n_end;  // output window (multiples of 128, m_end any in bf16 mode)
    int tiles_m, tiles_n;
};

// Dequantize one quarter (elements 4*part .. 4*part+3) of a finished K-block
// partial into the accumulator: 8 VALU ops, issued between two MFMAs.
__device__ __forceinline__ void dequant_quarter(f32x16 &acc, const i32x16 &pk, float scale, int part) {
#pragma unroll
    for (int r = part * 4; r < part * 4 + 4; ++r) acc[r] = __builtin_fmaf((float)pk[r], scale, acc[r]);
}

// Buffer resource for `rows` rows of K bytes starting at `base`: loads past
// the last row return zeros (raw buffer range check), which is how partial
// edge tiles are handled without clamping.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const int8_t *base, int64_t rows, int64_t K) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(base), (short)0, (int)(rows * K),
                                             kRsrcWord3);
}

// kMode: kBlockScaled (the block form), kPartials (test epilogue),
// kPostScaled (per-row / per-channel scales applied once at the end),
// kBf16 (bf16 operands, fp32 accumulation: the fallback's fast path; the
// sizes in Problem then count bytes along K) or kBlockResidual (the block
// form whose bf16 output o feeds a gated residual update in the epilogue:
// y = bf16(fl32(h + fl32(gate[row / L] * o))), read from Residual).
enum { kBlockScaled = 0, kPartialsOnly = 1, kPostScaled = 2, kBf16 = 3, kBlockResidual = 4 };

// Operands of the gated residual epilogue: residual stream h [M, N] (may be
// y itself), gate [M / L, N], L rows per gate row.
struct Residual {
    const uint16_t *h;
    const uint16_t *gate;
    int64_t L;
};

template <int kMode>
__global__ __launch_bounds__(kThreads) void gemm_i8_bs_kernel(
    const int8_t *__restrict__ qx, const float *__restrict__ sx, const int8_t *__restrict__ qw,
    const float *__restrict__ sw, const uint16_t *__restrict__ bias, uint16_t *__restrict__ y,
    int32_t *__restrict__ partials, const Problem p, const Residual res) {
    constexpr bool kBlockForm = kMode == kBlockScaled || kMode == kBlockResidual;
    constexpr bool kPartials = kMode == kPartialsOnly;
    constexpr bool kPost = kMode == kPostScaled;
    constexpr bool kBf = kMode == kBf16;
    __shared__ __attribute__((aligned(1024))) int8_t lds[2 * kStage];

    // ---- tile index: XCD-contiguous ranges, then grouped m-fastest order
    const int nwg = (int)gridDim.x;
    int t = (int)blockIdx.x;
    if ((nwg & 7) == 0) t = (t & 7) * (nwg >> 3) + (t >> 3);
    const int group_size = kGroupM * p.tiles_n;
    const int g = t / group_size;
    const int first_m = g * kGroupM;
    const int gm = min(p.tiles_m - first_m, kGroupM);
    const int in_group = t - g * group_size;
    const int64_t m_org = p.m_begin + (int64_t)(first_m + in_group % gm) * kTileM;
    const int64_t n_org = p.n_begin + (int64_t)(in_group / gm) * kTileN;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wn = wave & 1, wm = wave >> 1;
    const int64_t K = p.K;
    const int KB = (int)(K / kBlock);

    // ---- operand loads, global -> LDS: wave w fills rows [32w, 32w+32) of
    // both tiles, 8 rows (1 KiB, lane-linear in LDS) per instruction; row
    // lrow + 8i for instruction i.  Lane l writes LDS slot l%8, which holds
    // global chunk swz_slot(row, l%8).  That slot pattern depends on row bit
    // 3, so even and odd instructions need different per-lane offsets; the
    // rest (row block, K-block) is a scalar offset, the same for both operands.
    const __amdgpu_buffer_rsrc_t xr = tile_rsrc(qx + m_org * K, min((int64_t)kTileM, p.m_end - m_org), K);
    const __amdgpu_buffer_rsrc_t wr = tile_rsrc(qw + n_org * K, min((int64_t)kTileN, p.n_end - n_org), K);
    const int lrow = wave * 32 + (lane >> 3);
    uint32_t voff[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
        voff[b] = (uint32_t)(lrow * K) + (uint32_t)(swz_slot(lrow + 8 * b, lane & 7) * 16);
    auto issue_loads = [&](int stage, int kb) {
        int8_t *xs = lds + stage * kStage + wave * 32 * kBlock;
        int8_t *ws = xs + kTileM * kBlock;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t so = (uint32_t)(kb * kBlock) + (uint32_t)(i * 8 * K);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(xs + i * 8 * kBlock), 16, voff[i & 1], so,
                                                     0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)(ws + i * 8 * kBlock), 16, voff[i & 1], so,
                                                     0, 0);
        }
    };

    const bool active = (m_org + wm * kWaveM < p.m_end) && (n_org + wn * kWaveN < p.n_end);
    const int64_t mblk = (m_org + wm * kWaveM) / kBlock;
    const int64_t nblk = (n_org + wn * kWaveN) / kBlock;
    const float *sxr = kBlockForm ? sx + mblk * KB : nullptr;
    const float *swr = kBlockForm ? sw + nblk * KB : nullptr;
    // combined scales sx*sw of 64 consecutive K-blocks, one per lane; each
    // K-block reads its own with readlane (no scalar load, whose lgkmcnt
    // wait would also drain every LDS read in flight)
    // (only active wavefronts read scales: an inactive one's block row of a
    // partial edge tile may not exist)
    float sc_lane = 0.0f;
    auto load_scales = [&](int kb0) {
        if constexpr (kBlockForm) {
            const int kb = kb0 + lane;
            sc_lane = (active && kb < KB) ? sxr[kb] * swr[kb] : 0.0f;
        }
    };

    // sub-tile s = 2*i + j: weight rows 32i.., activation rows 32j.. of the wave tile
    // block form: fp32 accumulators; post-scale form: int32 accumulators
    // carried across all K-blocks by the MFMAs themselves
    f32x16 acc[8];
    i32x16 acci[kPost ? 8 : 1];
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            acc[s][r] = 0.0f;
            acci[kPost ? s : 0][r] = 0;
        }
    i32x16 pk[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) pk[0][r] = pk[1][r] = 0;
    float prev_scale = 0.0f;  // scale of the partials carried in pk[0] (last quarter) and pk[1]

    // fragment read addresses: row (32-aligned base) + frow; the swizzle only
    // depends on frow, so one per-lane byte offset per K-slice kk
    const int frow = lane & 31, fhalf = lane >> 5;
    int fofs[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) fofs[kk] = frow * kBlock + (swz_slot(frow, kk * 2 + fhalf) << 4);

    load_scales(0);
    issue_loads(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    const i32x16 zero = {0};
    for (int kb = 0; kb < KB; ++kb) {
        const int stage = kb & 1;
        if (kb + 1 < KB) issue_loads(stage ^ 1, kb + 1);

        if (active) {
            const int8_t *xs = lds + stage * kStage + wm * kWaveM * kBlock;
            const int8_t *ws = lds + stage * kStage + kTileM * kBlock + wn * kWaveN * kBlock;
            // first sub-tile's fragments in MFMA order, then the second
            // activation fragment set
            i32x4 fx[2][4], fw[2][4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                fw[0][kk] = *reinterpret_cast<const i32x4 *>(ws + fofs[kk]);
                fx[0][kk] = *reinterpret_cast<const i32x4 *>(xs + fofs[kk]);
            }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                fx[1][kk] = *reinterpret_cast<const i32x4 *>(xs + 32 * kBlock + fofs[kk]);
            float scale = 0.0f;
            if constexpr (kBlockForm)
                scale = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc_lane), kb & 63));

            // software pipeline: the MFMAs of sub-tile s run while the VALU
            // dequantizes sub-tile s-1 (for s = 0 and 1: sub-tiles 7 and 6 of
            // the previous K-block, carried across the barrier in pk[1], pk[0])
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int i = s >> 1, j = s & 1;
                if (j == 0 && i < 3) {
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        fw[(i + 1) & 1][kk] =
                            *reinterpret_cast<const i32x4 *>(ws + (i + 1) * 32 * kBlock + fofs[kk]);
                }
                if constexpr (kPost) {
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        acci[s] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fw[i & 1][kk], fx[j][kk], acci[s], 0, 0, 0);
                    continue;
                }
                if constexpr (kBf) {
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fw[i & 1][kk]),
                                                                         __builtin_bit_cast(bf16x8, fx[j][kk]), acc[s],
                                                                         0, 0, 0);
                    continue;
                }
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    // last quarter of sub-tile s-2, whose registers this MFMA reuses
                    if (!kPartials && kk == 0) {
                        if (s >= 2)
                            dequant_quarter(acc[s - 2], pk[s & 1], scale, 3);
                        else
                            dequant_quarter(acc[6 + s], pk[s & 1], prev_scale, 3);
                    }
                    pk[s & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fw[i & 1][kk], fx[j][kk],
                                                                      kk == 0 ? zero : pk[s & 1], 0, 0, 0);
                    if constexpr (!kPartials) {
                        if (kk > 0) {
                            if (s > 0)
                                dequant_quarter(acc[s - 1], pk[(s - 1) & 1], scale, kk - 1);
                            else
                                dequant_quarter(acc[7], pk[1], prev_scale, kk - 1);
                        }
                        // issue order MFMA, its dequant VALU ops, MFMA, ...: a
                        // hard scheduling fence per step (group barriers alone
                        // let the scheduler bunch 4 dependent MFMAs together)
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                if constexpr (kPartials) {
                    const int64_t m = m_org - p.m_begin + wm * kWaveM + j * 32 + frow;
                    const int64_t nt = p.n_end - p.n_begin;
                    int32_t *dst = partials + (m * nt + (n_org - p.n_begin) + wn * kWaveN + i * 32 +
                                                 fhalf * 4) * KB + kb;
#pragma unroll
                    for (int r = 0; r < 16; ++r) dst[((r >> 2) * 8 + (r & 3)) * KB] = pk[s & 1][r];
                }
            }
            prev_scale = scale;
        }
        if ((kb & 63) == 63 && kb + 1 < KB) load_scales(kb + 1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    if constexpr (!kPartials) {
        if (!active) return;
        if constexpr (kPost) {
            // post-scale epilogue: y = float(int32 sum over K) * sx[m] * sw[n]
            float sxm[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) sxm[j] = sx[m_org + wm * kWaveM + j * 32 + frow];
            const float *swp = sw + n_org + wn * kWaveN + fhalf * 4;
#pragma unroll
            for (int s = 0; s < 8; ++s)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 w4 = *reinterpret_cast<const f32x4 *>(swp + (s >> 1) * 32 + q * 8);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[s][q * 4 + e] = (float)acci[s][q * 4 + e] * sxm[s & 1] * w4[e];
                }
        } else if constexpr (!kBf) {
            dequant_quarter(acc[6], pk[0], prev_scale, 3);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) dequant_quarter(acc[7], pk[1], prev_scale, kk);
        }

        // ---- epilogue through LDS (free after the last barrier): each wave
        // writes its 64 (m) x 128 (n) bf16 tile as rows of 256 bytes with the
        // 16-byte chunk index XOR-swizzled by (row & 15), then stores whole
        // rows to Y with 16-byte, fully coalesced writes.
        if (bias) {
            const uint16_t *bp = bias + n_org + wn * kWaveN + fhalf * 4;
#pragma unroll
            for (int s = 0; s < 8; ++s)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x2 b = *reinterpret_cast<const u32x2 *>(bp + (s >> 1) * 32 + q * 8);
                    acc[s][q * 4 + 0] += bf16_to_f32(b.x & 0xFFFFu);
                    acc[s][q * 4 + 1] += bf16_to_f32(b.x >> 16);
                    acc[s][q * 4 + 2] += bf16_to_f32(b.y & 0xFFFFu);
                    acc[s][q * 4 + 3] += bf16_to_f32(b.y >> 16);
                }
        }
        int8_t *ot = lds + wave * (kWaveM * kWaveN * 2);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int i = s >> 1, j = s & 1;
            const int row = j * 32 + frow;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int chunk = i * 4 + q;  // 16-byte chunk (8 columns) inside the 128-column row
                u32x2 out;
                out.x = pack_bf16x2(acc[s][q * 4 + 0], acc[s][q * 4 + 1]);
                out.y = pack_bf16x2(acc[s][q * 4 + 2], acc[s][q * 4 + 3]);
                *reinterpret_cast<u32x2 *>(ot + row * 256 + ((chunk ^ (row & 15)) << 4) + fhalf * 8) = out;
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
        __builtin_amdgcn_wave_barrier();
        const int c = lane & 15;
        uint16_t *yrow = y + (m_org + wm * kWaveM) * p.N + n_org + wn * kWaveN + c * 8;
        const int64_t rows_left = p.m_end - (m_org + wm * kWaveM);  // < 64 only in a ragged last tile
        if constexpr (kMode == kBlockResidual) {
            // gated residual: every row's h and gate chunk is requested
            // before the first is used; the same lane reads h and writes y at
            // one address, so y may be h itself
            const int64_t off = (m_org + wm * kWaveM) * p.N + n_org + wn * kWaveN + c * 8;
            const uint32_t grow0 = (uint32_t)(m_org + wm * kWaveM), L = (uint32_t)res.L;
            const uint16_t *gcol = res.gate + n_org + wn * kWaveN + c * 8;
            i32x4 hv[kWaveM / 4], gv[kWaveM / 4];
#pragma unroll
            for (int it = 0; it < kWaveM / 4; ++it) {
                const int row = it * 4 + (lane >> 4);
                const bool in = row < rows_left;
                hv[it] = in ? __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(res.h + off + (int64_t)row * p.N))
                            : i32x4{0, 0, 0, 0};
                gv[it] = in ? *reinterpret_cast<const i32x4 *>(gcol + (int64_t)((grow0 + row) / L) * p.N)
                            : i32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int it = 0; it < kWaveM / 4; ++it) {
                const int row = it * 4 + (lane >> 4);
                const i32x4 v = *reinterpret_cast<const i32x4 *>(ot + row * 256 + ((c ^ (row & 15)) << 4));
                i32x4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t ow = (uint32_t)v[e], hw = (uint32_t)hv[it][e], gw = (uint32_t)gv[it][e];
                    const float y0 = bf16_to_f32(hw & 0xFFFFu) + bf16_to_f32(gw & 0xFFFFu) * bf16_to_f32(ow & 0xFFFFu);
                    const float y1 = bf16_to_f32(hw >> 16) + bf16_to_f32(gw >> 16) * bf16_to_f32(ow >> 16);
                    out[e] = (int)pack_bf16x2(y0, y1);
                }
                if (row < rows_left)
                    __builtin_nontemporal_store(out, reinterpret_cast<i32x4 *>(yrow + (int64_t)row * p.N));
            }
        } else {
#pragma unroll
            for (int it = 0; it < kWaveM / 4; ++it) {
                const int row = it * 4 + (lane >> 4);
                const i32x4 v = *reinterpret_cast<const i32x4 *>(ot + row * 256 + ((c ^ (row & 15)) << 4));
                if (row < rows_left)
                    __builtin_nontemporal_store(v, reinterpret_cast<i32x4 *>(yrow + (int64_t)row * p.N));
            }
        }
    }
}

template <int kMode>
hipError_t launch(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw,
                  const uint16_t *bias, uint16_t *y, int32_t *partials, Problem p, hipStream_t stream,
                  Residual res = Residual{nullptr, nullptr, 1}) {
    const int64_t tm = (p.m_end - p.m_begin + kTileM - 1) / kTileM;
    const int64_t tn = (p.n_end - p.n_begin + kTileN - 1) / kTileN;
    if (tm <= 0 || tn <= 0 || p.K < kBlock) return hipSuccess;
    if (tm * tn > 0x7FFFFFFF) return hipErrorInvalidValue;
    p.tiles_m = (int)tm;
    p.tiles_n = (int)tn;
    gemm_i8_bs_kernel<kMode><<<dim3((unsigned)(tm * tn)), dim3(kThreads), 0, stream>>>(
        qx, sx, qw, sw, bias, y, partials, p, res);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_i8_blockscale(const int8_t *qx, const float *sx, const int8_t *qw,
                                     const float *sw, const uint16_t *bias, int64_t M, int64_t N,
                                     int64_t K, uint16_t *y, hipStream_t stream) {
    Problem p{N, K, 0, M, 0, N, 0, 0};
    return launch<kBlockScaled>(qx, sx, qw, sw, bias, y, nullptr, p, stream);
}

hipError_t launch_gemm_i8_blockscale_residual(const int8_t *qx, const float *sx, const int8_t *qw,
                                              const float *sw, const uint16_t *bias, int64_t M, int64_t N,
                                              int64_t K, const uint16_t *h, const uint16_t *gate, int64_t L,
                                              uint16_t *y, hipStream_t stream) {
    if (L <= 0 || M > 0x7FFFFFFF) return hipErrorInvalidValue;  // 32-bit row arithmetic in the epilogue
    Problem p{N, K, 0, M, 0, N, 0, 0};
    return launch<kBlockResidual>(qx, sx, qw, sw, bias, y, nullptr, p, stream, Residual{h, gate, L});
}

hipError_t launch_kblock_partials(const int8_t *qx, const int8_t *qw, int64_t M, int64_t N,
                                  int64_t K, int64_t m0, int64_t mt, int64_t n0, int64_t nt,
                                  int32_t *partials, hipStream_t stream) {
    (void)M;
    // the partials epilogue reads no scale, bias or output
    Problem p{N, K, m0, m0 + mt, n0, n0 + nt, 0, 0};
    return launch<kPartialsOnly>(qx, nullptr, qw, nullptr, nullptr, nullptr, partials, p, stream);
}

hipError_t launch_gemm_bf16_tiled(const uint16_t *x, const uint16_t *w, const uint16_t *bias, int64_t M,
                                  int64_t N, int64_t K, uint16_t *y, hipStream_t stream) {
    // K in bytes along the rows: 64 bf16 values per 128-byte K-block
    Problem p{N, 2 * K, 0, M, 0, N, 0, 0};
    return launch<kBf16>(reinterpret_cast<const int8_t *>(x), nullptr, reinterpret_cast<const int8_t *>(w),
                         nullptr, bias, y, nullptr, p, stream);
}

hipError_t launch_gemm_i8_postscale(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw,
                                    const uint16_t *bias, int64_t M, int64_t N, int64_t K, uint16_t *y,
                                    hipStream_t stream) {
    Problem p{N, K, 0, M, 0, N, 0, 0};
    return launch<kPostScaled>(qx, sx, qw, sw, bias, y, nullptr, p, stream);
}

}  // namespace w8a8
