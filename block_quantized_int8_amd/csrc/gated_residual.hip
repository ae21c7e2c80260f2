// Gated residual update of a transformer block, alone, for gfx950.
//
// The fused-kernels paragraph of the TurboT2VA paper (architecture-aware
// inference stack) lists gated residual updates among the memory-bound
// patterns it fuses: the residual stream h takes the linear's output o
// scaled by a per-batch-entry, per-channel gate,
//
//   y[i, n] = bf16( fl32( h[i, n] + fl32( gate[i / L, n] * o[i, n] ) ) )
//
// (each fl32 one IEEE fp32 operation: the library is built without
// floating-point contraction; the product of two bf16 is exact in fp32;
// bf16 to nearest even).  The block-scaled GEMM applies the same update in
// its epilogue (gemm_i8_blockscale.hip), so that o never reaches HBM; this
// kernel is the update on its own, for the bf16 fallback path and as the
// unfused reference point.  Memory-bound: 6 bytes per element (h and o read
// once with nontemporal loads, y written), the gate [B, N] from cache.
//
// One thread per 16-byte chunk of 8 elements, four chunks per thread spaced
// a workgroup apart so four loads of each operand are in flight.  y may be
// h or o itself (each element is read and written by the same thread).
#include "w8a8_internal.h"

namespace w8a8 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kPerThread = 4;

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t update_word(uint32_t h, uint32_t g, uint32_t o) {
    const float y0 = lo_bf16(h) + lo_bf16(g) * lo_bf16(o);
    const float y1 = hi_bf16(h) + hi_bf16(g) * hi_bf16(o);
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{y0, y1}, bf16x2));  // nearest even
}

__global__ __launch_bounds__(kThreads) void gated_residual_kernel(const uint16_t *h, const uint16_t *o,
                                                                  const uint16_t *__restrict__ gate, int64_t L,
                                                                  int64_t N, int64_t chunks, uint16_t *y) {
    const int64_t chunks_per_row = N / 8;
    const int64_t base = (int64_t)blockIdx.x * (kThreads * kPerThread) + threadIdx.x;
    u32x4 hv[kPerThread], ov[kPerThread], gv[kPerThread];
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int64_t c = base + k * kThreads;
        if (c < chunks) {
            const int64_t row = c / chunks_per_row, col = (c - row * chunks_per_row) * 8;
            hv[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(h) + c);
            ov[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(o) + c);
            gv[k] = *reinterpret_cast<const u32x4 *>(gate + (row / L) * N + col);
        }
    }
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int64_t c = base + k * kThreads;
        if (c < chunks)
            reinterpret_cast<u32x4 *>(y)[c] = u32x4{update_word(hv[k].x, gv[k].x, ov[k].x),
                                                    update_word(hv[k].y, gv[k].y, ov[k].y),
                                                    update_word(hv[k].z, gv[k].z, ov[k].z),
                                                    update_word(hv[k].w, gv[k].w, ov[k].w)};
    }
}

}  // namespace

hipError_t launch_gated_residual(const uint16_t *h, const uint16_t *o, const uint16_t *gate, int64_t B, int64_t L,
                                 int64_t N, uint16_t *y, hipStream_t stream) {
    const int64_t chunks = B * L * (N / 8);
    if (chunks <= 0) return hipSuccess;
    const int64_t blocks = (chunks + kThreads * kPerThread - 1) / (kThreads * kPerThread);
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    gated_residual_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(h, o, gate, L, N, chunks, y);
    return hipGetLastError();
}

}  // namespace w8a8
