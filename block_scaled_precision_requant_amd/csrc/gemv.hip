// gemv.hip -- weight-streaming block-scaled GEMV for gfx950 (m <= 8).
//
// Same result definition as the GEMM (exact int32 dot product per 32-wide K
// block, FP32 rescale by fl32(a_s * w_s), FP32 accumulation, BF16 out) for the
// decode row counts, where the work is bound by reading W_i8 and W_scale from
// HBM once.  kGemvLanesPerCol lanes share one output column: lane g reads
// whole 32-byte blocks g, g + 16, ... of the weight row (a 16-lane group reads
// 512 contiguous bytes per step), dots them against every activation row with
// v_dot4_i32_i8, rescales per block, and the group reduces its FP32 partials
// at the end.  One kernel is compiled per row count 1, 2, 4, 8; other m take
// the next larger one with the extra rows skipped.
#include "bsr_internal.h"

namespace bsr {
namespace {

__device__ __forceinline__ int dot32(const uint4 &a0, const uint4 &a1, const uint4 &w0,
                                     const uint4 &w1) {
    int p = 0;
    p = __builtin_amdgcn_sdot4((int)a0.x, (int)w0.x, p, false);
    p = __builtin_amdgcn_sdot4((int)a0.y, (int)w0.y, p, false);
    p = __builtin_amdgcn_sdot4((int)a0.z, (int)w0.z, p, false);
    p = __builtin_amdgcn_sdot4((int)a0.w, (int)w0.w, p, false);
    p = __builtin_amdgcn_sdot4((int)a1.x, (int)w1.x, p, false);
    p = __builtin_amdgcn_sdot4((int)a1.y, (int)w1.y, p, false);
    p = __builtin_amdgcn_sdot4((int)a1.z, (int)w1.z, p, false);
    p = __builtin_amdgcn_sdot4((int)a1.w, (int)w1.w, p, false);
    return p;
}

template <int MR>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(
    const int8_t *__restrict__ a, const int8_t *__restrict__ w, const float *__restrict__ a_s,
    const float *__restrict__ w_s, uint16_t *__restrict__ out, uint32_t m, uint32_t n, uint32_t k) {
    const int g = threadIdx.x % kGemvLanesPerCol;
    const uint32_t col = blockIdx.x * kGemvColsPerWg + threadIdx.x / kGemvLanesPerCol;
    const bool live = col < n;
    const uint32_t c = live ? col : n - 1;
    const uint32_t nb = k / 32;
    const int8_t *wrow = w + (uint64_t)c * k;
    const float *wsrow = w_s + (uint64_t)c * nb;

    float acc[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) acc[r] = 0.0f;

    for (uint32_t b = g; b < nb; b += kGemvLanesPerCol) {
        const uint4 w0 = *reinterpret_cast<const uint4 *>(wrow + 32ull * b);
        const uint4 w1 = *reinterpret_cast<const uint4 *>(wrow + 32ull * b + 16);
        const float wsv = wsrow[b];
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            if (r < (int)m) {
                const int8_t *arow = a + (uint64_t)r * k + 32ull * b;
                const uint4 a0 = *reinterpret_cast<const uint4 *>(arow);
                const uint4 a1 = *reinterpret_cast<const uint4 *>(arow + 16);
                const int p = dot32(a0, a1, w0, w1);
                acc[r] = fmaf((float)p, a_s[(uint64_t)r * nb + b] * wsv, acc[r]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
        for (int off = kGemvLanesPerCol / 2; off >= 1; off >>= 1)
            acc[r] += __shfl_xor(acc[r], off, kGemvLanesPerCol);
    if (live && g == 0) {
#pragma unroll
        for (int r = 0; r < MR; ++r)
            if (r < (int)m) out[(uint64_t)r * n + col] = f32_to_bf16_rne(acc[r]);
    }
}

}  // namespace

hipError_t launch_gemv(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale,
                       const float *w_scale, uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                       hipStream_t s) {
    const dim3 grid((uint32_t)div_up(n, kGemvColsPerWg));
    const dim3 block(kGemvThreads);
    if (m <= 1)
        hipLaunchKernelGGL(gemv_kernel<1>, grid, block, 0, s, a_i8, w_i8, a_scale, w_scale, out, m, n, k);
    else if (m <= 2)
        hipLaunchKernelGGL(gemv_kernel<2>, grid, block, 0, s, a_i8, w_i8, a_scale, w_scale, out, m, n, k);
    else if (m <= 4)
        hipLaunchKernelGGL(gemv_kernel<4>, grid, block, 0, s, a_i8, w_i8, a_scale, w_scale, out, m, n, k);
    else
        hipLaunchKernelGGL(gemv_kernel<8>, grid, block, 0, s, a_i8, w_i8, a_scale, w_scale, out, m, n, k);
    return hipGetLastError();
}

}  // namespace bsr
