// gemm.hip -- int8 x int8 block-scaled GEMM for gfx950 (m > 8).
//
// Computes out[i,j] = bf16_rne( sum_b fl32(a_s[i,b] * w_s[j,b]) * P[i,j,b] ) with
// P the exact int32 dot product of 32-wide K block b -- the second launch of
// `int8_gemm_faith2_prefill` on page "metrale_model_layers/layers/ops/
// gemm_dense_int8.rs".
//
// One v_mfma_i32_32x32x32_i8 covers exactly one scale block of a 32 x 32
// output tile, so each block's P leaves the matrix core as int32 and is
// rescaled into FP32 accumulators in registers before the next block.
// A and W tiles of kGemmStageBlocks blocks are staged through LDS (rows padded
// so 8 consecutive rows start on distinct bank groups); the scales are staged
// transposed so a lane's four consecutive output rows read one 16-byte word.
#include "bsr_internal.h"

namespace bsr {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(kGemmThreads, 2) void gemm_kernel(
    const int8_t *__restrict__ a, const int8_t *__restrict__ w, const float *__restrict__ a_s,
    const float *__restrict__ w_s, uint16_t *__restrict__ out, uint32_t M, uint32_t N, uint32_t K,
    uint32_t tiles_n) {
    __shared__ __attribute__((aligned(16))) int8_t lds_a[kGemmBM * kGemmLdsRowStride];
    __shared__ __attribute__((aligned(16))) int8_t lds_w[kGemmBN * kGemmLdsRowStride];
    __shared__ __attribute__((aligned(16))) float lds_as[kGemmStageBlocks][kGemmBM];
    __shared__ __attribute__((aligned(16))) float lds_ws[kGemmStageBlocks][kGemmBN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const uint32_t tile = blockIdx.x;
    const uint32_t m0 = (tile / tiles_n) * kGemmBM;
    const uint32_t n0 = (tile % tiles_n) * kGemmBN;
    const uint32_t nb = K / 32;

    float acc[2][2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const v16i zero = {};
    constexpr int kChunksPerRow = kGemmStageBytes / 16;                       // 8
    constexpr int kChunkIters = kGemmBM * kChunksPerRow / kGemmThreads;       // 4
    constexpr int kScaleIters = kGemmBM * kGemmStageBlocks / kGemmThreads;    // 2

    for (uint32_t kb = 0; kb < nb; kb += kGemmStageBlocks) {
        const uint32_t nbs = min((uint32_t)kGemmStageBlocks, nb - kb);
        uint4 ra[kChunkIters], rw[kChunkIters];
        float rsa[kScaleIters], rsw[kScaleIters];
#pragma unroll
        for (int i = 0; i < kChunkIters; ++i) {
            const int c = tid + kGemmThreads * i;
            const int row = c / kChunksPerRow, col = c % kChunksPerRow;
            const bool on = (uint32_t)col < 2 * nbs;
            const uint64_t ga = (uint64_t)min(m0 + row, M - 1) * K + (uint64_t)kb * 32 + col * 16;
            const uint64_t gw = (uint64_t)min(n0 + row, N - 1) * K + (uint64_t)kb * 32 + col * 16;
            ra[i] = on ? *reinterpret_cast<const uint4 *>(a + ga) : make_uint4(0, 0, 0, 0);
            rw[i] = on ? *reinterpret_cast<const uint4 *>(w + gw) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < kScaleIters; ++i) {
            const int idx = tid + kGemmThreads * i;
            const int row = idx / kGemmStageBlocks, jb = idx % kGemmStageBlocks;
            const bool on = (uint32_t)jb < nbs;
            rsa[i] = on ? a_s[(uint64_t)min(m0 + row, M - 1) * nb + kb + jb] : 0.0f;
            rsw[i] = on ? w_s[(uint64_t)min(n0 + row, N - 1) * nb + kb + jb] : 0.0f;
        }
        __syncthreads();  // the previous stage's readers are done
#pragma unroll
        for (int i = 0; i < kChunkIters; ++i) {
            const int c = tid + kGemmThreads * i;
            const int row = c / kChunksPerRow, col = c % kChunksPerRow;
            *reinterpret_cast<uint4 *>(lds_a + row * kGemmLdsRowStride + col * 16) = ra[i];
            *reinterpret_cast<uint4 *>(lds_w + row * kGemmLdsRowStride + col * 16) = rw[i];
        }
#pragma unroll
        for (int i = 0; i < kScaleIters; ++i) {
            const int idx = tid + kGemmThreads * i;
            const int row = idx / kGemmStageBlocks, jb = idx % kGemmStageBlocks;
            lds_as[jb][row] = rsa[i];
            lds_ws[jb][row] = rsw[i];
        }
        __syncthreads();

        for (uint32_t j = 0; j < nbs; ++j) {
            v4i af[2], bf[2];
            float wsv[2];
            float asv[2][16];
#pragma unroll
            for (int sm = 0; sm < 2; ++sm) {
                const int row = wm * 64 + sm * 32 + (lane & 31);
                af[sm] = *reinterpret_cast<const v4i *>(lds_a + row * kGemmLdsRowStride + j * 32 +
                                                        (lane >> 5) * 16);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float4 f = *reinterpret_cast<const float4 *>(
                        &lds_as[j][wm * 64 + sm * 32 + 8 * g + 4 * (lane >> 5)]);
                    asv[sm][4 * g + 0] = f.x;
                    asv[sm][4 * g + 1] = f.y;
                    asv[sm][4 * g + 2] = f.z;
                    asv[sm][4 * g + 3] = f.w;
                }
            }
#pragma unroll
            for (int sn = 0; sn < 2; ++sn) {
                const int row = wn * 64 + sn * 32 + (lane & 31);
                bf[sn] = *reinterpret_cast<const v4i *>(lds_w + row * kGemmLdsRowStride + j * 32 +
                                                        (lane >> 5) * 16);
                wsv[sn] = lds_ws[j][row];
            }
#pragma unroll
            for (int sm = 0; sm < 2; ++sm)
#pragma unroll
                for (int sn = 0; sn < 2; ++sn) {
                    const v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[sm], bf[sn], zero, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[sm][sn][r] = fmaf((float)p[r], asv[sm][r] * wsv[sn], acc[sm][sn][r]);
                }
        }
    }

    // Output layout of a 32x32 MFMA tile: lane l holds column l % 32 and, in
    // register r, row 8 * (r / 4) + 4 * (l / 32) + r % 4.
#pragma unroll
    for (int sm = 0; sm < 2; ++sm)
#pragma unroll
        for (int sn = 0; sn < 2; ++sn) {
            const uint32_t col = n0 + wn * 64 + sn * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const uint32_t row = m0 + wm * 64 + sm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row < M && col < N) out[(uint64_t)row * N + col] = f32_to_bf16_rne(acc[sm][sn][r]);
            }
        }
}

}  // namespace

hipError_t launch_gemm(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale,
                       const float *w_scale, uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                       hipStream_t s) {
    const uint32_t tiles_m = (uint32_t)div_up(m, kGemmBM);
    const uint32_t tiles_n = (uint32_t)div_up(n, kGemmBN);
    hipLaunchKernelGGL(gemm_kernel, dim3(tiles_m * tiles_n), dim3(kGemmThreads), 0, s, a_i8, w_i8,
                       a_scale, w_scale, out, m, n, k, tiles_n);
    return hipGetLastError();
}

}  // namespace bsr
