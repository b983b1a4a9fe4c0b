// gemv.hip -- weight-streaming block-scaled GEMV for gfx950 (m <= 8).
//
// Same result definition as the GEMM (page "metrale_model_layers/layers/ops/
// gemm_dense_int8.rs", second launch of `int8_gemm_faith2_prefill`): exact
// int32 dot product per 32-wide K block, FP32 rescale by fl32(a_s * w_s), FP32
// accumulation, BF16 out -- here for decode row counts, where the kernel is
// bound by reading W_i8 and W_scale from HBM once.
//
// Mapping.  Workgroup = kGemvCols (16) output columns x all of K; its waves
// split K into contiguous ranges.  A wave step covers 64 bytes of K (two scale
// blocks) for its 16 columns: lane l loads 16 bytes of weight row (n0 + l % 16)
// at byte 16 * (l / 16) of the step -- 16 rows x 64 contiguous bytes per
// instruction -- and, if l % 16 < m, 16 bytes of activation row l % 16 at the
// same offset.  One v_mfma_i32_16x16x64_i8 with the activation quarters 2-3
// zeroed gives the first block's P, one with quarters 0-1 zeroed the second's:
// lanes pair A and B bytes by (quarter, byte), so the zeroed quarters drop out
// exactly.  Output lane l holds column l % 16, rows 4 * (l / 16) + r (r < 4),
// so lanes 0-31 hold all m <= 8 rows.
#include "bsr_internal.h"

namespace bsr {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Scales of blocks idx..idx+3 of one row: one 16-byte load when every row
// holds a multiple of 4 blocks (then idx, a multiple of 4, is 16-byte aligned
// and idx + 3 < nb), else four loads clamped to the row.
template <bool VEC>
__device__ __forceinline__ v4f load_f4(const float *p, uint32_t idx, uint32_t nb) {
    if (VEC) return *reinterpret_cast<const v4f *>(p + idx);
    const v4f r = {p[min(idx, nb - 1)], p[min(idx + 1, nb - 1)], p[min(idx + 2, nb - 1)],
                   p[min(idx + 3, nb - 1)]};
    return r;
}

__device__ __forceinline__ float f4(const v4f &v, int i) { return v[i]; }

template <bool VEC>
__global__ __launch_bounds__(kGemvMaxWaves * 64) void gemv_kernel(
    const int8_t *__restrict__ a, const int8_t *__restrict__ w, const float *__restrict__ a_s,
    const float *__restrict__ w_s, uint16_t *__restrict__ out, uint32_t m, uint32_t n, uint32_t k,
    uint32_t blocks_per_wave) {
    __shared__ float red[kGemvMaxWaves][64][4];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = blockDim.x >> 6;
    const int q = lane >> 4;                      // 16-byte quarter of a 64-byte step
    const uint32_t n0 = blockIdx.x * kGemvCols;
    const uint32_t col = min(n0 + (lane & 15), n - 1);
    const uint32_t arow = lane & 15;              // activation row this lane feeds
    const bool a_live = arow < m;
    const uint32_t nb = k / 32;
    // scale rows this lane's outputs need: 4q + r (only q < 2 carries real rows)
    const uint32_t srow0 = min(4u * (uint32_t)q, m - 1);

    const int8_t *wrow = w + (uint64_t)col * k;
    const int8_t *arowp = a + (uint64_t)min(arow, m - 1) * k;
    const float *wsrow = w_s + (uint64_t)col * nb;

    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t b_begin = wave * blocks_per_wave;
    const uint32_t b_end = min(nb, b_begin + blocks_per_wave);
    const v4i zero4 = {0, 0, 0, 0};

    // One iteration = kGemvBlocksPerIter blocks = kSteps 64-byte steps.  Every
    // load of the iteration is issued before any is used, so each wave keeps
    // kSteps * 1 KB of weight bytes in flight.
    constexpr int kSteps = kGemvBlocksPerIter / 2;
    constexpr int kQuads = kGemvBlocksPerIter / 4;
    for (uint32_t b0 = b_begin; b0 < b_end; b0 += kGemvBlocksPerIter) {
        v4i wv[kSteps], av[kSteps];
        bool live[kSteps];
#pragma unroll
        for (int t = 0; t < kSteps; ++t) {
            const uint32_t blk = b0 + 2 * t + (q >> 1);  // block of this lane's quarter
            const uint64_t off = min((uint64_t)b0 * 32 + 64 * t + 16 * q, (uint64_t)k - 16);
            wv[t] = *reinterpret_cast<const v4i *>(wrow + off);
            av[t] = *reinterpret_cast<const v4i *>(arowp + off);  // dead lanes zeroed below
            live[t] = a_live && blk < b_end;
        }
        v4f wsv[kQuads], asv[kQuads][4];
#pragma unroll
        for (int h = 0; h < kQuads; ++h) {
            wsv[h] = load_f4<VEC>(wsrow, b0 + 4 * h, nb);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                asv[h][r] = load_f4<VEC>(a_s + (uint64_t)min(srow0 + r, m - 1) * nb, b0 + 4 * h, nb);
        }
#pragma unroll
        for (int t = 0; t < kSteps; ++t) {
            const v4i avl = live[t] ? av[t] : zero4;
            const v4i lo = q < 2 ? avl : zero4;  // first block of the step
            const v4i hi = q < 2 ? zero4 : avl;  // second block
            const v4i p0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(lo, wv[t], zero4, 0, 0, 0);
            const v4i p1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(hi, wv[t], zero4, 0, 0, 0);
            // blocks past b_end have zero activations, so P = 0 and they add nothing
            const int h = t >> 1, e = 2 * (t & 1);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc[r] = fmaf((float)p0[r], f4(asv[h][r], e) * f4(wsv[h], e), acc[r]);
                acc[r] = fmaf((float)p1[r], f4(asv[h][r], e + 1) * f4(wsv[h], e + 1), acc[r]);
            }
        }
    }

    // add the waves' partial sums in wave order
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][lane][r] = acc[r];
    __syncthreads();
    if (wave == 0 && lane < 32) {
        float tot[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int v = 0; v < nwaves; ++v)
#pragma unroll
            for (int r = 0; r < 4; ++r) tot[r] += red[v][lane][r];
        const uint32_t c = n0 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t row = 4 * q + r;
            if (row < m && c < n) out[(uint64_t)row * n + c] = f32_to_bf16_rne(tot[r]);
        }
    }
}

}  // namespace

hipError_t launch_gemv(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale,
                       const float *w_scale, uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                       hipStream_t s) {
    // Waves per workgroup: enough that the whole launch has ~24 waves per CU
    // (6144 waves over 256 CUs), but at least one iteration per wave.
    const uint32_t tiles = (uint32_t)div_up(n, kGemvCols);
    const uint32_t nb = k / 32;
    uint32_t waves = (uint32_t)div_up(6144, tiles);
    waves = max(1u, min(waves, (uint32_t)kGemvMaxWaves));
    waves = min(waves, (uint32_t)div_up(nb, kGemvBlocksPerIter));
    uint32_t bpw = (uint32_t)div_up(nb, waves);
    bpw = (uint32_t)div_up(bpw, kGemvBlocksPerIter) * kGemvBlocksPerIter;
    waves = (uint32_t)div_up(nb, bpw);
    if (nb % 4 == 0)
        hipLaunchKernelGGL(gemv_kernel<true>, dim3(tiles), dim3(64 * waves), 0, s, a_i8, w_i8, a_scale,
                           w_scale, out, m, n, k, bpw);
    else
        hipLaunchKernelGGL(gemv_kernel<false>, dim3(tiles), dim3(64 * waves), 0, s, a_i8, w_i8, a_scale,
                           w_scale, out, m, n, k, bpw);
    return hipGetLastError();
}

}  // namespace bsr
