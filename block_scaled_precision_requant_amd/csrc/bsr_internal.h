// bsr_internal.h -- launchers and device helpers shared by the kernels and
// the C-ABI layer.  The launch geometry constants live in bsr_geometry.h: the
// kernels are compiled against those values and the host derives grids from
// them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsr_geometry.h"

namespace bsr {

// Launchers (no validation: the C-ABI layer has checked every argument).
hipError_t launch_requant_w(const uint8_t *w_packed, const uint8_t *w_e4m3, float scale2,
                            int8_t *w_i8, float *w_scale, uint64_t nblocks, hipStream_t s);
hipError_t launch_requant_a(const uint16_t *a_bf16, int8_t *a_i8, float *a_scale,
                            uint64_t nblocks, hipStream_t s);
hipError_t launch_silu_requant(const uint16_t *gate, const uint16_t *up, uint32_t ld, int8_t *a_i8,
                               float *a_scale, uint32_t m, uint32_t k, hipStream_t s);
hipError_t launch_w4a16(const uint16_t *x, const uint8_t *w_packed, const uint8_t *w_e4m3, float scale2,
                        uint16_t *out, uint32_t m, uint32_t n, uint32_t k, hipStream_t s);
hipError_t launch_quant_act(const uint16_t *a_bf16, uint8_t *q, float *scale, uint32_t m, uint32_t k,
                            uint32_t group, bool e4m3, hipStream_t s);
// a_scale row r, block b: a_scale[r * a_ld + (b >> a_shift)] (a_ld = k / 32 and
// a_shift = 0 for one activation scale per block).
// split_k: small grids may split K inside a workgroup (a different FP32 sum
// order per output); false keeps every output one chain over the blocks.
hipError_t launch_gemm(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale, uint32_t a_ld,
                       uint32_t a_shift, const float *w_scale, uint16_t *out, uint32_t m, uint32_t n,
                       uint32_t k, bool split_k, hipStream_t s);
// The GEMM with K split across workgroups (plan from gemm_split_plan, slices
// >= 2): FP32 slice tiles into `partial` (plan.bytes, 16-byte aligned), then
// their ordered sum into out.
hipError_t launch_gemm_split(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale,
                             const float *w_scale, uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                             float *partial, const SplitPlan &plan, hipStream_t s);
// GEMV whose per-output accumulation follows the GEMM's block order.
hipError_t launch_gemv_chain(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale, uint32_t a_ld,
                             uint32_t a_shift, const float *w_scale, uint16_t *out, uint32_t m, uint32_t n,
                             uint32_t k, hipStream_t s);
// m <= kGemvMaxRows, or m <= kGemvStreamMaxRows with k % kGemvStreamKAlign == 0.
hipError_t launch_gemv(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale, uint32_t a_ld,
                       uint32_t a_shift, const float *w_scale, uint16_t *out, uint32_t m, uint32_t n,
                       uint32_t k, hipStream_t s);

}  // namespace bsr

namespace bsr {
// BF16 round-to-nearest-even of a finite or infinite binary32.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
}  // namespace bsr
