// bsr_internal.h -- launch geometry and device helpers shared by the kernels
// and the C-ABI layer.  Every geometry constant lives here once: the kernels
// are compiled against these values and the host derives grids from them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsr {

// ---- requant kernels ------------------------------------------------------
// Activation requant: one lane per 16-byte chunk (8 BF16), four lanes per
// 32-element block, 256 lanes per workgroup.
constexpr int kRqaThreads = 256;
constexpr int kRqaLanesPerBlock = 4;
constexpr int kRqaUnroll = 2;        // chunks per lane, loads issued together
// Weight requant: one lane per 32-element block (16 packed bytes in,
// 32 int8 out), 256 lanes per workgroup.
constexpr int kRqwThreads = 256;
constexpr int kRqwUnroll = 2;        // blocks per lane, loads issued together
constexpr int kSiluMinPasses = 8;    // fewest passes per workgroup for the SiLU table kernel
constexpr int kSiluThreads = 512;    // lanes per workgroup of the SiLU table kernel

// ---- GEMM (m > 16) --------------------------------------------------------
// A workgroup computes a BM x BN output tile; each wave owns a WM x WN piece
// made of 32 x 32 MFMA tiles.  The K loop stages kGemmStageBlocks 32-wide
// blocks of A, W and their scales per LDS buffer, in a ring of 2 (or 3)
// buffers.  Workgroups are ordered so that each XCD runs a compact
// kGemmGroupM-tall group of output tiles.  Shapes: 128 x 128 with four
// 64 x 64 waves, and 64 x 64 with four 32 x 32 waves for grids of the large
// tile too small to give every CU two workgroups; both run two workgroups per
// CU.  Grids with at most one or two tiles per CU split K inside the
// workgroup over groups of waves (64 x 64 or 32 x 32 tiles).
constexpr int kGemmBM = 128;
constexpr int kGemmBN = 128;
constexpr int kGemmSmallTile = 64;
constexpr int kGemmTinyTile = 32;
constexpr int kGemmStageBlocks = 4;
constexpr int kGemmStageBytes = 32 * kGemmStageBlocks;    // 128 bytes of K per row: whole cache lines
constexpr int kGemmGroupM = 8;
constexpr int kXcds = 8;
constexpr int kGemmCus = 256;                             // compute units of an MI355X

// ---- GEMV (m <= 16) -------------------------------------------------------
// A workgroup owns kGemvCols output columns and splits K over its waves; each
// wave runs 16-row MFMA tiles on (activation rows padded to 16) x (16 weight
// rows): v_mfma_i32_16x16x32_i8 per 32-wide block in the streamed kernel (K a
// multiple of 256), else v_mfma_i32_16x16x64_i8 per 64-byte step with the two
// blocks separated by zeroing half of the activation operand.  The waves'
// FP32 partial sums are added in LDS in a fixed order.
constexpr int kGemvCols = 16;
constexpr int kGemvMaxWaves = 16;
constexpr int kGemvMaxRows = 16;  // the rows of one 16x16 MFMA output tile
// The streamed GEMV (K a multiple of kGemvStreamKAlign) takes up to four
// 16-row tiles; the automatic path uses it for m <= kGemvStreamAutoRows when
// the grid has at most one 16-column workgroup per CU.
constexpr int kGemvStreamMaxRows = 64;
constexpr int kGemvStreamAutoRows = 48;
constexpr int kGemvStreamKAlign = 256;
constexpr int kGemvBlocksPerIter = 4;   // K blocks per loop iteration of a wave (two MFMA steps)

// ---- W4A16 decode GEMV (m <= 16, straight from NVFP4) -----------------------
// Same workgroup shape as the int8 GEMV; K in super-steps of 128, at most
// kW4PassSteps per staging pass of a wave.
constexpr int kW4PassSteps = 8;

inline uint64_t div_up(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

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
