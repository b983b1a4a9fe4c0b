/*
 * bsr.h -- C ABI of the MI355X (gfx950) block-scaled int8 projection library.
 *
 * The projection Y[M,N] = A[M,K] * W[N,K]^T runs in three steps, each one
 * entry point below:
 *   1. requant_w_nvfp4_int8  -- one-time: NVFP4 weight -> int8 + F32 per 32;
 *   2. requant_a_int8        -- per call: BF16 activations -> int8 + F32 per 32;
 *   3. int8_gemm_blockscaled -- int8 x int8 with an exact int32 dot product per
 *      32-wide K block, each block rescaled in FP32 by a_scale * w_scale,
 *      accumulated in FP32 and written as BF16 (a weight-streaming GEMV for
 *      M <= 16, and up to M = 48 on narrow grids; an MFMA GEMM otherwise).
 * The operations are those of page "metrale_model_layers/layers/ops/
 * gemm_dense_int8.rs": the doc comments of `requant_w_nvfp4_int8` and
 * `int8_gemm_faith2_prefill` (the latter's two launches are entry points 2
 * and 3 here).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensors are dense row-major DEVICE buffers owned by the caller; the
 *   library allocates nothing, keeps no pointer after it returns and never
 *   synchronises.  Host pointers are not accepted (undefined behaviour).
 * - Work is enqueued on `stream` (a hipStream_t passed as void*, NULL = the
 *   default stream).  Calls on one stream run in order, so the output of
 *   requant_a_int8 may be passed straight to int8_gemm_blockscaled.
 * - Sizes are uint32_t; index arithmetic inside is 64-bit.
 * - Validation happens before any launch: on an error nothing is launched and
 *   no output byte is written.  There is no fallback to another path.
 * - m == 0 or n == 0 is a valid empty problem: BSR_OK, nothing launched.
 * - k must be a positive multiple of 32 (every K/2, K/16, K/32 is whole).
 * - Inputs outside the method's contract (NaN/Inf activations, NaN E4M3
 *   scale codes, a non-finite dequantized weight) give unspecified output.
 * - Outputs must not alias inputs (undefined behaviour, not checked).
 * - The calling thread's current HIP device must be a gfx950 GPU; the device
 *   check is cached per device, so the library is safe to call from several
 *   host threads.
 *
 * Number formats: E2M1 per the OCP Microscaling Formats v1.0 spec, element
 * 2j of a packed byte row in the LOW nibble of byte j; E4M3 per the OCP 8-bit
 * floating point spec (no infinities, S.1111.111 NaN); BF16 = upper half of
 * an IEEE binary32.
 *
 * Quantizer (steps 1 and 2), per 32-element block of a row:
 *   amax = max |v|;  s = fl32(amax / 127) (IEEE divide), stored as the scale;
 *   s == 0 (zero block or underflow): scale +0.0f and q = 0;
 *   else q = clamp(round_half_even(fl32(v / s)), -127, 127).
 * Results are bit-identical to that definition (subnormals included).
 */
#ifndef BSR_H
#define BSR_H

#include <stdint.h>

/* The library is built with hidden visibility: exactly the functions declared
 * here are exported from libbsr.so. */
#if defined(__GNUC__) || defined(__clang__)
#define BSR_API __attribute__((visibility("default")))
#else
#define BSR_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum bsr_status {
    BSR_OK = 0,
    BSR_EINVAL = 1,  /* k == 0, k % 32 != 0, unsupported size, or bad `path` */
    BSR_ENULL = 2,   /* a required pointer is NULL (m, n > 0)                */
    BSR_EALIGN = 3,  /* a pointer is not aligned as stated per argument      */
    BSR_EDEVICE = 4, /* no current HIP device, or it is not gfx950           */
    BSR_ELAUNCH = 5  /* the kernel launch reported an error                  */
};

/*
 * Step 1, one-time weight requant (page ".../gemm_dense_int8.rs", doc of
 * `requant_w_nvfp4_int8`).
 *   w_packed [n, k/2]  u8  two E2M1 codes per byte, low nibble first; 16-byte aligned
 *   w_e4m3   [n, k/16] u8  E4M3 scale of elements 16c..16c+15;       2-byte aligned
 *   scale2             f32 per-tensor scale, by value; must be finite
 *   w_i8     [n, k]    i8  output codes in [-127, 127];              16-byte aligned
 *   w_scale  [n, k/32] f32 output scale of each 32-block;             4-byte aligned
 * Dequantized value: v = fl32(fl32(e2m1 * e4m3) * scale2) (the first product
 * is exact), then the quantizer above.
 * Errors: BSR_EINVAL (k, or scale2 not finite), BSR_ENULL, BSR_EALIGN,
 * BSR_EDEVICE, BSR_ELAUNCH.
 */
BSR_API int requant_w_nvfp4_int8(const uint8_t *w_packed, const uint8_t *w_e4m3, float scale2,
                                 int8_t *w_i8, float *w_scale, uint32_t n, uint32_t k, void *stream);

/*
 * Step 2, per-call activation requant (page ".../gemm_dense_int8.rs", doc of
 * `int8_gemm_faith2_prefill`, its first launch).
 *   a_bf16  [m, k]    BF16 as raw u16;  16-byte aligned
 *   a_i8    [m, k]    i8 output;        16-byte aligned (caller-owned scratch)
 *   a_scale [m, k/32] f32 output;        4-byte aligned (caller-owned scratch)
 * Errors: BSR_EINVAL, BSR_ENULL, BSR_EALIGN, BSR_EDEVICE, BSR_ELAUNCH.
 */
BSR_API int requant_a_int8(const uint16_t *a_bf16, int8_t *a_i8, float *a_scale,
                           uint32_t m, uint32_t k, void *stream);

/*
 * Step 3, block-scaled GEMM (page ".../gemm_dense_int8.rs", doc of
 * `int8_gemm_faith2_prefill`, its second launch).
 *   a_i8    [m, k]    i8,  16-byte aligned     w_i8    [n, k]    i8,  16-byte aligned
 *   a_scale [m, k/32] f32,  4-byte aligned     w_scale [n, k/32] f32,  4-byte aligned
 *   out     [m, n]    BF16 as raw u16, 2-byte aligned
 * out[i,j] = bf16_rne( FP32 sum over blocks b of fl32(a_scale[i,b] * w_scale[j,b])
 *            * P[i,j,b] ), P the exact int32 dot product of block b.  The FP32
 * summation order is the kernel's own (not part of the contract); the result
 * is within 4e-3 relative or 1 BF16 ulp of the FP64 value, or within the
 * worst-case FP32 error of a K/32-term sum where that is larger.
 * Scales must be finite: a NaN or Inf in a_scale or w_scale is outside the
 * contract and may make other rows' outputs non-finite too (the kernels read
 * a few scales past a row's last block and zero their products by
 * multiplying by 0).
 * m <= 16 (one 16-row matrix-core tile) runs the weight-streaming GEMV; so
 * does m <= 48 when k is a multiple of 256 and n <= 4096 (16-column
 * workgroups at most one per CU); other shapes run the MFMA GEMM.
 * Limit: for m > 16, k < 2^25 (the GEMM addresses a tile's 128 rows with
 * 32-bit offsets).
 * Errors: BSR_EINVAL (k; m > 16 with k >= 2^25), BSR_ENULL, BSR_EALIGN,
 * BSR_EDEVICE, BSR_ELAUNCH.
 */
BSR_API int int8_gemm_blockscaled(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale,
                                  const float *w_scale, uint16_t *out, uint32_t m, uint32_t n,
                                  uint32_t k, void *stream);

/* Paths of int8_gemm_blockscaled_ex. */
enum bsr_path {
    BSR_PATH_AUTO = 0, /* as int8_gemm_blockscaled                       */
    BSR_PATH_GEMM = 1, /* the MFMA GEMM at any m (k < 2^25)              */
    BSR_PATH_GEMV = 2, /* the GEMV; requires m <= 16, or m <= 64 with k a
                        * multiple of 256, else BSR_EINVAL              */
    BSR_PATH_INVARIANT = 3 /* m <= 16: a GEMV that accumulates every output
                            * over the K blocks in increasing order, as the
                            * GEMM does; m > 16: the GEMM.  A row's output
                            * bits then depend on neither m nor the path
                            * (the invariants stated for `W8a8Weight::segment`
                            * on page "metrale_model_layers/layers/ops/
                            * w8a8_decode/parts.rs" and for `nvfp4_proj_mx`
                            * on page ".../w4a4_proj/fixed.rs"); slower
                            * decode than BSR_PATH_GEMV, whose waves split K */
};

/*
 * int8_gemm_blockscaled with an explicit path, so tests can run both kernels
 * on the same rows (same arguments and errors; BSR_EINVAL for an unknown path).
 */
BSR_API int int8_gemm_blockscaled_ex(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale,
                                     const float *w_scale, uint16_t *out, uint32_t m, uint32_t n,
                                     uint32_t k, void *stream, int path);

/*
 * Workspace bytes int8_gemm_blockscaled_ws needs for an (m, n, k) problem: 0
 * when that problem runs without a K split (then no workspace is used), else
 * at most 8 MiB.  Pure host arithmetic, no device call.
 */
BSR_API uint64_t int8_gemm_blockscaled_ws_bytes(uint32_t m, uint32_t n, uint32_t k);

/*
 * int8_gemm_blockscaled with a caller workspace, for grids too small to fill
 * the GPU: m > 32 rows in fewer 64 x 64 output tiles than compute units with
 * k >= 8192 (e.g. m = 48..192 at n = 4096, k = 14336), where it measured
 * faster than the paths without workspace.  Each tile's K range is cut into
 * slices of whole 128-element
 * stages, one workgroup per (tile, slice), each writing its FP32 tile to the
 * workspace; a second launch adds the slices in slice order and rounds to
 * BF16.  Same step as the GEMM launch of `int8_gemm_faith2_prefill` (page
 * "metrale_model_layers/layers/ops/gemm_dense_int8.rs"); the FP32 sum per
 * output is (sum over the slices, in order, of each slice's chain over its
 * blocks), within the same tolerance as int8_gemm_blockscaled.  Problems
 * with no split (int8_gemm_blockscaled_ws_bytes == 0) run exactly as
 * int8_gemm_blockscaled and do not touch the workspace.
 *   arguments 1-8 as int8_gemm_blockscaled
 *   workspace        device buffer of workspace_bytes, 16-byte aligned; its
 *                    contents on entry do not matter, on return they are
 *                    scratch; it must not alias any other argument, and two
 *                    calls that may overlap in time must not share it
 * Errors: as int8_gemm_blockscaled; when a split runs, BSR_ENULL (workspace
 * NULL), BSR_EALIGN (workspace), BSR_EINVAL (workspace_bytes below
 * int8_gemm_blockscaled_ws_bytes(m, n, k)).
 */
BSR_API int int8_gemm_blockscaled_ws(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale,
                                     const float *w_scale, uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                                     void *workspace, uint64_t workspace_bytes, void *stream);

/*
 * int8_gemm_blockscaled_ws for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the K-split workspace is the library's own static device array
 * of 8 MiB per GPU (the most any split plan asks for), held until the process
 * ends; the call allocates nothing.  Same arguments as int8_gemm_blockscaled
 * and the same results as int8_gemm_blockscaled_ws, bit for bit.
 * Every call on one GPU shares that GPU's array: calls that may overlap in
 * time on one GPU (different streams, or several host threads) race and give
 * undefined results; calls ordered on one stream do not.  Nothing in the
 * array must start at zero (each call overwrites what it reads).
 * Errors: as int8_gemm_blockscaled; BSR_EINVAL if a split would need more
 * than the 8 MiB array (no problem size does); BSR_EDEVICE if the array's
 * device address cannot be obtained.
 */
BSR_API int int8_gemm_blockscaled_noalloc(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale,
                                          const float *w_scale, uint16_t *out, uint32_t m, uint32_t n,
                                          uint32_t k, void *stream);

/*
 * Fused SiLU·mul -> int8 per-32 requant: the quantized input of the down
 * projection, straight from the gate and up halves of a gate+up output (the
 * SiLU-product quantizer `W8a8Kernels::quant_silu` of page
 * "metrale_model_layers/layers/ops/w8a8_decode/parts.rs" and the re-quantized
 * SiLU product of page ".../fp8_moe_grouped_tc_w8a8.rs", here with the int8
 * per-32 quantizer of step 2).
 *   gate, up [m, ld] BF16 as raw u16, 16-byte aligned; columns 0..k-1 of each
 *            row are used (ld >= k, ld a multiple of 8).  Both halves of one
 *            [m, 2I] buffer qualify: gate = buf, up = buf + I, ld = 2I.
 *   a_i8     [m, k]    i8 output, dense, 16-byte aligned
 *   a_scale  [m, k/32] f32 output, dense, 4-byte aligned
 * Per element: e = exp(-g) rounded once to binary32 (evaluated in binary64),
 * h = bf16_rne(fl32(fl32(g / fl32(1 + e)) * u)); then the quantizer above on
 * the 32-blocks of h, so the result equals requant_a_int8 applied to the BF16
 * SiLU product.  (Where exp(-g) overflows binary32, g < -88.72, silu is -0.)
 * Errors: BSR_EINVAL (k, ld < k, ld not a multiple of 8), BSR_ENULL,
 * BSR_EALIGN, BSR_EDEVICE, BSR_ELAUNCH.
 */
BSR_API int silu_mul_requant_int8(const uint16_t *gate, const uint16_t *up, uint32_t ld, int8_t *a_i8,
                                  float *a_scale, uint32_t m, uint32_t k, void *stream);

/*
 * W4A16 decode GEMV straight from the NVFP4 weight, no int8 requant (the
 * decode launcher of page "metrale_model_layers/layers/ops/gemv_sw.rs":
 * BF16 input, packed weight, E4M3 weight scale, F32 scale_2, BF16 output).
 *   x_bf16   [m, k]    BF16 as raw u16, 16-byte aligned, 1 <= m <= 16
 *   w_packed [n, k/2]  u8 (E2M1 pairs, low nibble first), 16-byte aligned
 *   w_e4m3   [n, k/16] u8, 16-byte aligned when k % 256 == 0, else 2-byte
 *   out      [m, n]    BF16 as raw u16, 2-byte aligned
 * out[i,j] = bf16_rne( fl32( S * scale2 ) ), S an FP32 evaluation of the sum
 * over k of x[i,k] * e2m1[j,k] * s16[j,k/16] in the kernel's own order (for
 * k % 256 == 0 the exact products x * e2m1 are summed per 16-element scale
 * block and each block sum is multiplied by its s16; otherwise the exact
 * products x * (e2m1 * s16) are summed): within 4e-3 relative or 1 BF16 ulp
 * of the FP64 value, or within the worst-case FP32 error of a (k + 16)-term
 * sum.
 * Errors: BSR_EINVAL (k, m > 16, scale2 not finite), BSR_ENULL, BSR_EALIGN,
 * BSR_EDEVICE, BSR_ELAUNCH.
 */
BSR_API int w4a16_gemv(const uint16_t *x_bf16, const uint8_t *w_packed, const uint8_t *w_e4m3, float scale2,
                       uint16_t *out, uint32_t m, uint32_t n, uint32_t k, void *stream);

/* Activation code formats of quantize_act. */
enum bsr_format {
    BSR_FMT_INT8 = 0, /* int8 codes, scale = amax / 127                    */
    BSR_FMT_E4M3 = 1  /* OCP E4M3 codes (bias 7, max 448), amax / 448      */
};

/*
 * Activation quantizer with another scale layout: one F32 scale per group of
 * `group` consecutive elements of a row (32 or 128) or per row (group = 0),
 * int8 or E4M3 codes (the W8A8 activation layouts `W8a8Scale::PerRow` /
 * `W8a8Scale::Block128` and the FP8 activation of page
 * "metrale_model_layers/layers/ops/w8a8_decode/parts.rs"; the per-(row, 128)
 * E4M3 quantizer of page ".../fp8_moe_grouped_tc_w8a8.rs").
 *   a_bf16 [m, k]         BF16 as raw u16, 16-byte aligned, k % 32 == 0
 *                         (k % 128 == 0 for group 128)
 *   q      [m, k]         u8 codes (int8 two's complement or E4M3), 8-byte aligned
 *   scale  [m, k / group] F32 ([m] for group 0), 4-byte aligned
 * Per group: s = fl32(amax / F), F = 127 (int8) or 448 (E4M3); s == 0 gives
 * scale +0 and codes 0; else q = clamp(rne(fl32(v / s)), -127, 127) for int8
 * and the E4M3 code nearest fl32(v / s) (ties to the even code) for E4M3.
 * group 32 with BSR_FMT_INT8 equals requant_a_int8.
 * Errors: BSR_EINVAL (k, group, format), BSR_ENULL, BSR_EALIGN, BSR_EDEVICE,
 * BSR_ELAUNCH.
 */
BSR_API int quantize_act(const uint16_t *a_bf16, uint8_t *q, float *scale, uint32_t m, uint32_t k,
                         uint32_t group, int format, void *stream);

/*
 * int8_gemm_blockscaled_ex with int8 activations whose scales come per group
 * of a_group elements (32 or 128) or per row (a_group = 0), as quantize_act
 * writes them: block b of row r is rescaled by fl32(a_scale[r, (32 b) /
 * a_group] * w_scale[n, b]) (a_scale[r] for a_group 0), so the result equals
 * int8_gemm_blockscaled with each activation scale repeated over its blocks.
 *   a_scale [m, k / a_group] F32 ([m] for a_group 0), 4-byte aligned
 * Other arguments, path and the output tolerance as int8_gemm_blockscaled_ex.
 * Errors: BSR_EINVAL (a_group not 0/32/128, a_group 128 with k % 128 != 0,
 * or as int8_gemm_blockscaled_ex), BSR_ENULL, BSR_EALIGN, BSR_EDEVICE,
 * BSR_ELAUNCH.
 */
BSR_API int int8_gemm_blockscaled_agroup(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale,
                                         uint32_t a_group, const float *w_scale, uint16_t *out, uint32_t m,
                                         uint32_t n, uint32_t k, void *stream, int path);

/* Human-readable name of a status code (static storage, never NULL). */
BSR_API const char *bsr_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* BSR_H */
