/*
 * bsr_oracle.c -- plain, slow CPU oracle of the block-scaled int8 projection.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load, call or
 * link this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library, and it never reads a value the GPU produced.
 *
 * What it follows (page "metrale_model_layers/layers/ops/gemm_dense_int8.rs"):
 *   - doc comment of `requant_w_nvfp4_int8`: an NVFP4 weight (packed E2M1,
 *     one E4M3 scale per 16 elements, one per-tensor F32 `scale2`) becomes
 *     signed int8 `W_i8[N,K]` with one F32 scale per 32 elements
 *     `W_scale[N,K/32]`;
 *   - doc comment of `int8_gemm_faith2_prefill`: BF16 activations `[M,K]`
 *     become int8 with one F32 scale per 32 elements, then an int8 x int8
 *     block-scaled GEMM writes BF16 `out[M,N]`.
 * The pages fix neither the number formats' bit layouts nor the quantizer's
 * rounding; the readings taken here are:
 *   - E2M1 and E4M3 follow the OCP Microscaling Formats v1.0 and OCP 8-bit
 *     Floating Point (E4M3, "fn": no infinities, S.1111.111 is NaN) specs;
 *   - element 2j of a packed row is the low nibble of byte j;
 *   - the dequantized weight is (e2m1 * s16) * scale2 in binary32 (the first
 *     product is exact, so only the multiply by scale2 rounds);
 *   - per 32-block: amax = max |v|, s = fl32(amax / 127) (IEEE divide),
 *     s == 0 stores +0.0f and q = 0, else q = clamp(rne(fl32(v / s)), -127, 127)
 *     with round-half-to-even;
 *   - the reference output is the FP64 sum over blocks of
 *     (double)a_s * (double)w_s * (double)P, P the exact int32 block dot product.
 *
 * Arithmetic: IEEE binary32 round-to-nearest-even on every float op, built
 * with -ffp-contract=off and without fast-math, subnormals honoured.
 * OpenMP spreads independent rows over threads; it changes no arithmetic.
 *
 * Status codes: 0 ok, -1 k not a positive multiple of 32, -2 a non-finite
 * input or dequantized value (outside the method's contract).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_EK (-1)
#define ORC_ENONFINITE (-2)

/* ---- O1: OCP FP4 E2M1.  Sign bit 3, exponent bits 2..1 with bias 1,
 * mantissa bit 0.  Exponent field 0 is subnormal: 0.5 * m. ---------------- */
float orc_e2m1_value(uint32_t code)
{
    uint32_t sign = (code >> 3) & 1u;
    uint32_t e = (code >> 1) & 3u;
    uint32_t m = code & 1u;
    float mag;
    if (e == 0)
        mag = 0.5f * (float)m;
    else
        mag = ldexpf(1.0f + 0.5f * (float)m, (int)e - 1);
    return sign ? -mag : mag;
}

/* ---- O2: OCP FP8 E4M3.  Sign bit 7, exponent bits 6..3 with bias 7,
 * mantissa bits 2..0.  Exponent field 0 is subnormal: 2^-6 * m/8.
 * S.1111.111 is NaN; there is no infinity (largest finite value 448). ---- */
float orc_e4m3_value(uint32_t code)
{
    uint32_t sign = (code >> 7) & 1u;
    uint32_t e = (code >> 3) & 15u;
    uint32_t m = code & 7u;
    float mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexpf((float)m / 8.0f, -6);
    else
        mag = ldexpf(1.0f + (float)m / 8.0f, (int)e - 7);
    return sign ? -mag : mag;
}

/* BF16 is the upper half of a binary32; widening is exact. */
static float bf16_to_f32(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* ---- O4: one 32-element block -> 32 int8 codes and one F32 scale. ------- */
static int quantize_block32(const float *v, int8_t *q, float *scale)
{
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
        if (!isfinite(v[i]))
            return ORC_ENONFINITE;
        float a = fabsf(v[i]);
        if (a > amax)
            amax = a;
    }
    float s = amax / 127.0f;
    if (s == 0.0f) {
        *scale = 0.0f; /* +0.0f, also when amax / 127 underflows */
        memset(q, 0, 32);
        return ORC_OK;
    }
    *scale = s;
    for (int i = 0; i < 32; ++i) {
        float r = v[i] / s;      /* IEEE binary32 divide by the stored scale */
        float t = nearbyintf(r); /* round half to even (default rounding mode) */
        if (t > 127.0f)
            t = 127.0f;
        if (t < -127.0f)
            t = -127.0f;
        q[i] = (int8_t)t;
    }
    return ORC_OK;
}

/* ---- a1: NVFP4 weight -> int8 + F32 per 32 (one-time weight requant). ----
 * w_packed [n, k/2] u8, w_e4m3 [n, k/16] u8, scale2 f32 by value,
 * w_i8 [n, k] i8, w_scale [n, k/32] f32.  All row-major host buffers. */
int orc_requant_w(const uint8_t *w_packed, const uint8_t *w_e4m3, float scale2,
                  int8_t *w_i8, float *w_scale, int64_t n, int64_t k)
{
    if (k <= 0 || k % 32 != 0)
        return ORC_EK;
    int status = ORC_OK;
    const int64_t nb = k / 32;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < n; ++row) {
        float v[32];
        for (int64_t b = 0; b < nb; ++b) {
            for (int j = 0; j < 32; ++j) {
                int64_t idx = 32 * b + j;
                uint8_t byte = w_packed[row * (k / 2) + idx / 2];
                uint32_t code = (idx & 1) ? (uint32_t)(byte >> 4) : (uint32_t)(byte & 15u);
                float s16 = orc_e4m3_value(w_e4m3[row * (k / 16) + idx / 16]);
                float t = orc_e2m1_value(code) * s16; /* exact */
                v[j] = t * scale2;                    /* the one rounding */
            }
            int rc = quantize_block32(v, w_i8 + row * k + 32 * b, w_scale + row * nb + b);
            if (rc != ORC_OK) {
#pragma omp atomic write
                status = rc;
            }
        }
    }
    return status;
}

/* ---- a2: BF16 activations -> int8 + F32 per 32 (per-call requant). ------
 * a_bf16 [m, k] as raw u16 bits, a_i8 [m, k], a_scale [m, k/32]. */
int orc_requant_a(const uint16_t *a_bf16, int8_t *a_i8, float *a_scale, int64_t m, int64_t k)
{
    if (k <= 0 || k % 32 != 0)
        return ORC_EK;
    int status = ORC_OK;
    const int64_t nb = k / 32;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < m; ++row) {
        float v[32];
        for (int64_t b = 0; b < nb; ++b) {
            for (int j = 0; j < 32; ++j)
                v[j] = bf16_to_f32(a_bf16[row * k + 32 * b + j]);
            int rc = quantize_block32(v, a_i8 + row * k + 32 * b, a_scale + row * nb + b);
            if (rc != ORC_OK) {
#pragma omp atomic write
                status = rc;
            }
        }
    }
    return status;
}

/* ---- f1: SiLU(gate) * up, rounded to BF16, then the per-32 quantizer. ----
 * The pages name a quantizer of a SiLU product (`W8a8Kernels::quant_silu` on
 * page "metrale_model_layers/layers/ops/w8a8_decode/parts.rs", and the
 * re-quantized SiLU product between gate+up and down in the module comment of
 * page "metrale_model_layers/layers/ops/fp8_moe_grouped_tc_w8a8.rs")
 * without fixing its arithmetic.  Reading taken here, for BF16 gate g and up u
 * (widened exactly):
 *   e = exp(-g) correctly rounded to binary32 (evaluated in binary64, rounded once),
 *   silu = fl32(g / fl32(1 + e)),   h = bf16_rne(fl32(silu * u)),
 * and the 32-blocks of h are quantized exactly as the activation requant does,
 * so the fused step equals "SiLU·mul to BF16, then requant". */

/* Round a binary32 to the nearest BF16 value (8 significant bits), ties to
 * even, by rescaling the significand: no bit manipulation of the encoding. */
static float round_to_bf16(float x)
{
    if (x == 0.0f || !isfinite(x))
        return x;
    if (fabsf(x) < ldexpf(1.0f, -126)) /* BF16 subnormal grid: multiples of 2^-133 */
        return ldexpf(nearbyintf(ldexpf(x, 133)), -133);
    int e;
    float m = frexpf(x, &e); /* x = m * 2^e, 0.5 <= |m| < 1 */
    return ldexpf(nearbyintf(ldexpf(m, 8)), e - 8);
}

float orc_bf16_round(float x) { return round_to_bf16(x); }

/* exp(-g) rounded once to binary32 */
float orc_exp_neg_f32(float g) { return (float)exp(-(double)g); }

float orc_silu_mul(float g, float u)
{
    float e = orc_exp_neg_f32(g);
    float d = 1.0f + e;
    float silu = g / d;
    return round_to_bf16(silu * u);
}

/* gate, up: [m, ld] BF16 bits (the first k of each row are used);
 * q [m, k] i8 and scale [m, k/32] f32, dense. */
int orc_silu_mul_requant(const uint16_t *gate, const uint16_t *up, int64_t ld, int8_t *q,
                         float *scale, int64_t m, int64_t k)
{
    if (k <= 0 || k % 32 != 0 || ld < k)
        return ORC_EK;
    int status = ORC_OK;
    const int64_t nb = k / 32;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < m; ++row) {
        float v[32];
        for (int64_t b = 0; b < nb; ++b) {
            for (int j = 0; j < 32; ++j) {
                int64_t idx = row * ld + 32 * b + j;
                v[j] = orc_silu_mul(bf16_to_f32(gate[idx]), bf16_to_f32(up[idx]));
            }
            int rc = quantize_block32(v, q + row * k + 32 * b, scale + row * nb + b);
            if (rc != ORC_OK) {
#pragma omp atomic write
                status = rc;
            }
        }
    }
    return status;
}

/* ---- f4: other activation scale layouts and E4M3 activations. -----------
 * The W8A8 parts of page "metrale_model_layers/layers/ops/w8a8_decode/parts.rs"
 * (`W8a8Scale::PerRow`, `W8a8Scale::Block128`, the `[rows, k]` E4M3 activation
 * with its FP32 scales) and the per-(row, 128) E4M3 quantizer of page
 * ".../fp8_moe_grouped_tc_w8a8.rs" fix the layouts but not the arithmetic.
 * Reading taken: the per-32 rule above with the group size G (32, 128 or the
 * whole row) and, for E4M3, the format's largest finite value in place of 127:
 *   int8: s = fl32(amax / 127), q = clamp(rne(fl32(v / s)), -127, 127);
 *   E4M3: s = fl32(amax / 448), q = the OCP E4M3 code nearest fl32(v / s),
 *         ties to the even code, magnitudes above 448 saturating to 448;
 * s == 0 gives +0.0f and code 0 in both. */

/* Nearest OCP E4M3 code of a binary32 (ties to even, saturating at 448). */
uint32_t orc_e4m3_encode(float x)
{
    uint32_t sign = signbit(x) ? 0x80u : 0u;
    double a = fabs((double)x);
    if (a >= 448.0)
        return sign | 0x7Eu;
    if (a == 0.0)
        return sign;
    /* the finite E4M3 magnitudes: subnormals m * 2^-9 (m < 8), normals
     * (8 + m) * 2^(e - 10) for e = 1..15, m = 0..7 (excluding the NaN code) */
    int e;
    frexp(a, &e);                 /* a = f * 2^e, 0.5 <= f < 1 */
    int ex = e - 1 + 7;           /* biased exponent if a is normal */
    double unit = ex >= 1 ? ldexp(1.0, e - 1 - 3) : ldexp(1.0, -9);
    double n = nearbyint(a / unit); /* exact quotient (power-of-two unit), ties to even */
    uint32_t code;
    if (ex >= 1) {
        /* n in [8, 16]; 16 means the next binade's 8 */
        code = n >= 16.0 ? (uint32_t)((ex + 1) << 3) : (uint32_t)((ex << 3) | ((uint32_t)n - 8u));
    } else {
        code = (uint32_t)n; /* 8 is the smallest normal, code 0x08 */
    }
    if (code > 0x7Eu)
        code = 0x7Eu;
    return sign | code;
}

static int quantize_group(const float *v, int64_t g, int e4m3, uint8_t *q, float *scale)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < g; ++i) {
        if (!isfinite(v[i]))
            return ORC_ENONFINITE;
        float a = fabsf(v[i]);
        if (a > amax)
            amax = a;
    }
    float s = amax / (e4m3 ? 448.0f : 127.0f);
    if (s == 0.0f) {
        *scale = 0.0f;
        memset(q, 0, (size_t)g);
        return ORC_OK;
    }
    *scale = s;
    for (int64_t i = 0; i < g; ++i) {
        float r = v[i] / s;
        if (e4m3) {
            q[i] = (uint8_t)orc_e4m3_encode(r);
        } else {
            float t = nearbyintf(r);
            if (t > 127.0f)
                t = 127.0f;
            if (t < -127.0f)
                t = -127.0f;
            q[i] = (uint8_t)(int8_t)t;
        }
    }
    return ORC_OK;
}

/* a_bf16 [m, k] -> q [m, k] (int8 or E4M3 codes as bytes), scale [m, k / g];
 * group g = 32, 128 or k (one scale per row); g must divide k. */
int orc_quant_act(const uint16_t *a_bf16, uint8_t *q, float *scale, int64_t m, int64_t k,
                  int64_t g, int e4m3)
{
    if (k <= 0 || k % 32 != 0 || g <= 0 || k % g != 0)
        return ORC_EK;
    int status = ORC_OK;
    const int64_t ng = k / g;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < m; ++row) {
        float *v = (float *)malloc((size_t)g * sizeof(float));
        for (int64_t b = 0; b < ng; ++b) {
            for (int64_t j = 0; j < g; ++j)
                v[j] = bf16_to_f32(a_bf16[row * k + g * b + j]);
            int rc = quantize_group(v, g, e4m3, q + row * k + g * b, scale + row * ng + b);
            if (rc != ORC_OK) {
#pragma omp atomic write
                status = rc;
            }
        }
        free(v);
    }
    return status;
}

/* Reference of the int8 GEMM with activation scales per group of g (32, 128
 * or k): term = a_scale[i][32 b / g] * w_scale[j][b] * P[i, j, b]. */
int orc_gemm_ref_agroup(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale,
                        const float *w_scale, const int64_t *rows, int64_t nrows,
                        double *y, double *t, int64_t n, int64_t k, int64_t g)
{
    if (k <= 0 || k % 32 != 0 || g <= 0 || g % 32 != 0 || k % g != 0)
        return ORC_EK;
    const int64_t nb = k / 32, ng = k / g;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows[r];
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0, mag = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                int32_t p = 0;
                for (int u = 0; u < 32; ++u)
                    p += (int32_t)a_i8[i * k + 32 * b + u] * (int32_t)w_i8[j * k + 32 * b + u];
                double term = (double)a_scale[i * ng + (32 * b) / g] * (double)w_scale[j * nb + b] * (double)p;
                acc += term;
                mag += fabs(term);
            }
            y[r * n + j] = acc;
            t[r * n + j] = mag;
        }
    }
    return ORC_OK;
}

/* ---- O5: exact int32 block partials P[m, n, k/32]. --------------------- */
int orc_block_partials(const int8_t *a_i8, const int8_t *w_i8, int32_t *p,
                       int64_t m, int64_t n, int64_t k)
{
    if (k <= 0 || k % 32 != 0)
        return ORC_EK;
    const int64_t nb = k / 32;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j)
            for (int64_t b = 0; b < nb; ++b) {
                int32_t acc = 0;
                for (int t = 0; t < 32; ++t)
                    acc += (int32_t)a_i8[i * k + 32 * b + t] * (int32_t)w_i8[j * k + 32 * b + t];
                p[(i * n + j) * nb + b] = acc;
            }
    return ORC_OK;
}

/* ---- O6: FP64 reference output for the listed activation rows. ---------
 * y[r, j] = sum_b (double)a_s[row_r, b] * (double)w_s[j, b] * (double)P,
 * t[r, j] = sum_b |same term| (the magnitude the FP32 error bound scales with).
 * rows: nrows indices into [0, m); y and t are [nrows, n]. */
int orc_gemm_ref(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale,
                 const float *w_scale, const int64_t *rows, int64_t nrows,
                 double *y, double *t, int64_t n, int64_t k)
{
    if (k <= 0 || k % 32 != 0)
        return ORC_EK;
    const int64_t nb = k / 32;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows[r];
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0, mag = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                int32_t p = 0;
                for (int u = 0; u < 32; ++u)
                    p += (int32_t)a_i8[i * k + 32 * b + u] * (int32_t)w_i8[j * k + 32 * b + u];
                double term = (double)a_scale[i * nb + b] * (double)w_scale[j * nb + b] * (double)p;
                acc += term;
                mag += fabs(term);
            }
            y[r * n + j] = acc;
            t[r * n + j] = mag;
        }
    }
    return ORC_OK;
}

/* ---- f3: W4A16 decode GEMV reference (page "metrale_model_layers/layers/ops/
 * gemv_sw.rs": BF16 activations times an NVFP4 weight -- packed E2M1, one E4M3
 * scale per 16, one F32 scale_2 -- with no int8 requant).  The page gives only
 * the launch; the reading taken: the weight is dequantized exactly as in the
 * weight requant, e2m1 * s16 * scale2, and
 *   y[i][j] = sum_k x[i][k] * e2m1[j][k] * s16[j][k/16] * scale2
 * in FP64, where every term is exact (8 + 2 + 4 + 24 significant bits); t is
 * the sum of the terms' magnitudes, for the FP32 error bound.
 * x [m, k] BF16 bits, w_packed [n, k/2], w_e4m3 [n, k/16]; y, t [nrows, n]. */
int orc_w4a16_ref(const uint16_t *x_bf16, const uint8_t *w_packed, const uint8_t *w_e4m3,
                  float scale2, const int64_t *rows, int64_t nrows, double *y, double *t,
                  int64_t n, int64_t k)
{
    if (k <= 0 || k % 32 != 0)
        return ORC_EK;
    int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < n; ++j) {
        for (int64_t r = 0; r < nrows; ++r) {
            const int64_t i = rows[r];
            double acc = 0.0, mag = 0.0;
            for (int64_t c = 0; c < k; ++c) {
                uint8_t byte = w_packed[j * (k / 2) + c / 2];
                uint32_t code = (c & 1) ? (uint32_t)(byte >> 4) : (uint32_t)(byte & 15u);
                double w = (double)orc_e2m1_value(code) * (double)orc_e4m3_value(w_e4m3[j * (k / 16) + c / 16]) *
                           (double)scale2;
                double term = (double)bf16_to_f32(x_bf16[i * k + c]) * w;
                acc += term;
                mag += fabs(term);
            }
            if (!isfinite(acc)) {
#pragma omp atomic write
                status = ORC_ENONFINITE;
            }
            y[r * n + j] = acc;
            t[r * n + j] = mag;
        }
    }
    return status;
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}
