// requant.hip -- the two per-32 int8 quantizers for gfx950.
//
// Both follow page "metrale_model_layers/layers/ops/gemm_dense_int8.rs": the
// doc comment of `requant_w_nvfp4_int8` (NVFP4 weight -> int8 + F32 per 32)
// and the first launch of `int8_gemm_faith2_prefill` (BF16 activations ->
// int8 + F32 per 32).  Per block: amax = max|v|, s = fl32(amax/127),
// q = clamp(rne(fl32(v/s)), -127, 127); s == 0 gives +0.0f and q = 0.
// Results are bit-identical to that definition; the code only reorganises
// how the quotient's rounding is obtained:
//
//  * BF16 path: q0 = v * r with r ~ 1/s.  |q0 - v/s| < 2^-15 for |q0| <= 128,
//    so whenever q0 sits more than 2^-14 away from a half-integer, rne(q0)
//    equals rne(fl32(v/s)).  Elements closer than that take the IEEE divide.
//    A power-of-two s has an exact reciprocal (q0 is then exact); a subnormal
//    s takes the IEEE divide and the clamp for the whole block.
//  * NVFP4 path: a half-block holds one E4M3 scale, so its 16 elements take at
//    most 8 magnitudes.  The 7 non-zero magnitudes of each half are quantized
//    once (same reciprocal fast path; an element worth exactly half the block
//    max, the common tie, gets its code from one exact FMA residual; other
//    near ties and subnormal s take the IEEE divide), and every element picks
//    its code with a byte permute.
#include "bsr_internal.h"

namespace bsr {
namespace {

constexpr float kTieGuard = 0.5f - 0x1p-14f;

// Max over the four lanes of a quad (the lanes of one 32-element block).
__device__ __forceinline__ float quad_max(float x) {
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true)));
    return x;
}

// Low bytes of a, b, c, d (two's complement codes) packed in that order.
__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
    const uint32_t ab = __builtin_amdgcn_perm((uint32_t)b, (uint32_t)a, 0x0C0C0400u);  // [a, b, 0, 0]
    const uint32_t cd = __builtin_amdgcn_perm((uint32_t)d, (uint32_t)c, 0x0C0C0400u);  // [c, d, 0, 0]
    return __builtin_amdgcn_perm(cd, ab, 0x05040100u);                                 // [a, b, c, d]
}

__device__ __forceinline__ float local_amax(const float (&v)[8]) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    return amax;
}

// int8 codes of 8 values of a block with scale s = fl32(amax / 127).
__device__ __forceinline__ uint2 int8_codes(const float (&v)[8], float s) {
    float t[8];
    if (s == 0.0f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = 0.0f;
    } else if (s < 0x1p-126f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = fminf(fmaxf(rintf(v[i] / s), -127.0f), 127.0f);
    } else {
        const uint32_t sb = __float_as_uint(s);
        const bool pow2 = (sb & 0x007FFFFFu) == 0;
        const float r = pow2 ? __uint_as_float(0x7F000000u - (sb & 0x7F800000u))
                             : __builtin_amdgcn_rcpf(s);
        // largest distance of a quotient from its rounding: only when some
        // element is within 2^-14 of a half-integer is the divide needed
        float dev = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float q0 = v[i] * r;
            t[i] = rintf(q0);
            dev = fmaxf(dev, fabsf(q0 - t[i]));
        }
        if (!pow2 && dev > kTieGuard) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (fabsf(v[i] * r - t[i]) > kTieGuard) t[i] = rintf(v[i] / s);
        }
    }
    return make_uint2(pack4_i8((int)t[0], (int)t[1], (int)t[2], (int)t[3]),
                      pack4_i8((int)t[4], (int)t[5], (int)t[6], (int)t[7]));
}

// Nearest OCP E4M3 code of x (ties to even, saturating at 448).  Normal
// range: round the binary32 significand to 3 bits with an integer add (a
// carry moves into the exponent); below 2^-6 the grid is m * 2^-9.
__device__ __forceinline__ uint32_t e4m3_rne(float x) {
    const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
    const float a = fminf(fabsf(x), 448.0f);
    uint32_t code;
    if (a < 0x1p-6f) {
        code = (uint32_t)rintf(a * 512.0f);  // 8 is the smallest normal, code 0x08
    } else {
        const uint32_t b = __float_as_uint(a);
        const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
        code = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
    }
    return sign | code;
}

// E4M3 codes of 8 values of a block with scale s = fl32(amax / 448): the
// nearest E4M3 value of fl32(v / s), with the IEEE divide.  (A reciprocal
// fast path as in int8_codes does not pay here: with BF16 values and
// 448 = 7 * 2^6 many quotients fall exactly on E4M3 midpoints, so nearly
// every wave would also run the divide for its tied elements -- measured
// 40 % slower.)
__device__ __forceinline__ uint2 e4m3_codes(const float (&v)[8], float s) {
    if (s == 0.0f) return make_uint2(0u, 0u);
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = e4m3_rne(v[i] / s);  // IEEE divide, as the definition
    return make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                      c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
}

// Quantize 8 values (BF16-representable) of a block whose 32 values sit on
// the four lanes of a quad; returns the 8 codes packed and the block scale.
__device__ __forceinline__ uint2 requant_a_vals(const float (&v)[8], float &s_out) {
    const float amax = quad_max(local_amax(v));
    const float s = amax / 127.0f;
    s_out = s;
    return int8_codes(v, s);
}

// One 16-byte chunk (8 BF16, element 2i in the low half of word i).
__device__ __forceinline__ uint2 requant_a_chunk(uint4 raw, float &s_out) {
    const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(wd[i] << 16);
        v[2 * i + 1] = __uint_as_float(wd[i] & 0xFFFF0000u);
    }
    return requant_a_vals(v, s_out);
}

// Each lane handles U chunks kRqaThreads apart (all U loads are issued before
// any is used); a quad's four lanes always hold the four chunks of one block.
template <int U>
__global__ __launch_bounds__(kRqaThreads) void requant_a_kernel(const uint4 *__restrict__ a,
                                                                uint2 *__restrict__ q,
                                                                float *__restrict__ scale,
                                                                uint64_t nchunks) {
    const uint64_t base = (uint64_t)blockIdx.x * kRqaThreads * U + threadIdx.x;
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) raw[u] = a[min(base + (uint64_t)u * kRqaThreads, nchunks - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        // nchunks is a multiple of 4 and so is every quad's first chunk: a
        // quad is either wholly live or wholly idle.
        const uint64_t c = base + (uint64_t)u * kRqaThreads;
        float s;
        const uint2 packed = requant_a_chunk(raw[u], s);
        if (c < nchunks) {
            q[c] = packed;
            if ((c & 3) == 0) scale[c >> 2] = s;
        }
    }
}

// ---- fused SiLU·mul -> int8 per-32 (the down projection's input) ----------
// The pages' SiLU-product quantizer (`W8a8Kernels::quant_silu`, page
// "metrale_model_layers/layers/ops/w8a8_decode/parts.rs") feeds the int8
// per-32 quantizer above: h = bf16_rne(fl32(fl32(g / fl32(1 + e)) * u)) with
// e = exp(-g) rounded once to binary32 from a binary64 evaluation, then the
// 32-blocks of h are quantized exactly like BF16 activations.

__device__ __forceinline__ float silu32(float g) {
    const float e = (float)exp(-(double)g);
    return g / (1.0f + e);
}

__device__ __forceinline__ uint32_t silu_mul_bf16(uint32_t g_bits, uint32_t u_bits) {
    const float g = __uint_as_float(g_bits << 16), u = __uint_as_float(u_bits << 16);
    return f32_to_bf16_rne(silu32(g) * u);
}

// SiLU by table.  silu32 depends only on the 16-bit gate, and outside a band
// it has a closed form:
//   |g| < 2^-25:  exp(-g) rounds to 1, so silu32(g) = g / 2 (exact, = g * 0.5);
//   g >= 32:      1 + exp(-g) rounds to 1, so silu32(g) = g;
//   g <= -128:    exp(-g) overflows binary32, so silu32(g) = g / inf = -0.
// The band -- gates of either sign with exponent -25..6 -- is 64 binades x 128
// BF16 values, tabulated with silu32 itself (the positive gates from 32 up
// hold silu32(g) = g like the closed form).  Within it the index is a bit
// field of the gate: magnitude minus the band's lowest key in bits 0-11, sign
// in bit 12.
constexpr int kSiluPosBinades = 32, kSiluNegBinades = 32;
constexpr int kSiluTable = (kSiluPosBinades + kSiluNegBinades) * 128;
constexpr uint32_t kSiluLoExp = 127 - 25;  // biased exponent of the band's lowest binade

__device__ __forceinline__ uint32_t silu_table_bits(int i) {  // BF16 gate of table entry i
    const bool neg = i >= kSiluPosBinades * 128;
    const int j = neg ? i - kSiluPosBinades * 128 : i;
    return (neg ? 0x8000u : 0u) | ((kSiluLoExp + j / 128) << 7) | (uint32_t)(j % 128);
}

// b: BF16 gate bits (16 bits).  key = magnitude bits; the band is keys
// [lo, pos_hi) for positive gates and [lo, neg_hi) for negative ones.
__device__ __forceinline__ float silu_lookup(uint32_t b, const float *tab) {
    constexpr uint32_t lo = kSiluLoExp << 7;
    constexpr uint32_t pos_hi = (kSiluLoExp + kSiluPosBinades) << 7, neg_hi = (kSiluLoExp + kSiluNegBinades) << 7;
    const uint32_t key = b & 0x7FFFu;
    const bool neg = b >> 15;
    const uint32_t hi = neg ? neg_hi : pos_hi;
    // index of the clamped key in its sign's half of the table (one median)
    const uint32_t base = neg ? kSiluPosBinades * 128 - lo : 0u - lo;
    const float t = tab[min(max(key, lo), hi - 1) + base];
    const float g = __uint_as_float(b << 16);
    const float outer = neg ? -0.0f : g;  // key >= hi
    return key < lo ? g * 0.5f : (key >= hi ? outer : t);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// SiLU(gate) * up of one chunk, rounded to BF16 values (v_cvt_pk_bf16_f32:
// round to nearest even, as f32_to_bf16_rne on every non-NaN value; a NaN
// stays a NaN, which the quantizer treats alike whatever its payload).  Every gate
// in the band reads its table entry at the bit-field index; a lane holding a
// gate outside it redoes its chunk with silu_lookup.
__device__ __forceinline__ void silu_mul_chunk(uint4 gr, uint4 ur, const float *tab, float (&h)[8]) {
    constexpr uint32_t lo = kSiluLoExp << 7, band = kSiluPosBinades * 128;
    static_assert(kSiluPosBinades == kSiluNegBinades && band == 4096, "index = 12 bits of magnitude + sign");
    const uint32_t gw[4] = {gr.x, gr.y, gr.z, gr.w};
    const uint32_t uw[4] = {ur.x, ur.y, ur.z, ur.w};
    uint32_t b[8];
    float u[8], sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // element 2i in the low half of word i
        b[2 * i] = gw[i] & 0xFFFFu;
        b[2 * i + 1] = gw[i] >> 16;
        u[2 * i] = __uint_as_float(uw[i] << 16);
        u[2 * i + 1] = __uint_as_float(uw[i] & 0xFFFF0000u);
    }
    uint32_t off = 0;  // largest (magnitude - lo) mod 2^15: >= band iff some gate is outside
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t d = b[e] - lo;
        off = max(off, d & 0x7FFFu);
        sv[e] = tab[(d & (band - 1)) | ((b[e] >> 3) & band)];
    }
    if (off >= band) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[e] = silu_lookup(b[e], tab);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x2_t p = {sv[2 * i] * u[2 * i], sv[2 * i + 1] * u[2 * i + 1]};
        const uint32_t r = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2_t));
        h[2 * i] = __uint_as_float(r << 16);
        h[2 * i + 1] = __uint_as_float(r & 0xFFFF0000u);
    }
}

// Offset of chunk c (8 elements) in the gate / up rows: row c / kc, columns
// 8 * (c % kc) .. + 7, rows ld elements apart.
__device__ __forceinline__ uint64_t silu_chunk_offset(uint64_t c, uint32_t kc, uint32_t ld) {
    return (c / kc) * ld + (c % kc) * 8;
}

// Direct kernel (small inputs): each lane handles U chunks kRqaThreads apart,
// loads first, SiLU evaluated per element.
template <int U>
__global__ __launch_bounds__(kRqaThreads) void silu_requant_kernel(const uint16_t *__restrict__ gate,
                                                                   const uint16_t *__restrict__ up,
                                                                   uint32_t ld, uint2 *__restrict__ q,
                                                                   float *__restrict__ scale,
                                                                   uint64_t nchunks, uint32_t kc) {
    const uint64_t base = (uint64_t)blockIdx.x * kRqaThreads * U + threadIdx.x;
    uint4 gr[U], ur[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t off = silu_chunk_offset(min(base + (uint64_t)u * kRqaThreads, nchunks - 1), kc, ld);
        gr[u] = *reinterpret_cast<const uint4 *>(gate + off);
        ur[u] = *reinterpret_cast<const uint4 *>(up + off);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t c = base + (uint64_t)u * kRqaThreads;
        const uint32_t gw[4] = {gr[u].x, gr[u].y, gr[u].z, gr[u].w};
        const uint32_t uw[4] = {ur[u].x, ur[u].y, ur[u].z, ur[u].w};
        uint32_t hw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)   // element 2i in the low half of word i
            hw[i] = silu_mul_bf16(gw[i] & 0xFFFFu, uw[i] & 0xFFFFu) |
                    (silu_mul_bf16(gw[i] >> 16, uw[i] >> 16) << 16);
        float s;
        const uint2 packed = requant_a_chunk(make_uint4(hw[0], hw[1], hw[2], hw[3]), s);
        if (c < nchunks) {
            q[c] = packed;
            if ((c & 3) == 0) scale[c >> 2] = s;
        }
    }
}

// Table kernel (large inputs): persistent workgroups each fill the SiLU table
// in LDS once, then stride over the chunks, one per lane and pass.  The loads
// run two passes ahead of the arithmetic (three register sets, the loop
// unrolled by three so each set keeps its registers): the first two passes'
// loads go out before the table fill, and every pass issues the loads of the
// pass after next before computing its own.  Each lane tracks the (row, column)
// of its next load incrementally instead of dividing.
__global__ __launch_bounds__(kSiluThreads) void silu_requant_table_kernel(
    const uint16_t *__restrict__ gate, const uint16_t *__restrict__ up, uint32_t ld,
    uint2 *__restrict__ q, float *__restrict__ scale, uint64_t nchunks, uint32_t kc) {
    __shared__ float tab[kSiluTable];
    const uint64_t stride = (uint64_t)gridDim.x * kSiluThreads;
    const uint64_t s_row = stride / kc;
    const uint32_t s_col = (uint32_t)(stride % kc);
    const uint64_t last = silu_chunk_offset(nchunks - 1, kc, ld);
    const uint64_t c0 = (uint64_t)blockIdx.x * kSiluThreads + threadIdx.x;
    uint64_t cl = c0, row = c0 / kc;  // chunk, row and column of the next load
    uint32_t col = (uint32_t)(c0 % kc);
    auto load = [&](uint4 &g, uint4 &u) {
        const uint64_t off = cl < nchunks ? row * ld + col * 8 : last;
        g = *reinterpret_cast<const uint4 *>(gate + off);
        u = *reinterpret_cast<const uint4 *>(up + off);
        cl += stride;
        col += s_col;
        row += s_row;
        if (col >= kc) {
            col -= kc;
            ++row;
        }
    };
    uint4 g0, u0, g1, u1, g2, u2;
    load(g0, u0);
    load(g1, u1);
    for (int i = threadIdx.x; i < kSiluTable; i += kSiluThreads)
        tab[i] = silu32(__uint_as_float(silu_table_bits(i) << 16));
    __syncthreads();
    uint64_t c = c0;  // chunk of the next computation
    auto compute = [&](const uint4 &g, const uint4 &u) {
        float h[8], s;
        silu_mul_chunk(g, u, tab, h);
        const uint2 packed = requant_a_vals(h, s);
        q[c] = packed;
        if ((c & 3) == 0) scale[c >> 2] = s;
        c += stride;
    };
    while (c < nchunks) {
        load(g2, u2);
        compute(g0, u0);
        if (c >= nchunks) break;
        load(g0, u0);
        compute(g1, u1);
        if (c >= nchunks) break;
        load(g1, u1);
        compute(g2, u2);
    }
}

// ---- activation quantizers with other groups / E4M3 ----------------------
// The W8A8 activation layouts of page "metrale_model_layers/layers/ops/
// w8a8_decode/parts.rs" (scales per row or per (row, 128), E4M3 codes): the
// per-32 rule with group size G and, for E4M3, 448 in place of 127 and the
// nearest E4M3 code.

// Max over the 16 lanes of a DPP row: quads, then rotations by 4 and 8.
__device__ __forceinline__ float row16_max(float x) {
    x = quad_max(x);
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xF, 0xF, true)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, true)));
    return x;
}

__device__ __forceinline__ void bf16_chunk(uint4 raw, float (&v)[8]) {
    const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(wd[i] << 16);
        v[2 * i + 1] = __uint_as_float(wd[i] & 0xFFFF0000u);
    }
}

// Groups of LPG chunks (LPG = 4: 32 elements, 16: 128 elements) on LPG
// consecutive lanes; U chunks per lane, kRqaThreads apart, loads first.
template <bool E4M3, int LPG, int U>
__global__ __launch_bounds__(kRqaThreads) void quant_group_kernel(const uint4 *__restrict__ a,
                                                                  uint2 *__restrict__ q,
                                                                  float *__restrict__ scale,
                                                                  uint64_t nchunks) {
    static_assert(LPG == 4 || LPG == 16, "group of 32 or 128 elements");
    const uint64_t base = (uint64_t)blockIdx.x * kRqaThreads * U + threadIdx.x;
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) raw[u] = a[min(base + (uint64_t)u * kRqaThreads, nchunks - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        // nchunks is a multiple of LPG and so is every group's first chunk
        const uint64_t c = base + (uint64_t)u * kRqaThreads;
        float v[8];
        bf16_chunk(raw[u], v);
        const float amax = LPG == 4 ? quad_max(local_amax(v)) : row16_max(local_amax(v));
        const float s = amax / (E4M3 ? 448.0f : 127.0f);
        const uint2 codes = E4M3 ? e4m3_codes(v, s) : int8_codes(v, s);
        if (c < nchunks) {
            q[c] = codes;
            if (c % LPG == 0) scale[c / LPG] = s;
        }
    }
}

// One scale per row: one workgroup per row.  U > 0: the row's chunks (at
// most U per lane) stay in registers between the amax and the quantization;
// U = 0: two passes over the row (the second re-reads it from the caches).
template <bool E4M3, int U>
__global__ __launch_bounds__(kRqaThreads) void quant_row_kernel(const uint4 *__restrict__ a,
                                                                uint2 *__restrict__ q,
                                                                float *__restrict__ scale, uint32_t kc) {
    __shared__ float wmax[kRqaThreads / 64];
    const uint64_t row0 = (uint64_t)blockIdx.x * kc;
    uint4 raw[U > 0 ? U : 1];
    float amax = 0.0f;
    if constexpr (U > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t c = threadIdx.x + u * kRqaThreads;
            raw[u] = c < kc ? a[row0 + c] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float v[8];
            bf16_chunk(raw[u], v);  // +0 past the row's end
            amax = fmaxf(amax, local_amax(v));
        }
    } else {
        for (uint32_t c = threadIdx.x; c < kc; c += kRqaThreads) {
            float v[8];
            bf16_chunk(a[row0 + c], v);
            amax = fmaxf(amax, local_amax(v));
        }
    }
    amax = row16_max(amax);
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kRqaThreads / 64; ++w) amax = fmaxf(amax, wmax[w]);
    const float s = amax / (E4M3 ? 448.0f : 127.0f);
    if constexpr (U > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t c = threadIdx.x + u * kRqaThreads;
            if (c < kc) {
                float v[8];
                bf16_chunk(raw[u], v);
                q[row0 + c] = E4M3 ? e4m3_codes(v, s) : int8_codes(v, s);
            }
        }
    } else {
        for (uint32_t c = threadIdx.x; c < kc; c += kRqaThreads) {
            float v[8];
            bf16_chunk(a[row0 + c], v);
            q[row0 + c] = E4M3 ? e4m3_codes(v, s) : int8_codes(v, s);
        }
    }
    if (threadIdx.x == 0) scale[blockIdx.x] = s;
}

// The per-row kernel for kc chunks a row: chunks per lane rounded up to 1,
// 2, 4 or 8, else two passes.
template <bool E4M3>
void launch_quant_row(const uint4 *a, uint2 *q, float *scale, uint32_t m, uint32_t kc, hipStream_t s) {
    const uint64_t per_lane = div_up(kc, kRqaThreads);
    const dim3 grid(m), blk(kRqaThreads);
    if (per_lane <= 1) hipLaunchKernelGGL((quant_row_kernel<E4M3, 1>), grid, blk, 0, s, a, q, scale, kc);
    else if (per_lane <= 2) hipLaunchKernelGGL((quant_row_kernel<E4M3, 2>), grid, blk, 0, s, a, q, scale, kc);
    else if (per_lane <= 4) hipLaunchKernelGGL((quant_row_kernel<E4M3, 4>), grid, blk, 0, s, a, q, scale, kc);
    else if (per_lane <= 8) hipLaunchKernelGGL((quant_row_kernel<E4M3, 8>), grid, blk, 0, s, a, q, scale, kc);
    else hipLaunchKernelGGL((quant_row_kernel<E4M3, 0>), grid, blk, 0, s, a, q, scale, kc);
}

// OCP E4M3 code -> binary32.  Its exponent and mantissa bits shifted into a
// binary32 give the value times 2^-120 (E4M3 subnormals land on binary32
// subnormals), so one exact multiply restores it.
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
    const float mag = __uint_as_float((code & 0x7Fu) << 20) * 0x1p120f;
    return (code & 0x80u) ? -mag : mag;
}

// E2M1 magnitude code (0..7) -> binary32: the 3 bits shifted into a binary32
// give the value times 2^-126 (code 1 lands on a subnormal).
__device__ __forceinline__ float e2m1_mag_to_f32(uint32_t mcode) {
    return __uint_as_float(mcode << 22) * 0x1p126f;
}

// Highest magnitude code (0..7) among the 16 nibbles of two packed dwords.
__device__ __forceinline__ uint32_t max_mag_code(uint32_t w0, uint32_t w1) {
    // perm with a byte table {1,2,4,...,128} turns each 3-bit code into a one-hot byte.
    const uint32_t t_lo = 0x08040201u, t_hi = 0x80402010u;
    uint32_t x = __builtin_amdgcn_perm(t_hi, t_lo, w0 & 0x07070707u) |
                 __builtin_amdgcn_perm(t_hi, t_lo, (w0 >> 4) & 0x07070707u) |
                 __builtin_amdgcn_perm(t_hi, t_lo, w1 & 0x07070707u) |
                 __builtin_amdgcn_perm(t_hi, t_lo, (w1 >> 4) & 0x07070707u);
    x |= x >> 16;
    x |= x >> 8;
    return 31u - (uint32_t)__builtin_clz(x & 0xFFu);  // x != 0: every nibble sets a bit
}

// 8 codes of one packed dword -> 8 int8 (two dwords), given the byte tables
// of the half: pos = q of magnitude codes 0..7, neg = their negations.
__device__ __forceinline__ uint2 lookup8(uint32_t w, uint32_t pos_lo, uint32_t pos_hi,
                                         uint32_t neg_lo, uint32_t neg_hi) {
    const uint32_t w4 = w >> 4;
    const uint32_t sel_e = w & 0x07070707u, sel_o = w4 & 0x07070707u;
    const uint32_t sg_e = w & 0x08080808u, sg_o = w4 & 0x08080808u;
    const uint32_t mask_e = (sg_e << 5) - (sg_e >> 3);  // 0xFF in bytes whose sign bit is set
    const uint32_t mask_o = (sg_o << 5) - (sg_o >> 3);
    const uint32_t ev = (mask_e & __builtin_amdgcn_perm(neg_hi, neg_lo, sel_e)) |
                        (~mask_e & __builtin_amdgcn_perm(pos_hi, pos_lo, sel_e));
    const uint32_t od = (mask_o & __builtin_amdgcn_perm(neg_hi, neg_lo, sel_o)) |
                        (~mask_o & __builtin_amdgcn_perm(pos_hi, pos_lo, sel_o));
    // interleave: elements 0..3 = ev.b0 od.b0 ev.b1 od.b1, elements 4..7 = ev.b2 od.b2 ev.b3 od.b3
    return make_uint2(__builtin_amdgcn_perm(od, ev, 0x05010400u),
                      __builtin_amdgcn_perm(od, ev, 0x07030602u));
}

// Codes of the non-zero magnitudes of one half-block: qm[c] (c = 1..7) is the
// signed int8 code of v_c = fl32(fl32(mag_c * s16) * scale2) in a block of
// scale s = fl32(amax / 127) != 0, i.e. rne(fl32(v_c / s)), clamped (reachable
// only for subnormal s).  Normal s uses the reciprocal fast path of the
// activation kernel (q0 = v * r within 2^-15 of v / s, so away from a
// half-integer rne(q0) is the answer), with one exception settled exactly:
//
//   an element worth exactly half the block max (|v| = amax / 2, the usual
//   source of ties in E2M1 data, e.g. magnitude 3 under a max of 6) has the
//   quotient fl32(amax / s) / 2.  As |amax / s - 127| < 2^-17 (s is amax / 127
//   rounded), fl32(amax / s) is 127 or a neighbour, so the code is 63 when
//   fl32(amax / s) < 127, i.e. when amax - 127 s < -2^-18 s, and 64 otherwise
//   (63.5 itself rounds to even).  Both sides of that comparison are exact:
//   the FMA residual has fewer than 8 significant bits above ulp(s), and the
//   power-of-two product stays normal for s >= 2^-100 (q_half is only used
//   there).
//
// Any other quotient within 2^-14 of a half-integer sends the half through
// one branch that recomputes those codes with the IEEE divide.
__device__ __forceinline__ void half_codes(float s16, float scale2, float amax, float s, float r,
                                           bool exact_r, bool sub, bool use_half, float q_half,
                                           int (&qm)[8]) {
    const float mags[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    const float half_amax = 0.5f * amax;
    const float q_half_signed = copysignf(q_half, s16 * scale2);  // every v_c has this sign
    float v[8], t[8];
    bool is_half[8], near[8];
    bool any_near = false;
#pragma unroll
    for (int c = 1; c < 8; ++c) {
        v[c] = (mags[c] * s16) * scale2;  // exact product, one rounding
        // a magnitude above the block max (|q0| > 128) occurs in no element of
        // this half: its table entry is never read, so it is kept off the tie check
        const float q0 = fminf(fmaxf(v[c] * r, -128.0f), 128.0f);
        const float tt = rintf(q0);
        is_half[c] = use_half && fabsf(v[c]) == half_amax;
        near[c] = !is_half[c] && fabsf(q0 - tt) > kTieGuard;
        t[c] = is_half[c] ? q_half_signed : tt;
        any_near |= near[c];
    }
    if (sub || (!exact_r && any_near)) {
#pragma unroll
        for (int c = 1; c < 8; ++c) {
            if (sub)
                t[c] = fminf(fmaxf(rintf(v[c] / s), -127.0f), 127.0f);
            else if (near[c])
                t[c] = rintf(v[c] / s);
        }
    }
    qm[0] = 0;
#pragma unroll
    for (int c = 1; c < 8; ++c) qm[c] = (int)t[c];
}

// Quantize one 32-element block: 16 packed bytes and its two E4M3 scales.
__device__ __forceinline__ void requant_w_block(uint4 p, uint32_t sc, float scale2, uint4 &lo,
                                                uint4 &hi, float &s_out) {
    const float s16[2] = {e4m3_to_f32(sc & 0xFFu), e4m3_to_f32(sc >> 8)};
    const uint32_t mc[2] = {max_mag_code(p.x, p.y), max_mag_code(p.z, p.w)};

    float amax = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) amax = fmaxf(amax, fabsf((e2m1_mag_to_f32(mc[h]) * s16[h]) * scale2));
    const float s = amax / 127.0f;

    lo = make_uint4(0, 0, 0, 0);
    hi = make_uint4(0, 0, 0, 0);
    if (s != 0.0f) {
        const uint32_t sb = __float_as_uint(s);
        const bool sub = s < 0x1p-126f;
        const bool pow2 = (sb & 0x007FFFFFu) == 0;
        const float r = pow2 ? __uint_as_float(0x7F000000u - (sb & 0x7F800000u)) : __builtin_amdgcn_rcpf(s);
        const bool use_half = s >= 0x1p-100f;
        const float q_half = fmaf(-127.0f, s, amax) < -0x1p-18f * s ? 63.0f : 64.0f;
        uint32_t tab[2][4];  // pos_lo, pos_hi, neg_lo, neg_hi per half
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            int qm[8];
            half_codes(s16[h], scale2, amax, s, r, pow2, sub, use_half, q_half, qm);
            tab[h][0] = pack4_i8(qm[0], qm[1], qm[2], qm[3]);
            tab[h][1] = pack4_i8(qm[4], qm[5], qm[6], qm[7]);
            tab[h][2] = pack4_i8(-qm[0], -qm[1], -qm[2], -qm[3]);
            tab[h][3] = pack4_i8(-qm[4], -qm[5], -qm[6], -qm[7]);
        }
        const uint2 e0 = lookup8(p.x, tab[0][0], tab[0][1], tab[0][2], tab[0][3]);
        const uint2 e1 = lookup8(p.y, tab[0][0], tab[0][1], tab[0][2], tab[0][3]);
        const uint2 e2 = lookup8(p.z, tab[1][0], tab[1][1], tab[1][2], tab[1][3]);
        const uint2 e3 = lookup8(p.w, tab[1][0], tab[1][1], tab[1][2], tab[1][3]);
        lo = make_uint4(e0.x, e0.y, e1.x, e1.y);
        hi = make_uint4(e2.x, e2.y, e3.x, e3.y);
    }
    s_out = s;
}

// Each lane handles U blocks kRqwThreads apart, all loads issued first.  The
// 64 consecutive blocks of a wave (2 KB of codes) go out through LDS, so every
// store instruction writes 1 KB of consecutive bytes.
template <int U>
__global__ __launch_bounds__(kRqwThreads) void requant_w_kernel(const uint4 *__restrict__ packed,
                                                                const uint16_t *__restrict__ e4m3,
                                                                float scale2,
                                                                uint4 *__restrict__ q,
                                                                float *__restrict__ scale,
                                                                uint64_t nblocks) {
    __shared__ uint4 stage[kRqwThreads * 2];
    const int lane = threadIdx.x & 63;
    uint4 *wst = stage + (threadIdx.x & ~63) * 2;  // this wave's 128 16-byte slots
    const uint64_t base = (uint64_t)blockIdx.x * kRqwThreads * U + threadIdx.x;
    uint4 p[U];
    uint32_t sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t b = min(base + (uint64_t)u * kRqwThreads, nblocks - 1);
        p[u] = packed[b];
        sc[u] = e4m3[b];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t b = base + (uint64_t)u * kRqwThreads;
        const uint64_t b0 = b - lane;  // the wave's first block
        uint4 lo, hi;
        float s;
        requant_w_block(p[u], sc[u], scale2, lo, hi, s);
        if (b < nblocks) scale[b] = s;
        wst[2 * lane] = lo;
        wst[2 * lane + 1] = hi;
        __builtin_amdgcn_wave_barrier();
        const uint4 v0 = wst[lane], v1 = wst[64 + lane];
        if (b0 + lane / 2 < nblocks) q[2 * b0 + lane] = v0;
        if (b0 + 32 + lane / 2 < nblocks) q[2 * b0 + 64 + lane] = v1;
        __builtin_amdgcn_wave_barrier();
    }
}

}  // namespace

hipError_t launch_requant_a(const uint16_t *a_bf16, int8_t *a_i8, float *a_scale, uint64_t nblocks,
                            hipStream_t s) {
    const uint64_t nchunks = nblocks * kRqaLanesPerBlock;
    const uint64_t grid = div_up(nchunks, (uint64_t)kRqaThreads * kRqaUnroll);
    hipLaunchKernelGGL(requant_a_kernel<kRqaUnroll>, dim3((uint32_t)grid), dim3(kRqaThreads), 0, s,
                       reinterpret_cast<const uint4 *>(a_bf16), reinterpret_cast<uint2 *>(a_i8),
                       a_scale, nchunks);
    return hipGetLastError();
}

hipError_t launch_silu_requant(const uint16_t *gate, const uint16_t *up, uint32_t ld, int8_t *a_i8,
                               float *a_scale, uint32_t m, uint32_t k, hipStream_t s) {
    const uint32_t kc = k / 8;
    const uint64_t nchunks = (uint64_t)m * kc;
    // Table kernel once there is work for at least one workgroup per CU with
    // kSiluMinPasses passes each (its table costs ~16 SiLU evaluations per
    // lane); up to 4 workgroups of 8 waves per CU (LDS: 32 KB each).
    const uint64_t table_grid = min(div_up(nchunks, (uint64_t)kSiluThreads * kSiluMinPasses), (uint64_t)4 * kGemmCus);
    if (table_grid >= (uint64_t)kGemmCus) {
        hipLaunchKernelGGL(silu_requant_table_kernel, dim3((uint32_t)table_grid), dim3(kSiluThreads),
                           0, s, gate, up, ld, reinterpret_cast<uint2 *>(a_i8), a_scale, nchunks, kc);
    } else {
        const uint64_t grid = div_up(nchunks, (uint64_t)kRqaThreads * kRqaUnroll);
        hipLaunchKernelGGL(silu_requant_kernel<kRqaUnroll>, dim3((uint32_t)grid), dim3(kRqaThreads), 0, s,
                           gate, up, ld, reinterpret_cast<uint2 *>(a_i8), a_scale, nchunks, kc);
    }
    return hipGetLastError();
}

hipError_t launch_quant_act(const uint16_t *a_bf16, uint8_t *q, float *scale, uint32_t m, uint32_t k,
                            uint32_t group, bool e4m3, hipStream_t s) {
    const uint32_t kc = k / 8;
    const uint64_t nchunks = (uint64_t)m * kc;
    const uint4 *a = reinterpret_cast<const uint4 *>(a_bf16);
    uint2 *qq = reinterpret_cast<uint2 *>(q);
    const dim3 blk(kRqaThreads);
    const dim3 grid((uint32_t)div_up(nchunks, (uint64_t)kRqaThreads * kRqaUnroll));
    if (group == 0) {
        if (e4m3) launch_quant_row<true>(a, qq, scale, m, kc, s);
        else launch_quant_row<false>(a, qq, scale, m, kc, s);
    } else if (group == 32) {
        if (e4m3) hipLaunchKernelGGL((quant_group_kernel<true, 4, kRqaUnroll>), grid, blk, 0, s, a, qq, scale, nchunks);
        else hipLaunchKernelGGL((quant_group_kernel<false, 4, kRqaUnroll>), grid, blk, 0, s, a, qq, scale, nchunks);
    } else {
        if (e4m3) hipLaunchKernelGGL((quant_group_kernel<true, 16, kRqaUnroll>), grid, blk, 0, s, a, qq, scale, nchunks);
        else hipLaunchKernelGGL((quant_group_kernel<false, 16, kRqaUnroll>), grid, blk, 0, s, a, qq, scale, nchunks);
    }
    return hipGetLastError();
}

hipError_t launch_requant_w(const uint8_t *w_packed, const uint8_t *w_e4m3, float scale2,
                            int8_t *w_i8, float *w_scale, uint64_t nblocks, hipStream_t s) {
    const uint64_t grid = div_up(nblocks, (uint64_t)kRqwThreads * kRqwUnroll);
    hipLaunchKernelGGL(requant_w_kernel<kRqwUnroll>, dim3((uint32_t)grid), dim3(kRqwThreads), 0, s,
                       reinterpret_cast<const uint4 *>(w_packed),
                       reinterpret_cast<const uint16_t *>(w_e4m3), scale2,
                       reinterpret_cast<uint4 *>(w_i8), w_scale, nblocks);
    return hipGetLastError();
}

}  // namespace bsr
