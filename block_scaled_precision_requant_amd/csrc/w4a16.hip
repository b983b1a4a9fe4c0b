// w4a16.hip -- decode GEMV straight from the NVFP4 weight (no int8 requant).
//
// Page "metrale_model_layers/layers/ops/gemv_sw.rs" launches a W4A16 decode
// GEMV: BF16 activations times an NVFP4 weight (packed E2M1, one E4M3 scale
// per 16 elements, one F32 scale_2).  Result definition used here:
//   out[i, j] = bf16_rne( fl32( S[i, j] * scale_2 ) ),
//   S[i, j]   = FP32 sum over k of x[i, k] * (e2m1[j, k] * s16[j, k / 16]),
// where every product is exact (e2m1 * s16 has at most 6 significant bits, so
// it is a BF16 value, and BF16 x BF16 is exact in FP32); only the FP32 sum
// (order: the kernel's own) and the two final roundings are inexact.
//
// Mapping.  Workgroup = 16 output columns x all of K, K split over its waves
// in super-steps of 128.  In a super-step lane l (column c = l % 16, quarter
// q = l / 16) owns K range [128 T + 32 q, +32): it loads those 16 packed bytes
// of weight row n0 + c (16 rows x 64 contiguous bytes per instruction), turns
// each dword (8 codes) into 8 BF16 weights with byte-table lookups, and feeds
// four v_mfma_f32_16x16x32_bf16 whose activation operand is the matching 8
// BF16 of activation row c (rows >= m only feed outputs that are dropped).
// Within an MFMA the K order is a lane's own, the same for both operands, so
// the pairing of x and w is exact.  Activations are staged per wave in LDS
// (global_load_lds); each pass of at most kW4PassSteps super-steps issues all
// of its weight and scale loads before any is used.
#include "bsr_internal.h"

namespace bsr {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kStepK = 128;  // K per super-step

// OCP E4M3 code -> binary32 (exact): exponent and mantissa bits shifted into a
// binary32 give the value times 2^-120.
__device__ __forceinline__ float e4m3_value(uint32_t code) {
    const float mag = __uint_as_float((code & 0x7Fu) << 20) * 0x1p120f;
    return (code & 0x80u) ? -mag : mag;
}

// BF16 of e2m1_magnitude(c) * s for c = 0..7, as byte tables: hi*/lo* hold
// the high / low bytes of codes 0-3 (suffix 0) and 4-7 (suffix 1).
struct ByteTable {
    uint32_t hi0, hi1, lo0, lo1;
};

__device__ __forceinline__ ByteTable make_table(uint32_t scale_code) {
    const float s = e4m3_value(scale_code);
    // the products are exact (<= 6 significant bits): their upper halves are the BF16 values
    const uint32_t b1 = __float_as_uint(0.5f * s), b2 = __float_as_uint(s), b3 = __float_as_uint(1.5f * s);
    const uint32_t b4 = __float_as_uint(2.0f * s), b5 = __float_as_uint(3.0f * s);
    const uint32_t b6 = __float_as_uint(4.0f * s), b7 = __float_as_uint(6.0f * s);
    const uint32_t p01 = __builtin_amdgcn_perm(b1, 0u, 0x07060302u);  // [bf16(0), bf16(v1)]
    const uint32_t p23 = __builtin_amdgcn_perm(b3, b2, 0x07060302u);
    const uint32_t p45 = __builtin_amdgcn_perm(b5, b4, 0x07060302u);
    const uint32_t p67 = __builtin_amdgcn_perm(b7, b6, 0x07060302u);
    ByteTable t;
    t.hi0 = __builtin_amdgcn_perm(p23, p01, 0x07050301u);
    t.lo0 = __builtin_amdgcn_perm(p23, p01, 0x06040200u);
    t.hi1 = __builtin_amdgcn_perm(p67, p45, 0x07050301u);
    t.lo1 = __builtin_amdgcn_perm(p67, p45, 0x06040200u);
    return t;
}

// 8 codes of one dword (element 2b in the low nibble of byte b, 2b+1 in the
// high one) -> 8 BF16 in element order.  Sign bit 3 of a code flips the sign
// bit of its BF16 (a negative scale is already in the table).
__device__ __forceinline__ v4i decode8(uint32_t w, const ByteTable &t) {
    const uint32_t w4 = w >> 4;
    const uint32_t se = w & 0x07070707u, so = w4 & 0x07070707u;
    const uint32_t ge = (w << 4) & 0x80808080u, go = w & 0x80808080u;
    const uint32_t hie = __builtin_amdgcn_perm(t.hi1, t.hi0, se) ^ ge;
    const uint32_t loe = __builtin_amdgcn_perm(t.lo1, t.lo0, se);
    const uint32_t hio = __builtin_amdgcn_perm(t.hi1, t.hi0, so) ^ go;
    const uint32_t loo = __builtin_amdgcn_perm(t.lo1, t.lo0, so);
    const uint32_t e02 = __builtin_amdgcn_perm(hie, loe, 0x05010400u);  // [e0, e2]
    const uint32_t e46 = __builtin_amdgcn_perm(hie, loe, 0x07030602u);  // [e4, e6]
    const uint32_t e13 = __builtin_amdgcn_perm(hio, loo, 0x05010400u);  // [e1, e3]
    const uint32_t e57 = __builtin_amdgcn_perm(hio, loo, 0x07030602u);  // [e5, e7]
    v4i r;
    r.x = __builtin_amdgcn_perm(e13, e02, 0x05040100u);  // [e0, e1]
    r.y = __builtin_amdgcn_perm(e13, e02, 0x07060302u);  // [e2, e3]
    r.z = __builtin_amdgcn_perm(e57, e46, 0x05040100u);  // [e4, e5]
    r.w = __builtin_amdgcn_perm(e57, e46, 0x07060302u);  // [e6, e7]
    return r;
}

// s_waitcnt vmcnt(n); expcnt and lgkmcnt left at their maxima.
template <int n>
__device__ __forceinline__ void wait_vm_le() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
}

// Per-wave LDS region: m activation rows of a_pitch bytes (one pass of
// super-steps plus 16 bytes, so the 16 lanes of a quarter reading 16 rows at
// one offset spread over the banks).
__host__ __device__ inline uint32_t w4_pitch(uint32_t pass_steps) { return pass_steps * kStepK * 2 + 16; }

// VS: every weight row's scales start 16-byte aligned (K % 256 == 0) and
// every pass starts at an even super-step, so a lane reads its row's scale
// bytes for a pass with 16-byte loads (8 bytes per super-step); otherwise it
// reads its own two codes per super-step with 2-byte loads.
// PS: super-steps per staging pass (at most kW4PassSteps; even when VS).
// CT: 16-column tiles per workgroup; each wave runs all CT tiles over its K
// range with one staged copy of the activations, so larger m (whose
// activation bytes rival the weight bytes) copies them fewer times.
// (wp and we are not __restrict__: a restrict-qualified read-only load may be
// moved past the empty asm statements that keep a pass's loads ahead of its
// compute.)
template <bool VS, int PS, int CT>
__global__ __launch_bounds__(kGemvMaxWaves * 64) void w4a16_kernel(
    const uint16_t *__restrict__ x, const uint8_t *wp, const uint8_t *we,
    float scale2, uint16_t *__restrict__ out, uint32_t m, uint32_t n, uint32_t k, uint32_t steps_per_wave) {
    static_assert(PS >= 1 && PS <= kW4PassSteps, "pass length");
    static_assert(!VS || PS % 2 == 0, "16-byte scale loads cover two super-steps");
    constexpr uint32_t pass_steps = PS;
    extern __shared__ __attribute__((aligned(1024))) int8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = blockDim.x >> 6;
    const int q = lane >> 4;
    const uint32_t c = lane & 15;
    const uint32_t n0 = blockIdx.x * kGemvCols * CT;
    const uint32_t nsteps = (k + kStepK - 1) / kStepK;
    const uint32_t s_begin = wave * steps_per_wave;
    const uint32_t s_end = min(nsteps, s_begin + steps_per_wave);
    const uint32_t pitch = w4_pitch(pass_steps);
    int8_t *la = smem + (uint64_t)wave * (m * pitch);
    const uint32_t arow = min(c, m - 1);  // activation row this lane feeds
    const uint8_t *wrow[CT];
    const uint8_t *srow[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const uint32_t col = min(n0 + kGemvCols * ct + c, n - 1);
        wrow[ct] = wp + (uint64_t)col * (k / 2);
        srow[ct] = we + (uint64_t)col * (k / 16);
    }

    v4f acc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    for (uint32_t p0 = s_begin; p0 < s_end; p0 += pass_steps) {
        const uint32_t plen = min(pass_steps, s_end - p0);
        // 1. activations of the pass: m rows of plen * 128 BF16, 1 KB copies
        //    (lanes in a row's padding, or past K, re-read the row's last 16 bytes)
        const uint32_t a_bytes = m * pitch;
        for (uint32_t b0 = 0; b0 < a_bytes; b0 += 1024) {
            const uint32_t p = b0 + 16 * lane;
            const uint32_t r = min(p / pitch, m - 1);
            const uint64_t e = min((uint64_t)p0 * kStepK + (p % pitch) / 2, (uint64_t)k - 8);
            if (p < a_bytes)
                __builtin_amdgcn_global_load_lds(x + (uint64_t)r * k + e, (lds_void *)(la + b0), 16, 0, 0);
        }
        asm volatile("" ::: "memory");
        // 2. weights and scale codes, in the order the super-steps use them
        //    (clamped loads keep the code straight-line)
        v4i wv[CT][PS];
        uint32_t sc[CT][PS];
        auto load_w = [&](int ct, int j) {
            const uint32_t kk = min((p0 + min((uint32_t)j, plen - 1)) * kStepK + 32 * q, k - 32);
            wv[ct][j] = *reinterpret_cast<const v4i *>(wrow[ct] + kk / 2);
        };
        if constexpr (VS) {
            // 8 scale bytes per super-step: one 16-byte load per pair of super-steps;
            // the lane's two codes are bytes 8 j' + 2 q, i.e. dword 2 j' + q / 2
            v4i sv[CT][PS / 2];
#pragma unroll
            for (int h = 0; h < PS / 2; ++h) {
                const uint32_t g = min((p0 + 2 * h) * 8, k / 16 - 16);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    sv[ct][h] = *reinterpret_cast<const v4i *>(srow[ct] + g);
                    load_w(ct, 2 * h);
                    load_w(ct, 2 * h + 1);
                }
            }
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int j = 0; j < PS; ++j) {
                    const uint32_t d0 = (j & 1) ? sv[ct][j / 2].z : sv[ct][j / 2].x;
                    const uint32_t d1 = (j & 1) ? sv[ct][j / 2].w : sv[ct][j / 2].y;
                    const uint32_t d = (q >> 1) ? d1 : d0;
                    sc[ct][j] = (q & 1) ? d >> 16 : d & 0xFFFFu;
                }
        } else {
#pragma unroll
            for (int j = 0; j < PS; ++j) {
                const uint32_t g = min(((p0 + min((uint32_t)j, plen - 1)) * kStepK + 32 * q) / 16, k / 16 - 2);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    sc[ct][j] = *reinterpret_cast<const uint16_t *>(srow[ct] + g);
                    load_w(ct, j);
                }
            }
        }
        asm volatile("" ::: "memory");
        // 3. the copies were issued first and loads complete in order: waiting
        //    until only this pass's weight and scale loads may be outstanding
        //    means the activations are in LDS (the compiler then waits per
        //    super-step for just the loads that super-step reads)
        wait_vm_le<CT * (VS ? PS + PS / 2 : 2 * PS)>();

        const int8_t *xa = la + arow * pitch + 64 * q;  // this lane's 32 BF16 of a super-step
#pragma unroll
        for (int j = 0; j < PS; ++j) {
            if ((uint32_t)j >= plen) break;
            const bool live = (p0 + j) * kStepK + 32 * q < k;  // quarters past K contribute 0
            if constexpr (CT == 1) {
                const ByteTable t0 = make_table(sc[0][j] & 0xFFu), t1 = make_table(sc[0][j] >> 8);
                const uint32_t wd[4] = {(uint32_t)wv[0][j].x, (uint32_t)wv[0][j].y, (uint32_t)wv[0][j].z,
                                        (uint32_t)wv[0][j].w};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const v4i b = decode8(wd[t], t < 2 ? t0 : t1);
                    v4i a = *reinterpret_cast<const v4i *>(xa + j * (kStepK * 2) + 16 * t);
                    if (!live) a = v4i{0, 0, 0, 0};
                    acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                                     __builtin_bit_cast(bf16x8, b), acc[0], 0, 0, 0);
                }
                continue;
            }
            v4i a[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                a[t] = *reinterpret_cast<const v4i *>(xa + j * (kStepK * 2) + 16 * t);
                if (!live) a[t] = v4i{0, 0, 0, 0};
            }
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const ByteTable t0 = make_table(sc[ct][j] & 0xFFu), t1 = make_table(sc[ct][j] >> 8);
                const uint32_t wd[4] = {(uint32_t)wv[ct][j].x, (uint32_t)wv[ct][j].y, (uint32_t)wv[ct][j].z,
                                        (uint32_t)wv[ct][j].w};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const v4i b = decode8(wd[t], t < 2 ? t0 : t1);
                    acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[t]),
                                                                      __builtin_bit_cast(bf16x8, b), acc[ct], 0, 0, 0);
                }
            }
        }
        asm volatile("" ::: "memory");  // the next pass's copies overwrite this pass's activations
    }

    // partial sums of the waves, added in wave order; then scale_2 and BF16
    __syncthreads();
    float *red = reinterpret_cast<float *>(smem);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[((ct * kGemvMaxWaves + wave) * 64 + lane) * 4 + r] = acc[ct][r];
    __syncthreads();
    if (wave < CT) {
        const int ct = wave;
        float tot[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int v = 0; v < nwaves; ++v)
#pragma unroll
            for (int r = 0; r < 4; ++r) tot[r] += red[((ct * kGemvMaxWaves + v) * 64 + lane) * 4 + r];
        const uint32_t oc = n0 + kGemvCols * ct + c;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t row = 4 * q + r;
            if (row < m && oc < n) out[(uint64_t)row * n + oc] = f32_to_bf16_rne(tot[r] * scale2);
        }
    }
}

}  // namespace

hipError_t launch_w4a16(const uint16_t *x, const uint8_t *w_packed, const uint8_t *w_e4m3, float scale2,
                        uint16_t *out, uint32_t m, uint32_t n, uint32_t k, hipStream_t s) {
    // Column tiles per workgroup: two from m = 4 on, where the activation
    // bytes a workgroup stages (2 m per K element) approach the weight bytes
    // of one 16-column tile (9 per K element) -- if that still leaves a
    // workgroup for every CU.  Waves per workgroup as for the
    // int8 GEMV (~24 waves per CU over the launch), at most 16 (and with two
    // tiles, one of them reduces each tile's partial sums); then the smallest
    // number of passes whose activation staging fits in LDS.
    const uint32_t ct = m >= 4 && div_up(n, 2 * kGemvCols) >= (uint64_t)kGemmCus ? 2 : 1;
    const uint32_t tiles = (uint32_t)div_up(n, kGemvCols * ct);
    const uint32_t nsteps = (uint32_t)div_up(k, kStepK);
    uint32_t waves = (uint32_t)div_up(6144, tiles);
    waves = max(ct, min(waves, (uint32_t)kGemvMaxWaves));
    waves = min(waves, max(nsteps, ct));
    const bool vs = k % 256 == 0;  // then nsteps is even
    uint32_t spw = (uint32_t)div_up(nsteps, waves);
    if (vs) spw += spw & 1u;  // even: every pass starts at an even super-step
    waves = max((uint32_t)div_up(nsteps, spw), ct);
    const uint32_t red = ct * kGemvMaxWaves * 64 * 4 * 4;
    // pass length: the whole per-wave range when its staging fits in LDS,
    // else the largest that fits (even when the scales are read 16 bytes at a
    // time); launched with PS rounded up to an instantiated length
    uint32_t pass = min(spw, ct == 2 ? 6u : (uint32_t)kW4PassSteps);  // two tiles: 6 keeps 128 VGPRs
    const uint32_t step = vs ? 2u : 1u;
    while (pass > step && (uint64_t)waves * m * w4_pitch(pass) > 160 * 1024) pass -= step;
    pass = vs ? max(2u, (pass + 1) & ~1u) : (pass <= 2 ? pass : (pass + 1) & ~1u);
    const uint32_t lds = max((uint32_t)(waves * m * w4_pitch(pass)), red);
    if (lds > 160 * 1024) return hipErrorInvalidValue;
#define BSR_W4_LAUNCH(V, P, C)                                                                            \
    hipLaunchKernelGGL((w4a16_kernel<V, P, C>), dim3(tiles), dim3(64 * waves), lds, s, x, w_packed, w_e4m3, \
                       scale2, out, m, n, k, spw)
    if (ct == 2) {
        switch ((vs ? 16 : 0) + pass) {
        case 16 + 6: BSR_W4_LAUNCH(true, 6, 2); break;
        case 16 + 4: BSR_W4_LAUNCH(true, 4, 2); break;
        case 16 + 2: BSR_W4_LAUNCH(true, 2, 2); break;
        case 6: BSR_W4_LAUNCH(false, 6, 2); break;
        case 4: BSR_W4_LAUNCH(false, 4, 2); break;
        case 2: BSR_W4_LAUNCH(false, 2, 2); break;
        default: BSR_W4_LAUNCH(false, 1, 2); break;
        }
    } else {
        switch ((vs ? 16 : 0) + pass) {
        case 16 + 8: BSR_W4_LAUNCH(true, 8, 1); break;
        case 16 + 6: BSR_W4_LAUNCH(true, 6, 1); break;
        case 16 + 4: BSR_W4_LAUNCH(true, 4, 1); break;
        case 16 + 2: BSR_W4_LAUNCH(true, 2, 1); break;
        case 8: BSR_W4_LAUNCH(false, 8, 1); break;
        case 6: BSR_W4_LAUNCH(false, 6, 1); break;
        case 4: BSR_W4_LAUNCH(false, 4, 1); break;
        case 2: BSR_W4_LAUNCH(false, 2, 1); break;
        default: BSR_W4_LAUNCH(false, 1, 1); break;
        }
    }
#undef BSR_W4_LAUNCH
    return hipGetLastError();
}

}  // namespace bsr
