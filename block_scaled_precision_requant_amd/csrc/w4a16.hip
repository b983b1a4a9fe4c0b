// w4a16.hip -- decode GEMV straight from the NVFP4 weight (no int8 requant).
//
// Page "metrale_model_layers/layers/ops/gemv_sw.rs" launches a W4A16 decode
// GEMV: BF16 activations times an NVFP4 weight (packed E2M1, one E4M3 scale
// per 16 elements, one F32 scale_2).  Result definition used here:
//   out[i, j] = bf16_rne( fl32( S[i, j] * scale_2 ) ),
//   S[i, j]   = an FP32 evaluation of the sum over k of x[i, k] * e2m1[j, k] *
//               s16[j, k / 16] (order: the kernel's own).
// Two kernels.  The streamed one (K a multiple of 256, below) sums the exact
// products x * e2m1 per 16-element block and adds s16 times each block sum;
// the register-decode one sums the exact products x * (e2m1 * s16) (e2m1 *
// s16 has at most 6 significant bits, a BF16 value, and BF16 x BF16 is exact
// in FP32).  Either way only FP32 sums, one product per block or none, and
// the two final roundings are inexact.
//
// Register-decode kernel mapping.  Workgroup = 16 output columns x all of K, K split over its waves
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

// A lane reads its own two E4M3 codes per super-step with 2-byte loads (this
// kernel runs for K % 256 != 0, where scale rows need not be 16-byte aligned).
// PS: super-steps per staging pass (at most kW4PassSteps).
// CT: 16-column tiles per workgroup; each wave runs all CT tiles over its K
// range with one staged copy of the activations, so larger m (whose
// activation bytes rival the weight bytes) copies them fewer times.
// (wp and we are not __restrict__: a restrict-qualified read-only load may be
// moved past the empty asm statements that keep a pass's loads ahead of its
// compute.)
template <int PS, int CT>
__global__ __launch_bounds__(kGemvMaxWaves * 64) void w4a16_kernel(
    const uint16_t *__restrict__ x, const uint8_t *wp, const uint8_t *we,
    float scale2, uint16_t *__restrict__ out, uint32_t m, uint32_t n, uint32_t k, uint32_t steps_per_wave) {
    static_assert(PS >= 1 && PS <= kW4PassSteps, "pass length");
    constexpr uint32_t pass_steps = PS;
    extern __shared__ __attribute__((aligned(1024))) int8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = blockDim.x >> 6;
    const int q = lane >> 4;
    const uint32_t c = lane & 15;
    const uint32_t n0 = blockIdx.x * kGemvCols * CT;
    const uint32_t nsteps = (k + kW4StepK - 1) / kW4StepK;
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
            const uint64_t e = min((uint64_t)p0 * kW4StepK + (p % pitch) / 2, (uint64_t)k - 8);
            if (p < a_bytes)
                __builtin_amdgcn_global_load_lds(x + (uint64_t)r * k + e, (lds_void *)(la + b0), 16, 0, 0);
        }
        asm volatile("" ::: "memory");
        // 2. weights and scale codes, in the order the super-steps use them
        //    (clamped loads keep the code straight-line)
        v4i wv[CT][PS];
        uint32_t sc[CT][PS];
        auto load_w = [&](int ct, int j) {
            const uint32_t kk = min((p0 + min((uint32_t)j, plen - 1)) * kW4StepK + 32 * q, k - 32);
            wv[ct][j] = *reinterpret_cast<const v4i *>(wrow[ct] + kk / 2);
        };
#pragma unroll
        for (int j = 0; j < PS; ++j) {
            const uint32_t g = min(((p0 + min((uint32_t)j, plen - 1)) * kW4StepK + 32 * q) / 16, k / 16 - 2);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                sc[ct][j] = *reinterpret_cast<const uint16_t *>(srow[ct] + g);
                load_w(ct, j);
            }
        }
        asm volatile("" ::: "memory");
        // 3. the copies were issued first and loads complete in order: waiting
        //    until only this pass's weight and scale loads may be outstanding
        //    means the activations are in LDS (the compiler then waits per
        //    super-step for just the loads that super-step reads)
        wait_vm_le<CT * 2 * PS>();

        const int8_t *xa = la + arow * pitch + 64 * q;  // this lane's 32 BF16 of a super-step
#pragma unroll
        for (int j = 0; j < PS; ++j) {
            if ((uint32_t)j >= plen) break;
            const bool live = (p0 + j) * kW4StepK + 32 * q < k;  // quarters past K contribute 0
            if constexpr (CT == 1) {
                const ByteTable t0 = make_table(sc[0][j] & 0xFFu), t1 = make_table(sc[0][j] >> 8);
                const uint32_t wd[4] = {(uint32_t)wv[0][j].x, (uint32_t)wv[0][j].y, (uint32_t)wv[0][j].z,
                                        (uint32_t)wv[0][j].w};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const v4i b = decode8(wd[t], t < 2 ? t0 : t1);
                    v4i a = *reinterpret_cast<const v4i *>(xa + j * (kW4StepK * 2) + 16 * t);
                    if (!live) a = v4i{0, 0, 0, 0};
                    acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                                     __builtin_bit_cast(bf16x8, b), acc[0], 0, 0, 0);
                }
                continue;
            }
            v4i a[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                a[t] = *reinterpret_cast<const v4i *>(xa + j * (kW4StepK * 2) + 16 * t);
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

// ---------------------------------------------------------------- stream

// Streamed W4A16 (K a multiple of 256).  Same workgroup shape (16 columns,
// K split over the waves); each wave brings its run of 256-element chunks --
// 16 weight rows of packed codes, their E4M3 codes and the activation rows --
// through a private 2-buffer LDS ring with global_load_lds.  Per 16-element
// scale block: the lane's 4 codes become BF16 E2M1 values through
// v_cvt_scalef32_pk_bf16_fp4 (scale 1, exact), one v_mfma_f32_16x16x16bf16_1k
// gives the block's FP32 partial sums P (products exact, 16 terms), and the
// accumulators take fma(P, s16, acc) with s16 from v_cvt_f32_fp8 (OCP E4M3,
// exact).  So S[i, j] = FP32 sum over blocks of s16 * (FP32 sum over the block
// of x * e2m1): the same real value as the sum over k of x * (e2m1 * s16),
// evaluated in another FP32 order (within the K + 16 term bound).
constexpr int kW4ChunkK = 256;
constexpr int kW4ChunkBlocks = kW4ChunkK / 16;
constexpr int kW4WRowBytes = kW4ChunkK / 2;  // 128: 8 slots of 16 bytes
constexpr int kW4ARowBytes = kW4ChunkK * 2;  // 512: 32 slots of 16 bytes
constexpr int kW4StreamMaxWaves = 8;
// LDS rows are unpadded and XOR-swizzled by 16-byte slot: slot s of weight row
// r holds slot s ^ (r & 7) of the row, slot s of activation row r holds slot
// s ^ (r & 15), so 16 rows read at one offset spread over the banks.
template <int ROWS>
struct W4Buf {
    static constexpr int kARows = ROWS < 2 ? 2 : ROWS;
    uint8_t w[kGemvCols * kW4WRowBytes];
    uint8_t a[kARows * kW4ARowBytes];
    uint8_t s[kGemvCols * kW4ChunkBlocks];  // E4M3 codes, [row][block]
};
template <int ROWS>
constexpr int w4_stream_copies() {  // copy instructions per chunk
    return kGemvCols * kW4WRowBytes / 1024 + W4Buf<ROWS>::kARows * kW4ARowBytes / 1024 + 1;
}

typedef short short4_ __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// OCP E4M3 code in byte b of a dword -> binary32 (v_cvt_f32_fp8, exact; the
// byte select is an immediate).
__device__ __forceinline__ float e4m3_byte(uint32_t codes, int b) {
    switch (b) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)codes, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)codes, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)codes, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)codes, 3);
    }
}

// Wait until at most C * later copies are outstanding (later <= N): s_waitcnt
// takes an immediate, so one branch per count.
template <int C, int N>
__device__ __forceinline__ void wait_vm_later(uint32_t later) {
    if constexpr (N > 0) {
        if (later == (uint32_t)N) {
            wait_vm_le<C * N>();
            return;
        }
        wait_vm_later<C, N - 1>(later);
    } else {
        wait_vm_le<0>();
    }
}

template <int ROWS, int RING>
__global__ __launch_bounds__(kW4StreamMaxWaves * 64) void w4a16_stream_kernel(
    const uint16_t *__restrict__ x, const uint8_t *wp, const uint8_t *we, float scale2,
    uint16_t *__restrict__ out, uint32_t m, uint32_t n, uint32_t k, uint32_t cpw) {
    using Buf = W4Buf<ROWS>;
    constexpr int NC = w4_stream_copies<ROWS>();
    static_assert(NC * (RING - 1) < 64, "the copies in flight fit the vmcnt range");
    static_assert(ROWS <= kGemvMaxRows, "one 16-row MFMA tile");
    extern __shared__ __attribute__((aligned(1024))) int8_t smem[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = blockDim.x >> 6;
    const int q = lane >> 4;
    const uint32_t c16 = lane & 15;
    const uint32_t n0 = blockIdx.x * kGemvCols;
    const uint32_t c_begin = wave * cpw;
    const uint32_t nchunks = min(k / kW4ChunkK, c_begin + cpw) - c_begin;  // >= 1
    Buf *ring = reinterpret_cast<Buf *>(smem) + wave * RING;

    auto issue = [&](int bi, uint32_t chunk) {
        Buf &b = ring[bi];
        const uint32_t kc = (c_begin + chunk) * kW4ChunkK;
#pragma unroll
        for (int i = 0; i < kGemvCols * kW4WRowBytes / 1024; ++i) {  // 8 rows x 128 bytes per copy
            const uint32_t r = 8 * i + (lane >> 3), slot = lane & 7;
            const uint8_t *src = wp + (uint64_t)min(n0 + r, n - 1) * (k / 2) + kc / 2 + ((slot ^ (r & 7)) << 4);
            __builtin_amdgcn_global_load_lds(src, (lds_void *)(b.w + i * 1024), 16, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < Buf::kARows * kW4ARowBytes / 1024; ++i) {  // 2 rows x 512 bytes per copy
            const uint32_t r = 2 * i + (lane >> 5), slot = lane & 31;
            const uint16_t *src = x + (uint64_t)min(r, m - 1) * k + kc + ((slot ^ (r & 15)) << 3);
            __builtin_amdgcn_global_load_lds(src, (lds_void *)(b.a + i * 1024), 16, 0, 0);
        }
        if (lane < kGemvCols)  // 16 rows x 16 scale codes
            __builtin_amdgcn_global_load_lds(we + (uint64_t)min(n0 + lane, n - 1) * (k / 16) + kc / 16,
                                             (lds_void *)b.s, 16, 0, 0);
    };

    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t arow = min(c16, (uint32_t)ROWS - 1);
    const uint32_t wshift = 16 * (q & 1);  // this lane's 2 code bytes within a dword
    auto compute = [&](int bi) {
        const Buf &b = ring[bi];
        const v4f zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int g = 0; g < kW4ChunkBlocks / 4; ++g) {
            const uint32_t scodes = *reinterpret_cast<const uint32_t *>(b.s + c16 * kW4ChunkBlocks + 4 * g);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int j = 4 * g + jj;  // block of the chunk
                // activations: elements 16 j + 4 q .. + 3 of row arow
                const uint32_t aslot = (uint32_t)(2 * j) + (q >> 1);
                const short4_ av = *reinterpret_cast<const short4_ *>(
                    b.a + arow * kW4ARowBytes + ((aslot ^ (arow & 15)) << 4) + 8 * (q & 1));
                // weights: code bytes 2 q, 2 q + 1 of block j of row c16
                const uint32_t wslot = (uint32_t)j >> 1;
                const uint32_t wd = *reinterpret_cast<const uint32_t *>(
                    b.w + c16 * kW4WRowBytes + ((wslot ^ (c16 & 7)) << 4) + 8 * (j & 1) + 4 * (q >> 1));
                const uint32_t wb = wd >> wshift;
                const auto w01 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wb, 1.0f, 0);
                const auto w23 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wb, 1.0f, 1);
                const u32x2 wpair = {__builtin_bit_cast(uint32_t, w01), __builtin_bit_cast(uint32_t, w23)};
                const short4_ wv = __builtin_bit_cast(short4_, wpair);  // elements 4q .. 4q + 3
                const v4f p = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, wv, zero4, 0, 0, 0);
                const float sc = e4m3_byte(scodes, jj);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = fmaf(p[r], sc, acc[r]);
            }
        }
    };
    auto reads_done = [&]() {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        asm volatile("" ::: "memory");
    };

    // Chunks c + 1 .. c + RING - 1 are in flight while chunk c is computed.
#pragma unroll
    for (int r = 0; r < RING - 1; ++r)
        if ((uint32_t)r < nchunks) issue(r, r);
    for (uint32_t c0 = 0; c0 < nchunks; c0 += RING) {
#pragma unroll
        for (int u = 0; u < RING; ++u) {
            const uint32_t c = c0 + u;
            if (c >= nchunks) break;
            // buffer (u + RING - 1) % RING held chunk c - 1, whose reads are done
            if (c + RING - 1 < nchunks) issue((u + RING - 1) % RING, c + RING - 1);
            wait_vm_later<NC, RING - 1>(min(nchunks - 1 - c, (uint32_t)RING - 1));
            asm volatile("" ::: "memory");
            compute(u);
            reads_done();
        }
    }

    // partial sums of the waves, added in wave order; then scale_2 and BF16
    __syncthreads();
    float *red = reinterpret_cast<float *>(smem);
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * 64 + lane) * 4 + r] = acc[r];
    __syncthreads();
    if (wave == 0) {
        float tot[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int v = 0; v < nwaves; ++v)
#pragma unroll
            for (int r = 0; r < 4; ++r) tot[r] += red[(v * 64 + lane) * 4 + r];
        const uint32_t oc = n0 + c16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t row = 4 * q + r;
            if (row < m && oc < n) out[(uint64_t)row * n + oc] = f32_to_bf16_rne(tot[r] * scale2);
        }
    }
}

constexpr int kW4StreamRing = 2;
template <int ROWS, int RING = kW4StreamRing>
hipError_t launch_w4a16_stream(const uint16_t *x, const uint8_t *w_packed, const uint8_t *w_e4m3, float scale2,
                               uint16_t *out, uint32_t m, uint32_t n, uint32_t k, hipStream_t s) {
    constexpr uint32_t ring_bytes = RING * sizeof(W4Buf<ROWS>);
    constexpr uint32_t lds_waves = 160u * 1024u / ring_bytes;
    constexpr uint32_t max_waves = lds_waves < (uint32_t)kW4StreamMaxWaves ? lds_waves : kW4StreamMaxWaves;
    const uint32_t tiles = (uint32_t)div_up(n, kGemvCols);
    const uint32_t nchunks = k / kW4ChunkK;
    // as many waves (2 to 8) as let the workgroups a CU must run share its LDS
    // at once, except that m <= 2 always takes 8 (N = 14336, K = 4096: 9.6-9.7 us
    // against 9.9 with the 6 that fit four workgroups per CU; m = 8 wants 2)
    const uint32_t wg_per_cu = (uint32_t)div_up(tiles, kGemmCus);
    uint32_t waves = ROWS <= 2 ? max_waves : max(2u, (160u * 1024u / wg_per_cu) / ring_bytes);
    waves = min(min(waves, max_waves), nchunks);
    const uint32_t cpw = (uint32_t)div_up(nchunks, waves);
    waves = (uint32_t)div_up(nchunks, cpw);
    const uint32_t lds = max(waves * ring_bytes, (uint32_t)(kW4StreamMaxWaves * 64 * 4 * 4));
    hipLaunchKernelGGL((w4a16_stream_kernel<ROWS, RING>), dim3(tiles), dim3(64 * waves), lds, s, x, w_packed, w_e4m3,
                       scale2, out, m, n, k, cpw);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_w4a16(const uint16_t *x, const uint8_t *w_packed, const uint8_t *w_e4m3, float scale2,
                        uint16_t *out, uint32_t m, uint32_t n, uint32_t k, hipStream_t s) {
    if (k % kW4ChunkK == 0) {
        if (m <= 1) return launch_w4a16_stream<1>(x, w_packed, w_e4m3, scale2, out, m, n, k, s);
        if (m <= 2) return launch_w4a16_stream<2>(x, w_packed, w_e4m3, scale2, out, m, n, k, s);
        if (m <= 4) return launch_w4a16_stream<4>(x, w_packed, w_e4m3, scale2, out, m, n, k, s);
        if (m <= 8) return launch_w4a16_stream<8>(x, w_packed, w_e4m3, scale2, out, m, n, k, s);
        return launch_w4a16_stream<16>(x, w_packed, w_e4m3, scale2, out, m, n, k, s);
    }
    // Other K: the register-decode kernel, with the plan of bsr_geometry.h.
    const W4Plan p = w4a16_reg_plan(m, n, k);
    if (p.lds > kLdsBytes) return hipErrorInvalidValue;
#define BSR_W4_LAUNCH(P, C)                                                                                 \
    hipLaunchKernelGGL((w4a16_kernel<P, C>), dim3(p.tiles), dim3(64 * p.waves), p.lds, s, x, w_packed, w_e4m3, \
                       scale2, out, m, n, k, p.spw)
    if (p.ct == 2) {
        switch (p.pass) {
        case 6: BSR_W4_LAUNCH(6, 2); break;
        case 4: BSR_W4_LAUNCH(4, 2); break;
        case 2: BSR_W4_LAUNCH(2, 2); break;
        default: BSR_W4_LAUNCH(1, 2); break;
        }
    } else {
        switch (p.pass) {
        case 8: BSR_W4_LAUNCH(8, 1); break;
        case 6: BSR_W4_LAUNCH(6, 1); break;
        case 4: BSR_W4_LAUNCH(4, 1); break;
        case 2: BSR_W4_LAUNCH(2, 1); break;
        default: BSR_W4_LAUNCH(1, 1); break;
        }
    }
#undef BSR_W4_LAUNCH
    return hipGetLastError();
}

}  // namespace bsr
