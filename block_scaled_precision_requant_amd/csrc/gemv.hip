// gemv.hip -- weight-streaming block-scaled GEMV for gfx950 (m <= 16).
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
// instruction -- and takes 16 bytes of activation row l % 16 (clamped to the
// last row; rows >= m only feed outputs that are never stored) at the same
// offset.  One v_mfma_i32_16x16x64_i8 with the activation quarters 2-3 zeroed
// gives the first block's P, one with quarters 0-1 zeroed the second's: lanes
// pair A and B bytes by (quarter, byte), so the zeroed quarters drop out
// exactly.  Output lane l holds column l % 16, rows 4 * (l / 16) + r (r < 4):
// the 16 rows of the MFMA cover m <= 16 at no extra matrix-core cost.
//
// Kernels:
//  * stream (K a multiple of 256): each wave brings its K range through a
//    private LDS ring with global_load_lds, 1 KB copies of whole cache lines
//    -- weight rows, activation rows and scales alike -- and takes one
//    v_mfma_i32_16x16x32_i8 per block; about three times the per-CU copy
//    rate of loading 16 rows x 64 bytes per instruction into registers;
//  * staged: the workgroup first copies its activations, activation scales
//    and the scales of its 16 weight rows into LDS (global_load_lds), so the
//    only global loads of the K loop are weight bytes -- one 1 KB instruction
//    per wave step;
//  * direct: every operand comes from global memory.  Used when the staged
//    copies do not fit in LDS or K is not a multiple of 128;
//  * chain (the path-invariant GEMV): each output is the same FP32 chain
//    acc = fma(P_b, fl32(a_s * w_s), acc), b = 0, 1, ..., that the GEMM
//    evaluates, held on one lane from the first block to the last -- its
//    BF16 bits equal the GEMM's.  On grids of at most one workgroup per CU
//    (K % 256 == 0) producer waves stream the chunks and take the block
//    products, and chain waves run the chains from an LDS exchange (relay);
//    on wider grids one wave per workgroup walks all of K (the streamed
//    kernel's loop); other K take the one-wave LDS-ring form (K % 128 == 0)
//    or the register form.
#include <type_traits>

#include "bsr_internal.h"

namespace bsr {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kSteps = kGemvBlocksPerIter / 2;  // 64-byte MFMA steps per iteration
constexpr int kQuads = kGemvBlocksPerIter / 4;  // groups of 4 scales per iteration
static_assert(kGemvBlocksPerIter % 4 == 0, "scales are read 4 blocks at a time");

// Operands of one iteration (kGemvBlocksPerIter blocks) of one lane.
struct IterOps {
    v4i wv[kSteps], av[kSteps];
    v4f wsv[kQuads], asv[kQuads][4];  // asv[h][r]: activation row 4q + r
};

// Rescale-accumulate one iteration.  Blocks at or past b_end (and rows >= m)
// get zero activations, so their P is 0 and they add nothing.
__device__ __forceinline__ void gemv_iter(float (&acc)[4], const IterOps &x, uint32_t b0,
                                          uint32_t b_end, bool a_live, int q) {
    const v4i zero4 = {0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
        const uint32_t blk = b0 + 2 * t + (q >> 1);  // block of this lane's quarter
        const bool live = a_live && blk < b_end;
        const v4i avl = live ? x.av[t] : zero4;
        const v4i lo = q < 2 ? avl : zero4;  // first block of the step
        const v4i hi = q < 2 ? zero4 : avl;  // second block
        const v4i p0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(lo, x.wv[t], zero4, 0, 0, 0);
        const v4i p1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(hi, x.wv[t], zero4, 0, 0, 0);
        const int h = t >> 1, e = 2 * (t & 1);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            acc[r] = fmaf((float)p0[r], x.asv[h][r][e] * x.wsv[h][e], acc[r]);
            acc[r] = fmaf((float)p1[r], x.asv[h][r][e + 1] * x.wsv[h][e + 1], acc[r]);
        }
    }
}

// Add the waves' partial sums in wave order and store the live outputs.
// `red` holds kGemvMaxWaves x 64 x 4 floats; the caller has made it free.
__device__ __forceinline__ void gemv_reduce_store(float *red, const float (&acc)[4], int wave,
                                                  int nwaves, int lane, uint32_t n0, uint32_t m,
                                                  uint32_t n, uint16_t *out) {
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * 64 + lane) * 4 + r] = acc[r];
    __syncthreads();
    if (wave == 0) {
        float tot[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int v = 0; v < nwaves; ++v)
#pragma unroll
            for (int r = 0; r < 4; ++r) tot[r] += red[(v * 64 + lane) * 4 + r];
        const uint32_t c = n0 + (lane & 15);
        const int q = lane >> 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t row = 4 * q + r;
            if (row < m && c < n) out[(uint64_t)row * n + c] = f32_to_bf16_rne(tot[r]);
        }
    }
}

// s_waitcnt vmcnt(n); expcnt and lgkmcnt left at their maxima.
template <int n>
__device__ __forceinline__ void wait_vm_le() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
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

// Workgroup barrier without the fences of __syncthreads(), whose release
// side waits for every outstanding vector-memory operation (vmcnt(0)) and
// so would drain the LDS copies a ring keeps in flight across the barrier.
// Callers wait for what the barrier publishes: lgkmcnt(0) for their LDS
// reads and writes, vmcnt for their own copies that the next step reads.
// The memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

// ---------------------------------------------------------------- direct

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

// Activation scales of blocks idx..idx+3 of one row with a scale per 2^shift
// blocks (shift >= 2): idx is a multiple of 4, so one scale covers all four.
__device__ __forceinline__ v4f load_group_f4(const float *p, uint32_t idx, uint32_t nb, uint32_t shift) {
    const float v = p[min(idx, nb - 1) >> shift];
    const v4f r = {v, v, v, v};
    return r;
}

// VEC: 16-byte scale loads (nb % 4 == 0).  AGROUP: activation scales per 2^a_shift
// blocks (a_shift >= 2), rows a_ld floats apart; else one per block, a_ld = nb.
template <bool VEC, bool AGROUP>
__global__ __launch_bounds__(kGemvMaxWaves * 64) void gemv_direct_kernel(
    const int8_t *__restrict__ a, const int8_t *__restrict__ w, const float *__restrict__ a_s,
    const float *__restrict__ w_s, uint16_t *__restrict__ out, uint32_t m, uint32_t n, uint32_t k,
    uint32_t a_ld, uint32_t a_shift, uint32_t blocks_per_wave) {
    __shared__ float red[kGemvMaxWaves * 64 * 4];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = blockDim.x >> 6;
    const int q = lane >> 4;                      // 16-byte quarter of a 64-byte step
    const uint32_t n0 = blockIdx.x * kGemvCols;
    const uint32_t col = min(n0 + (lane & 15), n - 1);
    const uint32_t arow = lane & 15;              // activation row this lane feeds
    const bool a_live = arow < m;
    const uint32_t nb = k / 32;
    const uint32_t srow0 = min(4u * (uint32_t)q, m - 1);  // scale rows 4q + r

    const int8_t *wrow = w + (uint64_t)col * k;
    const int8_t *arowp = a + (uint64_t)min(arow, m - 1) * k;
    const float *wsrow = w_s + (uint64_t)col * nb;

    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t b_begin = wave * blocks_per_wave;
    const uint32_t b_end = min(nb, b_begin + blocks_per_wave);
    // Every load of an iteration is issued before any is used.
    for (uint32_t b0 = b_begin; b0 < b_end; b0 += kGemvBlocksPerIter) {
        IterOps x;
#pragma unroll
        for (int t = 0; t < kSteps; ++t) {
            const uint64_t off = min((uint64_t)b0 * 32 + 64 * t + 16 * q, (uint64_t)k - 16);
            x.wv[t] = *reinterpret_cast<const v4i *>(wrow + off);
            x.av[t] = *reinterpret_cast<const v4i *>(arowp + off);
        }
#pragma unroll
        for (int h = 0; h < kQuads; ++h) {
            x.wsv[h] = load_f4<VEC>(wsrow, b0 + 4 * h, nb);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float *ar = a_s + (uint64_t)min(srow0 + r, m - 1) * a_ld;
                x.asv[h][r] = AGROUP ? load_group_f4(ar, b0 + 4 * h, nb, a_shift) : load_f4<VEC>(ar, b0 + 4 * h, nb);
            }
        }
        gemv_iter(acc, x, b0, b_end, a_live, q);
    }
    gemv_reduce_store(red, acc, wave, nwaves, lane, n0, m, n, out);
}

// ---------------------------------------------------------------- chain

constexpr int kChainDepth = 4;  // iterations whose loads are in flight ahead of the compute

// One wave, 16 columns, all of K in increasing block order: per output, the
// blocks' rescaled products enter a single FP32 accumulator in the GEMM's
// order, which makes the result independent of the path and of m.  Loads run
// kChainDepth iterations ahead in a register ring (the ring index is static
// in the unrolled body); past the last iteration they re-read it.
template <bool VEC, bool AGROUP>
__global__ __launch_bounds__(64) void gemv_chain_kernel(
    const int8_t *__restrict__ a, const int8_t *w, const float *__restrict__ a_s,
    const float *__restrict__ w_s, uint16_t *__restrict__ out, uint32_t m, uint32_t n, uint32_t k,
    uint32_t a_ld, uint32_t a_shift) {
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4;
    const uint32_t n0 = blockIdx.x * kGemvCols;
    const uint32_t col = min(n0 + (lane & 15), n - 1);
    const uint32_t arow = lane & 15;
    const bool a_live = arow < m;
    const uint32_t nb = k / 32;
    const uint32_t niter = (nb + kGemvBlocksPerIter - 1) / kGemvBlocksPerIter;
    const uint32_t srow0 = min(4u * (uint32_t)q, m - 1);

    const int8_t *wrow = w + (uint64_t)col * k;
    const int8_t *arowp = a + (uint64_t)min(arow, m - 1) * k;
    const float *wsrow = w_s + (uint64_t)col * nb;
    auto load = [&](IterOps &x, uint32_t it) {
        const uint32_t b0 = it * kGemvBlocksPerIter;
#pragma unroll
        for (int t = 0; t < kSteps; ++t) {
            const uint64_t off = min((uint64_t)b0 * 32 + 64 * t + 16 * q, (uint64_t)k - 16);
            x.wv[t] = *reinterpret_cast<const v4i *>(wrow + off);
            x.av[t] = *reinterpret_cast<const v4i *>(arowp + off);
        }
#pragma unroll
        for (int h = 0; h < kQuads; ++h) {
            x.wsv[h] = load_f4<VEC>(wsrow, b0 + 4 * h, nb);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float *ar = a_s + (uint64_t)min(srow0 + r, m - 1) * a_ld;
                x.asv[h][r] = AGROUP ? load_group_f4(ar, b0 + 4 * h, nb, a_shift) : load_f4<VEC>(ar, b0 + 4 * h, nb);
            }
        }
    };

    IterOps ring[kChainDepth];
#pragma unroll
    for (int u = 0; u < kChainDepth; ++u) load(ring[u], min((uint32_t)u, niter - 1));
    asm volatile("" ::: "memory");
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (uint32_t it0 = 0; it0 < niter; it0 += kChainDepth) {
#pragma unroll
        for (int u = 0; u < kChainDepth; ++u) {
            // past the last iteration every block is >= nb: zero activations, P = 0,
            // and acc + 0 * s leaves acc unchanged (acc is never -0)
            gemv_iter(acc, ring[u], (it0 + u) * kGemvBlocksPerIter, nb, a_live, q);
            load(ring[u], min(it0 + u + kChainDepth, niter - 1));
            // keep the refill here: the compiler would otherwise sink it to its
            // use kChainDepth iterations later and the loads would not overlap
            asm volatile("" ::: "memory");
        }
    }
    const uint32_t c = n0 + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t row = 4 * q + r;
        if (row < m && c < n) out[(uint64_t)row * n + c] = f32_to_bf16_rne(acc[r]);
    }
}

// Streamed chain kernel (K a multiple of 128): the same FP32 chain, with W, A
// and both scales brought into an LDS ring by global_load_lds in chunks of
// kChainChunkBlocks blocks, so the wave's only waits are for a whole chunk
// that was requested one chunk earlier.  The block products come from
// v_mfma_i32_16x16x32_i8 (K = 32: one block, no zeroed operand quarters):
// lane (c = l % 16, q = l / 16) gives bytes 8q..8q+7 of a block of
// activation row c and of weight row n0 + c; A and B pair by (quarter, byte),
// so the sum over lanes is the block's exact dot product.
constexpr int kChainChunkBlocks = 32;
constexpr int kChainRowPitch = kChainChunkBlocks * 32 + 16;  // bytes; +16 spreads 16 rows over the banks
constexpr int kChainSPitch = kChainChunkBlocks + 4;          // floats per scale row
// ROWS: activation rows the ring holds (m <= ROWS): copies and LDS scale
// with the rows actually used.
template <int ROWS>
struct ChainBuf {
    static constexpr int kSRows = kGemvCols + ROWS;  // w_s rows, then a_s rows
    int8_t w[kGemvCols * kChainRowPitch];
    int8_t a[ROWS * kChainRowPitch];
    float s[kSRows * kChainSPitch];
};

// Copies of one chunk issued by the wave: one 1 KB copy per weight and
// activation row, the scale rows flattened into 16-byte copies (4-byte copies
// for grouped activation scales, expanded to one per block).  Every copy
// instruction has live lanes, so each one counts once in vmcnt.
template <bool AGROUP, int ROWS>
struct ChainCopies {
    static constexpr int kScale16 = AGROUP ? (kGemvCols * kChainSPitch + 255) / 256
                                           : ((kGemvCols + ROWS) * kChainSPitch + 255) / 256;
    static constexpr int kScale4 = AGROUP ? (ROWS * kChainSPitch + 63) / 64 : 0;
    static constexpr int kTotal = kGemvCols + ROWS + kScale16 + kScale4;
};

// Operands of one iteration (4 blocks) of the streamed chain kernel: per
// block 8 activation and 8 weight bytes, and the scale pair this lane feeds
// into the scale-product MFMA (activation row l % 16, weight column l % 16,
// block l / 16 of the iteration).
struct ChainOps {
    long av[4], wv[4];
    float as, ws;
};
typedef float v16f __attribute__((ext_vector_type(16)));

template <bool AGROUP, int RING, int ROWS>
__global__ __launch_bounds__(64) void gemv_chain_lds_kernel(
    const int8_t *__restrict__ a, const int8_t *w, const float *__restrict__ a_s,
    const float *__restrict__ w_s, uint16_t *__restrict__ out, uint32_t m, uint32_t n, uint32_t k,
    uint32_t a_ld, uint32_t a_shift) {
    using Buf = ChainBuf<ROWS>;
    __shared__ __attribute__((aligned(16))) Buf ring[RING];
    constexpr int NC = ChainCopies<AGROUP, ROWS>::kTotal;
    static_assert(NC * (RING - 1) < 64, "the copies in flight fit the vmcnt range");

    const int lane = threadIdx.x & 63;
    const int q = lane >> 4;
    const uint32_t c16 = lane & 15;
    const uint32_t n0 = blockIdx.x * kGemvCols;
    const uint32_t nb = k / 32;  // a multiple of 4
    const uint32_t nchunks = (nb + kChainChunkBlocks - 1) / kChainChunkBlocks;

    auto issue = [&](int bi, uint32_t chunk) {
        Buf &b = ring[bi];
        // row bases are wave-uniform (scalar registers); lanes add a 32-bit offset
        const uint32_t off = min(chunk * (uint32_t)kChainChunkBlocks * 32 + 16 * lane, k - 16);
#pragma unroll
        for (int r = 0; r < kGemvCols; ++r) {
            const int8_t *row = w + (uint64_t)min(n0 + r, n - 1) * k;
            __builtin_amdgcn_global_load_lds(row + off, (lds_void *)(b.w + r * kChainRowPitch), 16, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const int8_t *row = a + (uint64_t)min((uint32_t)r, m - 1) * k;
            __builtin_amdgcn_global_load_lds(row + off, (lds_void *)(b.a + r * kChainRowPitch), 16, 0, 0);
        }
        const uint32_t bb0 = chunk * kChainChunkBlocks;
        constexpr uint32_t s_rows16 = AGROUP ? kGemvCols : Buf::kSRows;
#pragma unroll
        for (int i = 0; i < ChainCopies<AGROUP, ROWS>::kScale16; ++i) {
            const uint32_t p = i * 256 + 4 * lane;  // float index in the region
            const uint32_t r = min(p / kChainSPitch, s_rows16 - 1);
            const uint32_t cb = min(bb0 + min(p % kChainSPitch, (uint32_t)kChainChunkBlocks - 4), nb - 4);
            const float *src = r < kGemvCols ? w_s + (uint64_t)min(n0 + r, n - 1) * nb + cb
                                             : a_s + (uint64_t)min(r - kGemvCols, m - 1) * a_ld + cb;
            if (p < s_rows16 * kChainSPitch)  // lanes past the region stay idle
                __builtin_amdgcn_global_load_lds(src, (lds_void *)(b.s + i * 256), 16, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < ChainCopies<AGROUP, ROWS>::kScale4; ++i) {
            const uint32_t p = i * 64 + lane;
            const uint32_t r = min(p / kChainSPitch, (uint32_t)ROWS - 1);
            const uint32_t cb = min(bb0 + min(p % kChainSPitch, (uint32_t)kChainChunkBlocks - 1), nb - 1);
            if (p < ROWS * kChainSPitch)
                __builtin_amdgcn_global_load_lds(a_s + (uint64_t)min(r, m - 1) * a_ld + (cb >> a_shift),
                                                 (lds_void *)(b.s + kGemvCols * kChainSPitch + i * 64), 4, 0, 0);
        }
    };

    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    // One chunk from LDS: blocks in increasing order, one FP32 chain per
    // output; each iteration's LDS reads are issued before the previous
    // iteration's arithmetic, which hides their latency.
    auto compute = [&](int bi, uint32_t chunk, auto full_chunk) {
        constexpr bool full = decltype(full_chunk)::value;
        const Buf &b = ring[bi];
        const int8_t *wr = b.w + c16 * kChainRowPitch + 8 * q;
        const int8_t *ar = b.a + min(c16, (uint32_t)ROWS - 1) * kChainRowPitch + 8 * q;
        const float *wsr = b.s + c16 * kChainSPitch + q;
        const float *asr = b.s + (kGemvCols + min(c16, m - 1)) * kChainSPitch + q;
        auto read = [&](ChainOps &x, int i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x.av[j] = *reinterpret_cast<const long *>(ar + (4 * i + j) * 32);
                x.wv[j] = *reinterpret_cast<const long *>(wr + (4 * i + j) * 32);
            }
            x.as = asr[4 * i];
            x.ws = wsr[4 * i];
        };
        const uint32_t bb0 = chunk * kChainChunkBlocks;
        const v4i zero4 = {0, 0, 0, 0};
        const v16f zero16 = {};
        ChainOps x[2];
        read(x[0], 0);
#pragma unroll
        for (int i = 0; i < kChainChunkBlocks / 4; ++i) {
            if (i + 1 < kChainChunkBlocks / 4) read(x[(i + 1) & 1], i + 1);
            __builtin_amdgcn_sched_barrier(0);
            const ChainOps &cur = x[i & 1];
            v4i p[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // only the last chunk can hold blocks past K: zero activations
                // there, so P = 0 and acc + 0 * s = acc
                const long avl = (full || bb0 + 4 * i + j < nb) ? cur.av[j] : 0;
                p[j] = __builtin_amdgcn_mfma_i32_16x16x32_i8(avl, cur.wv[j], zero4, 0, 0, 0);
            }
            // the 4 blocks' scale outer products a_s x w_s, one rounded product
            // per output: block j in registers 4j..4j+3, laid out like P
            const v16f sc = __builtin_amdgcn_mfma_f32_16x16x1f32(cur.as, cur.ws, zero16, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = fmaf((float)p[j][r], sc[4 * j + r], acc[r]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Reads of a buffer are complete before copies into it are issued.
    auto reads_done = [&]() {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt at their maxima
        asm volatile("" ::: "memory");
    };
    // Before computing chunk c: wait for its copies; the copies of the chunks
    // after it that were issued (at most RING - 1) may stay in flight.
    auto wait_chunk = [&](uint32_t c) {
        const uint32_t ahead = min(nchunks - 1 - c, (uint32_t)RING - 1);
        if (RING > 2 && ahead >= 2) wait_vm_le<NC * (RING - 1 > 1 ? 2 : 1)>();
        else if (ahead >= 1) wait_vm_le<NC>();
        else wait_vm_le<0>();
        asm volatile("" ::: "memory");
    };

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
            wait_chunk(c);
            if ((c + 1) * kChainChunkBlocks <= nb) compute(u, c, std::true_type());
            else compute(u, c, std::false_type());
            reads_done();
        }
    }
    const uint32_t col = n0 + c16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t row = 4 * q + r;
        if (row < m && col < n) out[(uint64_t)row * n + col] = f32_to_bf16_rne(acc[r]);
    }
}

// ---------------------------------------------------------------- staged

// Each wave stages the slices of A, a_s and w_s that its own K range needs
// into a private LDS region, so no barrier precedes the K loop.  Region of a
// wave (bytes): m activation rows of a_pitch bytes, then m activation-scale
// rows and kGemvCols weight-scale rows of s_pitch floats.  The 16-byte row
// padding of a_pitch shifts consecutive rows by 4 banks, so the 16 lanes of a
// quarter (16 rows, one offset) hit 16 distinct banks; s_pitch is padded by 4
// floats when bpw / 4 is even, for the same reason on the weight-scale rows.
struct StagedGeo {
    uint32_t a_pitch, s_pitch, wave_bytes;
};

__host__ __device__ inline StagedGeo staged_geo(uint32_t m, uint32_t bpw) {
    StagedGeo g;
    g.a_pitch = bpw * 32 + 16;
    g.s_pitch = ((bpw / 4) & 1) ? bpw : bpw + 4;
    g.wave_bytes = (m * g.a_pitch + (m + kGemvCols) * g.s_pitch * 4 + 15) / 16 * 16;
    return g;
}

constexpr uint32_t kRedBytes = kGemvMaxWaves * 64 * 4 * 4;
constexpr int kStagedMaxIters = 8;                   // iterations per wave (unrolled)

// Staged kernel with every iteration of a wave unrolled (at most
// kStagedMaxIters): straight-line code, so the compiler's vmcnt waits count
// exactly the weight loads issued after the ones an iteration needs.
// (The weight pointer is not __restrict__: a restrict-qualified read-only
// load may be moved across the empty asm statements that order the loads.)
__global__ __launch_bounds__(kGemvMaxWaves * 64) void gemv_staged_kernel(
    const int8_t *__restrict__ a, const int8_t *w, const float *__restrict__ a_s,
    const float *__restrict__ w_s, uint16_t *__restrict__ out, uint32_t m, uint32_t n, uint32_t k,
    uint32_t a_ld, uint32_t a_shift, uint32_t bpw) {
    extern __shared__ __attribute__((aligned(1024))) int8_t smem[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = blockDim.x >> 6;
    const int q = lane >> 4;
    const uint32_t n0 = blockIdx.x * kGemvCols;
    const uint32_t nb = k / 32;
    const StagedGeo g = staged_geo(m, bpw);
    const uint32_t b_begin = wave * bpw;
    const uint32_t b_end = min(nb, b_begin + bpw);
    const uint32_t len = b_end - b_begin;          // a multiple of 4, at least 4
    const uint32_t niter = len / kGemvBlocksPerIter;
    int8_t *la = smem + (uint64_t)wave * g.wave_bytes;
    float *ls = reinterpret_cast<float *>(la + m * g.a_pitch);

    const uint32_t col = min(n0 + (lane & 15), n - 1);
    const uint32_t arow = lane & 15;
    const bool a_live = arow < m;
    const int8_t *wrow = w + (uint64_t)col * k + (uint64_t)b_begin * 32 + 16 * q;
    auto load_w = [&](v4i (&wv)[kSteps], uint32_t it) {
#pragma unroll
        for (int t = 0; t < kSteps; ++t)
            wv[t] = *reinterpret_cast<const v4i *>(wrow + (uint64_t)it * kGemvBlocksPerIter * 32 + 64 * t);
    };

    // First iteration's weights, then the staging copies, then one wait for
    // all of them: the weight bytes arrive during the staging latency.
    v4i wv0[kSteps], wv1[kSteps];
    load_w(wv0, 0);
    asm volatile("" ::: "memory");
    // A slice: m rows of len * 32 bytes, flattened in 1 KB copies; lanes past
    // the region are masked, lanes in a row's padding re-read its last chunk.
    const uint32_t a_bytes = m * g.a_pitch;
    for (uint32_t p0 = 0; p0 < a_bytes; p0 += 1024) {
        const uint32_t p = p0 + 16 * lane;
        const uint32_t r = p / g.a_pitch, c = min(p % g.a_pitch, len * 32 - 16);
        if (p < a_bytes)
            __builtin_amdgcn_global_load_lds(a + (uint64_t)min(r, m - 1) * k + (uint64_t)b_begin * 32 + c,
                                             (lds_void *)(la + p0), 16, 0, 0);
    }
    // Scale slices: m rows of a_s then 16 rows of w_s, len floats each, in
    // 16-byte copies (b_begin and len are multiples of 4 and so is nb).  With
    // a_shift > 0 the activation rows are expanded to one scale per block by
    // 4-byte copies, so the K loop reads the same layout either way.
    const uint32_t s_floats = (m + kGemvCols) * g.s_pitch;
    const uint32_t as_floats = a_shift ? m * g.s_pitch : 0;
    for (uint32_t p0 = as_floats & ~255u; p0 < s_floats; p0 += 256) {
        const uint32_t p = p0 + 4 * lane;
        const uint32_t r = min(p / g.s_pitch, m + kGemvCols - 1), c = min(p % g.s_pitch, len - 4);
        const float *src = r < m ? a_s + (uint64_t)r * a_ld
                                 : w_s + (uint64_t)min(n0 + (r - m), n - 1) * nb;
        if (p < s_floats && p >= as_floats)
            __builtin_amdgcn_global_load_lds(src + b_begin + c, (lds_void *)(ls + p0), 16, 0, 0);
    }
    for (uint32_t p0 = 0; p0 < as_floats; p0 += 64) {
        const uint32_t p = p0 + lane;
        const uint32_t r = min(p / g.s_pitch, m - 1), c = min(p % g.s_pitch, len - 1);
        if (p < as_floats)
            __builtin_amdgcn_global_load_lds(a_s + (uint64_t)r * a_ld + ((b_begin + c) >> a_shift),
                                             (lds_void *)(ls + p0), 4, 0, 0);
    }
    wait_vm_le<0>();

    const int8_t *la_row = la + min(arow, m - 1) * g.a_pitch + 16 * q;
    const float *lws_row = ls + (m + (lane & 15)) * g.s_pitch;
    const float *las_row[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) las_row[r] = ls + min(4u * q + r, m - 1) * g.s_pitch;
    auto load_lds = [&](IterOps &x, uint32_t it) {
        const uint32_t c = it * kGemvBlocksPerIter;
#pragma unroll
        for (int t = 0; t < kSteps; ++t) x.av[t] = *reinterpret_cast<const v4i *>(la_row + c * 32 + 64 * t);
#pragma unroll
        for (int h = 0; h < kQuads; ++h) {
            x.wsv[h] = *reinterpret_cast<const v4f *>(lws_row + c + 4 * h);
#pragma unroll
            for (int r = 0; r < 4; ++r) x.asv[h][r] = *reinterpret_cast<const v4f *>(las_row[r] + c + 4 * h);
        }
    };

    // Iteration it computes with weights loaded one iteration earlier; its own
    // step issues the next iteration's weight and LDS loads first.  Loads are
    // clamped to the last iteration rather than skipped, keeping the code
    // straight-line.
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    IterOps x[2];
    load_lds(x[0], 0);
#pragma unroll
    for (int it = 0; it < kStagedMaxIters; ++it) {
        const uint32_t nxt = min((uint32_t)it + 1, niter - 1);
        if (it & 1) load_w(wv0, nxt); else load_w(wv1, nxt);
        load_lds(x[(it + 1) & 1], nxt);
        __builtin_amdgcn_sched_barrier(0);
        IterOps &cur = x[it & 1];
#pragma unroll
        for (int t = 0; t < kSteps; ++t) cur.wv[t] = (it & 1) ? wv1[t] : wv0[t];
        gemv_iter(acc, cur, b_begin + it * kGemvBlocksPerIter, b_end, a_live, q);
        if ((uint32_t)it + 1 >= niter) break;
    }

    __syncthreads();  // every wave is done with its staged operands
    gemv_reduce_store(reinterpret_cast<float *>(smem), acc, wave, nwaves, lane, n0, m, n, out);
}

// ---------------------------------------------------------------- stream

// Streamed GEMV (K a multiple of 256): the waves split K into contiguous
// ranges of 8-block chunks, and each wave brings its chunks -- 16 weight
// rows, the activation rows and both scale tiles -- through a private LDS
// ring with global_load_lds, 1 KB per copy (4 rows of 256 bytes, whole cache
// lines), RING - 1 chunks in flight while one is computed.  Per 4 blocks and
// 16-row activation tile: four v_mfma_i32_16x16x32_i8 and one
// v_mfma_f32_16x16x1f32 of scale products, as in the chain kernel; up to four
// tiles (m <= 64) share each weight chunk.  The waves' partial sums are added
// in wave order at the end.  AGROUP: activation scales per 2^a_shift blocks,
// expanded to one per block by 4-byte copies.
constexpr int kStreamChunkBlocks = kGemvStreamKAlign / 32;
constexpr int kStreamRowBytes = kStreamChunkBlocks * 32;  // 256: 16 slots of 16 bytes
constexpr int kStreamRowsPerCopy = 1024 / kStreamRowBytes;
// LDS rows are unpadded; 16-byte slot c of row r holds chunk c ^ (r & 15), so
// the 16 rows a quarter-wave reads at one offset fall in 16 distinct slots.
template <int ROWS>
struct StreamBuf {
    static constexpr int kARows = ROWS < kStreamRowsPerCopy ? kStreamRowsPerCopy : ROWS;
    static constexpr int kSRows = kGemvCols + ROWS;  // w_s rows, then a_s rows
    int8_t w[kGemvCols * kStreamRowBytes];
    int8_t a[kARows * kStreamRowBytes];
    float s[kSRows][kStreamChunkBlocks];
};
template <int ROWS, bool AGROUP>
struct StreamCopies {  // copy instructions per chunk, each with live lanes
    static constexpr int kScale16 = AGROUP ? 1 : (kGemvCols + ROWS + 31) / 32;  // 32 rows per copy
    static constexpr int kScale4 = AGROUP ? (ROWS + 7) / 8 : 0;                  // 8 rows per copy
    static constexpr int kTotal =
        kGemvCols / kStreamRowsPerCopy + StreamBuf<ROWS>::kARows / kStreamRowsPerCopy + kScale16 + kScale4;
};

// At most kStreamMaxWaves waves per workgroup (the launcher's rule; the rings
// of 16 rows fit no more), so each may take up to 256 registers.
constexpr int kStreamMaxWaves = 8;

template <int ROWS, int RING, bool AGROUP>
__global__ __launch_bounds__(kStreamMaxWaves * 64) void gemv_stream_kernel(
    const int8_t *__restrict__ a, const int8_t *w, const float *__restrict__ a_s,
    const float *__restrict__ w_s, uint16_t *__restrict__ out, uint32_t m, uint32_t n, uint32_t k,
    uint32_t a_ld, uint32_t a_shift, uint32_t cpw) {
    using Buf = StreamBuf<ROWS>;
    using Copies = StreamCopies<ROWS, AGROUP>;
    constexpr int NC = Copies::kTotal;
    constexpr int RT = (ROWS + 15) / 16;  // 16-row MFMA tiles
    static_assert(NC * (RING - 1) < 64, "the copies in flight fit the vmcnt range");
    static_assert(ROWS <= kGemvStreamMaxRows && (ROWS <= 16 || ROWS % 16 == 0), "whole 16-row tiles");
    extern __shared__ __attribute__((aligned(1024))) int8_t smem[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = blockDim.x >> 6;
    const int q = lane >> 4;
    const uint32_t c16 = lane & 15;
    const uint32_t n0 = blockIdx.x * kGemvCols;
    const uint32_t nb = k / 32;  // a multiple of 8
    const uint32_t c_begin = wave * cpw;
    const uint32_t nchunks = min(nb / kStreamChunkBlocks, c_begin + cpw) - c_begin;  // >= 1
    Buf *ring = reinterpret_cast<Buf *>(smem) + wave * RING;

    // Copy lane roles: byte copies take row (lane / 16) of a 4-row group and
    // LDS slot lane % 16, fetching chunk slot ^ row; a 16-byte scale copy takes
    // row 32 i + lane / 2 (weight rows, then per-block activation rows) and
    // half lane % 2; a 4-byte grouped-scale copy takes activation row
    // 8 i + lane / 8 and block lane % 8.
    const uint32_t slot = lane & 15;
    auto issue = [&](int bi, uint32_t chunk) {
        Buf &b = ring[bi];
        const uint32_t kb = (c_begin + chunk) * kStreamChunkBlocks;
#pragma unroll
        for (int i = 0; i < kGemvCols / kStreamRowsPerCopy; ++i) {
            const uint32_t r = i * kStreamRowsPerCopy + (lane >> 4);
            const int8_t *src = w + (uint64_t)min(n0 + r, n - 1) * k + kb * 32 + ((slot ^ (r & 15)) << 4);
            __builtin_amdgcn_global_load_lds(src, (lds_void *)(b.w + i * 1024), 16, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < Buf::kARows / kStreamRowsPerCopy; ++i) {
            const uint32_t r = i * kStreamRowsPerCopy + (lane >> 4);
            const int8_t *src = a + (uint64_t)min(r, m - 1) * k + kb * 32 + ((slot ^ (r & 15)) << 4);
            __builtin_amdgcn_global_load_lds(src, (lds_void *)(b.a + i * 1024), 16, 0, 0);
        }
        constexpr uint32_t s16_rows = AGROUP ? kGemvCols : kGemvCols + ROWS;
#pragma unroll
        for (int i = 0; i < Copies::kScale16; ++i) {
            const uint32_t srow = 32 * i + (lane >> 1);
            const float *src = srow < (uint32_t)kGemvCols
                                   ? w_s + (uint64_t)min(n0 + srow, n - 1) * nb
                                   : a_s + (uint64_t)min(srow - kGemvCols, m - 1) * a_ld;
            if (srow < s16_rows)
                __builtin_amdgcn_global_load_lds(src + kb + 4 * (lane & 1), (lds_void *)(&b.s[32 * i][0]), 16, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < Copies::kScale4; ++i) {
            const uint32_t r = 8 * i + (lane >> 3);
            if (r < (uint32_t)ROWS)
                __builtin_amdgcn_global_load_lds(a_s + (uint64_t)min(r, m - 1) * a_ld + ((kb + (lane & 7)) >> a_shift),
                                                 (lds_void *)(&b.s[kGemvCols + 8 * i][0]), 4, 0, 0);
        }
    };

    float acc[RT][4];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][r] = 0.0f;
    uint32_t arow[RT];  // LDS activation row of this lane in tile t
#pragma unroll
    for (int t = 0; t < RT; ++t) arow[t] = min(16u * t + c16, (uint32_t)ROWS - 1);
    // Operands of 4 blocks: this lane's 8 bytes of each block for its weight
    // row and activation rows, and the scale pair it feeds the scale-product
    // MFMA with (block l / 16 of the 4).
    struct Ops {
        long wv[4], av[RT][4];
        float ws, as[RT];
    };
    auto compute = [&](int bi) {
        const Buf &b = ring[bi];
        const int8_t *wr = b.w + c16 * kStreamRowBytes;
        auto off = [&](uint32_t r, int blk) {  // byte offset of this lane's 8 bytes of a block
            return ((((uint32_t)(2 * blk) + (q >> 1)) ^ (r & 15)) << 4) + 8 * (q & 1);
        };
        auto read = [&](Ops &o, int i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) o.wv[j] = *reinterpret_cast<const long *>(wr + off(c16, 4 * i + j));
            o.ws = b.s[c16][4 * i + q];
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                const int8_t *ar = b.a + arow[t] * kStreamRowBytes;
#pragma unroll
                for (int j = 0; j < 4; ++j) o.av[t][j] = *reinterpret_cast<const long *>(ar + off(arow[t], 4 * i + j));
                o.as[t] = b.s[kGemvCols + arow[t]][4 * i + q];
            }
        };
        const v4i zero4 = {0, 0, 0, 0};
        const v16f zero16 = {};
        // the next 4 blocks' LDS reads are issued before the current ones'
        // arithmetic, so a lone wave (the path-invariant use) hides their latency
        Ops x[2];
        read(x[0], 0);
#pragma unroll
        for (int i = 0; i < kStreamChunkBlocks / 4; ++i) {
            if (i + 1 < kStreamChunkBlocks / 4) read(x[(i + 1) & 1], i + 1);
            __builtin_amdgcn_sched_barrier(0);
            const Ops &cur = x[i & 1];
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                v4i p[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    p[j] = __builtin_amdgcn_mfma_i32_16x16x32_i8(cur.av[t][j], cur.wv[j], zero4, 0, 0, 0);
                // the 4 blocks' scale outer products a_s x w_s, one rounded
                // product per output: block j in registers 4j..4j+3, laid out like P
                const v16f sc = __builtin_amdgcn_mfma_f32_16x16x1f32(cur.as[t], cur.ws, zero16, 0, 0, 0);
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[t][r] = fmaf((float)p[j][r], sc[4 * j + r], acc[t][r]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto reads_done = [&]() {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        asm volatile("" ::: "memory");
    };
    // Before computing chunk c (after issuing chunk c + RING - 1): its copies
    // are done; those of the up to RING - 1 later chunks may stay in flight.
    auto wait_chunk = [&](uint32_t c) {
        wait_vm_later<NC, RING - 1>(min(nchunks - 1 - c, (uint32_t)RING - 1));
        asm volatile("" ::: "memory");
    };

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
            wait_chunk(c);
            compute(u);
            reads_done();
        }
    }

    // Per tile: the waves' partial sums added in wave order (alternating
    // between two LDS buffers, so one barrier per tile suffices).
    __syncthreads();  // every wave is done with its ring
    float *red = reinterpret_cast<float *>(smem);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        float *rb = red + (t & 1) * (kGemvMaxWaves * 64 * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) rb[(wave * 64 + lane) * 4 + r] = acc[t][r];
        __syncthreads();
        if (wave == t % nwaves) {
            float tot[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int v = 0; v < nwaves; ++v)
#pragma unroll
                for (int r = 0; r < 4; ++r) tot[r] += rb[(v * 64 + lane) * 4 + r];
            const uint32_t col = n0 + c16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t row = 16 * t + 4 * q + r;
                if (row < m && col < n) out[(uint64_t)row * n + col] = f32_to_bf16_rne(tot[r]);
            }
        }
    }
}

// Path-invariant GEMV for grids of at most one workgroup per CU (K a
// multiple of 256): each output's FP32 chain stays on one lane of a chain
// wave, the work that feeds the chains is spread over PW producer waves.  A
// round covers PW * G consecutive chunks of 8 blocks; producer p takes
// chunks g * PW + p of it (g < G), streams them through its own LDS ring as
// the streamed GEMV does, takes one v_mfma_i32_16x16x32_i8 per block, and
// writes P (converted to float) of its live outputs and the chunk's scales
// into the chunk's slot of an exchange buffer.  The CW chain waves then run,
// for every block in increasing order, acc = fma(P_b, a_s * w_s, acc) with
// the scale product rounded once to binary32 -- the GEMM's chain, so the
// bits equal the GEMM's -- one output per lane (16 * ROWS outputs over 64
// CW lanes).  In round r the producers fill exchange buffer r % 2 while the
// chain waves read buffer (r - 1) % 2; a barrier ends each round.
//
// Exchange slot of a chunk: P of the F = 16 ROWS live outputs as [F][8
// blocks], then the chunk's scales as the ring holds them: [16 weight rows
// + ROWS activation rows][8 blocks].  Output f is row 4 q + r, column c of
// the tile for f = r * 16 QG + 16 q + c (QG live 4-row groups; the MFMA lane
// 16 q + c holds rows 4 q .. 4 q + 3 of column c).
template <int ROWS>
struct RelayGeo {
    static constexpr int kQG = (ROWS + 3) / 4;  // live 4-row groups: lanes 0 .. 16 kQG - 1
    static constexpr int kRP = ROWS < 4 ? ROWS : 4;  // live rows of such a lane
    static constexpr int kF = 16 * kQG * kRP;        // live outputs (16 ROWS)
    static constexpr int kCW = (kF + 63) / 64;       // chain waves
    static constexpr int kSFloats = (kGemvCols + ROWS) * kStreamChunkBlocks;
    static constexpr int kChunkFloats = kF * kStreamChunkBlocks + kSFloats;
};

template <int ROWS, int PW, int RING, int G, bool AGROUP>
__global__ __launch_bounds__((PW + RelayGeo<ROWS>::kCW) * 64) void gemv_chain_relay_kernel(
    const int8_t *__restrict__ a, const int8_t *w, const float *__restrict__ a_s,
    const float *__restrict__ w_s, uint16_t *__restrict__ out, uint32_t m, uint32_t n, uint32_t k,
    uint32_t a_ld, uint32_t a_shift) {
    using Buf = StreamBuf<ROWS>;
    using Copies = StreamCopies<ROWS, AGROUP>;
    using RG = RelayGeo<ROWS>;
    typedef float v4f_ __attribute__((ext_vector_type(4)));
    constexpr int NC = Copies::kTotal;
    constexpr int F = RG::kF;
    constexpr int CB = kStreamChunkBlocks;
    constexpr uint32_t kSlots = PW * G;  // chunks per round
    static_assert(NC * (RING - 1) < 64, "the copies in flight fit the vmcnt range");
    static_assert(ROWS <= kGemvMaxRows && (ROWS & (ROWS - 1)) == 0, "1, 2, 4, 8 or 16 rows");
    static_assert(CB == 8, "two 16-byte LDS accesses per output and chunk");
    static_assert(sizeof(Buf::s) == RG::kSFloats * sizeof(float) && RG::kSFloats <= 64 * 4,
                  "one 16-byte copy per lane moves a chunk's scales");
    extern __shared__ __attribute__((aligned(1024))) int8_t smem[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q = lane >> 4;
    const uint32_t c16 = lane & 15;
    const uint32_t n0 = blockIdx.x * kGemvCols;
    const uint32_t nb = k / 32;                          // a multiple of 8
    const uint32_t nchunks = nb / CB;
    const uint32_t rounds = (nchunks + kSlots - 1) / kSlots;
    float *xch = reinterpret_cast<float *>(smem);        // [2][kSlots][chunk floats]
    Buf *ring = reinterpret_cast<Buf *>(smem + 2 * kSlots * RG::kChunkFloats * sizeof(float));

    if (wave < RG::kCW) {
        // a chain wave: output f = 64 wave + lane, blocks in increasing order
        const uint32_t f = 64 * wave + lane;
        const uint32_t g = f % (16 * RG::kQG);
        const uint32_t row = 4 * (g / 16) + f / (16 * RG::kQG), col = g % 16;
        float acc = 0.0f;
        auto chain = [&](const float *xc) {  // one chunk's 8 blocks
            const float *pe = xc + f * CB;
            const float *we = xc + F * CB + col * CB;
            const float *ae = xc + F * CB + (kGemvCols + row) * CB;
            const v4f_ p0 = *reinterpret_cast<const v4f_ *>(pe), p1 = *reinterpret_cast<const v4f_ *>(pe + 4);
            const v4f_ w0 = *reinterpret_cast<const v4f_ *>(we), w1 = *reinterpret_cast<const v4f_ *>(we + 4);
            const v4f_ a0 = *reinterpret_cast<const v4f_ *>(ae), a1 = *reinterpret_cast<const v4f_ *>(ae + 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = fmaf(p0[j], a0[j] * w0[j], acc);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = fmaf(p1[j], a1[j] * w1[j], acc);
        };
        for (uint32_t r = 0; r <= rounds; ++r) {
            if (r > 0 && f < (uint32_t)F) {
                const float *xb = xch + ((r - 1) & 1) * kSlots * RG::kChunkFloats;
                const uint32_t live = min(kSlots, nchunks - (r - 1) * kSlots);
                if (live == kSlots) {
#pragma unroll
                    for (uint32_t c = 0; c < kSlots; ++c) chain(xb + c * RG::kChunkFloats);
                } else {
                    for (uint32_t c = 0; c < live; ++c) chain(xb + c * RG::kChunkFloats);
                }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this round's reads are done
            ring_barrier();
        }
        if (f < (uint32_t)F && row < m && n0 + col < n) out[(uint64_t)row * n + n0 + col] = f32_to_bf16_rne(acc);
        return;
    }

    // a producer: its i-th chunk is chunk (i / G) kSlots + (i % G) PW + pw,
    // increasing in i, so the chunks below nchunks are its first `mine`
    const uint32_t pw = wave - RG::kCW;
    auto chunk_of = [&](uint32_t i) { return (i / G) * kSlots + (i % G) * PW + pw; };
    uint32_t mine = 0;
    if (nchunks > pw) {
        const uint32_t full = (nchunks - pw) / kSlots, rest = (nchunks - pw) % kSlots;  // rest < kSlots
        mine = full * G + min((uint32_t)G, (rest + PW - 1) / PW);
    }
    Buf *pring = ring + pw * RING;
    const uint32_t slot = lane & 15;
    auto issue = [&](int bi, uint32_t i) {
        Buf &b = pring[bi];
        const uint32_t kb = chunk_of(i) * CB;
#pragma unroll
        for (int t = 0; t < kGemvCols / kStreamRowsPerCopy; ++t) {
            const uint32_t r = t * kStreamRowsPerCopy + (lane >> 4);
            const int8_t *src = w + (uint64_t)min(n0 + r, n - 1) * k + kb * 32 + ((slot ^ (r & 15)) << 4);
            __builtin_amdgcn_global_load_lds(src, (lds_void *)(b.w + t * 1024), 16, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < Buf::kARows / kStreamRowsPerCopy; ++t) {
            const uint32_t r = t * kStreamRowsPerCopy + (lane >> 4);
            const int8_t *src = a + (uint64_t)min(r, m - 1) * k + kb * 32 + ((slot ^ (r & 15)) << 4);
            __builtin_amdgcn_global_load_lds(src, (lds_void *)(b.a + t * 1024), 16, 0, 0);
        }
        constexpr uint32_t s16_rows = AGROUP ? kGemvCols : kGemvCols + ROWS;
#pragma unroll
        for (int t = 0; t < Copies::kScale16; ++t) {
            const uint32_t srow = 32 * t + (lane >> 1);
            const float *src = srow < (uint32_t)kGemvCols
                                   ? w_s + (uint64_t)min(n0 + srow, n - 1) * nb
                                   : a_s + (uint64_t)min(srow - kGemvCols, m - 1) * a_ld;
            if (srow < s16_rows)
                __builtin_amdgcn_global_load_lds(src + kb + 4 * (lane & 1), (lds_void *)(&b.s[32 * t][0]), 16, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < Copies::kScale4; ++t) {
            const uint32_t r = 8 * t + (lane >> 3);
            if (r < (uint32_t)ROWS)
                __builtin_amdgcn_global_load_lds(a_s + (uint64_t)min(r, m - 1) * a_ld + ((kb + (lane & 7)) >> a_shift),
                                                 (lds_void *)(&b.s[kGemvCols + 8 * t][0]), 4, 0, 0);
        }
    };
    const uint32_t arow = min(c16, (uint32_t)ROWS - 1);
    // one chunk: its block products and its scales into exchange slot xs
    auto produce = [&](int bi, float *xs) {
        const Buf &b = pring[bi];
        if (lane < RG::kSFloats / 4) {
            const v4f_ sv = reinterpret_cast<const v4f_ *>(&b.s[0][0])[lane];
            reinterpret_cast<v4f_ *>(xs + F * CB)[lane] = sv;
        }
        const int8_t *wr = b.w + c16 * kStreamRowBytes;
        const int8_t *ar = b.a + arow * kStreamRowBytes;
        auto off = [&](uint32_t r, int blk) {
            return ((((uint32_t)(2 * blk) + (q >> 1)) ^ (r & 15)) << 4) + 8 * (q & 1);
        };
        const v4i zero4 = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < CB / 4; ++i) {
            v4i p[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const long wv = *reinterpret_cast<const long *>(wr + off(c16, 4 * i + j));
                const long av = *reinterpret_cast<const long *>(ar + off(arow, 4 * i + j));
                p[j] = __builtin_amdgcn_mfma_i32_16x16x32_i8(av, wv, zero4, 0, 0, 0);
            }
            if (q < RG::kQG) {
#pragma unroll
                for (int r = 0; r < RG::kRP; ++r) {
                    const v4f_ pv = {(float)p[0][r], (float)p[1][r], (float)p[2][r], (float)p[3][r]};
                    *reinterpret_cast<v4f_ *>(xs + (r * 16 * RG::kQG + lane) * CB + 4 * i) = pv;
                }
            }
        }
    };

#pragma unroll
    for (int r = 0; r < RING - 1; ++r)
        if ((uint32_t)r < mine) issue(r, r);
    for (uint32_t r = 0; r <= rounds; ++r) {
        float *xb = xch + (r & 1) * kSlots * RG::kChunkFloats;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint32_t i = r * G + g;
            if (i < mine) {
                // ring buffer (i + RING - 1) % RING held chunk i - 1, whose reads are done
                if (i + RING - 1 < mine) issue((i + RING - 1) % RING, i + RING - 1);
                wait_vm_later<NC, RING - 1>(min(mine - 1 - i, (uint32_t)RING - 1));
                asm volatile("" ::: "memory");
                produce(i % RING, xb + (g * PW + pw) * RG::kChunkFloats);
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): ring reads and exchange writes are done
                asm volatile("" ::: "memory");
            }
        }
        ring_barrier();  // the copies of later chunks stay in flight
    }
}

// LDS bytes of the relay kernel: the exchange (two buffers of PW G chunks)
// and the producers' rings.
template <int ROWS, int PW, int RING, int G>
constexpr uint32_t relay_lds() {
    return 2 * PW * G * RelayGeo<ROWS>::kChunkFloats * sizeof(float) + PW * RING * sizeof(StreamBuf<ROWS>);
}

}  // namespace

namespace {

// The path-invariant GEMV through the streamed kernel with one wave per
// workgroup: that wave walks every chunk in K order, so each output is the
// single FP32 chain acc = fma(P_b, fl32(a_s * w_s), acc) over b = 0, 1, ...
// (and the final wave sum adds it to +0, which changes no value: acc is
// never -0).  Used for grids of more than one workgroup per CU, whose waves
// then share the CU (N = 14336, K = 4096: 15.5-16 us against 16.5-22 for the
// chain kernel); with one workgroup per CU the lone wave's arithmetic bounds
// both kernels and the chain kernel's 1 KB rows measured faster (22-25 us
// against 27 at N = 4096, K = 14336, even with six chunks in flight).
template <int ROWS, bool AGROUP>
hipError_t launch_chain_stream(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale, uint32_t a_ld,
                               uint32_t a_shift, const float *w_scale, uint16_t *out, uint32_t m, uint32_t n,
                               uint32_t k, hipStream_t s) {
    const uint32_t tiles = (uint32_t)div_up(n, kGemvCols);
    const uint32_t nchunks = k / kGemvStreamKAlign;
#define BSR_CHAIN_STREAM(RG)                                                                                      \
    hipLaunchKernelGGL((gemv_stream_kernel<ROWS, RG, AGROUP>), dim3(tiles), dim3(64),                            \
                       max((uint32_t)(RG * sizeof(StreamBuf<ROWS>)), kRedBytes), s, a_i8, w_i8, a_scale, w_scale, \
                       out, m, n, k, a_ld, a_shift, nchunks)
    BSR_CHAIN_STREAM(4);
#undef BSR_CHAIN_STREAM
    return hipGetLastError();
}

// The relay kernel's producer waves, ring depth and chunks per producer and
// round per row count: as many producers as LDS holds with RING - 1 chunks
// in flight each.
template <int ROWS>
struct RelayCfg {
    static constexpr int kPW = ROWS <= 1 ? 6 : ROWS <= 2 ? 8 : ROWS <= 4 ? 7 : 4;
    static constexpr int kRing = ROWS <= 1 ? 3 : 2;
    static constexpr int kG = ROWS <= 1 ? 3 : ROWS <= 8 ? 2 : 1;
};
template <int ROWS, bool AGROUP>
hipError_t launch_chain_relay(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale, uint32_t a_ld,
                              uint32_t a_shift, const float *w_scale, uint16_t *out, uint32_t m, uint32_t n,
                              uint32_t k, hipStream_t s) {
    constexpr int PW = RelayCfg<ROWS>::kPW, RING = RelayCfg<ROWS>::kRing, G = RelayCfg<ROWS>::kG;
    constexpr uint32_t lds = relay_lds<ROWS, PW, RING, G>();
    static_assert(lds <= kLdsBytes, "exchange and rings fit in LDS");
    hipLaunchKernelGGL((gemv_chain_relay_kernel<ROWS, PW, RING, G, AGROUP>), dim3((uint32_t)div_up(n, kGemvCols)),
                       dim3(64 * (PW + RelayGeo<ROWS>::kCW)), lds, s, a_i8, w_i8, a_scale, w_scale, out, m, n, k, a_ld, a_shift);
    return hipGetLastError();
}

template <bool AGROUP>
hipError_t launch_chain_relay_rows(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale, uint32_t a_ld,
                                   uint32_t a_shift, const float *w_scale, uint16_t *out, uint32_t m, uint32_t n,
                                   uint32_t k, hipStream_t s) {
    if (m <= 1) return launch_chain_relay<1, AGROUP>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
    if (m <= 2) return launch_chain_relay<2, AGROUP>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
    if (m <= 4) return launch_chain_relay<4, AGROUP>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
    if (m <= 8) return launch_chain_relay<8, AGROUP>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
    return launch_chain_relay<16, AGROUP>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
}

template <bool AGROUP>
hipError_t launch_chain_stream_rows(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale, uint32_t a_ld,
                                    uint32_t a_shift, const float *w_scale, uint16_t *out, uint32_t m, uint32_t n,
                                    uint32_t k, hipStream_t s) {
    if (m <= 1) return launch_chain_stream<1, AGROUP>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
    if (m <= 2) return launch_chain_stream<2, AGROUP>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
    if (m <= 4) return launch_chain_stream<4, AGROUP>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
    if (m <= 8) return launch_chain_stream<8, AGROUP>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
    return launch_chain_stream<16, AGROUP>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
}

}  // namespace

hipError_t launch_gemv_chain(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale, uint32_t a_ld,
                             uint32_t a_shift, const float *w_scale, uint16_t *out, uint32_t m, uint32_t n,
                             uint32_t k, hipStream_t s) {
    if (k % kGemvStreamKAlign == 0 && div_up(n, kGemvCols) > (uint64_t)kGemmCus) {
        if (a_shift) return launch_chain_stream_rows<true>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
        return launch_chain_stream_rows<false>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
    }
    if (k % kGemvStreamKAlign == 0) {
        if (a_shift) return launch_chain_relay_rows<true>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
        return launch_chain_relay_rows<false>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
    }
    const dim3 grid((uint32_t)div_up(n, kGemvCols)), blk(64);
    const uint32_t nb = k / 32;
    if (nb % 4 == 0) {
        // few column tiles: one workgroup per CU, so a deeper ring costs nothing
        const bool deep = grid.x <= (uint32_t)kGemmCus;
        const uint32_t rows = m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : m <= 8 ? 8 : 16;
#define BSR_CHAIN(AG, RG, RW)                                                                              \
    hipLaunchKernelGGL((gemv_chain_lds_kernel<AG, RG, RW>), grid, blk, 0, s, a_i8, w_i8, a_scale, w_scale, \
                       out, m, n, k, a_ld, a_shift)
#define BSR_CHAIN_ROWS(AG, RG)                  \
    switch (rows) {                             \
    case 1: BSR_CHAIN(AG, RG, 1); break;        \
    case 2: BSR_CHAIN(AG, RG, 2); break;        \
    case 4: BSR_CHAIN(AG, RG, 4); break;        \
    default: BSR_CHAIN(AG, RG, 8); break;       \
    }
        if (rows == 16) {  // (37 or 44 copies per chunk: one chunk in flight)
            if (a_shift) BSR_CHAIN(true, 2, 16);
            else BSR_CHAIN(false, 2, 16);
        } else if (a_shift) {  // (its copies per chunk allow one chunk in flight)
            BSR_CHAIN_ROWS(true, 2)
        } else if (deep) {
            BSR_CHAIN_ROWS(false, 3)
        } else {
            BSR_CHAIN_ROWS(false, 2)
        }
#undef BSR_CHAIN_ROWS
#undef BSR_CHAIN
        return hipGetLastError();
    }
    if (a_shift)
        hipLaunchKernelGGL((gemv_chain_kernel<false, true>), grid, blk, 0, s, a_i8, w_i8, a_scale, w_scale, out,
                           m, n, k, a_ld, a_shift);
    else if (nb % 4 == 0)
        hipLaunchKernelGGL((gemv_chain_kernel<true, false>), grid, blk, 0, s, a_i8, w_i8, a_scale, w_scale, out,
                           m, n, k, a_ld, a_shift);
    else
        hipLaunchKernelGGL((gemv_chain_kernel<false, false>), grid, blk, 0, s, a_i8, w_i8, a_scale, w_scale, out,
                           m, n, k, a_ld, a_shift);
    return hipGetLastError();
}

namespace {

// Streamed GEMV launch (k a multiple of 256).  Waves per workgroup: about
// 2048 waves over the grid, 2 to 8 per workgroup (4 for grids of 1024
// workgroups or more); each wave gets an equal run of chunks.  The ring is
// double-buffered: deeper rings measured no faster once the grid holds ~8
// waves per CU.
template <int ROWS, bool AGROUP>
hipError_t launch_stream(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale, uint32_t a_ld,
                         uint32_t a_shift, const float *w_scale, uint16_t *out, uint32_t m, uint32_t n,
                         uint32_t k, hipStream_t s) {
    constexpr int kRing = 2;
    const uint32_t tiles = (uint32_t)div_up(n, kGemvCols);
    const uint32_t nchunks = k / 32 / kStreamChunkBlocks;
    constexpr uint32_t ring_bytes = kRing * sizeof(StreamBuf<ROWS>);
    constexpr uint32_t max_waves = kLdsBytes / ring_bytes;  // 8 up to 16 rows, 3 at 64
    static_assert(max_waves >= 3, "three waves' rings fit in LDS");
    uint32_t waves = tiles >= 1024 ? 4u : max(2u, min((uint32_t)kStreamMaxWaves, 2048u / tiles));
    waves = min(min(waves, max_waves), nchunks);
    const uint32_t cpw = (uint32_t)div_up(nchunks, waves);
    waves = (uint32_t)div_up(nchunks, cpw);
    const uint32_t lds = max(waves * ring_bytes, (ROWS > 16 ? 2 : 1) * kRedBytes);
    hipLaunchKernelGGL((gemv_stream_kernel<ROWS, kRing, AGROUP>), dim3(tiles), dim3(64 * waves), lds, s, a_i8, w_i8,
                       a_scale, w_scale, out, m, n, k, a_ld, a_shift, cpw);
    return hipGetLastError();
}

template <bool AGROUP>
hipError_t launch_stream_rows(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale, uint32_t a_ld,
                              uint32_t a_shift, const float *w_scale, uint16_t *out, uint32_t m, uint32_t n,
                              uint32_t k, hipStream_t s) {
    if (m <= 1) return launch_stream<1, AGROUP>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
    if (m <= 2) return launch_stream<2, AGROUP>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
    if (m <= 4) return launch_stream<4, AGROUP>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
    if (m <= 8) return launch_stream<8, AGROUP>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
    if (m <= 16) return launch_stream<16, AGROUP>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
    if (m <= 32) return launch_stream<32, AGROUP>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
    if (m <= 48) return launch_stream<48, AGROUP>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
    return launch_stream<64, AGROUP>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
}

}  // namespace

hipError_t launch_gemv(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale, uint32_t a_ld,
                       uint32_t a_shift, const float *w_scale, uint16_t *out, uint32_t m, uint32_t n,
                       uint32_t k, hipStream_t s) {
    if (k % kGemvStreamKAlign == 0) {
        if (a_shift) return launch_stream_rows<true>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
        return launch_stream_rows<false>(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s);
    }
    // Other K: the staged kernel when its slices fit in LDS, else the direct one.
    // Waves per workgroup: enough that the whole launch has ~24 waves per CU
    // (6144 waves over 256 CUs), but at least one iteration per wave.  The
    // staged kernel also needs at most kStagedMaxIters iterations per wave.
    const uint32_t tiles = (uint32_t)div_up(n, kGemvCols);
    const uint32_t nb = k / 32;
    const bool stageable = nb % kGemvBlocksPerIter == 0 &&
                           nb <= (uint32_t)(kGemvMaxWaves * kStagedMaxIters * kGemvBlocksPerIter);
    uint32_t waves = (uint32_t)div_up(6144, tiles);
    if (stageable) waves = max(waves, (uint32_t)div_up(nb, kStagedMaxIters * kGemvBlocksPerIter));
    waves = max(1u, min(waves, (uint32_t)kGemvMaxWaves));
    waves = min(waves, (uint32_t)div_up(nb, kGemvBlocksPerIter));
    uint32_t bpw = (uint32_t)div_up(nb, waves);
    bpw = (uint32_t)div_up(bpw, kGemvBlocksPerIter) * kGemvBlocksPerIter;
    waves = (uint32_t)div_up(nb, bpw);
    if (stageable) {
        const uint32_t lds = max(staged_geo(m, bpw).wave_bytes * waves, kRedBytes);
        if (lds <= kLdsBytes) {
            hipLaunchKernelGGL(gemv_staged_kernel, dim3(tiles), dim3(64 * waves), lds, s, a_i8, w_i8,
                               a_scale, w_scale, out, m, n, k, a_ld, a_shift, bpw);
            return hipGetLastError();
        }
    }
    const dim3 grid(tiles), blk(64 * waves);
    if (a_shift)
        hipLaunchKernelGGL((gemv_direct_kernel<false, true>), grid, blk, 0, s, a_i8, w_i8, a_scale, w_scale,
                           out, m, n, k, a_ld, a_shift, bpw);
    else if (nb % 4 == 0)
        hipLaunchKernelGGL((gemv_direct_kernel<true, false>), grid, blk, 0, s, a_i8, w_i8, a_scale, w_scale,
                           out, m, n, k, a_ld, a_shift, bpw);
    else
        hipLaunchKernelGGL((gemv_direct_kernel<false, false>), grid, blk, 0, s, a_i8, w_i8, a_scale, w_scale,
                           out, m, n, k, a_ld, a_shift, bpw);
    return hipGetLastError();
}

}  // namespace bsr
