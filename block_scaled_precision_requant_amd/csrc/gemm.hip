// gemm.hip -- int8 x int8 block-scaled GEMM for gfx950 (m > 16).
//
// Computes out[i,j] = bf16_rne( sum_b fl32(a_s[i,b] * w_s[j,b]) * P[i,j,b] ) with
// P the exact int32 dot product of 32-wide K block b -- the second launch of
// `int8_gemm_faith2_prefill` on page "metrale_model_layers/layers/ops/
// gemm_dense_int8.rs".
//
// Matrix-core work per 32 x 32 output tile and pair of K blocks:
//   * two v_mfma_i32_32x32x32_i8, each one whole scale block -> exact P;
//   * one v_mfma_f32_32x32x1_2b_f32, the outer products a_s x w_s of both
//     blocks (a single product per output, so each is fl32(a_s * w_s)).
// What is left for the vector ALU is one int -> float conversion and one FMA
// per output and block.
//
// Operand staging: a stage is kGemmStageBlocks blocks (128 bytes of every A
// and W row, i.e. whole cache lines) plus the matching scales, copied straight
// from global memory into LDS with global_load_lds (no registers held while
// the copy is in flight) into a ring of RING buffers; the next RING - 1
// stages are in flight while the current one is computed, with one barrier
// per stage.
#include "bsr_internal.h"

namespace bsr {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kChunksPerRow = kGemmStageBytes / 16;   // 8
constexpr int kRowsPerCopy = 64 / kChunksPerRow;      // 8 rows per 1 KB wave copy
static_assert(kChunksPerRow == 8, "the chunk swizzle permutes 8 chunks per row");
static_assert(kGemmStageBlocks % 2 == 0, "the 2-block f32 MFMA covers pairs of blocks");

// Geometry of one tile shape.
template <int BM, int BN, int WM, int WN>
struct Geo {
    static constexpr int kTM = WM / 32, kTN = WN / 32;  // 32x32 MFMA tiles per wave
    static constexpr int kWavesM = BM / WM, kWavesN = BN / WN;
    static constexpr int kWaves = kWavesM * kWavesN;
    static constexpr int kThreads = 64 * kWaves;
    static_assert(BM % (kRowsPerCopy) == 0 && BN % kRowsPerCopy == 0, "whole 1 KB copy segments");
    static_assert((BM * kGemmStageBlocks) % 64 == 0 && (BN * kGemmStageBlocks) % 64 == 0,
                  "whole 64-float scale segments");
};

// Workgroup -> output tile.  Workgroups are dispatched round-robin over the
// XCDs; renumber them so each XCD gets a contiguous run, then walk the runs in
// groups of kGemmGroupM tile rows so an XCD's concurrent tiles share A and W
// rows in its L2.
__device__ __forceinline__ void tile_of(uint32_t wg, uint32_t tiles_m, uint32_t tiles_n,
                                        uint32_t &tm, uint32_t &tn) {
    const uint32_t total = tiles_m * tiles_n;
    const uint32_t q = total / kXcds, r = total % kXcds;
    const uint32_t x = wg % kXcds, j = wg / kXcds;
    const uint32_t v = x * q + min(x, r) + j;
    const uint32_t per_group = kGemmGroupM * tiles_n;
    const uint32_t first_m = (v / per_group) * kGemmGroupM;
    const uint32_t gsize = min(tiles_m - first_m, (uint32_t)kGemmGroupM);
    const uint32_t in_group = v % per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

// LDS rows are 128 bytes with no padding; 16-byte chunk c of row r sits at
// slot c ^ swz(r).  Eight consecutive rows read at one chunk then hit eight
// distinct slots, and sixteen consecutive rows hit distinct (row parity, slot)
// pairs, so a 64-lane ds_read_b128 is conflict-free on 32- or 64-bank LDS.
__device__ __forceinline__ uint32_t chunk_swz(uint32_t r) { return (r & 7) ^ ((r >> 3) & 1); }

// Scale tiles are [row][block] with the 4 blocks of row r permuted by
// scale_swz(r): 32 consecutive rows read at one block then fall in 32 distinct
// banks (32- or 64-bank LDS), instead of 4 rows per bank.
__device__ __forceinline__ uint32_t scale_swz(uint32_t r) { return (r >> 3) & 3; }
static_assert(kGemmStageBlocks == 4, "scale_swz permutes 4 blocks");

template <int BM, int BN>
struct Stage {
    int8_t a[BM * kGemmStageBytes];
    int8_t w[BN * kGemmStageBytes];
    float as[BM][kGemmStageBlocks];  // [row][block ^ scale_swz(row)]
    float ws[BN][kGemmStageBlocks];
};

// Issue one stage's global -> LDS copies.  A wave's copy fills LDS in lane
// order (16 or 4 bytes per lane); the lane whose LDS slot is (row, slot)
// fetches chunk slot ^ swz(row).  Rows past M or N re-read the last row (their
// outputs are never stored); K chunks and scale blocks past the last block
// re-read the last one, and the compute zeroes the scale product of any block
// past K.  Scale copies map consecutive lanes to consecutive blocks of a row,
// so one copy touches 16 rows' worth of contiguous bytes.
// One tile's copies: NSEGS 1 KB segments of 8 rows x 128 bytes, segment `seg`
// issued by wave seg % NWAVES (compile-time trip counts, fully unrolled).
template <int NSEGS, int NWAVES>
__device__ __forceinline__ void copy_rows(int8_t *dst, const int8_t *src, uint32_t rows_limit,
                                          uint32_t r0, uint32_t K, uint32_t kb, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < (NSEGS + NWAVES - 1) / NWAVES; ++i) {
        const int seg = wave + i * NWAVES;
        if (NSEGS % NWAVES != 0 && seg >= NSEGS) break;
        const uint32_t row = seg * kRowsPerCopy + lane / kChunksPerRow;
        const uint32_t chunk = (lane % kChunksPerRow) ^ chunk_swz(row);
        const uint64_t kof = min((uint64_t)kb * 32 + chunk * 16, (uint64_t)K - 16);
        __builtin_amdgcn_global_load_lds(src + (uint64_t)min(r0 + row, rows_limit - 1) * K + kof,
                                         (lds_void *)(dst + seg * 1024), 16, 0, 0);
    }
}

// One scale tile's copies: NSEGS segments of 64 floats, consecutive lanes on
// the (swizzled) blocks of a row.  Block b of row r reads src[r * ld + (b >>
// shift)]: ld = nb, shift = 0 for a scale per block; an activation scale per
// 128 elements has ld = nb / 4, shift = 2, one per row ld = 1, shift = 31.
template <int NSEGS, int NWAVES>
__device__ __forceinline__ void copy_scales(float *dst, const float *src, uint32_t rows_limit,
                                            uint32_t r0, uint32_t ld, uint32_t shift, uint32_t nb,
                                            uint32_t kb, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < (NSEGS + NWAVES - 1) / NWAVES; ++i) {
        const int seg = wave + i * NWAVES;
        if (NSEGS % NWAVES != 0 && seg >= NSEGS) break;
        const uint32_t idx = seg * 64 + lane;  // = row * kGemmStageBlocks + slot
        const uint32_t row = idx / kGemmStageBlocks;
        const uint32_t blk = min(kb + ((idx % kGemmStageBlocks) ^ scale_swz(row)), nb - 1);
        __builtin_amdgcn_global_load_lds(src + (uint64_t)min(r0 + row, rows_limit - 1) * ld + (blk >> shift),
                                         (lds_void *)(dst + seg * 64), 4, 0, 0);
    }
}

template <class G, int BM, int BN>
__device__ __forceinline__ void issue_stage(Stage<BM, BN> &st, const int8_t *a, const int8_t *w,
                                            const float *a_s, const float *w_s, uint32_t M,
                                            uint32_t N, uint32_t K, uint32_t nb, uint32_t a_ld,
                                            uint32_t a_shift, uint32_t m0, uint32_t n0, uint32_t kb,
                                            int wave, int lane) {
    copy_rows<BM / kRowsPerCopy, G::kWaves>(st.a, a, M, m0, K, kb, wave, lane);
    copy_rows<BN / kRowsPerCopy, G::kWaves>(st.w, w, N, n0, K, kb, wave, lane);
    copy_scales<BM * kGemmStageBlocks / 64, G::kWaves>(&st.as[0][0], a_s, M, m0, a_ld, a_shift, nb, kb, wave, lane);
    copy_scales<BN * kGemmStageBlocks / 64, G::kWaves>(&st.ws[0][0], w_s, N, n0, nb, 0, nb, kb, wave, lane);
}

// Copies one wave issues per stage, when every operand's segments divide
// evenly among the waves (required for rings deeper than 2, whose waits count
// the copies of later stages).
template <class G, int BM, int BN>
constexpr int stage_copies() {
    return (BM / kRowsPerCopy + BN / kRowsPerCopy + BM * kGemmStageBlocks / 64 + BN * kGemmStageBlocks / 64) /
           G::kWaves;
}
template <class G, int BM, int BN>
constexpr bool even_copies() {
    return (BM / kRowsPerCopy) % G::kWaves == 0 && (BN / kRowsPerCopy) % G::kWaves == 0 &&
           (BM * kGemmStageBlocks / 64) % G::kWaves == 0 && (BN * kGemmStageBlocks / 64) % G::kWaves == 0;
}

// Wait until at most n of this wave's global -> LDS copies are outstanding.
// Copies complete in issue order, so this waits for every older stage.
// (s_waitcnt on gfx9: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt
// 11:8 left at their maxima.)
template <int n>
__device__ __forceinline__ void wait_copies() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
}

// Wait for a stage's copies while the copies of the `later` stages issued
// after it (C per stage, later <= N) stay in flight: s_waitcnt takes an
// immediate, so one branch per count.
template <int C, int N>
__device__ __forceinline__ void wait_later_stages(uint32_t later) {
    if constexpr (N > 0) {
        if (later == (uint32_t)N) {
            wait_copies<C * N>();
            return;
        }
        wait_later_stages<C, N - 1>(later);
    } else {
        wait_copies<0>();
    }
}

// Workgroup barrier without the release/acquire fences of __syncthreads():
// those would wait for every copy in flight (vmcnt(0)) and drain the ring.
// Visibility is handled explicitly: copies are waited for with wait_copies()
// before the barrier, and a wave's LDS reads of a stage have returned before
// its compute (which consumes them) ends.  The memory clobber keeps the
// compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Empty asm that reads and "writes" 16 accumulators: the compiler must finish
// the FMAs feeding them before this point, so a stage's compute cannot drift
// past the following wait-for-copies and barrier.
#define BSR_PIN16(x)                                                                         \
    asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), \
                 "+v"(x[6]), "+v"(x[7]), "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]),    \
                 "+v"(x[12]), "+v"(x[13]), "+v"(x[14]), "+v"(x[15]))

// KG: K groups.  With KG > 1 the workgroup holds KG copies of the wave grid,
// each with its own ring, walking its own contiguous range of stages; at the
// end the groups' FP32 tiles are added in group order through LDS.  This
// splits K inside a workgroup (no memory beyond the output) for grids too
// small to fill the CUs; the per-output order is then the groups' sum of
// sequential chains, so the path-invariant mode keeps KG = 1.
template <int BM, int BN, int WM, int WN, int WG_PER_CU, int KG, int RING>
__global__ __launch_bounds__(BM * BN / (WM * WN) * 64 * KG, WG_PER_CU) void gemm_kernel(
    const int8_t *__restrict__ a, const int8_t *__restrict__ w, const float *__restrict__ a_s,
    const float *__restrict__ w_s, uint16_t *__restrict__ out, uint32_t M, uint32_t N, uint32_t K,
    uint32_t a_ld, uint32_t a_shift, uint32_t tiles_m, uint32_t tiles_n) {
    using G = Geo<BM, BN, WM, WN>;
    constexpr int TM = G::kTM, TN = G::kTN;
    using St = Stage<BM, BN>;
    __shared__ __attribute__((aligned(1024))) St rings[KG][RING];
    static_assert(RING >= 2, "a ring of at least two buffers");
    static_assert(RING == 2 || even_copies<G, BM, BN>(), "deeper rings count uniform copies per wave");
    constexpr int kCopies = stage_copies<G, BM, BN>();
    static_assert(kCopies * (RING - 2) < 64, "the copies in flight fit the vmcnt range");
    static_assert(KG == 1 || sizeof(rings) >= sizeof(float) * KG * BM * BN, "the reduction reuses the rings");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave_all / G::kWaves;      // K group
    const int wave = wave_all % G::kWaves;     // wave within the group's grid
    St *ring = rings[grp];
    const int wm = wave / G::kWavesN, wn = wave % G::kWavesN;
    uint32_t tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const uint32_t m0 = tm * BM, n0 = tn * BN;
    const uint32_t nb = K / 32;
    const uint32_t all_stages = (nb + kGemmStageBlocks - 1) / kGemmStageBlocks;
    // this group's stages [s_first, s_first + nstages); every group steps
    // through spg barriers, so groups with fewer stages idle in their tail
    // (KG == 1: the whole K, with the bounds folded to constants of the loop)
    const uint32_t spg = KG == 1 ? all_stages : (all_stages + KG - 1) / KG;
    const uint32_t s_first = KG == 1 ? 0 : min(grp * spg, all_stages);
    const uint32_t nstages = KG == 1 ? all_stages : min(spg, all_stages - s_first);
    const uint32_t kend = KG == 1 ? nb : min(nb, (s_first + nstages) * kGemmStageBlocks);  // blocks past it add nothing

    // Per-lane LDS offsets of the MFMA operands (constant over the K loop):
    // lane l reads row (l % 32) of its 32-row tile and, for block j, the 16-byte
    // half (l / 32) of it.
    const uint32_t sw = chunk_swz(lane & 31);
    const int half = lane >> 5;
    // (rows of a tile differ by 32 * 128 bytes, a constant the compiler folds
    // into the ds_read offset, so one offset per block is kept)
    int off_a[kGemmStageBlocks], off_w[kGemmStageBlocks];
#pragma unroll
    for (int j = 0; j < kGemmStageBlocks; ++j) {
        const int chunk = 2 * j + half;
        off_a[j] = (wm * WM + (lane & 31)) * kGemmStageBytes + ((chunk ^ sw) << 4);
        off_w[j] = (wn * WN + (lane & 31)) * kGemmStageBytes + ((chunk ^ sw) << 4);
    }

    float acc[TM][TN][16];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const v16i zero16 = {};
    const v32f zero32 = {};

    // A block pair (blocks jp, jp + 1 of the stage) = 2 * TM * TN units (tile
    // t = sm * TN + sn, block j).  The matrix-core result of unit u + 1 (and the
    // scale products of its tile) is requested before unit u is rescaled, so
    // each rescale reads a result that finished while the previous unit's 32
    // VALU instructions ran.
    auto pair = [&](const St &cur, uint32_t kb, int jp) {
        v4i af[TM][2], bf[TN][2];
        float asv[TM], wsv[TN];
        // lanes 0-31 carry block jp, lanes 32-63 block jp + 1 (zero if past
        // the group's range)
        const bool blk_live = kb + jp + half < kend;
#pragma unroll
        for (int t = 0; t < TM; ++t) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
                af[t][j] = *reinterpret_cast<const v4i *>(cur.a + off_a[jp + j] + t * 32 * kGemmStageBytes);
            const uint32_t ra = wm * WM + t * 32 + (lane & 31);
            const float av = cur.as[ra][(jp + half) ^ scale_swz(ra)];
            asv[t] = blk_live ? av : 0.0f;
        }
#pragma unroll
        for (int t = 0; t < TN; ++t) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bf[t][j] = *reinterpret_cast<const v4i *>(cur.w + off_w[jp + j] + t * 32 * kGemmStageBytes);
            const uint32_t rw = wn * WN + t * 32 + (lane & 31);
            wsv[t] = cur.ws[rw][(jp + half) ^ scale_swz(rw)];
        }
        constexpr int kUnits = 2 * TM * TN;
        v32f sc[2];
        v16i p[2];
        sc[0] = __builtin_amdgcn_mfma_f32_32x32x1f32(asv[0], wsv[0], zero32, 0, 0, 0);
        p[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[0][0], bf[0][0], zero16, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            const int t = u >> 1, j = u & 1;
            if (u + 1 < kUnits) {
                const int t1 = (u + 1) >> 1, j1 = (u + 1) & 1;
                if (j1 == 0)
                    sc[t1 & 1] = __builtin_amdgcn_mfma_f32_32x32x1f32(asv[t1 / TN], wsv[t1 % TN], zero32, 0, 0, 0);
                p[(u + 1) & 1] =
                    __builtin_amdgcn_mfma_i32_32x32x32_i8(af[t1 / TN][j1], bf[t1 % TN][j1], zero16, 0, 0, 0);
            }
            float *ac = acc[t / TN][t % TN];
#pragma unroll
            for (int r = 0; r < 16; ++r) ac[r] = fmaf((float)p[u & 1][r], sc[t & 1][16 * j + r], ac[r]);
        }
    };
    auto compute = [&](const St &cur, uint32_t kb) {
#pragma unroll
        for (int jp = 0; jp < kGemmStageBlocks; jp += 2) {
            pair(cur, kb, jp);
            // read the next pair's operands only after this pair: bounds live registers
            asm volatile("" ::: "memory");
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) BSR_PIN16(acc[i][j]);
    };
    auto issue = [&](St &buf, uint32_t stage) {
        issue_stage<G>(buf, a, w, a_s, w_s, M, N, K, nb, a_ld, a_shift, m0, n0, (s_first + stage) * kGemmStageBlocks,
                       wave, lane);
    };
    // Stage s lives in buffer s % RING.  At the top of stage s each wave waits
    // for its own copies of stage s (those of the up to RING - 2 later stages
    // already issued may stay in flight), the barrier publishes every wave's
    // copies and frees buffer (s - 1) % RING (its reads are done), and the
    // copies of stage s + RING - 1 go into it before stage s is computed.
    auto step = [&](int u, uint32_t s) {
        wait_later_stages<kCopies, RING - 2>(s < nstages ? min(nstages - 1 - s, (uint32_t)RING - 2) : 0);
        stage_barrier();
        if (s + RING - 1 < nstages) issue(ring[(u + RING - 1) % RING], s + RING - 1);
        if (KG == 1 || s < nstages) compute(ring[u], (s_first + s) * kGemmStageBlocks);
    };
#pragma unroll
    for (int r = 0; r < RING - 1; ++r)
        if ((KG == 1 && r == 0) || (uint32_t)r < nstages) issue(ring[r], r);  // (KG == 1: K has a stage)
    for (uint32_t s = 0; s < spg; s += RING) {
#pragma unroll
        for (int u = 0; u < RING; ++u) {
            if (u > 0 && s + u >= spg) break;
            step(u, s + u);
        }
    }

    if constexpr (KG > 1) {
        // Groups' tiles through LDS (the rings are free once every wave has
        // passed this barrier), summed in group order by group 0.
        __syncthreads();
        float *red = reinterpret_cast<float *>(&rings[0][0]);
        constexpr int kTile = TM * TN * 16;  // floats per lane
        const uint32_t slot = (uint32_t)(wave * 64 + lane) * kTile;
        constexpr uint32_t kGroupFloats = G::kWaves * 64 * kTile;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) red[grp * kGroupFloats + slot + (i * TN + j) * 16 + r] = acc[i][j][r];
        __syncthreads();
        if (grp != 0) return;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float t = red[slot + (i * TN + j) * 16 + r];
                    for (int g = 1; g < KG; ++g) t += red[g * kGroupFloats + slot + (i * TN + j) * 16 + r];
                    acc[i][j][r] = t;
                }
    }

    // Output layout of a 32x32 MFMA tile: lane l holds column l % 32 and, in
    // register r, row 8 * (r / 4) + 4 * (l / 32) + r % 4.
#pragma unroll
    for (int sm = 0; sm < TM; ++sm)
#pragma unroll
        for (int sn = 0; sn < TN; ++sn) {
            const uint32_t col = n0 + wn * WN + sn * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const uint32_t row = m0 + wm * WM + sm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row < M && col < N) out[(uint64_t)row * N + col] = f32_to_bf16_rne(acc[sm][sn][r]);
            }
        }
}

template <int BM, int BN, int WM, int WN, int WG_PER_CU, int KG = 1, int RING = 2>
hipError_t launch_tiles(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale,
                        const float *w_scale, uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                        uint32_t a_ld, uint32_t a_shift, hipStream_t s) {
    const uint32_t tiles_m = (uint32_t)div_up(m, BM);
    const uint32_t tiles_n = (uint32_t)div_up(n, BN);
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, WG_PER_CU, KG, RING>), dim3(tiles_m * tiles_n),
                       dim3(Geo<BM, BN, WM, WN>::kThreads * KG), 0, s, a_i8, w_i8, a_scale, w_scale, out, m, n,
                       k, a_ld, a_shift, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale, uint32_t a_ld,
                       uint32_t a_shift, const float *w_scale, uint16_t *out, uint32_t m, uint32_t n,
                       uint32_t k, bool split_k, hipStream_t s) {
    // Grids of at least two 128x128 tiles per CU: two 4-wave 128x128
    // workgroups per CU (LDS 2 x 72 KB, 2 x 4 waves of about 230 VGPRs); their
    // barriers fall at different times, so one computes while the other waits
    // (measured faster than one 8-wave 256x128 workgroup per CU at
    // 2048x4096x4096 and 4096x28672x4096).  Smaller grids -- every m <= 128,
    // and e.g. m = 512 at n = 4096 -- take 64x64 tiles of four 32x32 waves:
    // four times the workgroups, 1.1-2.5x faster from m = 17 to 1024 on the
    // decode and attention widths.  Per output the blocks are accumulated in
    // the same order in both, so the bits do not depend on the shape chosen.
    const uint64_t big_tiles = div_up(m, kGemmBM) * div_up(n, kGemmBN);
    if (m > (uint32_t)kGemmBM && big_tiles >= 2 * (uint64_t)kGemmCus)
        return launch_tiles<kGemmBM, kGemmBN, 64, 64, 2>(a_i8, w_i8, a_scale, w_scale, out, m, n, k, a_ld,
                                                         a_shift, s);
    // Small grids, when K may be split inside a workgroup (its K groups each
    // walk a contiguous range of stages; the FP32 tiles are summed in group
    // order at the end) and K has a stage for every group:
    //  * at most one 32x32 tile per CU: 8 one-wave groups per workgroup
    //    (144 KB of LDS), e.g. m <= 64 at n = 4096, 2x faster than 64x64 tiles;
    //  * at most two: 4 groups, two workgroups per CU (72 KB each) -- also
    //    pads m = 17-32 to 32 rows instead of 64;
    //  * at most one 64x64 tile per CU: 2 groups of four 32x32 waves, each
    //    with a 3-deep ring (two stages in flight while one is computed).
    const uint64_t t32 = div_up(m, kGemmTinyTile) * div_up(n, kGemmTinyTile);
    const uint64_t small_tiles = div_up(m, kGemmSmallTile) * div_up(n, kGemmSmallTile);
    const uint32_t stages = (k / 32 + kGemmStageBlocks - 1) / kGemmStageBlocks;
    if (split_k && t32 <= (uint64_t)kGemmCus && stages >= 8)
        return launch_tiles<kGemmTinyTile, kGemmTinyTile, 32, 32, 1, 8>(a_i8, w_i8, a_scale, w_scale, out, m, n, k,
                                                                         a_ld, a_shift, s);
    if (split_k && t32 <= 2 * (uint64_t)kGemmCus && stages >= 4)
        return launch_tiles<kGemmTinyTile, kGemmTinyTile, 32, 32, 2, 4>(a_i8, w_i8, a_scale, w_scale, out, m, n, k,
                                                                         a_ld, a_shift, s);
    if (split_k && small_tiles <= (uint64_t)kGemmCus && stages >= 2)
        return launch_tiles<kGemmSmallTile, kGemmSmallTile, 32, 32, 1, 2, 3>(a_i8, w_i8, a_scale, w_scale, out, m,
                                                                             n, k, a_ld, a_shift, s);
    return launch_tiles<kGemmSmallTile, kGemmSmallTile, 32, 32, 2>(a_i8, w_i8, a_scale, w_scale, out, m, n, k,
                                                                   a_ld, a_shift, s);
}

}  // namespace bsr
