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
// from global memory into LDS with buffer loads (no registers held while the
// copy is in flight, and per-lane offsets fixed for the whole K loop) into a
// ring of RING buffers; the next RING - 1 stages are in flight while the
// current one is computed, with one barrier per stage.  A copy costs about
// one cycle of the CU's load path per cache line it touches, whatever its
// bytes, so the 256 x 128 and 128 x 128 shapes and the 64 x 64 shape with a
// ring of 4 stage their scales 8 blocks (32 bytes of a row) at a time, every
// other stage, and
// spread the next stage's copies over the units that compute the stage before
// it instead of issuing them all after the barrier, where the eight waves of
// a CU queued behind each other.
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
// groups of GROUP tile rows so an XCD's concurrent tiles share A and W rows in
// its L2.
template <uint32_t GROUP>
__device__ __forceinline__ void tile_of(uint32_t wg, uint32_t tiles_m, uint32_t tiles_n,
                                        uint32_t &tm, uint32_t &tn) {
    const uint32_t total = tiles_m * tiles_n;
    const uint32_t q = total / kXcds, r = total % kXcds;
    const uint32_t x = wg % kXcds, j = wg / kXcds;
    const uint32_t v = x * q + min(x, r) + j;
    const uint32_t per_group = GROUP * tiles_n;
    const uint32_t first_m = (v / per_group) * GROUP;
    const uint32_t gsize = min(tiles_m - first_m, GROUP);
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

// The 128 x 128 shape (ring of 2) and the 64 x 64 shapes with a ring of 4
// keep their scales apart from the operand ring: one scale stage covers two
// operand stages (8 blocks, 32 bytes of every scale row), so a scale copy
// touches 8 rows' cache lines instead of 16.  Its 8
// blocks of row r are permuted by scale_swz8(r): 32 consecutive rows read at
// one block then hit 32 distinct banks (32- or 64-bank LDS).
template <int BM, int BN>
struct OpStage {
    int8_t a[BM * kGemmStageBytes];
    int8_t w[BN * kGemmStageBytes];
};
constexpr int kSc8Blocks = 2 * kGemmStageBlocks;
template <int BM, int BN>
struct Sc8Stage {
    float as[BM][kSc8Blocks];  // [row][block ^ scale_swz8(row)]
    float ws[BN][kSc8Blocks];
};
__device__ __forceinline__ uint32_t scale_swz8(uint32_t r) { return (r >> 2) & 7; }

// Operand staging: buffer loads straight into LDS.  A wave's copy fills LDS
// in lane order (16 bytes per lane for operand rows, 4 for scales); the lane
// whose LDS slot is (row, slot) fetches chunk slot ^ chunk_swz(row), and scale
// copies map consecutive lanes to the (swizzled) blocks of a row: an operand
// copy covers 8 rows, a scale copy 16 rows of 4 blocks (8 rows of 8 blocks in
// the 8-block scale stages).  Every lane's byte offset within
// its workgroup's rows is fixed for the whole K loop -- only the scalar K
// offset of a stage changes -- so a stage's copies cost no vector address
// arithmetic.  Each operand's buffer starts at the workgroup's first row and
// ends at its last row inside M (N), so rows past the matrix, and K bytes past
// the last row's end, read as zero (the buffer range check); other bytes past
// K in a row read the next row's first blocks, whose scale products the
// compute zeroes.  Offsets are 32-bit: a tile's rows span less than 4 GiB
// (k < kGemmMaxK, checked before launch).  Block b of an activation-scale row
// r reads a_s[r * ld + (b >> shift)]: ld = nb, shift = 0 for a scale per
// block; a scale per 128 elements has ld = nb / 4, shift = 2, one per row
// ld = 1, shift = 31.
template <int BM, int BN, int NWAVES, bool SC8 = false>
struct BufStage {
    static constexpr int kSegA = BM / kRowsPerCopy, kSegW = BN / kRowsPerCopy;
    // scale copies: 64 lanes = 16 rows x 4 blocks, or 8 rows x 8 blocks (SC8)
    static constexpr int kScBlocks = SC8 ? kSc8Blocks : kGemmStageBlocks;
    static constexpr int kSegAs = BM * kScBlocks / 64, kSegWs = BN * kScBlocks / 64;
    static constexpr int kNA = (kSegA + NWAVES - 1) / NWAVES, kNW = (kSegW + NWAVES - 1) / NWAVES;
    static constexpr int kNAs = (kSegAs + NWAVES - 1) / NWAVES, kNWs = (kSegWs + NWAVES - 1) / NWAVES;
    __amdgpu_buffer_rsrc_t ra, rw, ras, rws;
    uint32_t oa[kNA], ow[kNW], oas[kNAs], ows[kNWs];
    uint32_t a_shift;

    static constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit elements (gfx9)

    __device__ __forceinline__ void init(const int8_t *a, const int8_t *w, const float *a_s, const float *w_s,
                                         uint32_t M, uint32_t N, uint32_t K, uint32_t nb, uint32_t a_ld,
                                         uint32_t shift, uint32_t m0, uint32_t n0, int wave, int lane) {
        const uint32_t rows_a = min((uint32_t)BM, M - m0), rows_w = min((uint32_t)BN, N - n0);
        ra = __builtin_amdgcn_make_buffer_rsrc((void *)(a + (uint64_t)m0 * K), (short)0, (int)(rows_a * K), kRsrcWord3);
        rw = __builtin_amdgcn_make_buffer_rsrc((void *)(w + (uint64_t)n0 * K), (short)0, (int)(rows_w * K), kRsrcWord3);
        ras = __builtin_amdgcn_make_buffer_rsrc((void *)(a_s + (uint64_t)m0 * a_ld), (short)0, (int)(rows_a * a_ld * 4),
                                                kRsrcWord3);
        rws = __builtin_amdgcn_make_buffer_rsrc((void *)(w_s + (uint64_t)n0 * nb), (short)0, (int)(rows_w * nb * 4),
                                                kRsrcWord3);
        a_shift = shift;
#pragma unroll
        for (int i = 0; i < kNA; ++i) {
            const uint32_t row = (wave + i * NWAVES) * kRowsPerCopy + lane / kChunksPerRow;
            oa[i] = row * K + (((lane % kChunksPerRow) ^ chunk_swz(row)) << 4);
        }
#pragma unroll
        for (int i = 0; i < kNW; ++i) {
            const uint32_t row = (wave + i * NWAVES) * kRowsPerCopy + lane / kChunksPerRow;
            ow[i] = row * K + (((lane % kChunksPerRow) ^ chunk_swz(row)) << 4);
        }
#pragma unroll
        for (int i = 0; i < kNAs; ++i) {
            const uint32_t idx = (wave + i * NWAVES) * 64 + lane, row = idx / kScBlocks;
            const uint32_t blk = (idx % kScBlocks) ^ (SC8 ? scale_swz8(row) : scale_swz(row));
            // a scale per 2^shift blocks; a stage's first block is a multiple of 4
            oas[i] = row * a_ld * 4 + (shift >= 31 ? 0u : (blk >> shift) * 4);
        }
#pragma unroll
        for (int i = 0; i < kNWs; ++i) {
            const uint32_t idx = (wave + i * NWAVES) * 64 + lane, row = idx / kScBlocks;
            const uint32_t blk = (idx % kScBlocks) ^ (SC8 ? scale_swz8(row) : scale_swz(row));
            ows[i] = row * nb * 4 + blk * 4;
        }
    }

    // SC8, one copy I (compile-time) of a stage's kAll: the operand segments
    // of the stage from block kb into (sa, sw), then the wave's copies of half
    // a scale stage -- the A scale rows of the 8 blocks from kbs into sas when
    // !wside, else the W scale rows into sws (every count divides evenly among
    // the waves; when the halves differ, as for 256 x 128 tiles, the smaller
    // one skips its last copies).
    static constexpr int kNSc = kNAs > kNWs ? kNAs : kNWs;  // copies of the larger scale half
    static constexpr int kAll = kNA + kNW + kNSc;
    template <int I>
    __device__ __forceinline__ void issue_one(int8_t *sa, int8_t *sw, float *sas, float *sws, uint32_t kb,
                                              uint32_t kbs, bool wside, int wave) const {
        static_assert(SC8 && kSegA % NWAVES == 0 && kSegW % NWAVES == 0 && kSegAs % NWAVES == 0 &&
                          kSegWs % NWAVES == 0,
                      "uniform copies");
        if constexpr (I < kNA) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(sa + (wave + I * NWAVES) * 1024), 16, oa[I],
                                                     kb * 32, 0, 0);
        } else if constexpr (I < kNA + kNW) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void *)(sw + (wave + (I - kNA) * NWAVES) * 1024), 16,
                                                     ow[I - kNA], kb * 32, 0, 0);
        } else if constexpr (I < kAll) {
            constexpr int J = I - kNA - kNW;
            const int seg = wave + J * NWAVES;
            if (wside ? J < kNWs : J < kNAs)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wside ? rws : ras,
                                                         (lds_void *)((wside ? sws : sas) + seg * 64), 4,
                                                         wside ? ows[J < kNWs ? J : 0] : oas[J < kNAs ? J : 0],
                                                         wside ? kbs * 4 : (kbs >> a_shift) * 4, 0, 0);
        }
    }

    // SC8, all of a stage's copies: its operands and the wave's copies of one
    // scale half (as issue_one over [0, kAll))
    __device__ __forceinline__ void issue_stage(int8_t *sa, int8_t *sw, float *sas, float *sws, uint32_t kb,
                                               uint32_t kbs, bool wside, int wave) const {
        if (sa != nullptr) {
#pragma unroll
            for (int i = 0; i < kNA; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(sa + (wave + i * NWAVES) * 1024), 16, oa[i],
                                                         kb * 32, 0, 0);
#pragma unroll
            for (int i = 0; i < kNW; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void *)(sw + (wave + i * NWAVES) * 1024), 16, ow[i],
                                                         kb * 32, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < kNSc; ++j) {
            const int seg = wave + j * NWAVES;
            if (wside ? j < kNWs : j < kNAs)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wside ? rws : ras,
                                                         (lds_void *)((wside ? sws : sas) + seg * 64), 4,
                                                         wside ? ows[j < kNWs ? j : 0] : oas[j < kNAs ? j : 0],
                                                         wside ? kbs * 4 : (kbs >> a_shift) * 4, 0, 0);
        }
    }

    // copies [LO, HI) of a stage
    template <int LO, int HI>
    __device__ __forceinline__ void issue_range(int8_t *sa, int8_t *sw, float *sas, float *sws, uint32_t kb,
                                                uint32_t kbs, bool wside, int wave) const {
        if constexpr (LO < HI) {
            issue_one<LO>(sa, sw, sas, sws, kb, kbs, wside, wave);
            issue_range<LO + 1, HI>(sa, sw, sas, sws, kb, kbs, wside, wave);
        }
    }

    // One stage's copies (first block kb): 1 KB per row-segment instruction,
    // 256 bytes per scale-segment instruction; segment `seg` of an operand is
    // issued by wave seg % NWAVES.
    __device__ __forceinline__ void issue(Stage<BM, BN> &st, uint32_t kb, int wave) const {
        issue_parts(st.a, st.w, &st.as[0][0], &st.ws[0][0], kb, wave);
    }
    __device__ __forceinline__ void issue_parts(int8_t *sta, int8_t *stw, float *stas, float *stws, uint32_t kb,
                                                int wave) const {
#pragma unroll
        for (int i = 0; i < kNA; ++i) {
            const int seg = wave + i * NWAVES;
            if (kSegA % NWAVES != 0 && seg >= kSegA) break;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(sta + seg * 1024), 16, oa[i], kb * 32, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < kNW; ++i) {
            const int seg = wave + i * NWAVES;
            if (kSegW % NWAVES != 0 && seg >= kSegW) break;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void *)(stw + seg * 1024), 16, ow[i], kb * 32, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < kNAs; ++i) {
            const int seg = wave + i * NWAVES;
            if (kSegAs % NWAVES != 0 && seg >= kSegAs) break;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ras, (lds_void *)(stas + seg * 64), 4, oas[i],
                                                     (kb >> a_shift) * 4, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < kNWs; ++i) {
            const int seg = wave + i * NWAVES;
            if (kSegWs % NWAVES != 0 && seg >= kSegWs) break;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rws, (lds_void *)(stws + seg * 64), 4, ows[i], kb * 4,
                                                     0, 0);
        }
    }
};

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

// The first of C copies that unit g of U issues: two each for the first
// C - U units, one each after them (C <= 2 U).
template <int C, int U>
constexpr int spread_first(int g) { return g + (g < C - U ? g : C - U); }

}  // namespace

namespace gemm_kernels {

// KG: K groups.  With KG > 1 the workgroup holds KG copies of the wave grid,
// each with its own ring, walking its own contiguous range of stages; at the
// end the groups' FP32 tiles are added in group order through LDS.  This
// splits K inside a workgroup (no memory beyond the output) for grids too
// small to fill the CUs; the per-output order is then the groups' sum of
// sequential chains, so the path-invariant mode keeps KG = 1.
// SPLIT: K split across workgroups.  Workgroup g runs tile g % tiles over the
// slice_stages stages of slice g / tiles and writes its FP32 tile to
// partial[slice * pitch + row * N + col] instead of BF16 out; the slices are
// added in slice order by split_reduce_kernel.
template <int BM, int BN, int WM, int WN, int WG_PER_CU, int KG, int RING, bool SPLIT>
__global__ __launch_bounds__(BM * BN / (WM * WN) * 64 * KG, WG_PER_CU) void gemm_kernel(
    const int8_t *__restrict__ a, const int8_t *__restrict__ w, const float *__restrict__ a_s,
    const float *__restrict__ w_s, uint16_t *__restrict__ out, uint32_t M, uint32_t N, uint32_t K,
    uint32_t a_ld, uint32_t a_shift, uint32_t tiles_m, uint32_t tiles_n, float *__restrict__ partial,
    uint64_t pitch, uint32_t slice_stages) {
    static_assert(!(SPLIT && KG > 1), "one K split at a time");
    using G = Geo<BM, BN, WM, WN>;
    constexpr int TM = G::kTM, TN = G::kTN;
    using St = Stage<BM, BN>;
    // kSc8 -- the 256 x 128 and 128 x 128 shapes with a ring of 2 and the 64 x 64
    // shape with a ring of 4 (K split or not): operands in RING OpStage buffers, scales in
    // Sc8Stage buffers of 8 blocks (2 for a ring of 2; 3 for a ring of 4,
    // whose copies run three stages ahead), and each stage's copies spread
    // over the units that compute the stage before them.
    constexpr bool kSc8 = (RING == 2 && KG == 1 && !SPLIT && (BM == 128 || BM == kGemmTallBM) && BN == 128) ||
                          (RING == 4 && KG == 1 && BM == 64 && BN == 64);
    constexpr int kScBufs = RING == 2 ? 2 : 3;
    // units that carry the copies: a ring of 2 leaves the copies one stage to
    // land, so only the first pair's units carry them; a ring of 4, all units
    constexpr int kSpreadUnits = RING == 2 ? 2 * TM * TN : 4 * TM * TN;
    using Op = OpStage<BM, BN>;
    using Sc = Sc8Stage<BM, BN>;
    constexpr size_t kLds = kSc8 ? RING * sizeof(Op) + kScBufs * sizeof(Sc) : sizeof(St) * KG * RING;
    __shared__ __attribute__((aligned(1024))) char lds[kLds];
    St(*rings)[RING] = reinterpret_cast<St(*)[RING]>(lds);
    Op *ops = reinterpret_cast<Op *>(lds);
    Sc *scs = reinterpret_cast<Sc *>(lds + RING * sizeof(Op));
    static_assert(RING >= 2, "a ring of at least two buffers");
    static_assert(RING == 2 || even_copies<G, BM, BN>(), "deeper rings count uniform copies per wave");
    constexpr int kCopies = stage_copies<G, BM, BN>();
    static_assert(kCopies * (RING - 2) < 64, "the copies in flight fit the vmcnt range");
    static_assert(KG == 1 || kLds >= sizeof(float) * KG * BM * BN, "the reduction reuses the rings");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave_all / G::kWaves;      // K group
    const int wave = wave_all % G::kWaves;     // wave within the group's grid
    St *ring = rings[grp];
    const int wm = wave / G::kWavesN, wn = wave % G::kWavesN;
    uint32_t tm, tn, tile = blockIdx.x, slice = 0;
    if constexpr (SPLIT) {
        slice = blockIdx.x / (tiles_m * tiles_n);
        tile = blockIdx.x % (tiles_m * tiles_n);
    }
    tile_of<BM == kGemmTallBM ? kGemmTallGroupM : kGemmGroupM>(tile, tiles_m, tiles_n, tm, tn);
    const uint32_t m0 = tm * BM, n0 = tn * BN;
    const uint32_t nb = K / 32;
    const uint32_t all_stages = (nb + kGemmStageBlocks - 1) / kGemmStageBlocks;
    // this group's (slice's) stages [s_first, s_first + nstages); every group
    // steps through spg barriers, so groups with fewer stages idle in their
    // tail (no split: the whole K, with the bounds folded to constants of the
    // loop)
    constexpr bool kRange = KG > 1 || SPLIT;
    const uint32_t spg = SPLIT ? slice_stages : (KG == 1 ? all_stages : (all_stages + KG - 1) / KG);
    const uint32_t s_first = SPLIT ? slice * slice_stages : (KG == 1 ? 0 : min(grp * spg, all_stages));
    const uint32_t nstages = kRange ? min(spg, all_stages - min(s_first, all_stages)) : all_stages;
    const uint32_t kend = kRange ? min(nb, (s_first + nstages) * kGemmStageBlocks) : nb;  // blocks past it add nothing

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
    BufStage<BM, BN, G::kWaves, kSc8> bufst;
    bufst.init(a, w, a_s, w_s, M, N, K, nb, a_ld, a_shift, m0, n0, wave, lane);
    // the next stage's copies (kSc8): operand slot, scale half, blocks
    int8_t *nx_a = nullptr, *nx_w = nullptr;
    float *nx_as = nullptr, *nx_ws = nullptr;
    uint32_t nx_kb = 0, nx_kbs = 0;
    bool nx_wside = false;
    constexpr int kScRow = kSc8 ? kSc8Blocks : kGemmStageBlocks;
    auto sidx = [&](uint32_t row, uint32_t blk) {
        return row * kScRow + (blk ^ (kSc8 ? scale_swz8(row) : scale_swz(row)));
    };

    // A block pair (blocks jp, jp + 1 of the stage) = 2 * TM * TN units (tile
    // t = sm * TN + sn, block j).  The matrix-core result of unit u + 1 (and the
    // scale products of its tile) is requested before unit u is rescaled, so
    // each rescale reads a result that finished while the previous unit's 32
    // VALU instructions ran.
    // operands ca / cw, scale rows cas / cws whose block boff is the stage's first
    auto pair = [&](const int8_t *ca, const int8_t *cw, const float *cas, const float *cws, uint32_t boff,
                    uint32_t kb, int jp) __attribute__((always_inline)) {
        v4i af[TM][2], bf[TN][2];
        float asv[TM], wsv[TN];
        // lanes 0-31 carry block jp, lanes 32-63 block jp + 1 (zero if past
        // the group's range)
        const bool blk_live = kb + jp + half < kend;
#pragma unroll
        for (int t = 0; t < TM; ++t) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
                af[t][j] = *reinterpret_cast<const v4i *>(ca + off_a[jp + j] + t * 32 * kGemmStageBytes);
            const uint32_t ra = wm * WM + t * 32 + (lane & 31);
            const float av = cas[sidx(ra, boff + jp + half)];
            asv[t] = blk_live ? av : 0.0f;
        }
#pragma unroll
        for (int t = 0; t < TN; ++t) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bf[t][j] = *reinterpret_cast<const v4i *>(cw + off_w[jp + j] + t * 32 * kGemmStageBytes);
            const uint32_t rw = wn * WN + t * 32 + (lane & 31);
            wsv[t] = cws[sidx(rw, boff + jp + half)];
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
                // The wave issuing matrix-core work goes ahead of the other
                // wave's rescale on the same SIMD, so the matrix core is fed
                // as soon as its operands are ready.
                __builtin_amdgcn_s_setprio(1);
                if (j1 == 0)
                    sc[t1 & 1] = __builtin_amdgcn_mfma_f32_32x32x1f32(asv[t1 / TN], wsv[t1 % TN], zero32, 0, 0, 0);
                p[(u + 1) & 1] =
                    __builtin_amdgcn_mfma_i32_32x32x32_i8(af[t1 / TN][j1], bf[t1 % TN][j1], zero16, 0, 0, 0);
                __builtin_amdgcn_s_setprio(0);
            }
            if constexpr (kSc8) {
                // unit g of the stage (over its pairs) issues copies
                // [first(g), first(g + 1)) of the next stage's kAll: two each
                // for the first kAll - kSpreadUnits units, then one each
                using BS = decltype(bufst);
                static_assert(BS::kAll >= kSpreadUnits && BS::kAll <= 2 * kSpreadUnits, "one or two per unit");
                const int g = (jp / 2) * kUnits + u;
#define BSR_UNIT(G)                                                                                   \
    case G:                                                                                           \
        if constexpr (G < kSpreadUnits)                                                               \
            bufst.template issue_range<spread_first<BS::kAll, kSpreadUnits>(G),                        \
                                       spread_first<BS::kAll, kSpreadUnits>(G + 1)>(                   \
                nx_a, nx_w, nx_as, nx_ws, nx_kb, nx_kbs, nx_wside, wave);                            \
        break;
                switch (g) {
                    BSR_UNIT(0)
                    BSR_UNIT(1)
                    BSR_UNIT(2)
                    BSR_UNIT(3)
                    BSR_UNIT(4)
                    BSR_UNIT(5)
                    BSR_UNIT(6)
                    BSR_UNIT(7)
                default: break;
                }
#undef BSR_UNIT
            }
            float *ac = acc[t / TN][t % TN];
#pragma unroll
            for (int r = 0; r < 16; ++r) ac[r] = fmaf((float)p[u & 1][r], sc[t & 1][16 * j + r], ac[r]);
        }
    };
    auto compute = [&](const int8_t *ca, const int8_t *cw, const float *cas, const float *cws, uint32_t boff,
                       uint32_t kb) {
#pragma unroll
        for (int jp = 0; jp < kGemmStageBlocks; jp += 2) {
            pair(ca, cw, cas, cws, boff, kb, jp);
            // read the next pair's operands only after this pair: bounds live registers
            asm volatile("" ::: "memory");
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) BSR_PIN16(acc[i][j]);
    };
    auto issue = [&](St &buf, uint32_t stage) { bufst.issue(buf, (s_first + stage) * kGemmStageBlocks, wave); };
    // kSc8: the copies of stage t are its operands (into slot t % RING) and
    // half of a scale stage: for odd t the A rows of scale stage (t + 1) / 2,
    // for even t the W rows of scale stage t / 2, so both halves of scale
    // stage j have landed by the top of stage 2j, and each goes into the
    // buffer scale stage j - kScBufs left, which the stages before the
    // current one finished with.  Past the group's last stage the copies
    // re-read in-range blocks into buffers nobody reads any more.
    auto set_next = [&](uint32_t t) {
        const uint32_t last = nstages - 1;
        nx_a = ops[t % RING].a;
        nx_w = ops[t % RING].w;
        nx_kb = (s_first + min(t, last)) * kGemmStageBlocks;
        nx_wside = t % 2 == 0;
        const uint32_t sst = nx_wside ? t / 2 : (t + 1) / 2;
        nx_as = &scs[sst % kScBufs].as[0][0];
        nx_ws = &scs[sst % kScBufs].ws[0][0];
        nx_kbs = (s_first + min(2 * sst, last)) * kGemmStageBlocks;
    };
    // Stage s lives in buffer s % RING.  At the top of stage s each wave waits
    // for its own copies of stage s (those of the up to RING - 2 later stages
    // already issued may stay in flight), the barrier publishes every wave's
    // copies and frees buffer (s - 1) % RING (its reads are done), and the
    // copies of stage s + RING - 1 go into it before stage s is computed.
    auto step = [&](int u, uint32_t s) {
        wait_later_stages<kCopies, RING - 2>(s < nstages ? min(nstages - 1 - s, (uint32_t)RING - 2) : 0);
        stage_barrier();
        if constexpr (kSc8) {
            // Stage s reads operand slot u and scale stage s / 2 (blocks from
            // (s % 2) * 4); its units bring the copies of stage s + RING - 1.
            set_next(s + RING - 1);
            if (!kRange || s < nstages) {
                const Sc &sc = scs[(s / 2) % kScBufs];
                compute(ops[u].a, ops[u].w, &sc.as[0][0], &sc.ws[0][0], (s % 2) * kGemmStageBlocks,
                        (s_first + s) * kGemmStageBlocks);
            }
        } else {
            if (s + RING - 1 < nstages) issue(ring[(u + RING - 1) % RING], s + RING - 1);
            if (!kRange || s < nstages)
                compute(ring[u].a, ring[u].w, &ring[u].as[0][0], &ring[u].ws[0][0], 0,
                        (s_first + s) * kGemmStageBlocks);
        }
    };
    if constexpr (kSc8) {
        // the A half of scale stage 0 (stage 0's copies bring its W half), then
        // the copies of stages 0 .. RING - 2
        bufst.issue_stage(nullptr, nullptr, &scs[0].as[0][0], nullptr, 0, s_first * kGemmStageBlocks, false, wave);
#pragma unroll
        for (int t = 0; t < RING - 1; ++t) {
            set_next(t);
            bufst.issue_stage(nx_a, nx_w, nx_as, nx_ws, nx_kb, nx_kbs, nx_wside, wave);
        }
    } else {
#pragma unroll
        for (int r = 0; r < RING - 1; ++r)
            if ((!kRange && r == 0) || (uint32_t)r < nstages) issue(ring[r], r);  // (no split: K has a stage)
    }
    for (uint32_t s = 0; s < spg; s += RING) {
#pragma unroll
        for (int u = 0; u < RING; ++u) {
            if (u > 0 && s + u >= spg) break;
            step(u, s + u);
        }
    }
    if constexpr (kSc8) wait_copies<0>();  // the copies issued by the last stage land before the workgroup ends

    if constexpr (KG > 1) {
        // Groups' tiles through LDS (the rings are free once every wave has
        // passed this barrier), summed in group order by group 0.
        __syncthreads();
        float *red = reinterpret_cast<float *>(lds);
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
                if (row < M && col < N) {
                    if constexpr (SPLIT)
                        partial[slice * pitch + (uint64_t)row * N + col] = acc[sm][sn][r];
                    else
                        out[(uint64_t)row * N + col] = f32_to_bf16_rne(acc[sm][sn][r]);
                }
            }
        }
}

// The K slices of a split GEMM: out = bf16_rne(((p_0 + p_1) + p_2) + ...), the
// FP32 slice tiles added in slice order (4 consecutive outputs per lane; each
// slice holds `pitch` floats, m * n rounded up to a multiple of 4).
__global__ __launch_bounds__(256) void split_reduce_kernel(const float *__restrict__ partial,
                                                           uint16_t *__restrict__ out, uint64_t mn, uint64_t pitch,
                                                           uint32_t slices) {
    const uint64_t i = ((uint64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= mn) return;
    typedef float v4f __attribute__((ext_vector_type(4)));
    v4f acc = *reinterpret_cast<const v4f *>(partial + i);
    for (uint32_t sl = 1; sl < slices; ++sl) {
        const v4f v = *reinterpret_cast<const v4f *>(partial + sl * pitch + i);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    const float r[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (i + j < mn) out[i + j] = f32_to_bf16_rne(r[j]);
}


// Explicit instantiations of every launched shape: clang otherwise left the
// host launch symbols of some instantiations undefined.
#define BSR_GEMM_INST(BM, BN, WM, WN, WGC, KG, RING, SPLIT)                                                 \
    template __global__ void gemm_kernel<BM, BN, WM, WN, WGC, KG, RING, SPLIT>(                             \
        const int8_t *__restrict__, const int8_t *__restrict__, const float *__restrict__,                  \
        const float *__restrict__, uint16_t *__restrict__, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, \
        uint32_t, uint32_t, float *__restrict__, uint64_t, uint32_t);
BSR_GEMM_INST(256, 128, 64, 64, 1, 1, 2, false)
BSR_GEMM_INST(128, 128, 64, 64, 2, 1, 2, false)
BSR_GEMM_INST(32, 32, 32, 32, 1, 8, 2, false)
BSR_GEMM_INST(32, 32, 32, 32, 2, 4, 2, false)
BSR_GEMM_INST(64, 64, 32, 32, 1, 2, 3, false)
BSR_GEMM_INST(64, 64, 32, 32, 2, 1, 4, false)
BSR_GEMM_INST(64, 64, 32, 32, 2, 1, 4, true)
#undef BSR_GEMM_INST

}  // namespace gemm_kernels

namespace {

using gemm_kernels::gemm_kernel;
using gemm_kernels::split_reduce_kernel;

template <int BM, int BN, int WM, int WN, int WG_PER_CU, int KG = 1, int RING = 2>
hipError_t launch_tiles(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale,
                        const float *w_scale, uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                        uint32_t a_ld, uint32_t a_shift, hipStream_t s) {
    const uint32_t tiles_m = (uint32_t)div_up(m, BM);
    const uint32_t tiles_n = (uint32_t)div_up(n, BN);
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, WG_PER_CU, KG, RING, false>), dim3(tiles_m * tiles_n),
                       dim3(Geo<BM, BN, WM, WN>::kThreads * KG), 0, s, a_i8, w_i8, a_scale, w_scale, out, m, n, k,
                       a_ld, a_shift, tiles_m, tiles_n, nullptr, 0, 0);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale, uint32_t a_ld,
                       uint32_t a_shift, const float *w_scale, uint16_t *out, uint32_t m, uint32_t n,
                       uint32_t k, bool split_k, hipStream_t s) {
    // Grids of at least two 128x128 tiles per CU: one 8-wave 256x128
    // workgroup per CU (LDS 120 KB, 8 waves of about 214 VGPRs) where its
    // 256-row tiling pads M no more than 128-row tiles and K < 2^24, else two
    // 4-wave 128x128 workgroups per CU (LDS 2 x 80 KB, 216 VGPRs), whose
    // barriers fall at different times.  Smaller grids -- every m <= 128,
    // and e.g. m = 512 at n = 4096 -- take 64x64 tiles of four 32x32 waves:
    // four times the workgroups, 1.1-2.5x faster from m = 17 to 1024 on the
    // decode and attention widths; their 4-deep ring (three stages in flight)
    // and 8-block scale stages fit 76 KB of LDS, two workgroups per CU.  Per
    // output the blocks are accumulated in the same order in both, so the bits
    // do not depend on the shape chosen.
    if (gemm_tall_tiles(m, n, k))
        return launch_tiles<kGemmTallBM, kGemmBN, 64, 64, 1>(a_i8, w_i8, a_scale, w_scale, out, m, n, k, a_ld,
                                                             a_shift, s);
    if (gemm_big_tiles(m, n))
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
    return launch_tiles<kGemmSmallTile, kGemmSmallTile, 32, 32, 2, 1, 4>(a_i8, w_i8, a_scale, w_scale, out, m, n,
                                                                         k, a_ld, a_shift, s);
}

hipError_t launch_gemm_split(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale,
                             const float *w_scale, uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                             float *partial, const SplitPlan &plan, hipStream_t s) {
    // 64 x 64 tiles of four 32 x 32 waves, two workgroups per CU, each with a
    // 4-deep ring (three stages in flight: a slice streams its A and W rows
    // from HBM with ~54 KB per workgroup outstanding)
    const uint32_t tiles_m = (uint32_t)div_up(m, kSplitTile), tiles_n = (uint32_t)div_up(n, kSplitTile);
    const uint32_t grid = tiles_m * tiles_n * plan.slices;
    hipLaunchKernelGGL((gemm_kernel<kSplitTile, kSplitTile, 32, 32, 2, 1, 4, true>), dim3(grid),
                       dim3(Geo<kSplitTile, kSplitTile, 32, 32>::kThreads), 0, s, a_i8, w_i8, a_scale, w_scale,
                       out, m, n, k, k / 32, 0u, tiles_m, tiles_n, partial, plan.pitch, plan.stages);
    if (hipError_t e = hipGetLastError()) return e;
    const uint64_t mn = (uint64_t)m * n;
    hipLaunchKernelGGL(split_reduce_kernel, dim3((uint32_t)div_up(mn, 4 * 256)), dim3(256), 0, s, partial, out, mn,
                       plan.pitch, plan.slices);
    return hipGetLastError();
}

}  // namespace bsr
