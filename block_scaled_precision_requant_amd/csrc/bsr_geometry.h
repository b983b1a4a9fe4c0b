// bsr_geometry.h -- launch geometry of every kernel, and the host-side
// launch plans that derive grids and LDS sizes from it.  Plain C++ with no HIP
// header, so host-only tests can compile the same plan code the launchers run.
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define BSR_HD __host__ __device__
#else
#define BSR_HD
#endif

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
constexpr int kRqwUnroll = 1;        // blocks per lane (one: stores staged through LDS per wave)
constexpr int kSiluMinPasses = 8;    // fewest passes per workgroup for the SiLU table kernel
constexpr int kSiluThreads = 512;    // lanes per workgroup of the SiLU table kernel

// ---- GEMM (m > 16) --------------------------------------------------------
// A workgroup computes a BM x BN output tile; each wave owns a WM x WN piece
// made of 32 x 32 MFMA tiles.  The K loop stages kGemmStageBlocks 32-wide
// blocks of A, W and their scales per LDS buffer, in a ring of 2 (or 3)
// buffers.  Workgroups are ordered so that each XCD runs a compact
// kGemmGroupM-tall group of output tiles.  Shapes: 256 x 128 with eight
// 64 x 64 waves, one workgroup per CU, and 128 x 128 with four 64 x 64 waves,
// two per CU, for grids that give every CU two 128 x 128 tiles; 64 x 64 with
// four 32 x 32 waves, two per CU, for smaller grids.  Grids with at most one
// or two tiles per CU split K inside the workgroup over groups of waves
// (64 x 64 or 32 x 32 tiles).
constexpr int kGemmBM = 128;
constexpr int kGemmBN = 128;
constexpr int kGemmSmallTile = 64;
constexpr int kGemmTinyTile = 32;
constexpr int kGemmStageBlocks = 4;
constexpr int kGemmStageBytes = 32 * kGemmStageBlocks;    // 128 bytes of K per row: whole cache lines
constexpr int kGemmGroupM = 8;
constexpr int kXcds = 8;
constexpr int kGemmCus = 256;                             // compute units of an MI355X
// The GEMM stages operands with 32-bit buffer offsets from a tile's first row:
// the rows of a tile must span less than 4 GiB, so k < 2^25 for 128 rows.
constexpr uint32_t kGemmMaxK = 1u << 25;

// The tall tile, 256 x 128: per staged byte it computes a third more output
// than the 128 x 128 tile (a copy's cost follows the cache lines it touches),
// at the price of one workgroup per CU whose eight waves meet at every
// barrier; measured 0.9-1.9 % faster at 2048x4096x4096, 4096x28672x4096 and
// 8192x28672x8192, bit-identical.  Its XCD groups are 4 tile rows tall, so
// an XCD's 32 concurrent tiles span 1024 A rows and 1024 W rows, and its 256
// rows need k < 2^24.
constexpr int kGemmTallBM = 256;
constexpr int kGemmTallGroupM = 4;
constexpr uint32_t kGemmTallMaxK = 1u << 24;


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

// Grids that give every CU two 128 x 128 tiles (and m > 128) run the tall
// tile when its 256-row tiling pads M no more than the 128-row one (m % 256
// is 0 or above 128) and K allows it; else the 128 x 128 tile.
inline bool gemm_big_tiles(uint32_t m, uint32_t n) {
    return m > (uint32_t)kGemmBM && div_up(m, kGemmBM) * div_up(n, kGemmBN) >= 2 * (uint64_t)kGemmCus;
}
inline bool gemm_tall_tiles(uint32_t m, uint32_t n, uint32_t k) {
    return gemm_big_tiles(m, n) && div_up(m, kGemmTallBM) * 2 == div_up(m, kGemmBM) && k < kGemmTallMaxK;
}

constexpr uint32_t kLdsBytes = 160u * 1024u;  // LDS of one CU (gfx950)

// ---- GEMM with K split across workgroups (caller workspace) ---------------
// For grids of fewer 64 x 64 tiles than CUs, each tile's K range is cut into
// `slices` contiguous ranges of whole stages, one workgroup per (tile, slice);
// every slice writes its FP32 tile to the workspace ([slice][m][n], each
// slice `pitch` floats), and a second kernel adds the slices in slice order
// and rounds to BF16.  slices * tiles <= kSplitMaxWorkgroups, so the
// workspace never exceeds kSplitMaxWorkgroups * 64 * 64 * 4 bytes (8 MiB).
constexpr uint32_t kSplitTile = 64;
constexpr uint32_t kSplitMaxWorkgroups = 2 * kGemmCus;  // two workgroups per CU
constexpr uint32_t kSplitMaxSlices = 16;
// K stages per slice, at least: slices of 4 stages spent more on each
// slice's pipeline start than they gained in workgroups (n = 2048,
// k = 8192, m = 40 / 48 / 64: 16.3 / 17.0 / 18.1 us with 16 slices of 4
// stages, 13.1 / 13.3 / 13.9 with 8 of 8, against 15.3 / 15.8 / 19.9 without
// workspace)
constexpr uint32_t kSplitMinStages = 8;
// Where the split measured faster than the paths without workspace: more
// rows than the streamed GEMV's two 16-row tiles, and K long enough (64
// stages, K >= 8192) to hide each slice's pipeline start and the second
// launch (n = 4096, k = 14336: m = 40 / 48 / 64 / 128 in 22.4 / 23.4 / 24.6 /
// 34.5 us against 25.0 / 26.5 / 33.7 / 54.4; m = 17-32 at n = 4096: level to
// 2.4 us slower; at k = 4096, n = 4096, m <= 64: 1.7-2.3 us slower, n = 14336,
// m = 40-64: 1-2 % faster).
constexpr uint32_t kSplitMinRows = 33;
constexpr uint32_t kSplitMinKStages = 64;
constexpr uint64_t kSplitMaxBytes = (uint64_t)kSplitMaxWorkgroups * kSplitTile * kSplitTile * 4;

struct SplitPlan {
    uint32_t slices;       // 0: no split (the ordinary paths run)
    uint32_t stages;       // K stages (of kGemmStageBlocks blocks) per slice
    uint64_t pitch;        // floats per slice in the workspace (m * n rounded up to 4)
    uint64_t bytes;        // workspace bytes the split needs
};

inline SplitPlan gemm_split_plan(uint32_t m, uint32_t n, uint32_t k) {
    SplitPlan p{0, 0, 0, 0};
    if (m < kSplitMinRows || k == 0 || k % 32 != 0) return p;
    const uint64_t tiles = div_up(m, kSplitTile) * div_up(n, kSplitTile);
    const uint32_t stages = (uint32_t)div_up(k / 32, kGemmStageBlocks);
    if (tiles >= (uint64_t)kGemmCus || stages < kSplitMinKStages) return p;
    uint64_t s = kSplitMaxWorkgroups / tiles;
    s = s < kSplitMaxSlices ? s : kSplitMaxSlices;
    s = s < stages / kSplitMinStages ? s : stages / kSplitMinStages;
    if (s < 2) return p;
    p.stages = (uint32_t)div_up(stages, s);
    p.slices = (uint32_t)div_up(stages, p.stages);  // every slice non-empty
    if (p.slices < 2) return SplitPlan{0, 0, 0, 0};
    p.pitch = ((uint64_t)m * n + 3) & ~(uint64_t)3;
    p.bytes = (uint64_t)p.slices * p.pitch * 4;
    return p;
}

// ---- W4A16 register-decode kernel (K % 256 != 0) --------------------------
constexpr int kW4StepK = 128;  // K per super-step

// Per-wave LDS region: m activation rows of pitch bytes (one pass of
// super-steps plus 16 bytes, so the 16 lanes of a quarter reading 16 rows at
// one offset spread over the banks).
BSR_HD inline uint32_t w4_pitch(uint32_t pass_steps) { return pass_steps * kW4StepK * 2 + 16; }

// Launch plan of the register-decode W4A16 kernel.
//   ct:    16-column tiles per workgroup (two from m = 4 on, where the
//          activation bytes a workgroup stages, 2 m per K element, approach
//          the weight bytes of one tile, 9 per K element, if that still leaves
//          a workgroup for every CU);
//   waves: as for the int8 GEMV (~24 waves per CU over the launch), at most
//          16, at least ct (with two tiles one wave reduces each tile);
//   spw:   super-steps per wave;
//   pass:  super-steps per staging pass: the whole per-wave range when its
//          activation staging fits in LDS, else the largest that fits, then
//          rounded DOWN to an instantiated length (1, 2, 4, 6 or 8; 6 at most
//          with two tiles, which keeps 128 VGPRs) so the LDS size only shrinks;
//   lds:   dynamic LDS bytes (staging, or the cross-wave reduction if larger);
//          above kLdsBytes the launcher reports an error instead of launching.
struct W4Plan {
    uint32_t ct, tiles, waves, spw, pass, lds;
};

inline W4Plan w4a16_reg_plan(uint32_t m, uint32_t n, uint32_t k) {
    W4Plan p;
    p.ct = m >= 4 && div_up(n, 2 * kGemvCols) >= (uint64_t)kGemmCus ? 2 : 1;
    p.tiles = (uint32_t)div_up(n, kGemvCols * p.ct);
    const uint32_t nsteps = (uint32_t)div_up(k, kW4StepK);
    uint32_t waves = (uint32_t)div_up(6144, p.tiles);
    waves = waves < (uint32_t)kGemvMaxWaves ? waves : (uint32_t)kGemvMaxWaves;
    waves = waves > p.ct ? waves : p.ct;
    const uint32_t cap = nsteps > p.ct ? nsteps : p.ct;
    waves = waves < cap ? waves : cap;
    p.spw = (uint32_t)div_up(nsteps, waves);
    p.waves = (uint32_t)div_up(nsteps, p.spw);
    p.waves = p.waves > p.ct ? p.waves : p.ct;
    const uint32_t red = p.ct * kGemvMaxWaves * 64 * 4 * 4;
    uint32_t pass = p.spw < (p.ct == 2 ? 6u : (uint32_t)kW4PassSteps) ? p.spw : (p.ct == 2 ? 6u : (uint32_t)kW4PassSteps);
    while (pass > 1 && (uint64_t)p.waves * m * w4_pitch(pass) > kLdsBytes) --pass;
    p.pass = pass <= 2 ? pass : pass & ~1u;
    const uint64_t stage = (uint64_t)p.waves * m * w4_pitch(p.pass);
    p.lds = (uint32_t)(stage > red ? stage : red);
    return p;
}

}  // namespace bsr
