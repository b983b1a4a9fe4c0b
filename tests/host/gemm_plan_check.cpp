// Host-only check of the GEMM's big-tile choice (bsr_geometry.h, the code the
// launcher runs): the 256 x 128 tile is taken only for grids of at least two
// 128 x 128 tiles per CU, only where its 256-row tiling pads M no more than
// the 128-row one, and only for K whose 256 rows stay within 32-bit offsets;
// the prefill workloads take it.
#include <cstdio>

#include "bsr_geometry.h"

int main() {
    using namespace bsr;
    long cases = 0, tall = 0;
    const uint32_t ns[] = {1, 128, 4096, 4097, 14336, 28672, 65536};
    const uint32_t ks[] = {32, 4096, 8192, 14336, (1u << 24) - 32, 1u << 24, (1u << 25) - 32};
    for (uint32_t m = 1; m <= 20000; m += (m < 1100 ? 1 : 37))
        for (uint32_t n : ns)
            for (uint32_t k : ks) {
                ++cases;
                if (!gemm_tall_tiles(m, n, k)) continue;
                ++tall;
                const bool ok = gemm_big_tiles(m, n) && div_up(m, kGemmTallBM) * kGemmTallBM == div_up(m, kGemmBM) * kGemmBM &&
                                (uint64_t)kGemmTallBM * k < (1ull << 32);
                if (!ok) {
                    std::printf("FAIL m=%u n=%u k=%u\n", m, n, k);
                    return 1;
                }
            }
    const uint32_t work[][3] = {{2048, 4096, 4096}, {4096, 28672, 4096}, {4096, 4096, 14336}, {8192, 28672, 8192}};
    for (const auto &w : work)
        if (!gemm_tall_tiles(w[0], w[1], w[2])) {
            std::printf("FAIL: %u x %u x %u does not take the tall tile\n", w[0], w[1], w[2]);
            return 1;
        }
    if (gemm_tall_tiles(1100, 7400, 1056) || !gemm_big_tiles(1100, 7400) || !gemm_tall_tiles(1200, 7400, 1056)) {
        std::printf("FAIL: the ragged test shapes\n");
        return 1;
    }
    std::printf("ok %ld %ld\n", cases, tall);
    return 0;
}
