// Host-only check of the K-split plan (bsr_geometry.h, the code the launcher
// runs): slices are non-empty and cover K exactly, the grid stays within two
// workgroups per CU, and the workspace within its stated maximum.
#include <cstdio>

#include "bsr_geometry.h"

int main() {
    using namespace bsr;
    const uint32_t ms[] = {1, 16, 17, 31, 32, 33, 48, 63, 64, 65, 100, 128, 200, 256, 512, 1024, 2048};
    const uint32_t ns[] = {1, 7, 64, 100, 1024, 4096, 4097, 8192, 14336, 28672};
    long cases = 0, split = 0;
    for (uint32_t m : ms)
        for (uint32_t n : ns)
            for (uint32_t k = 32; k <= 65536; k += (k < 4096 ? 32 : 1024)) {
                const SplitPlan p = gemm_split_plan(m, n, k);
                ++cases;
                if (p.slices == 0) continue;
                ++split;
                const uint32_t stages = (uint32_t)div_up(k / 32, kGemmStageBlocks);
                const uint64_t tiles = div_up(m, kSplitTile) * div_up(n, kSplitTile);
                const bool ok = m >= kSplitMinRows && stages >= kSplitMinKStages && p.slices >= 2 && p.slices <= kSplitMaxSlices &&
                                p.stages >= kSplitMinStages && (uint64_t)(p.slices - 1) * p.stages < stages &&
                                (uint64_t)p.slices * p.stages >= stages && tiles * p.slices <= kSplitMaxWorkgroups &&
                                p.pitch >= (uint64_t)m * n && p.pitch % 4 == 0 &&
                                p.bytes == (uint64_t)p.slices * p.pitch * 4 && p.bytes <= kSplitMaxBytes;
                if (!ok) {
                    std::printf("FAIL m=%u n=%u k=%u: slices=%u stages=%u pitch=%llu bytes=%llu\n", m, n, k, p.slices,
                                p.stages, (unsigned long long)p.pitch, (unsigned long long)p.bytes);
                    return 1;
                }
            }
    // the workloads the split is for: narrow N, long K, 17..64 rows
    const SplitPlan d = gemm_split_plan(64, 4096, 14336);
    if (d.slices < 4) {
        std::printf("FAIL: 64 x 4096 x 14336 gets %u slices\n", d.slices);
        return 1;
    }
    std::printf("ok %ld %ld\n", cases, split);
    return 0;
}
