// Host-only check of the register-decode W4A16 launch plan (bsr_geometry.h,
// the code the launcher runs): for every m <= 16 and every K that is a
// multiple of 32 but not of 256 up to 65536, at the widths of the decode
// workloads and a few ragged ones, the plan must fit the CU's LDS and name an
// instantiated pass length that the kernel's loop can use.
#include <cstdio>

#include "bsr_geometry.h"

int main() {
    using namespace bsr;
    const uint32_t widths[] = {1, 15, 16, 17, 333, 4096, 4112, 8192, 14336, 28672};
    long cases = 0;
    for (uint32_t m = 1; m <= (uint32_t)kGemvMaxRows; ++m)
        for (uint32_t n : widths)
            for (uint32_t k = 32; k <= 65536; k += 32) {
                if (k % 256 == 0) continue;
                const W4Plan p = w4a16_reg_plan(m, n, k);
                const uint32_t nsteps = (uint32_t)div_up(k, kW4StepK);
                const bool pass_ok = p.ct == 2 ? (p.pass == 1 || p.pass == 2 || p.pass == 4 || p.pass == 6)
                                               : (p.pass == 1 || p.pass == 2 || p.pass == 4 || p.pass == 6 ||
                                                  p.pass == 8);
                const bool ok = p.lds <= kLdsBytes && pass_ok && p.pass <= p.spw &&
                                (uint64_t)p.waves * p.spw >= nsteps && p.waves >= p.ct &&
                                p.waves <= (uint32_t)kGemvMaxWaves &&
                                (uint64_t)p.tiles * kGemvCols * p.ct >= n &&
                                (uint64_t)p.waves * m * w4_pitch(p.pass) <= p.lds;
                ++cases;
                if (!ok) {
                    std::printf("FAIL m=%u n=%u k=%u: ct=%u tiles=%u waves=%u spw=%u pass=%u lds=%u\n", m, n, k,
                                p.ct, p.tiles, p.waves, p.spw, p.pass, p.lds);
                    return 1;
                }
            }
    std::printf("ok %ld\n", cases);
    return 0;
}
