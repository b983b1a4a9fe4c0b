// api.hip -- the C ABI of libbsr: argument validation, the GEMV/GEMM dispatch
// and the launches.  Every check happens before the first launch; an error
// launches nothing.  The only state is a per-device cache of the gfx950 check.
#include <atomic>
#include <cmath>
#include <cstring>

#include "bsr.h"
#include "bsr_internal.h"

namespace {

constexpr int kMaxDevices = 256;
std::atomic<int> g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return BSR_EDEVICE;
    if (dev >= kMaxDevices) return BSR_EDEVICE;
    int state = g_device_ok[dev].load(std::memory_order_relaxed);
    if (state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return BSR_EDEVICE;
        state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_device_ok[dev].store(state, std::memory_order_relaxed);
    }
    return state == 1 ? BSR_OK : BSR_EDEVICE;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Scratch of the allocation-free GEMM entry point: the K-split workspace of
// int8_gemm_blockscaled_noalloc, one copy per GPU, held until the process
// ends.  Its size is the largest workspace a split plan asks for.  Host code
// never uses the symbol itself (that is a host-side stand-in, not a device
// address): scratch_ptr() looks up, once per device, the address of that
// device's copy.
static __device__ __align__(256) float scratch[bsr::kSplitMaxBytes / sizeof(float)];
std::atomic<void *> g_scratch[kMaxDevices];

// The current device's scratch address (nullptr if the lookup failed).
void *scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch[dev].store(p, std::memory_order_release);  // the same value if two threads race here
    }
    return p;
}

bool k_ok(uint32_t k) { return k != 0 && k % 32 == 0; }

// Rows the GEMV takes: one 16-row tile at any K, up to four when K suits the
// streamed kernel.
bool gemv_rows_ok(uint32_t m, uint32_t k) {
    return m <= (uint32_t)bsr::kGemvMaxRows ||
           (m <= (uint32_t)bsr::kGemvStreamMaxRows && k % bsr::kGemvStreamKAlign == 0);
}

// Grids stay below 2^31 workgroups.
constexpr uint64_t kMaxGrid = (1ull << 31) - 1;

int launched(hipError_t e) { return e == hipSuccess ? BSR_OK : BSR_ELAUNCH; }

int gemm_args_check(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale,
                    const float *w_scale, const uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                    int path) {
    if (!k_ok(k)) return BSR_EINVAL;
    if (path != BSR_PATH_AUTO && path != BSR_PATH_GEMM && path != BSR_PATH_GEMV && path != BSR_PATH_INVARIANT)
        return BSR_EINVAL;
    if (m == 0 || n == 0) return BSR_OK;
    if (path == BSR_PATH_GEMV && !gemv_rows_ok(m, k)) return BSR_EINVAL;
    if ((path == BSR_PATH_GEMM || m > (uint32_t)bsr::kGemvMaxRows) && k >= bsr::kGemmMaxK) return BSR_EINVAL;
    if (!a_i8 || !w_i8 || !a_scale || !w_scale || !out) return BSR_ENULL;
    if (!aligned(a_i8, 16) || !aligned(w_i8, 16) || !aligned(a_scale, 4) || !aligned(w_scale, 4) ||
        !aligned(out, 2))
        return BSR_EALIGN;
    const uint64_t tiles = bsr::div_up(m, bsr::kGemmSmallTile) * bsr::div_up(n, bsr::kGemmSmallTile);
    if (tiles > kMaxGrid) return BSR_EINVAL;
    return BSR_OK;
}

int gemm_launch(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale, uint32_t a_ld,
                uint32_t a_shift, const float *w_scale, uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                void *stream, int path) {
    if (int st = check_device()) return st;
    const bool small = m <= (uint32_t)bsr::kGemvMaxRows;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (path == BSR_PATH_INVARIANT && small)
        return launched(bsr::launch_gemv_chain(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s));
    // The automatic path also takes the streamed GEMV for a few tiles of rows
    // when the grid is narrow (measured faster than the GEMM's small-grid
    // tiles up to 48 rows at n <= 4096; slower at n = 14336).
    const bool narrow = bsr::div_up(n, bsr::kGemvCols) <= (uint64_t)bsr::kGemmCus;
    const bool stream_rows = m <= (uint32_t)bsr::kGemvStreamAutoRows && k % bsr::kGemvStreamKAlign == 0 && narrow;
    const bool gemv = path == BSR_PATH_GEMV || (path == BSR_PATH_AUTO && (small || stream_rows));
    if (gemv) return launched(bsr::launch_gemv(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, s));
    return launched(bsr::launch_gemm(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k,
                                     path != BSR_PATH_INVARIANT, s));
}

}  // namespace

extern "C" {

int requant_w_nvfp4_int8(const uint8_t *w_packed, const uint8_t *w_e4m3, float scale2,
                         int8_t *w_i8, float *w_scale, uint32_t n, uint32_t k, void *stream) {
    if (!k_ok(k) || !std::isfinite(scale2)) return BSR_EINVAL;
    if (n == 0) return BSR_OK;
    if (!w_packed || !w_e4m3 || !w_i8 || !w_scale) return BSR_ENULL;
    if (!aligned(w_packed, 16) || !aligned(w_e4m3, 2) || !aligned(w_i8, 16) || !aligned(w_scale, 4))
        return BSR_EALIGN;
    const uint64_t nblocks = (uint64_t)n * (k / 32);
    if (bsr::div_up(nblocks, bsr::kRqwThreads) > kMaxGrid) return BSR_EINVAL;
    if (int st = check_device()) return st;
    return launched(bsr::launch_requant_w(w_packed, w_e4m3, scale2, w_i8, w_scale, nblocks,
                                          static_cast<hipStream_t>(stream)));
}

int requant_a_int8(const uint16_t *a_bf16, int8_t *a_i8, float *a_scale, uint32_t m, uint32_t k,
                   void *stream) {
    if (!k_ok(k)) return BSR_EINVAL;
    if (m == 0) return BSR_OK;
    if (!a_bf16 || !a_i8 || !a_scale) return BSR_ENULL;
    if (!aligned(a_bf16, 16) || !aligned(a_i8, 16) || !aligned(a_scale, 4)) return BSR_EALIGN;
    const uint64_t nblocks = (uint64_t)m * (k / 32);
    if (bsr::div_up(nblocks * bsr::kRqaLanesPerBlock, bsr::kRqaThreads) > kMaxGrid) return BSR_EINVAL;
    if (int st = check_device()) return st;
    return launched(bsr::launch_requant_a(a_bf16, a_i8, a_scale, nblocks, static_cast<hipStream_t>(stream)));
}

int silu_mul_requant_int8(const uint16_t *gate, const uint16_t *up, uint32_t ld, int8_t *a_i8,
                          float *a_scale, uint32_t m, uint32_t k, void *stream) {
    if (!k_ok(k) || ld < k || ld % 8 != 0) return BSR_EINVAL;
    if (m == 0) return BSR_OK;
    if (!gate || !up || !a_i8 || !a_scale) return BSR_ENULL;
    if (!aligned(gate, 16) || !aligned(up, 16) || !aligned(a_i8, 16) || !aligned(a_scale, 4))
        return BSR_EALIGN;
    const uint64_t nchunks = (uint64_t)m * (k / 8);
    if (bsr::div_up(nchunks, bsr::kRqaThreads) > kMaxGrid) return BSR_EINVAL;
    if (int st = check_device()) return st;
    return launched(bsr::launch_silu_requant(gate, up, ld, a_i8, a_scale, m, k, static_cast<hipStream_t>(stream)));
}

int w4a16_gemv(const uint16_t *x_bf16, const uint8_t *w_packed, const uint8_t *w_e4m3, float scale2,
               uint16_t *out, uint32_t m, uint32_t n, uint32_t k, void *stream) {
    if (!k_ok(k) || !std::isfinite(scale2) || m > (uint32_t)bsr::kGemvMaxRows) return BSR_EINVAL;
    if (m == 0 || n == 0) return BSR_OK;
    if (!x_bf16 || !w_packed || !w_e4m3 || !out) return BSR_ENULL;
    if (!aligned(x_bf16, 16) || !aligned(w_packed, 16) || !aligned(out, 2)) return BSR_EALIGN;
    if (k % 256 == 0 ? !aligned(w_e4m3, 16) : !aligned(w_e4m3, 2)) return BSR_EALIGN;
    if (bsr::div_up(n, bsr::kGemvCols) > kMaxGrid) return BSR_EINVAL;
    if (int st = check_device()) return st;
    return launched(bsr::launch_w4a16(x_bf16, w_packed, w_e4m3, scale2, out, m, n, k, static_cast<hipStream_t>(stream)));
}

int int8_gemm_blockscaled_ex(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale,
                             const float *w_scale, uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                             void *stream, int path) {
    if (int st = gemm_args_check(a_i8, w_i8, a_scale, w_scale, out, m, n, k, path)) return st;
    if (m == 0 || n == 0) return BSR_OK;
    return gemm_launch(a_i8, w_i8, a_scale, k / 32, 0, w_scale, out, m, n, k, stream, path);
}

int int8_gemm_blockscaled(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale,
                          const float *w_scale, uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                          void *stream) {
    return int8_gemm_blockscaled_ex(a_i8, w_i8, a_scale, w_scale, out, m, n, k, stream, BSR_PATH_AUTO);
}

uint64_t int8_gemm_blockscaled_ws_bytes(uint32_t m, uint32_t n, uint32_t k) {
    return bsr::gemm_split_plan(m, n, k).bytes;
}

int int8_gemm_blockscaled_ws(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale,
                             const float *w_scale, uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                             void *workspace, uint64_t workspace_bytes, void *stream) {
    if (int st = gemm_args_check(a_i8, w_i8, a_scale, w_scale, out, m, n, k, BSR_PATH_AUTO)) return st;
    if (m == 0 || n == 0) return BSR_OK;
    const bsr::SplitPlan plan = bsr::gemm_split_plan(m, n, k);
    if (plan.slices == 0)
        return gemm_launch(a_i8, w_i8, a_scale, k / 32, 0, w_scale, out, m, n, k, stream, BSR_PATH_AUTO);
    if (!workspace) return BSR_ENULL;
    if (!aligned(workspace, 16)) return BSR_EALIGN;
    if (workspace_bytes < plan.bytes) return BSR_EINVAL;
    if (int st = check_device()) return st;
    return launched(bsr::launch_gemm_split(a_i8, w_i8, a_scale, w_scale, out, m, n, k,
                                           static_cast<float *>(workspace), plan, static_cast<hipStream_t>(stream)));
}

int int8_gemm_blockscaled_noalloc(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale,
                                  const float *w_scale, uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                                  void *stream) {
    if (int st = gemm_args_check(a_i8, w_i8, a_scale, w_scale, out, m, n, k, BSR_PATH_AUTO)) return st;
    if (m == 0 || n == 0) return BSR_OK;
    const bsr::SplitPlan plan = bsr::gemm_split_plan(m, n, k);
    if (plan.slices == 0)
        return gemm_launch(a_i8, w_i8, a_scale, k / 32, 0, w_scale, out, m, n, k, stream, BSR_PATH_AUTO);
    if (plan.bytes > sizeof(scratch)) return BSR_EINVAL;  // beyond the scratch (no plan asks for more)
    if (int st = check_device()) return st;
    void *ws = scratch_ptr();
    if (ws == nullptr) return BSR_EDEVICE;
    return launched(bsr::launch_gemm_split(a_i8, w_i8, a_scale, w_scale, out, m, n, k, static_cast<float *>(ws),
                                           plan, static_cast<hipStream_t>(stream)));
}

int int8_gemm_blockscaled_agroup(const int8_t *a_i8, const int8_t *w_i8, const float *a_scale,
                                 uint32_t a_group, const float *w_scale, uint16_t *out, uint32_t m,
                                 uint32_t n, uint32_t k, void *stream, int path) {
    if (a_group != 0 && a_group != 32 && a_group != 128) return BSR_EINVAL;
    if (a_group == 128 && k % 128 != 0) return BSR_EINVAL;
    if (int st = gemm_args_check(a_i8, w_i8, a_scale, w_scale, out, m, n, k, path)) return st;
    if (m == 0 || n == 0) return BSR_OK;
    const uint32_t a_ld = a_group == 0 ? 1 : k / a_group;
    const uint32_t a_shift = a_group == 0 ? 31 : (a_group == 128 ? 2 : 0);
    return gemm_launch(a_i8, w_i8, a_scale, a_ld, a_shift, w_scale, out, m, n, k, stream, path);
}

int quantize_act(const uint16_t *a_bf16, uint8_t *q, float *scale, uint32_t m, uint32_t k,
                 uint32_t group, int format, void *stream) {
    if (!k_ok(k) || (group != 0 && group != 32 && group != 128)) return BSR_EINVAL;
    if (group == 128 && k % 128 != 0) return BSR_EINVAL;
    if (format != BSR_FMT_INT8 && format != BSR_FMT_E4M3) return BSR_EINVAL;
    if (m == 0) return BSR_OK;
    if (!a_bf16 || !q || !scale) return BSR_ENULL;
    if (!aligned(a_bf16, 16) || !aligned(q, 8) || !aligned(scale, 4)) return BSR_EALIGN;
    const uint64_t nchunks = (uint64_t)m * (k / 8);
    if (m > kMaxGrid || bsr::div_up(nchunks, bsr::kRqaThreads) > kMaxGrid) return BSR_EINVAL;
    if (int st = check_device()) return st;
    return launched(bsr::launch_quant_act(a_bf16, q, scale, m, k, group, format == BSR_FMT_E4M3,
                                          static_cast<hipStream_t>(stream)));
}

const char *bsr_status_string(int status) {
    switch (status) {
    case BSR_OK: return "BSR_OK";
    case BSR_EINVAL: return "BSR_EINVAL: invalid size or argument";
    case BSR_ENULL: return "BSR_ENULL: null pointer";
    case BSR_EALIGN: return "BSR_EALIGN: misaligned pointer";
    case BSR_EDEVICE: return "BSR_EDEVICE: no current gfx950 device";
    case BSR_ELAUNCH: return "BSR_ELAUNCH: kernel launch failed";
    default: return "unknown bsr status";
    }
}

}  // extern "C"
