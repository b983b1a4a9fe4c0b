// read_probe.hip -- a plain streaming-read kernel: the achievable-bandwidth
// context that bench.py reports beside the method's kernels.  It is a
// measurement aid, not a step of the method, and lives in its own library
// (libbsr_read.so) so that libbsr.so exports only the method's entry points.
//
// Each lane reads 16-byte words in a grid-stride loop and folds them with XOR
// (so no load can be dropped); each workgroup stores one word.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kReadThreads = 256;

__global__ __launch_bounds__(kReadThreads) void read_kernel(const uint4 *__restrict__ p, uint64_t n16,
                                                            uint32_t *__restrict__ out) {
    uint32_t acc = 0;
    const uint64_t stride = (uint64_t)gridDim.x * kReadThreads;
    for (uint64_t i = (uint64_t)blockIdx.x * kReadThreads + threadIdx.x; i < n16; i += stride) {
        const uint4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __shared__ uint32_t red[kReadThreads];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int j = 0; j < kReadThreads; ++j) t ^= red[j];
        out[blockIdx.x] = t;
    }
}

}  // namespace

// Read `bytes` (a multiple of 16, 16-byte aligned device memory) with `grid`
// workgroups of 256 lanes; `out` holds `grid` words.  Returns 0, or 1 if the
// arguments are invalid or the launch failed.
extern "C" __attribute__((visibility("default"))) int read_probe(const void *p, uint64_t bytes, uint32_t *out,
                                                                 uint32_t grid, void *stream) {
    if (!p || !out || grid == 0 || bytes % 16 || reinterpret_cast<uintptr_t>(p) % 16) return 1;
    hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(kReadThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4 *>(p), bytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}
