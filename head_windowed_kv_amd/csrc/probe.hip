// HBM reference kernels, built into libhwkv_probe.so (not part of the hwkv
// C ABI).  The benchmark uses them for two figures:
//   - probe_read: a plain streaming read of a large buffer, the practical
//     read-bandwidth ceiling that the decode split kernel is compared with;
//   - probe_copy: a copy of known size, whose FETCH_SIZE / WRITE_SIZE
//     counter readings calibrate the counters of the decode kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void probe_read_kernel(const u32x4* __restrict__ src,
                                                              uint64_t n16, uint32_t* out) {
    uint32_t acc = 0;
    const uint64_t stride = (uint64_t)gridDim.x * kThreads * kUnroll;
    for (uint64_t i = (uint64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; i < n16;
         i += stride) {
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const uint64_t j = i + (uint64_t)u * kThreads;
            if (j < n16) {
                const u32x4 x = __builtin_nontemporal_load(src + j);
                acc ^= x.x ^ x.y ^ x.z ^ x.w;
            }
        }
    }
    if (acc == 0x9e3779b9u) out[0] = acc;  // keeps the loads live; almost never taken
}

__global__ __launch_bounds__(kThreads) void probe_copy_kernel(const u32x4* __restrict__ src,
                                                              u32x4* __restrict__ dst,
                                                              uint64_t n16) {
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
}

}  // namespace

extern "C" int hwkv_probe_read(const void* src, uint64_t bytes, void* out4, int grid,
                               hipStream_t stream) {
    if (!src || !out4 || grid < 1 || bytes % 16) return 1;
    hipLaunchKernelGGL(probe_read_kernel, dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(src), bytes / 16, static_cast<uint32_t*>(out4));
    return hipGetLastError() == hipSuccess ? 0 : 6;
}

extern "C" int hwkv_probe_copy(const void* src, void* dst, uint64_t bytes, int grid,
                               hipStream_t stream) {
    if (!src || !dst || grid < 1 || bytes % 16) return 1;
    hipLaunchKernelGGL(probe_copy_kernel, dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 6;
}
