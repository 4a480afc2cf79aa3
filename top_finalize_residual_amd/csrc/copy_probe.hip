// Plain device copy of a known number of bytes, used only to calibrate
// hardware counters (bytes fetched / written per dispatch) and as a
// measured bandwidth ceiling next to the fused kernel. Not part of the op.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void mfr_copy_probe_kernel(const u32x4* __restrict__ src,
                                                              u32x4* __restrict__ dst, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = __builtin_nontemporal_load(src + i);
}

// Copies `bytes` (a multiple of 16; both pointers 16-byte aligned) on
// `stream` with `grid` workgroups of 256 threads. Returns 0 on success, 1 on
// bad arguments, 2 if the launch failed.
extern "C" int mfr_copy_probe(const void* src, void* dst, int64_t bytes, int grid, hipStream_t stream) {
    if (!src || !dst || bytes < 0 || (bytes & 15) || grid <= 0) return 1;
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) return 1;
    if (bytes == 0) return 0;
    hipLaunchKernelGGL(mfr_copy_probe_kernel, dim3(grid), dim3(256), 0, stream,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
