// Bandwidth probes of known byte counts, used only by the benchmark: a plain
// device copy (to calibrate the FETCH_SIZE / WRITE_SIZE counters against a
// kernel whose traffic is known, and as a measured read+write ceiling), a
// read-only sweep (a read ceiling), a write-only fill (a write ceiling), and
// an empty kernel (the per-launch floor). Not part of the fused op.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // 16-byte vectors in flight per thread per iteration

__global__ __launch_bounds__(kThreads) void mfr_copy_probe_kernel(const u32x4* __restrict__ src,
                                                                  u32x4* __restrict__ dst,
                                                                  int64_t n) {
    const int64_t chunk = static_cast<int64_t>(kThreads) * kUnroll;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * chunk; base < n;
         base += static_cast<int64_t>(gridDim.x) * chunk) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + u * kThreads + threadIdx.x;
            if (i < n) v[u] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + u * kThreads + threadIdx.x;
            if (i < n) dst[i] = v[u];
        }
    }
}

// Reads n vectors and writes one dword per workgroup (so the reads cannot be
// removed); out must hold gridDim.x dwords. NT: non-temporal loads (the read
// ceiling) or ordinary loads (which leave the data resident in the caches,
// to set a known cache state).
template <bool NT>
__global__ __launch_bounds__(kThreads) void mfr_read_probe_kernel(const u32x4* __restrict__ src,
                                                                  uint32_t* __restrict__ out,
                                                                  int64_t n) {
    const int64_t chunk = static_cast<int64_t>(kThreads) * kUnroll;
    uint32_t acc = 0;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * chunk; base < n;
         base += static_cast<int64_t>(gridDim.x) * chunk) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + u * kThreads + threadIdx.x;
            v[u] = i < n ? (NT ? __builtin_nontemporal_load(src + i) : src[i]) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    __shared__ uint32_t red[kThreads];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int i = 0; i < kThreads; ++i) r ^= red[i];
        out[blockIdx.x] = r;
    }
}

// Writes n vectors of one constant pattern.
__global__ __launch_bounds__(kThreads) void mfr_write_probe_kernel(u32x4* __restrict__ dst,
                                                                   int64_t n, uint32_t pattern) {
    const int64_t chunk = static_cast<int64_t>(kThreads) * kUnroll;
    const u32x4 v = {pattern, pattern, pattern, pattern};
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * chunk; base < n;
         base += static_cast<int64_t>(gridDim.x) * chunk) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + u * kThreads + threadIdx.x;
            if (i < n) dst[i] = v;
        }
    }
}

// Does nothing: its launch-to-completion time is the floor under any kernel.
__global__ __launch_bounds__(1024) void mfr_empty_probe_kernel() {}

// Copies `bytes` (a multiple of 16; both pointers 16-byte aligned) on
// `stream` with `grid` workgroups of 256 threads. Returns 0 on success, 1 on
// bad arguments, 2 if the launch failed.
extern "C" int mfr_copy_probe(const void* src, void* dst, int64_t bytes, int grid, hipStream_t stream) {
    if (!src || !dst || bytes < 0 || (bytes & 15) || grid <= 0) return 1;
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) return 1;
    if (bytes == 0) return 0;
    hipLaunchKernelGGL(mfr_copy_probe_kernel, dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Reads `bytes` (a multiple of 16, 16-byte aligned) with `grid` workgroups;
// `out` must hold `grid` dwords. Returns 0 on success, 1 on bad arguments, 2
// if the launch failed.
extern "C" int mfr_read_probe(const void* src, void* out, int64_t bytes, int grid, hipStream_t stream) {
    if (!src || !out || bytes < 0 || (bytes & 15) || grid <= 0) return 1;
    if (reinterpret_cast<uintptr_t>(src) & 15) return 1;
    if (bytes == 0) return 0;
    hipLaunchKernelGGL(mfr_read_probe_kernel<true>, dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(src), static_cast<uint32_t*>(out), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// As mfr_read_probe, with ordinary (cache-allocating) loads.
extern "C" int mfr_touch_probe(const void* src, void* out, int64_t bytes, int grid,
                               hipStream_t stream) {
    if (!src || !out || bytes < 0 || (bytes & 15) || grid <= 0) return 1;
    if (reinterpret_cast<uintptr_t>(src) & 15) return 1;
    if (bytes == 0) return 0;
    hipLaunchKernelGGL(mfr_read_probe_kernel<false>, dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(src), static_cast<uint32_t*>(out), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Fills `bytes` (a multiple of 16, 16-byte aligned) of dst with `pattern`
// using `grid` workgroups of 256 threads. Returns 0 on success, 1 on bad
// arguments, 2 if the launch failed.
extern "C" int mfr_write_probe(void* dst, int64_t bytes, uint32_t pattern, int grid,
                               hipStream_t stream) {
    if (!dst || bytes < 0 || (bytes & 15) || grid <= 0) return 1;
    if (reinterpret_cast<uintptr_t>(dst) & 15) return 1;
    if (bytes == 0) return 0;
    hipLaunchKernelGGL(mfr_write_probe_kernel, dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<u32x4*>(dst), bytes / 16, pattern);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Launches the empty kernel with `grid` workgroups of `threads` threads (at
// most 1024). Returns 0 on success, 1 on bad arguments, 2 if the launch
// failed.
extern "C" int mfr_empty_probe(int grid, int threads, hipStream_t stream) {
    if (grid <= 0 || threads <= 0 || threads > 1024) return 1;
    hipLaunchKernelGGL(mfr_empty_probe_kernel, dim3(grid), dim3(threads), 0, stream);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
