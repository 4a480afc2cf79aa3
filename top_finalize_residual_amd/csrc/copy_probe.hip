// Bandwidth probes of known byte counts, used only by the benchmark: a plain
// device copy (to calibrate the FETCH_SIZE / WRITE_SIZE counters against a
// kernel whose traffic is known, and as a measured read+write ceiling), a
// read-only sweep (a read ceiling), a write-only fill (a write ceiling), a
// mixed stream that reads and writes in the fused op's own proportions (the
// ceiling of that mix, with no gather and no arithmetic), and an empty kernel
// (the per-launch floor). Not part of the fused op.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

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

// Mixed stream. One unit of work is a block of A * kThreads 16-byte vectors
// read and B * kThreads written: each thread issues its A non-temporal loads
// at once, then stores B vectors, each the XOR of every B-th loaded vector
// (so no load can be dropped). Each unit's accesses go through buffer
// descriptors that cover exactly that unit's bytes. AUX: cache-policy bits of
// the stores (0 write-back, 16 write-through). Two forms:
//   * one unit per workgroup pass, units spread over the grid in turn (with
//     one workgroup per unit, the fused op's own launch);
//   * pipelined: each workgroup walks its units and issues the next unit's
//     loads before the current unit's stores, so a unit's reads are always
//     in flight (the persistent multi-token kernel's schedule).
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t unit_rsrc(const void* base, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(nbytes), 0x00020000);
}

template <int A>
__device__ __forceinline__ void unit_loads(const u32x4* src, int64_t u, u32x4 (&v)[A]) {
    const rsrc_t rs = unit_rsrc(src + u * (A * kThreads), A * kThreads * 16u);
#pragma unroll
    for (int i = 0; i < A; ++i)
        v[i] = __builtin_amdgcn_raw_buffer_load_b128(
            rs, static_cast<int>((i * kThreads + threadIdx.x) * 16u), 0, 2);
}

template <int A, int B>
__device__ __forceinline__ void unit_fold(const u32x4 (&v)[A], u32x4 (&x)[B]) {
#pragma unroll
    for (int j = 0; j < B; ++j) {
        x[j] = v[j];
#pragma unroll
        for (int i = j + B; i < A; i += B) x[j] ^= v[i];
    }
}

template <int B, int AUX>
__device__ __forceinline__ void unit_stores(u32x4* dst, int64_t u, const u32x4 (&x)[B]) {
    const rsrc_t rd = unit_rsrc(dst + u * (B * kThreads), B * kThreads * 16u);
#pragma unroll
    for (int j = 0; j < B; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(
            x[j], rd, static_cast<int>((j * kThreads + threadIdx.x) * 16u), 0, AUX);
}

// The FP8-code form's second output: per thread and unit, B 8-byte stores
// (the two halves of each written vector folded together) into a region of
// its own, as the FP8 codes (one byte per element) sit beside residual_out
// (two bytes per element) in a buffer of their own.
template <int B, int AUX>
__device__ __forceinline__ void unit_stores8(u32x2* dst8, int64_t u, const u32x4 (&x)[B]) {
    const rsrc_t rd = unit_rsrc(dst8 + u * (B * kThreads), B * kThreads * 8u);
#pragma unroll
    for (int j = 0; j < B; ++j)
        __builtin_amdgcn_raw_buffer_store_b64(
            u32x2{x[j].x ^ x[j].z, x[j].y ^ x[j].w}, rd,
            static_cast<int>((j * kThreads + threadIdx.x) * 8u), 0, AUX);
}

// CODES: the B 16-byte stores of each unit are followed by B 8-byte stores
// into dst8 (null otherwise).
template <int A, int B, int AUX, bool CODES>
__global__ __launch_bounds__(kThreads) void mfr_mix_probe_kernel(const u32x4* __restrict__ src,
                                                                 u32x4* __restrict__ dst,
                                                                 u32x2* __restrict__ dst8,
                                                                 int64_t units) {
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
        u32x4 v[A];
        unit_loads<A>(src, u, v);
        __builtin_amdgcn_sched_barrier(0);  // every load in flight before the first use
        u32x4 x[B];
        unit_fold<A, B>(v, x);
        unit_stores<B, AUX>(dst, u, x);
        if constexpr (CODES) unit_stores8<B, AUX>(dst8, u, x);
    }
}

template <int A, int B, int AUX, bool CODES>
__global__ __launch_bounds__(kThreads) void mfr_mix_pipe_probe_kernel(const u32x4* __restrict__ src,
                                                                      u32x4* __restrict__ dst,
                                                                      u32x2* __restrict__ dst8,
                                                                      int64_t units) {
    int64_t u = blockIdx.x;
    if (u >= units) return;
    u32x4 v[A];
    unit_loads<A>(src, u, v);
    for (; u < units; u += gridDim.x) {
        u32x4 x[B];
        unit_fold<A, B>(v, x);
        const int64_t next = u + gridDim.x;
        if (next < units) unit_loads<A>(src, next, v);
        unit_stores<B, AUX>(dst, u, x);
        if constexpr (CODES) unit_stores8<B, AUX>(dst8, u, x);
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

// Streams reads and writes in a fixed proportion over src (src_bytes) and dst
// (dst_bytes), both 16-byte aligned. Per thread and unit of work, `reads`
// vectors in and `writes` out, one of the pairs (10, 2), (15, 3), (20, 4),
// (25, 5), (30, 6) and (40, 8), five to one as in the fused op with bf16
// output ((30, 6) is one token of it at 256 threads: 8 rows, shared and
// residual in, residual_out and normed_out out), or (20, 3) and (40, 6),
// twenty to three as with FP8 codes. flags: bit 0 writes through (else
// back), bit 1 selects the pipelined form (which needs grid > 0), bit 2 the
// FP8-code form, pair (30, 3) only: after its three 16-byte vectors each
// thread writes three 8-byte ones, to a second region that starts where the
// units' 16-byte writes end (one token of the fused op with FP8 output at
// 256 threads: residual_out and the codes, twenty to three as well). As many
// whole units as both buffers hold are processed; `grid` workgroups of 256
// threads, or one workgroup per unit when grid is 0. per_cu > 0 reserves
// enough dynamic LDS at launch that at most that many workgroups fit on a CU
// (the fused op's own residency cap); 0 leaves residency to the registers.
// *read_out and *write_out (if not NULL) receive the bytes moved. Returns 0
// on success, 1 on bad arguments (or buffers too small for one unit), 2 if
// the launch failed, 3 if the residency cannot be set that way.
namespace {

template <int A, int B, int AUX, bool PIPE, bool CODES>
int mix_launch(dim3 g, int per_cu, const u32x4* s, u32x4* d, u32x2* d8, int64_t units,
               hipStream_t stream) {
    const void* kern =
        PIPE ? reinterpret_cast<const void*>(&mfr_mix_pipe_probe_kernel<A, B, AUX, CODES>)
             : reinterpret_cast<const void*>(&mfr_mix_probe_kernel<A, B, AUX, CODES>);
    size_t lds = 0;
    if (per_cu > 0) {
        int dev = 0, lds_cu = 0, fit = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                                  dev) != hipSuccess)
            return 2;
        lds = (static_cast<size_t>(lds_cu) / (per_cu + 1) / 512 + 1) * 512;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&fit, kern, kThreads, lds) !=
                hipSuccess ||
            fit != per_cu)
            return 3;
    }
    void* args[] = {&s, &d, &d8, &units};
    return hipLaunchKernel(kern, g, dim3(kThreads), args, lds, stream) == hipSuccess ? 0 : 2;
}

template <int A, int B, bool CODES = false>
int mix_pick(int flags, dim3 g, int per_cu, const u32x4* s, u32x4* d, u32x2* d8, int64_t units,
             hipStream_t stream) {
    switch (flags & 3) {
        case 0: return mix_launch<A, B, 0, false, CODES>(g, per_cu, s, d, d8, units, stream);
        case 1: return mix_launch<A, B, 16, false, CODES>(g, per_cu, s, d, d8, units, stream);
        case 2: return mix_launch<A, B, 0, true, CODES>(g, per_cu, s, d, d8, units, stream);
        default: return mix_launch<A, B, 16, true, CODES>(g, per_cu, s, d, d8, units, stream);
    }
}

bool mix_pair_ok(int a, int b, bool codes) {
    if (codes) return a == 30 && b == 3;
    return (b * 5 == a && (a == 10 || a == 15 || a == 20 || a == 25 || a == 30 || a == 40)) ||
           (a == 20 && b == 3) || (a == 40 && b == 6);
}

}  // namespace

extern "C" int mfr_mix_probe(const void* src, int64_t src_bytes, void* dst, int64_t dst_bytes,
                             int reads, int writes, int flags, int grid, int per_cu,
                             int64_t* read_out, int64_t* write_out, hipStream_t stream) {
    const bool codes = (flags & 4) != 0;
    if (!src || !dst || src_bytes < 0 || dst_bytes < 0 || grid < 0 || flags < 0 || flags > 7 ||
        per_cu < 0 || per_cu > 32 || !mix_pair_ok(reads, writes, codes) ||
        ((flags & 2) && grid == 0))
        return 1;
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) return 1;
    const int64_t ru = static_cast<int64_t>(reads) * kThreads * 16;
    const int64_t w16 = static_cast<int64_t>(writes) * kThreads * 16;
    const int64_t wu = codes ? w16 + w16 / 2 : w16;
    const int64_t units = src_bytes / ru < dst_bytes / wu ? src_bytes / ru : dst_bytes / wu;
    if (units <= 0 || units > 0x7FFFFFFF) return 1;
    if (read_out) *read_out = units * ru;
    if (write_out) *write_out = units * wu;
    const dim3 g(static_cast<uint32_t>(grid == 0 ? units : grid));
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* d = static_cast<u32x4*>(dst);
    // the second region starts at units * w16, a multiple of 16 bytes
    u32x2* d8 = codes ? reinterpret_cast<u32x2*>(static_cast<char*>(dst) + units * w16) : nullptr;
    if (codes) return mix_pick<30, 3, true>(flags, g, per_cu, s, d, d8, units, stream);
    switch (reads * 100 + writes) {
        case 1002: return mix_pick<10, 2>(flags, g, per_cu, s, d, d8, units, stream);
        case 1503: return mix_pick<15, 3>(flags, g, per_cu, s, d, d8, units, stream);
        case 2004: return mix_pick<20, 4>(flags, g, per_cu, s, d, d8, units, stream);
        case 2505: return mix_pick<25, 5>(flags, g, per_cu, s, d, d8, units, stream);
        case 3006: return mix_pick<30, 6>(flags, g, per_cu, s, d, d8, units, stream);
        case 4008: return mix_pick<40, 8>(flags, g, per_cu, s, d, d8, units, stream);
        case 2003: return mix_pick<20, 3>(flags, g, per_cu, s, d, d8, units, stream);
        default: return mix_pick<40, 6>(flags, g, per_cu, s, d, d8, units, stream);
    }
}

// Launches the empty kernel with `grid` workgroups of `threads` threads (at
// most 1024). Returns 0 on success, 1 on bad arguments, 2 if the launch
// failed.
extern "C" int mfr_empty_probe(int grid, int threads, hipStream_t stream) {
    if (grid <= 0 || threads <= 0 || threads > 1024) return 1;
    hipLaunchKernelGGL(mfr_empty_probe_kernel, dim3(grid), dim3(threads), 0, stream);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
