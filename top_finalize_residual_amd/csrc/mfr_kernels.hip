// Fused MoE finalize + residual add + RMSNorm for MI355X (gfx950, CDNA4),
// and its C ABI (declared in include/moe_finalize_rmsnorm.h).
//
// What is computed (vLLM pull request #62174, Details): the top-k sum of the
// token's GEMM2 rows, the routed scaling, the shared-expert add, the
// all-reduce (identity on one GPU), the residual add and the RMSNorm, in one
// kernel, accumulating in FP32 and rounding once per output (Claims,
// Validation).
//
// The op is a gather-stream: per token it reads K rows of H bf16 plus the
// shared and residual rows and writes two rows, about 0.96 flop per byte, so
// it is bound by HBM bandwidth at large T and by latency at small T. Nothing
// here is a dense contraction, so no MFMA is used. Both kernels share one
// per-token body:
//   * a workgroup owns one token at a time; thread i handles the 16-byte
//     vectors i, i + NT, ..., i + (VPT-1)*NT of every row it touches, so each
//     wave instruction moves 1 KiB of one row, fully coalesced;
//   * shared, residual and gamma loads are issued first (they do not depend
//     on the routing), then the K routing indices and weights are read as
//     wave-uniform scalars and all valid rows' loads are issued together
//     before the first FMA (gathering the routes together keeps K rows in
//     flight per thread);
//   * FP32 FMA chain in slot order in VGPRs; s = (routed + shared) + residual;
//     residual_out is stored at once;
//   * sum of squares: per lane, then a DPP tree within each wave, then one
//     LDS step across waves behind a single barrier;
//   * normalisation from the registers still holding s (no second read).
// The token kernel (grid = T) is the latency path; the stream kernel runs a
// persistent grid sized to the device's occupancy that walks the tokens, for
// large T.

#include "mfr_device.h"
#include "moe_finalize_rmsnorm.h"

#include <atomic>
#include <cmath>
#include <cstdint>

namespace mfr {

struct Params {
    const u32x4* expert_out;
    const int32_t* perm_idx;
    const float* topk_w;
    const u32x4* shared_out;
    const u32x4* residual;  // may equal residual_out (in place)
    const u32x4* gamma;
    u32x4* residual_out;
    u32x4* normed_out;
    int64_t T;
    float eps;
    float scale;
    float h_f;  // H as float (exact: H <= 16384)
    int V;      // 16-byte vectors per row, H / 8
    int K;
};

constexpr int MAX_WAVES = 16;  // 1024 threads

// Loads the rows of slots [k0, k0 + 8) and folds them into acc in slot order.
// Straight-line code: the scalar index/weight loads, then all eight row loads,
// then the FMAs. A masked slot (index < 0) or a slot at or past K gets a
// zero-record descriptor and a zero weight: its loads return zeros without
// touching memory and its FMA adds +0, which leaves acc bit-for-bit unchanged
// (acc starts at +0 and an exact-zero sum rounds to +0). No branches.
template <int VPT, bool CHECK_K>
__device__ __forceinline__ void gather8(const Params& p, const int32_t* prow, const float* wrow,
                                        int k0, const uint32_t (&off)[VPT],
                                        float (&acc)[VPT][8]) {
    const uint32_t rowbytes = static_cast<uint32_t>(p.V) * 16u;
    // Both metadata arrays are read unconditionally (eight scalar loads each,
    // merged by the compiler), then the slot decisions are uniform selects.
    int32_t idx[8];
    float wr[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        // CHECK_K: clamp to a slot that exists so the scalar load stays in bounds.
        const int k = k0 + kk;
        const int kc = CHECK_K ? (k < p.K ? k : p.K - 1) : k;
        idx[kk] = prow[kc];
        wr[kk] = wrow[kc];
    }
    rsrc_t rows[8];
    float w[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        const bool use = idx[kk] >= 0 && (!CHECK_K || k0 + kk < p.K);
        rows[kk] = make_rsrc(p.expert_out + static_cast<int64_t>(use ? idx[kk] : 0) * p.V,
                             use ? rowbytes : 0u);
        const float ws = p.scale * wr[kk];
        w[kk] = use ? ws : 0.0f;
    }
    u32x4 r[8][VPT];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int j = 0; j < VPT; ++j) r[kk][j] = buf_load<kAuxStream>(rows[kk], off[j]);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int j = 0; j < VPT; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[j][e] = __builtin_fmaf(w[kk], vec_elem(r[kk][j], e), acc[j][e]);
}

// One token, end to end. KT: 8 = exactly eight slots (the GLM-5.x / DeepSeek
// top-8 case, no slot-count checks); 0 = any K in 1..16, as one or two
// chunks of eight. Thread i owns the byte offsets 16*(i + j*NT), j < VPT, of
// every row; offsets at or past the row end (a ragged last tile) fall outside
// the descriptors' range, so their loads return zero and their stores are
// dropped by the hardware.
template <int VPT, int KT>
__device__ __forceinline__ void finalize_token(const Params& p, const int64_t t, float* red) {
    const int tid = threadIdx.x;
    const int nt = blockDim.x;
    const uint32_t rowbytes = static_cast<uint32_t>(p.V) * 16u;
    const int64_t trow = t * static_cast<int64_t>(p.V);

    uint32_t off[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) off[j] = static_cast<uint32_t>(tid + j * nt) * 16u;

    // Inputs that do not depend on the routing go first.
    const rsrc_t sh_r = make_rsrc(p.shared_out + trow, rowbytes);
    const rsrc_t rs_r = make_rsrc(p.residual + trow, rowbytes);
    const rsrc_t gm_r = make_rsrc(p.gamma, rowbytes);
    u32x4 sh[VPT], rs[VPT], gm[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        sh[j] = buf_load<kAuxStream>(sh_r, off[j]);
        rs[j] = buf_load<kAuxStream>(rs_r, off[j]);
        gm[j] = buf_load<kAuxDefault>(gm_r, off[j]);
    }

    float acc[VPT][8];
#pragma unroll
    for (int j = 0; j < VPT; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = 0.0f;

    const int32_t* prow = p.perm_idx + t * p.K;
    const float* wrow = p.topk_w + t * p.K;
    if (KT == 8) {
        gather8<VPT, false>(p, prow, wrow, 0, off, acc);
    } else {
        gather8<VPT, true>(p, prow, wrow, 0, off, acc);
        if (p.K > 8) gather8<VPT, true>(p, prow, wrow, 8, off, acc);
    }

    // s = (routed + shared) + residual; residual_out = bf16(s); per-lane sum of squares.
    const rsrc_t ro_r = make_rsrc(p.residual_out + trow, rowbytes);
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[j][e] = (acc[j][e] + vec_elem(sh[j], e)) + vec_elem(rs[j], e);
            ss = __builtin_fmaf(acc[j][e], acc[j][e], ss);
        }
        u32x4 o;
        o.x = pack_bf16x2(acc[j][0], acc[j][1]);
        o.y = pack_bf16x2(acc[j][2], acc[j][3]);
        o.z = pack_bf16x2(acc[j][4], acc[j][5]);
        o.w = pack_bf16x2(acc[j][6], acc[j][7]);
        buf_store<kAuxDefault>(o, ro_r, off[j]);
    }

    // Row reduction: wave tree, then the waves' partial sums in order.
    const float wsum = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = wsum;
    __syncthreads();
    float tot = 0.0f;
    const int nw = nt >> 6;
    for (int w = 0; w < nw; ++w) tot += red[w];
    const float rstd = 1.0f / __builtin_sqrtf(tot / p.h_f + p.eps);

    const rsrc_t no_r = make_rsrc(p.normed_out + trow, rowbytes);
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = (acc[j][e] * rstd) * vec_elem(gm[j], e);
        u32x4 o;
        o.x = pack_bf16x2(y[0], y[1]);
        o.y = pack_bf16x2(y[2], y[3]);
        o.z = pack_bf16x2(y[4], y[5]);
        o.w = pack_bf16x2(y[6], y[7]);
        buf_store<kAuxDefault>(o, no_r, off[j]);
    }
}

// Launch bound per vectors-per-thread: keeps the register budget large enough
// that the row vectors in flight never spill.
template <int VPT>
struct Bound {
    static constexpr int kThreads = VPT == 1 ? 1024 : 512;
};

template <int VPT, int KT>
__global__ __launch_bounds__(Bound<VPT>::kThreads) void mfr_token_kernel(Params p) {
    __shared__ float red[MAX_WAVES];
    finalize_token<VPT, KT>(p, static_cast<int64_t>(blockIdx.x), red);
}

template <int VPT, int KT>
__global__ __launch_bounds__(Bound<VPT>::kThreads) void mfr_stream_kernel(Params p) {
    // Two reduction slots, alternated per token: a wave can only reach the
    // token after next once every wave has passed the next token's barrier,
    // i.e. after everyone has finished reading this token's slot.
    __shared__ float red[2][MAX_WAVES];
    int par = 0;
    for (int64_t t = blockIdx.x; t < p.T; t += gridDim.x) {
        finalize_token<VPT, KT>(p, t, red[par]);
        par ^= 1;
    }
}

}  // namespace mfr

// ---------------------------------------------------------------------------
// Host side: validation, path choice, launch.
// ---------------------------------------------------------------------------
namespace {

constexpr int64_t kHMax = 16384;
constexpr int64_t kKMax = 16;
constexpr int64_t kTMax = 2147483647;
constexpr int kVptMax = 4;
// Token counts up to this use the one-workgroup-per-token kernel.
constexpr int64_t kTokenPathMaxT = 256;
constexpr int kMaxDevices = 64;

std::atomic<int> g_force_path{0};
std::atomic<int> g_force_vpt{0};
std::atomic<int> g_force_wgpcu{0};
std::atomic<int> g_cu_count[kMaxDevices];
// occupancy cache: [device][vpt-1][threads/64 - 1]
std::atomic<int> g_occ[kMaxDevices][kVptMax][2][16];

int max_threads(int vpt) { return vpt == 1 ? 1024 : 512; }

int threads_for(int64_t V, int vpt) {
    int64_t n = (V + vpt - 1) / vpt;
    n = (n + 63) / 64 * 64;
    return static_cast<int>(n);
}

bool shape_ok(int64_t T, int64_t H, int64_t K) {
    return T >= 0 && T <= kTMax && H >= 8 && H <= kHMax && H % 8 == 0 && K >= 1 && K <= kKMax;
}

int choose_path(int64_t T) {
    const int f = g_force_path.load(std::memory_order_relaxed);
    if (f == MFR_PATH_TOKEN || f == MFR_PATH_STREAM) return f;
    return T <= kTokenPathMaxT ? MFR_PATH_TOKEN : MFR_PATH_STREAM;
}

// Vectors per thread: the token path spreads a row over as many threads as
// possible (latency); the stream path uses up to 256 threads per token so that
// more tokens are resident per CU (bandwidth).
int choose_vpt(int path, int64_t V) {
    const int f = g_force_vpt.load(std::memory_order_relaxed);
    if (f >= 1 && f <= kVptMax && threads_for(V, f) <= max_threads(f)) return f;
    if (path == MFR_PATH_TOKEN) {
        for (int v = 1; v <= kVptMax; ++v)
            if (threads_for(V, v) <= max_threads(v)) return v;
    } else {
        for (int v = 1; v <= kVptMax; ++v)
            if (threads_for(V, v) <= 256) return v;
        for (int v = 1; v <= kVptMax; ++v)
            if (threads_for(V, v) <= max_threads(v)) return v;
    }
    return kVptMax;
}

bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
    const uint64_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return na > 0 && nb > 0 && a0 < b0 + nb && b0 < a0 + na;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Kernel address for (path, vectors per thread, K == 8).
template <int VPT>
const void* pick(int path, bool k8) {
    if (path == MFR_PATH_TOKEN)
        return k8 ? reinterpret_cast<const void*>(&mfr::mfr_token_kernel<VPT, 8>)
                  : reinterpret_cast<const void*>(&mfr::mfr_token_kernel<VPT, 0>);
    return k8 ? reinterpret_cast<const void*>(&mfr::mfr_stream_kernel<VPT, 8>)
              : reinterpret_cast<const void*>(&mfr::mfr_stream_kernel<VPT, 0>);
}

const void* kernel_for(int path, int vpt, bool k8) {
    switch (vpt) {
        case 1: return pick<1>(path, k8);
        case 2: return pick<2>(path, k8);
        case 3: return pick<3>(path, k8);
        default: return pick<4>(path, k8);
    }
}

// Persistent grid size for the stream kernel: compute units times resident
// workgroups per CU (from the occupancy calculator, cached per device).
hipError_t stream_grid(const void* kern, int vpt, int variant, int nt, int64_t T, int64_t* grid) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int cus = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cus <= 0) {
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        g_cu_count[dev].store(cus, std::memory_order_relaxed);
    }
    int per_cu = g_force_wgpcu.load(std::memory_order_relaxed);
    if (per_cu <= 0) {
        const int slot = nt / 64 - 1;
        per_cu = g_occ[dev][vpt - 1][variant][slot].load(std::memory_order_relaxed);
        if (per_cu <= 0) {
            int nb = 0;
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, nt, 0);
            if (e != hipSuccess) return e;
            per_cu = nb > 0 ? nb : 1;
            g_occ[dev][vpt - 1][variant][slot].store(per_cu, std::memory_order_relaxed);
        }
    }
    const int64_t g = static_cast<int64_t>(cus) * per_cu;
    *grid = T < g ? T : g;
    return hipSuccess;
}

}  // namespace

extern "C" {

int moe_finalize_rmsnorm(const uint16_t* expert_out, const int32_t* perm_idx,
                         const float* topk_w, const uint16_t* shared_out,
                         const uint16_t* residual, const uint16_t* gamma,
                         float eps, float scale,
                         uint16_t* residual_out, uint16_t* normed_out,
                         int64_t T, int64_t H, int64_t K, hipStream_t stream) {
    if (!shape_ok(T, H, K)) return MFR_ERR_SHAPE;
    if (!(eps >= 0.0f) || !std::isfinite(eps) || !std::isfinite(scale)) return MFR_ERR_SCALAR;
    if (T == 0) return MFR_OK;
    if (!expert_out || !perm_idx || !topk_w || !shared_out || !residual || !gamma ||
        !residual_out || !normed_out)
        return MFR_ERR_NULL;
    if (!aligned(expert_out, 16) || !aligned(shared_out, 16) || !aligned(residual, 16) ||
        !aligned(gamma, 16) || !aligned(residual_out, 16) || !aligned(normed_out, 16) ||
        !aligned(perm_idx, 4) || !aligned(topk_w, 4))
        return MFR_ERR_ALIGN;

    const uint64_t act = static_cast<uint64_t>(T) * H * 2;  // bytes of a [T, H] bf16 tensor
    const uint64_t meta = static_cast<uint64_t>(T) * K * 4;
    const uint64_t gam = static_cast<uint64_t>(H) * 2;
    // residual_out may be exactly residual; any other overlap of an output is refused.
    if (residual_out != residual && overlaps(residual_out, act, residual, act)) return MFR_ERR_ALIAS;
    if (overlaps(residual_out, act, shared_out, act) || overlaps(residual_out, act, gamma, gam) ||
        overlaps(residual_out, act, perm_idx, meta) || overlaps(residual_out, act, topk_w, meta) ||
        overlaps(residual_out, act, normed_out, act) || overlaps(residual_out, act, expert_out, 16))
        return MFR_ERR_ALIAS;
    if (overlaps(normed_out, act, residual, act) || overlaps(normed_out, act, shared_out, act) ||
        overlaps(normed_out, act, gamma, gam) || overlaps(normed_out, act, perm_idx, meta) ||
        overlaps(normed_out, act, topk_w, meta) || overlaps(normed_out, act, expert_out, 16))
        return MFR_ERR_ALIAS;

    mfr::Params p;
    p.expert_out = reinterpret_cast<const mfr::u32x4*>(expert_out);
    p.perm_idx = perm_idx;
    p.topk_w = topk_w;
    p.shared_out = reinterpret_cast<const mfr::u32x4*>(shared_out);
    p.residual = reinterpret_cast<const mfr::u32x4*>(residual);
    p.gamma = reinterpret_cast<const mfr::u32x4*>(gamma);
    p.residual_out = reinterpret_cast<mfr::u32x4*>(residual_out);
    p.normed_out = reinterpret_cast<mfr::u32x4*>(normed_out);
    p.T = T;
    p.eps = eps;
    p.scale = scale;
    p.h_f = static_cast<float>(H);
    p.V = static_cast<int>(H / 8);
    p.K = static_cast<int>(K);

    const int path = choose_path(T);
    const int vpt = choose_vpt(path, p.V);
    const int nt = threads_for(p.V, vpt);
    const bool k8 = K == 8;
    const void* kern = kernel_for(path, vpt, k8);
    void* args[] = {&p};
    hipError_t e;
    if (path == MFR_PATH_TOKEN) {
        e = hipLaunchKernel(kern, dim3(static_cast<uint32_t>(T)), dim3(nt), args, 0, stream);
    } else {
        int64_t grid = 0;
        e = stream_grid(kern, vpt, k8 ? 1 : 0, nt, T, &grid);
        if (e == hipSuccess)
            e = hipLaunchKernel(kern, dim3(static_cast<uint32_t>(grid)), dim3(nt), args, 0, stream);
    }
    return e == hipSuccess ? MFR_OK : MFR_ERR_HIP;
}

int moe_finalize_rmsnorm_path(int64_t T, int64_t H, int64_t K) {
    if (!shape_ok(T, H, K)) return MFR_PATH_UNSUPPORTED;
    return choose_path(T == 0 ? 1 : T);
}

const char* moe_finalize_rmsnorm_strerror(int status) {
    switch (status) {
        case MFR_OK: return "success";
        case MFR_ERR_NULL: return "a required pointer is NULL";
        case MFR_ERR_SHAPE: return "T, H or K outside the supported limits (0<=T<2^31, 8<=H<=16384, H%8==0, 1<=K<=16)";
        case MFR_ERR_ALIGN: return "bf16 pointers must be 16-byte aligned, perm_idx/topk_w 4-byte aligned";
        case MFR_ERR_ALIAS: return "an output overlaps an input or the other output (only residual_out == residual is allowed)";
        case MFR_ERR_SCALAR: return "eps must be finite and >= 0, scale must be finite";
        case MFR_ERR_HIP: return "the HIP runtime refused the kernel launch";
        case MFR_ERR_ARG: return "invalid override value";
        default: return "unknown status";
    }
}

int moe_finalize_rmsnorm_force(int path, int vectors_per_thread, int wg_per_cu) {
    if (path < 0 || path > MFR_PATH_STREAM) return MFR_ERR_ARG;
    if (vectors_per_thread < 0 || vectors_per_thread > kVptMax) return MFR_ERR_ARG;
    if (wg_per_cu < 0 || wg_per_cu > 16) return MFR_ERR_ARG;
    g_force_path.store(path, std::memory_order_relaxed);
    g_force_vpt.store(vectors_per_thread, std::memory_order_relaxed);
    g_force_wgpcu.store(wg_per_cu, std::memory_order_relaxed);
    return MFR_OK;
}

}  // extern "C"
