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
// here is a dense contraction, so no MFMA is used.
//
// One workgroup owns one token (grid = T):
//   * thread i handles the 16-byte vectors i, i + NT, ..., i + (VPT-1)*NT of
//     every row it touches, so each wave instruction moves 1 KiB of one row,
//     fully coalesced, through raw buffer loads;
//   * shared, residual and gamma loads are issued first (they do not depend
//     on the routing), then the K routing indices and weights are read as
//     wave-uniform scalars and all valid rows' loads are issued together
//     before the first FMA (gathering the routes together keeps K rows in
//     flight per thread);
//   * FP32 FMA chain in slot order in VGPRs; s = (routed + shared) + residual;
//   * sum of squares: per lane, then a DPP tree within each wave, then one
//     LDS step across waves behind a single barrier;
//   * after the barrier, residual_out = bf16(s) (before it, in the dense bf16
//     tail) and the normalisation, both from the registers still holding s
//     (no second read).
// Two launch shapes ("paths") of the same kernel:
//   * token path (small T, latency): the widest workgroup, one 16-byte vector
//     per thread per row (768 threads at H = 6144), so the K row loads of a
//     lone token are spread over as many waves as possible;
//   * stream path (large T, bandwidth): 256 threads per token (3 vectors per
//     thread per row at H = 6144), so three tokens are resident per CU, and,
//     once the outputs outgrow the L2, write-through stores (sc1) that send
//     them straight on instead of through L2 write-back.
// A persistent variant (a grid sized to the CUs, each workgroup looping over
// tokens) measured 3-4% slower than this grid of tokens at T = 512 and 8192:
// the hardware dispatcher balances the tail better than a static assignment.

#include "mfr_device.h"
#include "mfr_tuning.h"
#include "moe_finalize_rmsnorm.h"

#include <atomic>
#include <cmath>
#include <mutex>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

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
    float eps;
    float scale;
    uint32_t rows;  // rows of expert_out, at most 2^31: an index at or past it is masked
    float inv_h;    // 1 / H rounded to fp32: the mean of squares is their sum times it
    int64_t T;
    uint8_t* normed_fp8;  // [T, H] E4M3 codes (FP8 output modes only)
    float* fp8_scale;     // [T] per-token scales (FP8 output modes only)
    int32_t* bad_index;   // optional: set to 1 when some slot's index is at or past R
    // Last, so that the kernels' scalar loads of the fields above, which
    // they use, do not take in these, which they get as leading arguments.
    // (The order above serves the same end: a run of three used 32-bit
    // fields is loaded as four, and a register filled with an unused field
    // may be reused at once, which waits for the load. rows, used only by
    // the checked kernels, therefore sits between scale and inv_h.)
    int V;  // 16-byte vectors per row, H / 8
    int K;
};

// What the normalisation writes: the bf16 normed row, the per-token FP8
// (E4M3) row with its scale, or both.
enum OutMode { kOutBf16 = 0, kOutFp8 = 1, kOutBoth = 2 };
constexpr float kE4m3Max = 448.0f;  // largest finite OCP E4M3 value

constexpr int MAX_WAVES = 16;  // 1024 threads

// Workgroup scratch in LDS: the per-wave partial results of the row
// reductions.
struct Lds {
    float red[2 * MAX_WAVES];  // sums of squares, then (FP8 modes) maxima of |s * gamma|
    double red64[MAX_WAVES];   // fp64 sums of squares (range rescue only)
    float redm[MAX_WAVES];     // maxima of |y| (range rescue, FP8 modes)
};

// Threads per workgroup at VPT vectors per thread: a row's V vectors spread
// over whole waves. The host launches exactly this many, so the kernels
// derive it from V (an argument they hold in registers from the start)
// instead of reading the workgroup size from the dispatch's implicit
// arguments, a scalar memory load ahead of the first row load.
template <int VPT>
__device__ __forceinline__ int threads_of(int V) {
    return ((V + VPT - 1) / VPT + 63) & ~63;
}

// The fp32 normalisation is used when mean(s^2) + eps lies in
// [kRescueBelow, FLT_MAX]. Above, the fp32 sum of squares has overflowed;
// below, fp32 subnormal squares (or squares flushed to zero) could decide
// rstd, which happens only with eps (nearly) 0. There the row is
// normalised again in fp64.
constexpr float kRescueBelow = 0x1p-100f;
constexpr float kFltMax = 0x1.fffffep127f;

// Routing metadata of slots [k0, k0 + 8): indices and weights, read
// unconditionally (wave-uniform scalar loads, merged by the compiler). With
// CHECK_K, slots at or past K re-read slot K-1 so every load stays in bounds;
// gather_rows8 ignores them. Those loads cannot be merged, and scalar loads
// complete out of order, so any use of one waits for all that are in
// flight: the scheduling barrier keeps every use below the last load, so
// that the sixteen loads cost one round trip rather than one each.
// The loads go through the constant address space: perm_idx and topk_w are
// never written while a kernel runs (every entry point refuses outputs that
// overlap them), and saying so keeps them scalar loads after a store, as in
// the persistent kernel's loop. There, a compiler that must assume the
// stores could change them emits vector loads instead, and vector loads and
// stores share one in-order counter: waiting for the metadata then waits for
// every store and row load issued before it, the next token's included.
template <bool CHECK_K>
__device__ __forceinline__ void load_meta8(const Params& p, const int32_t* prow, const float* wrow,
                                           int k0, int32_t (&idx)[8], float (&wr)[8]) {
    typedef const int32_t __attribute__((address_space(4)))* const_i32;
    typedef const float __attribute__((address_space(4)))* const_f32;
    const const_i32 prow_c = (const_i32)prow;
    const const_f32 wrow_c = (const_f32)wrow;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        const int k = k0 + kk;
        const int kc = CHECK_K ? (k < p.K ? k : p.K - 1) : k;
        idx[kk] = prow_c[kc];
        wr[kk] = wrow_c[kc];
    }
    if constexpr (CHECK_K) __builtin_amdgcn_sched_barrier(0);
}

// Issues the row loads of slots [k0, k0 + 8): every load is in flight when
// this returns, the rows in r and the scaled weights in w. A masked slot
// (index < 0), a slot whose index is at or past R, or a slot at or past K
// gets a zero-record descriptor and a zero weight: its loads return zeros
// without touching memory, and its FMA in fold_rows8 adds +0, which leaves
// acc bit-for-bit unchanged (acc starts at +0 and an exact-zero sum rounds to
// +0). No branches. ROWS (the entry point told R) also masks an index at or
// past the rows and, when the caller asked for the report, returns whether a
// slot within K held one (the indices are wave-uniform, so the result is
// too); without ROWS the code is the plain index >= 0 test. live = false
// (the persistent path, a slot past the last token) gives every slot a
// zero-record descriptor.
template <int VPT, bool CHECK_K, bool ROWS>
__device__ __forceinline__ bool issue_rows8(const Params& p, const int32_t (&idx)[8],
                                            const float (&wr)[8], int k0,
                                            const uint32_t (&off)[VPT], u32x4 (&r)[8][VPT],
                                            float (&w)[8], bool live = true) {
    const uint32_t rowbytes = static_cast<uint32_t>(p.V) * 16u;
    rsrc_t rows[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        // With ROWS, one unsigned compare masks both a negative index (it
        // wraps to 2^31 or more) and one at or past the rows.
        const bool in_range = ROWS ? static_cast<uint32_t>(idx[kk]) < p.rows : idx[kk] >= 0;
        const bool use = live && in_range && (!CHECK_K || k0 + kk < p.K);
        // the row offset in unsigned arithmetic (a used index is >= 0): a
        // zero extension needs nothing of the loaded value, where a sign
        // extension, placed by the compiler right after each index load,
        // would make every load wait for the one before
        const uint32_t row = use ? static_cast<uint32_t>(idx[kk]) : 0u;
        rows[kk] = make_rsrc(p.expert_out + static_cast<uint64_t>(row) * static_cast<uint32_t>(p.V),
                             use ? rowbytes : 0u);
        const float ws = p.scale * wr[kk];
        w[kk] = use ? ws : 0.0f;
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int j = 0; j < VPT; ++j) r[kk][j] = buf_load<kAuxRows>(rows[kk], off[j]);
    // Whether a slot within K held an index at or past the rows: only asked
    // for when the caller wants the report (a uniform branch).
    bool past_r = false;
    if (ROWS && p.bad_index != nullptr) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            past_r |= live && (!CHECK_K || k0 + kk < p.K) && idx[kk] >= 0 &&
                      static_cast<uint32_t>(idx[kk]) >= p.rows;
    }
    return past_r;
}

// Folds eight loaded rows into acc in slot order (an FMA chain per element).
template <int VPT>
__device__ __forceinline__ void fold_rows8(const u32x4 (&r)[8][VPT], const float (&w)[8],
                                           float (&acc)[VPT][8]) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int j = 0; j < VPT; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[j][e] = __builtin_fmaf(w[kk], vec_elem(r[kk][j], e), acc[j][e]);
}

// Loads the rows of slots [k0, k0 + 8) and folds them into acc in slot order.
// Straight-line code: all eight row loads are issued, then the FMAs.
template <int VPT, bool CHECK_K, bool ROWS>
__device__ __forceinline__ bool gather_rows8(const Params& p, const int32_t (&idx)[8],
                                             const float (&wr)[8], int k0,
                                             const uint32_t (&off)[VPT], float (&acc)[VPT][8]) {
    u32x4 r[8][VPT];
    float w[8];
    const bool past_r = issue_rows8<VPT, CHECK_K, ROWS>(p, idx, wr, k0, off, r, w);
    fold_rows8<VPT>(r, w, acc);
    return past_r;
}

// The normalisation of a row whose fp32 sum of squares cannot be used: it
// overflowed (|s| beyond about 2^64 / sqrt(H), where rstd would come out 0
// and the normed row as zeros), or it is so small that fp32 subnormal
// squares, or squares flushed to zero, would decide rstd (eps near 0 and
// |s| below about 2^-50; with eps = 0 and every square zero rstd would be
// infinite). RMSNorm is defined on the exact sum (vLLM pull request #62174,
// Validation: the fused result must match the unfused chain), and fp64 holds
// the square of every fp32 value, so the squares are summed again in fp64,
// in the same lane, wave and workgroup order, and rstd is taken in fp64.
// rstd itself may lie outside the fp32 range, so it is split as
// m * 2^k with m in [0.5, 1): y = ((s * 2^k) * m) * gamma in fp32, where
// the scaling by 2^k is exact and |s * 2^k| stays below 2 sqrt(H). The
// rounding steps are those of the fp32 path.
// Entered by the whole workgroup or by none of it (the condition depends
// only on the reduced sum, which every thread holds), so its barriers are
// uniform. It adds no registers to the common path.
// gamma is loaded again here rather than kept in registers past the
// barrier, which the FP8-only output does not otherwise need.
template <int VPT, int OUT_AUX, int QM>
__device__ __forceinline__ void normalise_wide(const Params& p, const int64_t t,
                                               const float (&acc)[VPT][8],
                                               const uint32_t (&off)[VPT], Lds& lds) {
    const int tid = threadIdx.x;
    const int nw = threads_of<VPT>(p.V) >> 6;
    const uint32_t rowbytes = static_cast<uint32_t>(p.V) * 16u;
    const int64_t trow = t * static_cast<int64_t>(p.V);
    const rsrc_t gm_r = make_rsrc(p.gamma, rowbytes);
    u32x4 gm[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) gm[j] = buf_load<kAuxGamma>(gm_r, off[j]);
    // One element at a time (a scheduling barrier after each), so that only
    // one converted value is live: this branch must not raise the register
    // count of the kernel, and with it the occupancy of the common path.
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < VPT; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const double v = acc[j][e];
            ss = __builtin_fma(v, v, ss);
            __builtin_amdgcn_sched_barrier(0);
        }
    const double wsum = wave_sum_f64(ss);
    if ((tid & 63) == 0) lds.red64[tid >> 6] = wsum;
    __syncthreads();
    double tot = 0.0;
#pragma unroll 1
    for (int w = 0; w < nw; ++w) tot += lds.red64[w];
    const double rstd = 1.0 / __builtin_sqrt(tot / (static_cast<double>(p.V) * 8.0) +
                                             static_cast<double>(p.eps));
    // rstd = m * 2^k; an infinite, zero or NaN rstd (an all-zero row with
    // eps = 0, an infinite or NaN s) is used as it is, as in the fp32 path.
    int k = 0;
    float m = static_cast<float>(rstd);
    if (rstd > 0.0 && rstd <= 0x1.fffffffffffffp1023) m = static_cast<float>(__builtin_frexp(rstd, &k));
    float y[VPT][8];
#pragma unroll
    for (int j = 0; j < VPT; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            y[j][e] = (__builtin_ldexpf(acc[j][e], k) * m) * vec_elem(gm[j], e);
    if (QM != kOutFp8) {
        const rsrc_t no_r = make_rsrc(p.normed_out + trow, rowbytes);
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            u32x4 o;
            o.x = pack_bf16x2(y[j][0], y[j][1]);
            o.y = pack_bf16x2(y[j][2], y[j][3]);
            o.z = pack_bf16x2(y[j][4], y[j][5]);
            o.w = pack_bf16x2(y[j][6], y[j][7]);
            buf_store<OUT_AUX>(o, no_r, off[j]);
        }
    }
    if (QM != kOutBf16) {
        // amax over the row's y (NaN elements aside), then the FP8 rule of
        // the fp32 path applied to y itself.
        float mx = 0.0f;
#pragma unroll
        for (int j = 0; j < VPT; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) mx = __builtin_fmaxf(mx, __builtin_fabsf(y[j][e]));
        const float wm = wave_max(mx);
        if ((tid & 63) == 0) lds.redm[tid >> 6] = wm;
        __syncthreads();
        float amax = 0.0f;
#pragma unroll 1
        for (int w = 0; w < nw; ++w) amax = __builtin_fmaxf(amax, lds.redm[w]);
        const bool zero_row = !(amax > 0.0f);
        const float qscale = zero_row ? 1.0f : amax / kE4m3Max;
        // rows whose amax is below 2^-100 are scaled by 2^64 first (exact),
        // so that 448 / amax cannot overflow
        const float a = (!zero_row && amax < 0x1p-100f) ? 0x1p64f : 1.0f;
        const float f = zero_row ? 0.0f : e4m3_factor(amax * a);
        const rsrc_t q_r = make_rsrc(p.normed_fp8 + t * static_cast<int64_t>(p.V) * 8,
                                     static_cast<uint32_t>(p.V) * 8u);
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (y[j][e] * a) * f;
            buf_store_b64<OUT_AUX>(pack_e4m3x8(v), q_r, off[j] >> 1);
        }
        if (tid == 0) buf_store_b32<kAuxDefault>(qscale, make_rsrc(p.fp8_scale + t, 4u), 0u);
    }
}

// The rest of one token once its sum is formed in registers: s = (routed +
// shared) + residual (the dense tail: x + residual), residual_out, the row
// reduction behind one barrier (per-wave partials in red, 2 * MAX_WAVES
// floats of LDS) and the normalised outputs. acc holds the routed part on
// entry (ignored in the dense tail) and s after.
template <int VPT, int KT, int OUT_AUX, int QM>
__device__ __forceinline__ void finish_token(const Params& p, const int64_t t,
                                             float (&acc)[VPT][8], const u32x4 (&sh)[VPT],
                                             const u32x4 (&rs)[VPT], const u32x4 (&gm)[VPT],
                                             const uint32_t (&off)[VPT], float* red, Lds& lds) {
    const int tid = threadIdx.x;
    const int nt = threads_of<VPT>(p.V);
    const uint32_t rowbytes = static_cast<uint32_t>(p.V) * 16u;
    const int64_t trow = t * static_cast<int64_t>(p.V);
    constexpr bool DENSE = KT < 0;

    // s = (routed + shared) + residual (dense: x + residual); per-lane sum of
    // squares, and (FP8 modes) sg = s * gamma with its per-lane max |sg|. s
    // stays in registers. residual_out = bf16(s) is stored after the barrier,
    // next to the normalised output, which keeps the stores off the path to
    // the barrier; the dense tail with bf16 output, half of whose bytes are
    // writes, stores it before the barrier instead (each choice measured the
    // faster for its variant on MI355X).
    constexpr bool EARLY_RO = DENSE && QM == kOutBf16;
    const rsrc_t ro_r = make_rsrc(p.residual_out + trow, rowbytes);
    float ss = 0.0f;
    float mg = 0.0f;
    float sg[VPT][8];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if constexpr (DENSE)
                acc[j][e] = vec_elem(sh[j], e) + vec_elem(rs[j], e);
            else
                acc[j][e] = (acc[j][e] + vec_elem(sh[j], e)) + vec_elem(rs[j], e);
            ss = __builtin_fmaf(acc[j][e], acc[j][e], ss);
            if (QM != kOutBf16) {
                sg[j][e] = acc[j][e] * vec_elem(gm[j], e);
                mg = __builtin_fmaxf(mg, __builtin_fabsf(sg[j][e]));
            }
        }
        if constexpr (EARLY_RO) {
            u32x4 o;
            o.x = pack_bf16x2(acc[j][0], acc[j][1]);
            o.y = pack_bf16x2(acc[j][2], acc[j][3]);
            o.z = pack_bf16x2(acc[j][4], acc[j][5]);
            o.w = pack_bf16x2(acc[j][6], acc[j][7]);
            buf_store<OUT_AUX>(o, ro_r, off[j]);
        }
    }

    // Row reduction: wave tree, then the waves' partial sums in order. The FP8
    // modes reduce max |s * gamma| alongside, through the same exchange and
    // barrier: since rstd > 0, max |y| = rstd * max |s * gamma|.
    // The slots of waves the workgroup does not have are set to +0 before the
    // barrier, so that afterwards every thread reads all MAX_WAVES slots at
    // once (one LDS round trip, no loop) and folds them in wave order. Every
    // partial is +0 or more (or NaN), so adding the +0 slots and taking their
    // max changes neither result.
    const float wsum = wave_sum(ss);
    const float wmg = QM != kOutBf16 ? wave_max(mg) : 0.0f;
    const int nw = nt >> 6;
    if ((tid & 63) == 0) {
        red[tid >> 6] = wsum;
        if (QM != kOutBf16) red[MAX_WAVES + (tid >> 6)] = wmg;
    }
    if (tid >= nw && tid < MAX_WAVES) {
        red[tid] = 0.0f;
        if (QM != kOutBf16) red[MAX_WAVES + tid] = 0.0f;
    }
    __syncthreads();
    constexpr int NRED = QM != kOutBf16 ? 2 * MAX_WAVES : MAX_WAVES;
    float part[NRED];
#pragma unroll
    for (int w = 0; w < NRED; ++w) part[w] = red[w];
    __builtin_amdgcn_sched_barrier(0);  // all slot reads in flight before the first use
    float tot = 0.0f;
#pragma unroll
    for (int w = 0; w < MAX_WAVES; ++w) tot += part[w];
    float rmg = 0.0f;
#pragma unroll
    for (int w = MAX_WAVES; w < NRED; ++w) rmg = __builtin_fmaxf(rmg, part[w]);
    // the mean of squares as a product with the rounded 1/H: within an ulp
    // of the quotient, and a multiply instead of the division's sequence on
    // the path from the barrier to the stores
    const float ms_eps = tot * p.inv_h + p.eps;

    // residual_out = bf16(s), one rounding
    if constexpr (!EARLY_RO) {
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            u32x4 o;
            o.x = pack_bf16x2(acc[j][0], acc[j][1]);
            o.y = pack_bf16x2(acc[j][2], acc[j][3]);
            o.z = pack_bf16x2(acc[j][4], acc[j][5]);
            o.w = pack_bf16x2(acc[j][6], acc[j][7]);
            buf_store<OUT_AUX>(o, ro_r, off[j]);
        }
    }

    // Outside the fp32 range of the sum of squares (or, FP8 modes, of
    // s * gamma), the row is normalised in fp64 instead. NaN lands there too
    // and stays NaN.
    bool wide = !(ms_eps >= kRescueBelow && ms_eps <= kFltMax);
    if (QM != kOutBf16) wide = wide || !(rmg <= kFltMax);
    if (wide) {
        normalise_wide<VPT, OUT_AUX, QM>(p, t, acc, off, lds);
        return;
    }
    // ms_eps is a normal number here, which v_rsq_f32 takes as it is
    const float rstd = __builtin_amdgcn_rsqf(ms_eps);

    if (QM != kOutFp8) {
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
            buf_store<OUT_AUX>(o, no_r, off[j]);
        }
    }

    if (QM != kOutBf16) {
        // Dynamic per-token FP8: amax = max |y| = rstd * max |sg|, scale =
        // amax / 448, codes = E4M3(y * 448 / amax). Since rstd > 0 is common
        // to y and amax, y * 448 / amax = sg * (448 / max |sg|): one multiply
        // per element, with no rstd in it.
        //   * The factor (e4m3_factor) is a reciprocal shrunk by 2^-21, so
        //     that max |sg| times it stays below 448: no element can pass 448
        //     and the conversion needs no clamp. The scale is amax times the
        //     rounded 1/448. Both are within 2^-20 of the quotients, and
        //     neither puts a division between the barrier and the stores.
        //   * Rows with max |sg| < 2^-100, whose factor could overflow, are
        //     scaled by 2^64 first (exact).
        //   * A row with amax = 0, or rstd NaN, 0 or infinite, keeps the
        //     direct form y * 0: codes 0, or NaN where y is NaN; scale 1.
        // NaN elements (a NaN gamma) stay NaN; the conversion maps them to
        // the NaN code.
        const float rmax = rmg * rstd;
        const bool zero_row = !(rmax > 0.0f);
        const float qscale = zero_row ? 1.0f : rmax * kInvE4m3Max;
        const rsrc_t q_r = make_rsrc(p.normed_fp8 + t * static_cast<int64_t>(p.V) * 8,
                                     static_cast<uint32_t>(p.V) * 8u);
        if (!zero_row && rmg >= 0x1p-100f) {
            const float f = e4m3_factor(rmg);
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = sg[j][e] * f;
                buf_store_b64<OUT_AUX>(pack_e4m3x8(v), q_r, off[j] >> 1);
            }
        } else {
            const float a = zero_row ? rstd : 0x1p64f;
            const float b = zero_row ? 0.0f : e4m3_factor(rmg * 0x1p64f);
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = (sg[j][e] * a) * b;
                buf_store_b64<OUT_AUX>(pack_e4m3x8(v), q_r, off[j] >> 1);
            }
        }
        if (tid == 0) {
            const rsrc_t s_r = make_rsrc(p.fp8_scale + t, 4u);
            buf_store_b32<kAuxDefault>(qscale, s_r, 0u);
        }
    }
}

// One token, end to end. KT: 8 = exactly eight slots (the GLM-5.x / DeepSeek
// top-8 case, no slot-count checks); 0 = any K in 1..16, as one or two
// chunks of eight; -1 = no routed part (the dense residual add + RMSNorm:
// shared_out holds x and s = x + residual). Thread i owns the byte offsets 16*(i + j*NT), j < VPT, of
// every row; offsets at or past the row end (a ragged last tile) fall outside
// the descriptors' range, so their loads return zero and their stores are
// dropped by the hardware.
template <int VPT, int KT, int OUT_AUX, int QM, bool ROWS>
__device__ __forceinline__ void finalize_token(const Params& p, const int64_t t, Lds& lds) {
    const int tid = threadIdx.x;
    const int nt = threads_of<VPT>(p.V);
    const uint32_t rowbytes = static_cast<uint32_t>(p.V) * 16u;
    const int64_t trow = t * static_cast<int64_t>(p.V);

    uint32_t off[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) off[j] = static_cast<uint32_t>(tid + j * nt) * 16u;

    // The routing metadata (scalar loads) and the loads that do not depend on
    // it (shared, residual, gamma) are all in flight before anything that
    // waits for the metadata; in the machine code the vector loads go out
    // first, then the metadata. The scheduling barrier keeps the compiler
    // from sinking those independent loads below the metadata wait, so every
    // workgroup starts streaming HBM one memory latency earlier.
    constexpr bool DENSE = KT < 0;
    constexpr bool CHECK_K = KT != 8;
    const int32_t* prow = p.perm_idx + t * p.K;
    const float* wrow = p.topk_w + t * p.K;
    int32_t idx[8];
    float wr[8];
    if constexpr (!DENSE) load_meta8<CHECK_K>(p, prow, wrow, 0, idx, wr);

    const rsrc_t sh_r = make_rsrc(p.shared_out + trow, rowbytes);
    const rsrc_t rs_r = make_rsrc(p.residual + trow, rowbytes);
    const rsrc_t gm_r = make_rsrc(p.gamma, rowbytes);
    u32x4 sh[VPT], rs[VPT], gm[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        sh[j] = buf_load<kAuxActIn>(sh_r, off[j]);
        rs[j] = buf_load<kAuxActIn>(rs_r, off[j]);
        gm[j] = buf_load<kAuxGamma>(gm_r, off[j]);
    }
    __builtin_amdgcn_sched_barrier(0);

    float acc[VPT][8];
#pragma unroll
    for (int j = 0; j < VPT; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = 0.0f;

    if constexpr (!DENSE) {
        bool past_r = gather_rows8<VPT, CHECK_K, ROWS>(p, idx, wr, 0, off, acc);
        if (CHECK_K && p.K > 8) {
            load_meta8<true>(p, prow, wrow, 8, idx, wr);
            past_r |= gather_rows8<VPT, true, ROWS>(p, idx, wr, 8, off, acc);
        }
        // Report an index past the rows (its slot was treated as masked).
        // Every workgroup that sees one writes the same value, so there is
        // no race on the result.
        if (ROWS && past_r && p.bad_index != nullptr && tid == 0)
            buf_store_u32<kAuxDefault>(1u, make_rsrc(p.bad_index, 4u), 0u);
    }

    finish_token<VPT, KT, OUT_AUX, QM>(p, t, acc, sh, rs, gm, off, lds.red, lds);
}

// Launch bound per vectors-per-thread: keeps the register budget large enough
// that the row vectors in flight never spill.
template <int VPT>
struct Bound {
    static constexpr int kThreads = VPT == 1 ? 1024 : 512;
};

// Token of workgroup b. The hardware hands a dispatch's workgroups to the 8
// XCDs in turn (b to XCD b mod 8), so token b is the default (G = 0). Given
// the grid size G instead, XCD x takes the contiguous tokens from
// x*q + min(x, r) on (q = G / 8, r = G mod 8: the first r XCDs take q + 1
// tokens, the others q). Both maps are bijections of [0, G) for any G,
// whatever the XCD count, so only the placement changes.
__device__ __forceinline__ uint32_t token_of(uint32_t b, uint32_t G) {
    if (G == 0) return b;
    const uint32_t q = G >> 3, r = G & 7u, x = b & 7u, i = b >> 3;
    return x * q + (x < r ? x : r) + i;
}

// One workgroup per token. OUT_AUX is the cache policy of the output stores
// (write-back, or write-through for outputs larger than the L2); QM the
// OutMode of the normalised output.
//
// The pointers and sizes the first loads need come as separate leading
// arguments, ahead of the Params block: built with kernel-argument preload,
// the dispatcher places them in SGPRs when the wave launches, so the routing
// metadata load starts at once instead of behind a scalar load of the
// argument block. The values are the same as in p; p's copies are replaced.
// Preloading covers 14 dwords: the six pointers, V and K packed into one
// (vk = V | K << 16; V <= 2048, K <= 16), and xcd_grid (0, or the grid size
// for the per-XCD token ranges of token_of), which the token index, and so
// the first load, depends on.
template <int VPT, int KT, int OUT_AUX, int QM, bool ROWS = false>
__global__ __launch_bounds__(Bound<VPT>::kThreads) void mfr_fused_kernel(
        const int32_t* perm_idx, const float* topk_w, const u32x4* shared_out,
        const u32x4* residual, const u32x4* gamma, const u32x4* expert_out, uint32_t vk,
        uint32_t xcd_grid, Params p) {
    // Per-wave partial results of the row reductions; 16-byte aligned for vector reads.
    __shared__ __align__(16) Lds lds;
    // Built field by field: each field of p is then a scalar load of its
    // own, made only where the kernel uses it, rather than part of a copy of
    // the whole block (whose wide loads would also fill registers with
    // fields never used, and reusing those registers early would wait for
    // the load).
    Params q;
    q.perm_idx = perm_idx;
    q.topk_w = topk_w;
    q.shared_out = shared_out;
    q.residual = residual;
    q.gamma = gamma;
    q.expert_out = expert_out;
    q.V = static_cast<int>(vk & 0xFFFFu);
    q.K = static_cast<int>(vk >> 16);
    q.residual_out = p.residual_out;
    q.normed_out = p.normed_out;
    q.T = p.T;
    q.eps = p.eps;
    q.scale = p.scale;
    q.inv_h = p.inv_h;
    q.rows = p.rows;
    q.normed_fp8 = p.normed_fp8;
    q.fp8_scale = p.fp8_scale;
    q.bad_index = p.bad_index;
    const uint32_t t = token_of(blockIdx.x, xcd_grid);
    finalize_token<VPT, KT, OUT_AUX, QM, ROWS>(q, static_cast<int64_t>(t), lds);
}


// ---------------------------------------------------------------------------
// Persistent multi-token path (large T): a grid sized to the GPU's resident
// capacity, each workgroup walking the tokens blockIdx.x, blockIdx.x + G,
// blockIdx.x + 2G, ... (G = gridDim.x), one 16-byte vector per thread per row.
// Software-pipelined over two register buffers: the next token's K row loads
// and its shared and residual loads are issued before the current token is
// reduced, normalised and stored, so each workgroup keeps a token's reads in
// flight while it finishes the previous one (the page's fix gathers the
// routes of a token together; here the gather of the next token also
// overlaps the tail of the current one: vLLM pull request #62174,
// Validation). The two buffers keep fixed roles in a loop unrolled by two, so
// no register holding a load in flight is ever copied. A step past the last
// token issues its loads through zero-record descriptors (no memory access),
// so every path through the loop issues the same instructions and the load
// counters stay exact. The reduction slots in LDS alternate between two sets
// by token parity: one barrier per token then suffices, because a wave
// writes a slot set again only after every wave has passed the next barrier,
// and so has read it.
// ---------------------------------------------------------------------------

// At most 768 threads (12 waves, 3 per SIMD), so that the two register
// buffers fit in the 168 VGPRs a wave may then hold: H up to 6144.
constexpr int kPersistMaxThreads = 768;

struct LdsPersist {
    Lds lds;                     // even tokens' slots (lds.red), the range-rescue slots
    float red_b[2 * MAX_WAVES];  // odd tokens' slots
};

// Issues every load of token t that depends on no reduction: shared and
// residual rows, then (routed kernels) the K <= 8 gathered rows, all in
// flight on return. live = false loads nothing (zero-record descriptors; t
// is then any valid token, only used to form addresses).
template <int KT, bool ROWS>
__device__ __forceinline__ bool issue_token(const Params& p, const int64_t t, const bool live,
                                            const int32_t (&idx)[8], const float (&wr)[8],
                                            const uint32_t (&off)[1], u32x4 (&r)[8][1],
                                            float (&w)[8], u32x4 (&sh)[1], u32x4 (&rs)[1]) {
    const uint32_t rowbytes = static_cast<uint32_t>(p.V) * 16u;
    const int64_t trow = t * static_cast<int64_t>(p.V);
    sh[0] = buf_load<kAuxActIn>(make_rsrc(p.shared_out + trow, live ? rowbytes : 0u), off[0]);
    rs[0] = buf_load<kAuxActIn>(make_rsrc(p.residual + trow, live ? rowbytes : 0u), off[0]);
    if constexpr (KT >= 0)
        return issue_rows8<1, KT != 8, ROWS>(p, idx, wr, 0, off, r, w, live);
    return false;
}

// The routing metadata of token t (clamped to the last token: a step past
// the end reads a valid row of perm_idx and topk_w and uses none of it).
template <int KT>
__device__ __forceinline__ void persist_meta(const Params& p, int64_t t, int32_t (&idx)[8],
                                             float (&wr)[8]) {
    if constexpr (KT >= 0) {
        if (t >= p.T) t = p.T - 1;
        load_meta8<KT != 8>(p, p.perm_idx + t * p.K, p.topk_w + t * p.K, 0, idx, wr);
    }
}

template <int KT, int OUT_AUX, int QM>
__device__ __forceinline__ void persist_finish(const Params& p, const int64_t t,
                                               const u32x4 (&r)[8][1], const float (&w)[8],
                                               const u32x4 (&sh)[1], const u32x4 (&rs)[1],
                                               const u32x4 (&gm)[1], const uint32_t (&off)[1],
                                               float* red, Lds& lds) {
    float acc[1][8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[0][e] = 0.0f;
    if constexpr (KT >= 0) fold_rows8<1>(r, w, acc);
    finish_token<1, KT, OUT_AUX, QM>(p, t, acc, sh, rs, gm, off, red, lds);
}

// KT: 8 or 0 (any K <= 8: the host routes K > 8 elsewhere) or -1 (dense).
// The grid is at most T workgroups, so every workgroup's first token exists.
template <int KT, int OUT_AUX, int QM, bool ROWS = false>
__global__ __launch_bounds__(kPersistMaxThreads) void mfr_persist_kernel(
        const int32_t* perm_idx, const float* topk_w, const u32x4* shared_out,
        const u32x4* residual, const u32x4* gamma, const u32x4* expert_out, int V, int K,
        Params p) {
    __shared__ __align__(16) LdsPersist L;
    p.perm_idx = perm_idx;
    p.topk_w = topk_w;
    p.shared_out = shared_out;
    p.residual = residual;
    p.gamma = gamma;
    p.expert_out = expert_out;
    p.V = V;
    p.K = K;
    const uint32_t off[1] = {static_cast<uint32_t>(threadIdx.x) * 16u};
    const int64_t G = gridDim.x;
    int64_t t = blockIdx.x;

    int32_t idx[8];
    float wr[8];
    u32x4 ra[8][1], rb[8][1], sha[1], rsa[1], shb[1], rsb[1];
    float wa[8], wb[8];
    bool past_r = false;
    // gamma: one row for every token, loaded once
    const u32x4 gm[1] = {buf_load<kAuxGamma>(make_rsrc(p.gamma, static_cast<uint32_t>(V) * 16u),
                                             off[0])};
    persist_meta<KT>(p, t, idx, wr);
    past_r |= issue_token<KT, ROWS>(p, t, true, idx, wr, off, ra, wa, sha, rsa);
    persist_meta<KT>(p, t + G, idx, wr);
    for (;;) {
        // buffer B <- token t + G; finish token t from buffer A
        const int64_t tb = t + G;
        const bool lb = tb < p.T;
        past_r |= issue_token<KT, ROWS>(p, lb ? tb : t, lb, idx, wr, off, rb, wb, shb, rsb);
        persist_meta<KT>(p, tb + G, idx, wr);
        persist_finish<KT, OUT_AUX, QM>(p, t, ra, wa, sha, rsa, gm, off, L.lds.red, L.lds);
        if (!lb) break;
        t = tb;
        // buffer A <- token t + G; finish token t from buffer B
        const int64_t ta = t + G;
        const bool la = ta < p.T;
        past_r |= issue_token<KT, ROWS>(p, la ? ta : t, la, idx, wr, off, ra, wa, sha, rsa);
        persist_meta<KT>(p, ta + G, idx, wr);
        persist_finish<KT, OUT_AUX, QM>(p, t, rb, wb, shb, rsb, gm, off, L.red_b, L.lds);
        if (!la) break;
        t = ta;
    }
    // An index past the rows was treated as masked; report it (every
    // workgroup that saw one writes the same value).
    if (ROWS && past_r && p.bad_index != nullptr && threadIdx.x == 0)
        buf_store_u32<kAuxDefault>(1u, make_rsrc(p.bad_index, 4u), 0u);
}

}  // namespace mfr

// ---------------------------------------------------------------------------
// Host side: validation, launch shape, launch.
// ---------------------------------------------------------------------------
namespace {

constexpr int64_t kHMax = 16384;
constexpr int64_t kKMax = 16;
// V (= H / 8) and K travel packed in one 32-bit kernel argument.
static_assert(kHMax / 8 < (1 << 16) && kKMax < (1 << 16), "V and K must fit 16 bits each");
constexpr int64_t kTMax = 2147483647;
constexpr int kVptMax = 4;
// Row bound of the entry points that are not told R: 2^31, above every
// non-negative int32 index, so no slot is ever treated as past the rows.
constexpr uint32_t kNoRowBound = 0x80000000u;
// Token counts up to this use the token path (widest workgroup per token),
// that is below two tokens per CU on the 256 CUs of an MI355X. Measured there
// at H = 6144 (HBM-cold, every shape interleaved): the widest workgroup is
// 1-2.6% faster than the 256-thread stream shape from T = 257 to 368 and
// level with it, within the run-to-run spread, from 384 to 512; from T = 640
// the stream shape is ahead.
constexpr int64_t kTokenPathMaxT = 511;
// Output bytes (both outputs) above which the stores write through. Measured
// on MI355X at H = 6144 in three sweeps: write-back wins at T = 512 (12 MiB of
// outputs, which the 32 MB of L2 absorbs, every CU finishing its two tokens
// together), write-through from T = 513 up (3-5% at 513, 2-3% at 640, level at
// 768, 3-5% from 2048), where the grid's last tokens run alone and written-
// back outputs would wait in the L2 for the end of the kernel.
constexpr uint64_t kWriteThroughAboveBytes = 12ull << 20;
// Token counts up to which the token path writes its bf16 outputs through
// too. Measured on MI355X at H = 6144 (decode harnesses, interleaved): at
// T = 1 to 64 write-through is 0.6-3% faster for the fused op with fresh
// inputs, with the same inputs re-read and right after a producer wrote the
// rows, and level to 4% faster for the dense tail; at T = 128 write-back is
// 1-2% ahead. The same holds at H = 4096 and 7168 (HBM-cold sweeps, 1-2.5%
// at T = 1, 28 and 64). With one token per CU the call ends with every
// output line written; written-back lines would still be in the L2 then,
// waiting for the end of the kernel. The FP8 output (codes and a four-byte
// scale per token) is 0.1-3.5% slower written through, so it keeps
// write-back.
constexpr int64_t kTokenWriteThroughMaxT = 64;
// The stream path's 256-thread, 3-vector kernels of the fused op with bf16
// or FP8 output (3 workgroups per CU by their registers) run with at most
// kCapPerCu workgroups per CU from kCapMinT tokens on, for H above kCapMinH
// (up to 6144, where those kernels end). Measured on MI355X, every
// alternative interleaved, at H = 6144 in five sweeps: bf16 0.6-1.9% faster
// at T = 4096 and 8192, with one buffer set, with the Infinity Cache flushed
// before each call and with alternating outputs alike, level to 0.7% faster
// at 2048, and level at T = 512 and 1024; FP8 0.3-1.0% faster at T = 8192,
// level to 1.2% faster at 2048 and 4096. At H = 5120 (bf16) level or mixed
// (-1% to +2%) in four sweeps, so the rule stops above it. At H = 4096
// (another kernel, 7 per CU) and for the dense tail (8 per CU) a cap of 2
// was slower.
constexpr int64_t kCapMinT = 2048;
constexpr int64_t kCapMinH = 5120;
constexpr int kCapPerCu = 2;

// The calling thread's launch override (mfr_tuning_force_launch); 0 =
// automatic. Thread-local, so that one thread's override never changes the
// launch shape of another thread's call.
thread_local int t_force_path = 0;
thread_local int t_force_vpt = 0;
thread_local int t_force_store = 0;
thread_local int t_force_residency = 0;  // workgroups per CU (0 = automatic)
thread_local int t_force_order = 0;      // an mfr_token_order value

// Environment switches, read once when the library is loaded:
//   MFR_PATH=auto|token|stream|persist  default launch path (a thread's
//                               override set through mfr_tuning_force_launch
//                               takes precedence);
//   MFR_LOG=1                   one line on stderr per launch: shape, path,
//                               vectors per thread, threads, store policy.
// An unrecognised MFR_PATH value is reported on stderr and ignored.
int env_path() {
    const char* v = std::getenv("MFR_PATH");
    if (!v || !*v || std::strcmp(v, "auto") == 0) return 0;
    if (std::strcmp(v, "token") == 0) return MFR_PATH_TOKEN;
    if (std::strcmp(v, "stream") == 0) return MFR_PATH_STREAM;
    if (std::strcmp(v, "persist") == 0) return MFR_PATH_PERSIST;
    std::fprintf(stderr,
                 "moe_finalize_rmsnorm: ignoring MFR_PATH=%s (auto, token, stream or persist)\n", v);
    return 0;
}

bool env_log() {
    const char* v = std::getenv("MFR_LOG");
    return v && *v && std::strcmp(v, "0") != 0;
}

const int g_env_path = env_path();
const bool g_env_log = env_log();

int max_threads(int vpt) { return vpt == 1 ? 1024 : 512; }

int threads_for(int64_t V, int vpt) {
    int64_t n = (V + vpt - 1) / vpt;
    n = (n + 63) / 64 * 64;
    return static_cast<int>(n);
}

bool shape_ok(int64_t T, int64_t H, int64_t K) {
    return T >= 0 && T <= kTMax && H >= 8 && H <= kHMax && H % 8 == 0 && K >= 1 && K <= kKMax;
}

// The persistent path keeps one 16-byte vector per thread per row and at
// most eight gathered rows in each of its two register buffers: H up to 6144
// (768 threads) and K up to 8 (any K for the dense tail, which gathers
// nothing).
bool persist_ok(int64_t H, int64_t K) {
    return threads_for(H / 8, 1) <= mfr::kPersistMaxThreads && K <= 8;
}

// Launch path of a shape (K = 1 for the dense tail). A forced path that
// cannot serve the shape falls back to the automatic choice.
int choose_path(int64_t T, int64_t H, int64_t K) {
    int f = t_force_path;
    if (f == 0) f = g_env_path;
    if (f == MFR_PATH_PERSIST && !persist_ok(H, K)) f = 0;
    if (f == MFR_PATH_TOKEN || f == MFR_PATH_STREAM || f == MFR_PATH_PERSIST) return f;
    return T <= kTokenPathMaxT ? MFR_PATH_TOKEN : MFR_PATH_STREAM;
}

// Vectors per thread: the token path spreads a row over as many threads as
// possible (latency); the stream path uses at most 256 threads per token so
// that more tokens are resident per CU (bandwidth).
int choose_vpt(int path, int64_t V) {
    const int f = t_force_vpt;
    if (f >= 1 && f <= kVptMax && threads_for(V, f) <= max_threads(f)) return f;
    if (path == MFR_PATH_STREAM) {
        for (int v = 1; v <= kVptMax; ++v)
            if (threads_for(V, v) <= 256) return v;
    }
    for (int v = 1; v <= kVptMax; ++v)
        if (threads_for(V, v) <= max_threads(v)) return v;
    return kVptMax;
}

// Output store encodings: write-back, write-through (sc1), and the two
// non-temporal ones the tuning interface can force on the top-8 bf16 kernels
// of the grid paths.
enum Store { kStoreWb = 0, kStoreWt = 1, kStoreNt = 2, kStoreNtWt = 3 };

// Routing variant of a launch: exactly eight slots, any K, or no routed part;
// the checked forms also bound the indices by the rows of expert_out.
enum Variant { kTop8 = 8, kAnyK = 0, kDense = -1, kTop8Rows = 108, kAnyKRows = 100 };

// Names for the MFR_LOG lines.
const char* variant_name(Variant v) {
    switch (v) {
        case kTop8: return "top8";
        case kAnyK: return "anyK";
        case kTop8Rows: return "top8-rows";
        case kAnyKRows: return "anyK-rows";
        default: return "dense";
    }
}

const char* out_name(int qm) {
    return qm == mfr::kOutFp8 ? "fp8" : qm == mfr::kOutBoth ? "bf16+fp8" : "bf16";
}

const char* store_name(int st) {
    switch (st) {
        case kStoreWt: return "write-through";
        case kStoreNt: return "nt";
        case kStoreNtWt: return "nt-sc1";
        default: return "write-back";
    }
}

int store_policy(int path, int64_t T, int64_t H, Variant v, int qm) {
    const int f = t_force_store;
    if (f == MFR_STORE_WRITE_BACK) return kStoreWb;
    if (f == MFR_STORE_WRITE_THROUGH) return kStoreWt;
    if ((f == MFR_STORE_NONTEMPORAL || f == MFR_STORE_NONTEMPORAL_WRITE_THROUGH) && v == kTop8 &&
        qm == mfr::kOutBf16 && path != MFR_PATH_PERSIST)
        return f == MFR_STORE_NONTEMPORAL ? kStoreNt : kStoreNtWt;
    if (path == MFR_PATH_TOKEN)
        return T <= kTokenWriteThroughMaxT && qm == mfr::kOutBf16 ? kStoreWt : kStoreWb;
    return static_cast<uint64_t>(T) * H * 4 > kWriteThroughAboveBytes ? kStoreWt : kStoreWb;
}

bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
    const uint64_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return na > 0 && nb > 0 && a0 < b0 + nb && b0 < a0 + na;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

template <int VPT, int KT, int QM, bool ROWS = false>
const void* pick_store(int st) {
    if constexpr (KT == 8 && QM == mfr::kOutBf16 && !ROWS) {
        if (st == kStoreNt)
            return reinterpret_cast<const void*>(
                &mfr::mfr_fused_kernel<VPT, KT, mfr::kAuxOutNt, QM, ROWS>);
        if (st == kStoreNtWt)
            return reinterpret_cast<const void*>(
                &mfr::mfr_fused_kernel<VPT, KT, mfr::kAuxOutNtWriteThrough, QM, ROWS>);
    }
    return st == kStoreWt ? reinterpret_cast<const void*>(
                                &mfr::mfr_fused_kernel<VPT, KT, mfr::kAuxWriteThrough, QM, ROWS>)
                          : reinterpret_cast<const void*>(
                                &mfr::mfr_fused_kernel<VPT, KT, mfr::kAuxOut, QM, ROWS>);
}

template <int VPT, int QM>
const void* pick_variant(Variant v, int st) {
    switch (v) {
        case kTop8: return pick_store<VPT, 8, QM>(st);
        case kAnyK: return pick_store<VPT, 0, QM>(st);
        case kTop8Rows: return pick_store<VPT, 8, QM, true>(st);
        case kAnyKRows: return pick_store<VPT, 0, QM, true>(st);
        default: return pick_store<VPT, -1, QM>(st);
    }
}

template <int VPT>
const void* pick(Variant v, int st, int qm) {
    switch (qm) {
        case mfr::kOutFp8: return pick_variant<VPT, mfr::kOutFp8>(v, st);
        case mfr::kOutBoth: return pick_variant<VPT, mfr::kOutBoth>(v, st);
        default: return pick_variant<VPT, mfr::kOutBf16>(v, st);
    }
}

// Kernel address for (vectors per thread, routing variant, store encoding,
// output mode).
const void* kernel_for(int vpt, Variant v, int st, int qm) {
    switch (vpt) {
        case 1: return pick<1>(v, st, qm);
        case 2: return pick<2>(v, st, qm);
        case 3: return pick<3>(v, st, qm);
        default: return pick<4>(v, st, qm);
    }
}

template <int KT, int QM, bool ROWS = false>
const void* pick_persist_store(bool wt) {
    return wt ? reinterpret_cast<const void*>(
                    &mfr::mfr_persist_kernel<KT, mfr::kAuxWriteThrough, QM, ROWS>)
              : reinterpret_cast<const void*>(&mfr::mfr_persist_kernel<KT, mfr::kAuxOut, QM, ROWS>);
}

// The persistent kernel serves every call except the checked ones with FP8
// output: those need more registers than its 768-thread workgroups leave
// (they spilled), so they take the automatic path instead.
bool persist_serves(Variant v, int qm) {
    return qm == mfr::kOutBf16 || (v != kTop8Rows && v != kAnyKRows);
}

template <int QM>
const void* pick_persist_variant(Variant v, bool wt) {
    switch (v) {
        case kTop8: return pick_persist_store<8, QM>(wt);
        case kAnyK: return pick_persist_store<0, QM>(wt);
        case kTop8Rows:
            if constexpr (QM == mfr::kOutBf16) return pick_persist_store<8, QM, true>(wt);
            return nullptr;  // not served (persist_serves)
        case kAnyKRows:
            if constexpr (QM == mfr::kOutBf16) return pick_persist_store<0, QM, true>(wt);
            return nullptr;  // not served (persist_serves)
        default: return pick_persist_store<-1, QM>(wt);
    }
}

// Persistent kernel for (routing variant, write-through outputs, output mode).
const void* persist_kernel_for(Variant v, bool wt, int qm) {
    switch (qm) {
        case mfr::kOutFp8: return pick_persist_variant<mfr::kOutFp8>(v, wt);
        case mfr::kOutBoth: return pick_persist_variant<mfr::kOutBoth>(v, wt);
        default: return pick_persist_variant<mfr::kOutBf16>(v, wt);
    }
}

// Compute units of the calling thread's current device, queried once per
// device (the only state the library keeps besides the per-kernel residency
// below; both are filled on first use and never change).
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

int cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    std::atomic<int>* slot = dev < kMaxDevices ? &g_cus[dev] : nullptr;
    int n = slot ? slot->load(std::memory_order_relaxed) : 0;
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        return 1;
    if (slot) slot->store(n, std::memory_order_relaxed);
    return n;
}

// Workgroups of nt threads of one kernel that fit on a CU at once (from the
// kernel's register and LDS use), queried once per (kernel, nt, device).
struct Residency {
    const void* kern;
    int nt, dev;
    int per_cu;
};
std::mutex g_res_mu;
Residency g_res[512];
int g_res_n = 0;

int resident_per_cu(const void* kern, int nt) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    std::lock_guard<std::mutex> lock(g_res_mu);
    for (int i = 0; i < g_res_n; ++i)
        if (g_res[i].kern == kern && g_res[i].nt == nt && g_res[i].dev == dev)
            return g_res[i].per_cu;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, nt, 0) != hipSuccess || n <= 0)
        return 1;
    if (g_res_n < 512) g_res[g_res_n++] = {kern, nt, dev, n};
    return n;
}

// Dynamic LDS for a grid-path launch of kern (nt threads) that leaves room
// for at most n of its workgroups on a CU: the smallest multiple of 512 bytes
// above an (n+1)-th of the CU's LDS, less the kernel's own. 0 (no
// reservation) where the kernel's registers already allow no more than n, or
// where no such size gives exactly n, as the occupancy query reports it.
// Computed once per (kernel, threads, n) and device.
struct LdsCap {
    const void* kern;
    int nt, n, dev;
    size_t bytes;
};
std::mutex g_cap_mu;
LdsCap g_cap[256];
int g_cap_n = 0;

size_t lds_for_residency_uncached(const void* kern, int nt, int n);

size_t lds_for_residency(const void* kern, int nt, int n) {
    if (n <= 0) return 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(g_cap_mu);
    for (int i = 0; i < g_cap_n; ++i)
        if (g_cap[i].kern == kern && g_cap[i].nt == nt && g_cap[i].n == n && g_cap[i].dev == dev)
            return g_cap[i].bytes;
    const size_t b = lds_for_residency_uncached(kern, nt, n);
    if (g_cap_n < 256) g_cap[g_cap_n++] = {kern, nt, n, dev, b};
    return b;
}

size_t lds_for_residency_uncached(const void* kern, int nt, int n) {
    if (resident_per_cu(kern, nt) <= n) return 0;
    int dev = 0, per_cu = 0, per_block = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
            hipSuccess ||
        hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess)
        return 0;
    hipFuncAttributes a;
    if (hipFuncGetAttributes(&a, kern) != hipSuccess) return 0;
    const size_t total = (static_cast<size_t>(per_cu) / (n + 1) / 512 + 1) * 512;
    if (total <= a.sharedSizeBytes || total > static_cast<size_t>(per_block)) return 0;
    const size_t dyn = total - a.sharedSizeBytes;
    int got = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&got, kern, nt, dyn) != hipSuccess ||
        got != n)
        return 0;
    return dyn;
}

// Aliasing rule shared by the entry points: no output may overlap another
// output or any input, except that residual_out may be exactly residual (the
// in-place residual update). Extents are in bytes; an empty extent never
// overlaps.
struct Extent {
    const void* p;
    uint64_t n;
};

int check_aliasing(const Extent* outs, int n_out, const Extent* ins, int n_in,
                   const void* residual_out, const void* residual) {
    for (int i = 0; i < n_out; ++i) {
        for (int j = i + 1; j < n_out; ++j)
            if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return MFR_ERR_ALIAS;
        for (int j = 0; j < n_in; ++j) {
            const bool in_place = outs[i].p == residual_out && ins[j].p == residual &&
                                  residual_out == residual && outs[i].n == ins[j].n;
            if (!in_place && overlaps(outs[i].p, outs[i].n, ins[j].p, ins[j].n)) return MFR_ERR_ALIAS;
        }
    }
    return MFR_OK;
}

// The work-item count of one dispatch (workgroups x threads per workgroup) is
// a 32-bit quantity on this hardware, so a launch of T workgroups of nt
// threads holds at most this many tokens; more are split over several
// dispatches.
int64_t tokens_per_dispatch(int nt) {
    return static_cast<int64_t>(0xFFFFFFFFu / static_cast<uint32_t>(nt));
}

// p with every per-token pointer moved to token t0, so that a dispatch whose
// workgroup 0 is token t0 addresses the same bytes as workgroup t0 of one
// undivided grid. expert_out (addressed through the indices), gamma and the
// report flag are shared by all tokens and stay as they are.
mfr::Params from_token(const mfr::Params& p, int64_t t0) {
    mfr::Params q = p;
    const int64_t vec = t0 * p.V;  // 16-byte vectors before token t0 in a [T, H] bf16 tensor
    if (p.perm_idx) q.perm_idx = p.perm_idx + t0 * p.K;
    if (p.topk_w) q.topk_w = p.topk_w + t0 * p.K;
    q.shared_out = p.shared_out + vec;
    q.residual = p.residual + vec;
    q.residual_out = p.residual_out + vec;
    if (p.normed_out) q.normed_out = p.normed_out + vec;
    if (p.normed_fp8) q.normed_fp8 = p.normed_fp8 + vec * 8;  // one byte per element
    if (p.fp8_scale) q.fp8_scale = p.fp8_scale + t0;
    return q;
}

// Fills the shape fields, picks the launch shape and enqueues the kernel: one
// dispatch, or several in stream order when T x threads needs more than 32
// bits. Every token's arithmetic is the same in any dispatch, so the split
// changes no result.
int launch(mfr::Params& p, int64_t T, int64_t H, Variant v, int qm, hipStream_t stream) {
    p.T = T;
    p.inv_h = 1.0f / static_cast<float>(H);
    p.V = static_cast<int>(H / 8);
    int path = choose_path(T, H, v == kDense ? 1 : p.K);
    if (path == MFR_PATH_PERSIST && !persist_serves(v, qm))
        path = T <= kTokenPathMaxT ? MFR_PATH_TOKEN : MFR_PATH_STREAM;
    const int st = store_policy(path, T, H, v, qm);
    const bool wt = st == kStoreWt;
    if (path == MFR_PATH_PERSIST) {
        // one launch, a grid of at most T workgroups sized to what the GPU
        // holds at once; each workgroup walks its tokens
        const int nt = threads_for(p.V, 1);
        const void* kern = persist_kernel_for(v, wt, qm);
        int per_cu = resident_per_cu(kern, nt);
        if (t_force_residency > 0 && t_force_residency < per_cu) per_cu = t_force_residency;
        const int64_t cap = static_cast<int64_t>(cu_count()) * per_cu;
        const int64_t grid = T < cap ? T : cap;
        if (g_env_log)
            std::fprintf(stderr,
                         "moe_finalize_rmsnorm: T=%lld H=%lld K=%d variant=%s out=%s path=persist "
                         "vpt=1 threads=%d stores=%s workgroups=%lld\n",
                         static_cast<long long>(T), static_cast<long long>(H), p.K,
                         variant_name(v), out_name(qm), nt, store_name(st),
                         static_cast<long long>(grid));
        void* args[] = {&p.perm_idx, &p.topk_w, &p.shared_out, &p.residual, &p.gamma,
                        &p.expert_out, &p.V, &p.K, &p};
        const hipError_t e =
            hipLaunchKernel(kern, dim3(static_cast<uint32_t>(grid)), dim3(nt), args, 0, stream);
        return e == hipSuccess ? MFR_OK : MFR_ERR_HIP;
    }
    const int vpt = choose_vpt(path, p.V);
    const int nt = threads_for(p.V, vpt);
    const void* kern = kernel_for(vpt, v, st, qm);
    const int64_t per = tokens_per_dispatch(nt);
    // Workgroups per CU, capped through reserved LDS: the tuning override,
    // else the automatic cap of the 3-vector bf16 and FP8 stream kernels at
    // large T.
    int cap = t_force_residency;
    if (cap == 0 && path == MFR_PATH_STREAM && vpt == 3 && qm != mfr::kOutBoth && v != kDense &&
        T >= kCapMinT && H > kCapMinH)
        cap = kCapPerCu;
    const size_t lds = lds_for_residency(kern, nt, cap);
    // tuning only: the per-XCD token ranges
    const bool xcd_ranges = t_force_order == MFR_ORDER_XCD_RANGES;
    if (g_env_log)
        std::fprintf(stderr,
                     "moe_finalize_rmsnorm: T=%lld H=%lld K=%d variant=%s out=%s path=%s vpt=%d "
                     "threads=%d stores=%s dispatches=%lld reserved_lds=%zu order=%s\n",
                     static_cast<long long>(T), static_cast<long long>(H), p.K, variant_name(v),
                     out_name(qm), path == MFR_PATH_TOKEN ? "token" : "stream", vpt, nt,
                     store_name(st), static_cast<long long>((T + per - 1) / per), lds,
                     xcd_ranges ? "xcd-ranges" : "default");
    for (int64_t t0 = 0; t0 < T; t0 += per) {
        const int64_t n = T - t0 < per ? T - t0 : per;
        mfr::Params q = t0 == 0 ? p : from_token(p, t0);
        q.T = n;
        uint32_t vk = static_cast<uint32_t>(q.V) | static_cast<uint32_t>(q.K) << 16;
        uint32_t xcd_grid = xcd_ranges ? static_cast<uint32_t>(n) : 0u;
        void* args[] = {&q.perm_idx, &q.topk_w, &q.shared_out, &q.residual, &q.gamma,
                        &q.expert_out, &vk, &xcd_grid, &q};
        const hipError_t e =
            hipLaunchKernel(kern, dim3(static_cast<uint32_t>(n)), dim3(nt), args, lds, stream);
        if (e != hipSuccess) return MFR_ERR_HIP;
    }
    return MFR_OK;
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
    // expert_out's extent is unknown (R is not passed): only its first 16
    // bytes are checked.
    const Extent outs[] = {{residual_out, act}, {normed_out, act}};
    const Extent ins[] = {{residual, act}, {shared_out, act}, {gamma, static_cast<uint64_t>(H) * 2},
                          {perm_idx, meta}, {topk_w, meta}, {expert_out, 16}};
    const int rc = check_aliasing(outs, 2, ins, 6, residual_out, residual);
    if (rc != MFR_OK) return rc;

    mfr::Params p = {};
    p.expert_out = reinterpret_cast<const mfr::u32x4*>(expert_out);
    p.perm_idx = perm_idx;
    p.topk_w = topk_w;
    p.shared_out = reinterpret_cast<const mfr::u32x4*>(shared_out);
    p.residual = reinterpret_cast<const mfr::u32x4*>(residual);
    p.gamma = reinterpret_cast<const mfr::u32x4*>(gamma);
    p.residual_out = reinterpret_cast<mfr::u32x4*>(residual_out);
    p.normed_out = reinterpret_cast<mfr::u32x4*>(normed_out);
    p.eps = eps;
    p.scale = scale;
    p.K = static_cast<int>(K);
    p.rows = kNoRowBound;
    return launch(p, T, H, K == 8 ? kTop8 : kAnyK, mfr::kOutBf16, stream);
}

int moe_finalize_rmsnorm_checked(const uint16_t* expert_out, int64_t R, const int32_t* perm_idx,
                                 const float* topk_w, const uint16_t* shared_out,
                                 const uint16_t* residual, const uint16_t* gamma, float eps,
                                 float scale, uint16_t* residual_out, uint16_t* normed_out,
                                 int32_t* bad_index, int64_t T, int64_t H, int64_t K,
                                 hipStream_t stream) {
    if (!shape_ok(T, H, K) || R < 0) return MFR_ERR_SHAPE;
    if (!(eps >= 0.0f) || !std::isfinite(eps) || !std::isfinite(scale)) return MFR_ERR_SCALAR;
    if (T == 0) return MFR_OK;
    // int32 indices address at most 2^31 rows: a larger R means the same.
    if (R > (int64_t{1} << 31)) R = int64_t{1} << 31;
    if (!perm_idx || !topk_w || !shared_out || !residual || !gamma || !residual_out ||
        !normed_out || (R > 0 && !expert_out))
        return MFR_ERR_NULL;
    if (!aligned(expert_out, 16) || !aligned(shared_out, 16) || !aligned(residual, 16) ||
        !aligned(gamma, 16) || !aligned(residual_out, 16) || !aligned(normed_out, 16) ||
        !aligned(perm_idx, 4) || !aligned(topk_w, 4) || (bad_index && !aligned(bad_index, 4)))
        return MFR_ERR_ALIGN;
    const uint64_t act = static_cast<uint64_t>(T) * H * 2;
    const uint64_t meta = static_cast<uint64_t>(T) * K * 4;
    // With R known, the whole of expert_out takes part in the overlap check.
    const Extent outs[] = {{residual_out, act}, {normed_out, act}, {bad_index, bad_index ? 4u : 0u}};
    const Extent ins[] = {{residual, act}, {shared_out, act}, {gamma, static_cast<uint64_t>(H) * 2},
                          {perm_idx, meta}, {topk_w, meta},
                          {expert_out, static_cast<uint64_t>(R) * static_cast<uint64_t>(H) * 2}};
    const int rc = check_aliasing(outs, 3, ins, 6, residual_out, residual);
    if (rc != MFR_OK) return rc;

    mfr::Params p = {};
    p.expert_out = reinterpret_cast<const mfr::u32x4*>(expert_out);
    p.perm_idx = perm_idx;
    p.topk_w = topk_w;
    p.shared_out = reinterpret_cast<const mfr::u32x4*>(shared_out);
    p.residual = reinterpret_cast<const mfr::u32x4*>(residual);
    p.gamma = reinterpret_cast<const mfr::u32x4*>(gamma);
    p.residual_out = reinterpret_cast<mfr::u32x4*>(residual_out);
    p.normed_out = reinterpret_cast<mfr::u32x4*>(normed_out);
    p.eps = eps;
    p.scale = scale;
    p.K = static_cast<int>(K);
    p.rows = static_cast<uint32_t>(R);
    p.bad_index = bad_index;
    return launch(p, T, H, K == 8 ? kTop8Rows : kAnyKRows, mfr::kOutBf16, stream);
}

int moe_finalize_rmsnorm_fp8(const uint16_t* expert_out, const int32_t* perm_idx,
                             const float* topk_w, const uint16_t* shared_out,
                             const uint16_t* residual, const uint16_t* gamma, float eps,
                             float scale, uint16_t* residual_out, uint16_t* normed_out,
                             uint8_t* normed_fp8, float* fp8_scale, int64_t T, int64_t H,
                             int64_t K, hipStream_t stream) {
    if (!shape_ok(T, H, K)) return MFR_ERR_SHAPE;
    if (!(eps >= 0.0f) || !std::isfinite(eps) || !std::isfinite(scale)) return MFR_ERR_SCALAR;
    if (T == 0) return MFR_OK;
    if (!expert_out || !perm_idx || !topk_w || !shared_out || !residual || !gamma ||
        !residual_out || !normed_fp8 || !fp8_scale)
        return MFR_ERR_NULL;
    if (!aligned(expert_out, 16) || !aligned(shared_out, 16) || !aligned(residual, 16) ||
        !aligned(gamma, 16) || !aligned(residual_out, 16) ||
        (normed_out && !aligned(normed_out, 16)) || !aligned(normed_fp8, 8) ||
        !aligned(fp8_scale, 4) || !aligned(perm_idx, 4) || !aligned(topk_w, 4))
        return MFR_ERR_ALIGN;
    const uint64_t act = static_cast<uint64_t>(T) * H * 2;
    const uint64_t meta = static_cast<uint64_t>(T) * K * 4;
    const Extent outs[] = {{residual_out, act},
                           {normed_fp8, static_cast<uint64_t>(T) * H},
                           {fp8_scale, static_cast<uint64_t>(T) * 4},
                           {normed_out, normed_out ? act : 0}};
    const Extent ins[] = {{residual, act}, {shared_out, act}, {gamma, static_cast<uint64_t>(H) * 2},
                          {perm_idx, meta}, {topk_w, meta}, {expert_out, 16}};
    const int rc = check_aliasing(outs, 4, ins, 6, residual_out, residual);
    if (rc != MFR_OK) return rc;

    mfr::Params p = {};
    p.expert_out = reinterpret_cast<const mfr::u32x4*>(expert_out);
    p.perm_idx = perm_idx;
    p.topk_w = topk_w;
    p.shared_out = reinterpret_cast<const mfr::u32x4*>(shared_out);
    p.residual = reinterpret_cast<const mfr::u32x4*>(residual);
    p.gamma = reinterpret_cast<const mfr::u32x4*>(gamma);
    p.residual_out = reinterpret_cast<mfr::u32x4*>(residual_out);
    p.normed_out = reinterpret_cast<mfr::u32x4*>(normed_out);
    p.normed_fp8 = normed_fp8;
    p.fp8_scale = fp8_scale;
    p.eps = eps;
    p.scale = scale;
    p.K = static_cast<int>(K);
    p.rows = kNoRowBound;
    return launch(p, T, H, K == 8 ? kTop8 : kAnyK, normed_out ? mfr::kOutBoth : mfr::kOutFp8,
                  stream);
}

int moe_finalize_rmsnorm_fp8_checked(const uint16_t* expert_out, int64_t R,
                                     const int32_t* perm_idx, const float* topk_w,
                                     const uint16_t* shared_out, const uint16_t* residual,
                                     const uint16_t* gamma, float eps, float scale,
                                     uint16_t* residual_out, uint16_t* normed_out,
                                     uint8_t* normed_fp8, float* fp8_scale, int32_t* bad_index,
                                     int64_t T, int64_t H, int64_t K, hipStream_t stream) {
    if (!shape_ok(T, H, K) || R < 0) return MFR_ERR_SHAPE;
    if (!(eps >= 0.0f) || !std::isfinite(eps) || !std::isfinite(scale)) return MFR_ERR_SCALAR;
    if (T == 0) return MFR_OK;
    if (R > (int64_t{1} << 31)) R = int64_t{1} << 31;
    if (!perm_idx || !topk_w || !shared_out || !residual || !gamma || !residual_out ||
        !normed_fp8 || !fp8_scale || (R > 0 && !expert_out))
        return MFR_ERR_NULL;
    if (!aligned(expert_out, 16) || !aligned(shared_out, 16) || !aligned(residual, 16) ||
        !aligned(gamma, 16) || !aligned(residual_out, 16) ||
        (normed_out && !aligned(normed_out, 16)) || !aligned(normed_fp8, 8) ||
        !aligned(fp8_scale, 4) || !aligned(perm_idx, 4) || !aligned(topk_w, 4) ||
        (bad_index && !aligned(bad_index, 4)))
        return MFR_ERR_ALIGN;
    const uint64_t act = static_cast<uint64_t>(T) * H * 2;
    const uint64_t meta = static_cast<uint64_t>(T) * K * 4;
    const Extent outs[] = {{residual_out, act},
                           {normed_fp8, static_cast<uint64_t>(T) * H},
                           {fp8_scale, static_cast<uint64_t>(T) * 4},
                           {normed_out, normed_out ? act : 0},
                           {bad_index, bad_index ? 4u : 0u}};
    const Extent ins[] = {{residual, act}, {shared_out, act}, {gamma, static_cast<uint64_t>(H) * 2},
                          {perm_idx, meta}, {topk_w, meta},
                          {expert_out, static_cast<uint64_t>(R) * static_cast<uint64_t>(H) * 2}};
    const int rc = check_aliasing(outs, 5, ins, 6, residual_out, residual);
    if (rc != MFR_OK) return rc;

    mfr::Params p = {};
    p.expert_out = reinterpret_cast<const mfr::u32x4*>(expert_out);
    p.perm_idx = perm_idx;
    p.topk_w = topk_w;
    p.shared_out = reinterpret_cast<const mfr::u32x4*>(shared_out);
    p.residual = reinterpret_cast<const mfr::u32x4*>(residual);
    p.gamma = reinterpret_cast<const mfr::u32x4*>(gamma);
    p.residual_out = reinterpret_cast<mfr::u32x4*>(residual_out);
    p.normed_out = reinterpret_cast<mfr::u32x4*>(normed_out);
    p.normed_fp8 = normed_fp8;
    p.fp8_scale = fp8_scale;
    p.eps = eps;
    p.scale = scale;
    p.K = static_cast<int>(K);
    p.rows = static_cast<uint32_t>(R);
    p.bad_index = bad_index;
    return launch(p, T, H, K == 8 ? kTop8Rows : kAnyKRows,
                  normed_out ? mfr::kOutBoth : mfr::kOutFp8, stream);
}

int residual_add_rmsnorm(const uint16_t* x, const uint16_t* residual, const uint16_t* gamma,
                         float eps, uint16_t* residual_out, uint16_t* normed_out, int64_t T,
                         int64_t H, hipStream_t stream) {
    if (!shape_ok(T, H, 1)) return MFR_ERR_SHAPE;
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return MFR_ERR_SCALAR;
    if (T == 0) return MFR_OK;
    if (!x || !residual || !gamma || !residual_out || !normed_out) return MFR_ERR_NULL;
    if (!aligned(x, 16) || !aligned(residual, 16) || !aligned(gamma, 16) ||
        !aligned(residual_out, 16) || !aligned(normed_out, 16))
        return MFR_ERR_ALIGN;
    const uint64_t act = static_cast<uint64_t>(T) * H * 2;
    const Extent outs[] = {{residual_out, act}, {normed_out, act}};
    const Extent ins[] = {{residual, act}, {x, act}, {gamma, static_cast<uint64_t>(H) * 2}};
    const int rc = check_aliasing(outs, 2, ins, 3, residual_out, residual);
    if (rc != MFR_OK) return rc;

    mfr::Params p = {};
    p.shared_out = reinterpret_cast<const mfr::u32x4*>(x);
    p.residual = reinterpret_cast<const mfr::u32x4*>(residual);
    p.gamma = reinterpret_cast<const mfr::u32x4*>(gamma);
    p.residual_out = reinterpret_cast<mfr::u32x4*>(residual_out);
    p.normed_out = reinterpret_cast<mfr::u32x4*>(normed_out);
    p.eps = eps;
    p.scale = 1.0f;
    p.K = 0;
    p.rows = kNoRowBound;
    return launch(p, T, H, kDense, mfr::kOutBf16, stream);
}

int residual_add_rmsnorm_fp8(const uint16_t* x, const uint16_t* residual, const uint16_t* gamma,
                             float eps, uint16_t* residual_out, uint16_t* normed_out,
                             uint8_t* normed_fp8, float* fp8_scale, int64_t T, int64_t H,
                             hipStream_t stream) {
    if (!shape_ok(T, H, 1)) return MFR_ERR_SHAPE;
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return MFR_ERR_SCALAR;
    if (T == 0) return MFR_OK;
    if (!x || !residual || !gamma || !residual_out || !normed_fp8 || !fp8_scale) return MFR_ERR_NULL;
    if (!aligned(x, 16) || !aligned(residual, 16) || !aligned(gamma, 16) ||
        !aligned(residual_out, 16) || (normed_out && !aligned(normed_out, 16)) ||
        !aligned(normed_fp8, 8) || !aligned(fp8_scale, 4))
        return MFR_ERR_ALIGN;
    const uint64_t act = static_cast<uint64_t>(T) * H * 2;
    const Extent outs[] = {{residual_out, act},
                           {normed_fp8, static_cast<uint64_t>(T) * H},
                           {fp8_scale, static_cast<uint64_t>(T) * 4},
                           {normed_out, normed_out ? act : 0}};
    const Extent ins[] = {{residual, act}, {x, act}, {gamma, static_cast<uint64_t>(H) * 2}};
    const int rc = check_aliasing(outs, 4, ins, 3, residual_out, residual);
    if (rc != MFR_OK) return rc;

    mfr::Params p = {};
    p.shared_out = reinterpret_cast<const mfr::u32x4*>(x);
    p.residual = reinterpret_cast<const mfr::u32x4*>(residual);
    p.gamma = reinterpret_cast<const mfr::u32x4*>(gamma);
    p.residual_out = reinterpret_cast<mfr::u32x4*>(residual_out);
    p.normed_out = reinterpret_cast<mfr::u32x4*>(normed_out);
    p.normed_fp8 = normed_fp8;
    p.fp8_scale = fp8_scale;
    p.eps = eps;
    p.scale = 1.0f;
    p.K = 0;
    p.rows = kNoRowBound;
    return launch(p, T, H, kDense, normed_out ? mfr::kOutBoth : mfr::kOutFp8, stream);
}

int moe_finalize_rmsnorm_path(int64_t T, int64_t H, int64_t K) {
    if (!shape_ok(T, H, K)) return MFR_PATH_UNSUPPORTED;
    return choose_path(T == 0 ? 1 : T, H, K);
}

const char* moe_finalize_rmsnorm_strerror(int status) {
    switch (status) {
        case MFR_OK: return "success";
        case MFR_ERR_NULL: return "a required pointer is NULL";
        case MFR_ERR_SHAPE:
            return "T, H or K outside the supported limits "
                   "(0<=T<2^31, 8<=H<=16384, H%8==0, 1<=K<=16)";
        case MFR_ERR_ALIGN: return "bf16 pointers must be 16-byte aligned, perm_idx/topk_w 4-byte aligned";
        case MFR_ERR_ALIAS: return "an output overlaps an input or the other output (only residual_out == residual is allowed)";
        case MFR_ERR_SCALAR: return "eps must be finite and >= 0, scale must be finite";
        case MFR_ERR_HIP: return "the HIP runtime refused the kernel launch";
        case MFR_ERR_ARG: return "invalid launch override value";
        default: return "unknown status";
    }
}

int mfr_tuning_force_launch(int path, int vectors_per_thread, int store_policy) {
    if (path < 0 || path > MFR_PATH_PERSIST) return MFR_ERR_ARG;
    if (vectors_per_thread < 0 || vectors_per_thread > kVptMax) return MFR_ERR_ARG;
    if (store_policy < 0 || store_policy > MFR_STORE_NONTEMPORAL_WRITE_THROUGH) return MFR_ERR_ARG;
    t_force_path = path;
    t_force_vpt = vectors_per_thread;
    t_force_store = store_policy;
    return MFR_OK;
}

int mfr_tuning_force_residency(int workgroups_per_cu) {
    if (workgroups_per_cu < 0) return MFR_ERR_ARG;
    t_force_residency = workgroups_per_cu;
    return MFR_OK;
}

int mfr_tuning_force_token_order(int order) {
    if (order != MFR_ORDER_DEFAULT && order != MFR_ORDER_XCD_RANGES) return MFR_ERR_ARG;
    t_force_order = order;
    return MFR_OK;
}

}  // extern "C"
