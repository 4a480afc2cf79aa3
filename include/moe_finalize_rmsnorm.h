/*
 * moe_finalize_rmsnorm.h - C ABI of the fused MoE finalize + residual add +
 * RMSNorm for MI355X (gfx950).
 *
 * The operation is the tail of a decode MoE layer whose top-k reduction was
 * left open by the experts and is completed inside the following layer's
 * input norm (vLLM pull request #62174, Overview and Details).
 * For each token t and hidden index h:
 *
 *   routed[h] = sum over slots k with perm_idx[t,k] >= 0 of
 *               topk_w[t,k] * expert_out[perm_idx[t,k], h]
 *   s[h]      = (scale * routed[h] + shared_out[t,h]) + residual[t,h]
 *   residual_out[t,h] = bf16(s[h])                                (one rounding)
 *   normed_out[t,h]   = bf16(s[h] / sqrt(mean_h(s^2) + eps) * gamma[h])
 *
 * The page's fused kernel does the top-k sum, the routed scaling, the shared
 * add, an all-reduce across tensor-parallel ranks, the residual add and the
 * RMSNorm in one launch (Details); on one GPU the all-reduce is the identity.
 * The page also says the kernel sums in FP32, and that its outputs moved
 * because the per-step roundings of the unfused chain are gone (Claims,
 * Validation): here the sum s is kept in fp32 registers, rounded to bf16 only
 * at the two outputs, and the norm is taken of the unrounded fp32 s.
 *
 * Entry points:
 *   moe_finalize_rmsnorm              the fused op
 *   moe_finalize_rmsnorm_checked      the fused op, told the row count R
 *   moe_finalize_rmsnorm_fp8          the fused op, normed output as per-token FP8
 *   moe_finalize_rmsnorm_fp8_checked  the two above together
 *   residual_add_rmsnorm              the same tail with no routed part
 *   residual_add_rmsnorm_fp8          the dense tail with FP8 output
 *   moe_finalize_rmsnorm_path         host-only: the launch path of a shape
 *   moe_finalize_rmsnorm_strerror     text of a status code
 *
 * Data types and layout (all row-major, contiguous, device memory):
 *   bf16 tensors are passed as raw 16-bit patterns (uint16_t).
 *   expert_out   [R, H]  bf16   GEMM2 output rows; R is not passed. Every
 *                               non-negative perm_idx must be < R (not checked:
 *                               an index >= R reads out of bounds on the GPU;
 *                               moe_finalize_rmsnorm_checked takes R and
 *                               checks).
 *   perm_idx     [T, K]  int32  row of expert_out for (token t, slot k);
 *                               any negative value marks a masked slot, whose
 *                               row is never read and whose weight is ignored.
 *   topk_w       [T, K]  fp32   routing weights. A zero weight on a valid index
 *                               is not a mask: the row is still read.
 *   shared_out   [T, H]  bf16   shared-expert output
 *   residual     [T, H]  bf16   residual stream
 *   gamma        [H]     bf16   RMSNorm weight
 *   eps                  fp32   >= 0 and finite (inside the square root)
 *   scale                fp32   finite routed scaling factor; callers whose
 *                               router folds the factor into topk_w pass 1.0
 *                               (the page requires the experts' factor to be
 *                               1.0 in that case: Details)
 *   residual_out [T, H]  bf16   output; may be exactly equal to residual
 *                               (in place), must not overlap anything else
 *   normed_out   [T, H]  bf16   output; must not overlap any other argument
 *
 * Range: s is accumulated in fp32, as the page's kernel accumulates (Claims),
 * so |s| must stay below 2^128 (the fp32 range; an overflowing s gives an
 * infinite residual_out on both the fused and the unfused chain, and a NaN or
 * zero normed row). Within that range every finite row is normalised: rows
 * whose fp32 sum of squares overflows (|s| above about 2^64 / sqrt(H)) or is
 * too small to use (mean(s^2) + eps below 2^-100, e.g. eps = 0 with
 * subnormal s) are normalised again with an fp64 sum of squares, by the same
 * kernel, at no cost to other rows. An all-zero row with eps = 0 gives NaN
 * (0 / 0); an infinite or NaN s propagates (inf / inf = NaN, others 0).
 *
 * Limits: 0 <= T <= 2^31-1, 8 <= H <= 16384 with H % 8 == 0, 1 <= K <= 16.
 * bf16 pointers must be 16-byte aligned; perm_idx and topk_w 4-byte aligned.
 * One workgroup serves one token, and a dispatch holds fewer than 2^32
 * work-items: a call whose T times the workgroup size (64 to 1024 threads)
 * reaches that is enqueued as several dispatches in stream order, with the
 * same results.
 *
 * Ownership and ordering: the caller owns every buffer; the library allocates
 * and frees nothing and keeps no per-call state (on the page, releasing the
 * deferred buffers is the consuming layer's job: Details). The work is enqueued on `stream` (NULL = the
 * device's null stream) and the call returns without synchronising; buffers
 * must stay valid until the stream has passed the kernel. Calls may be
 * captured into a HIP graph. Results are deterministic: no atomics, and a
 * fixed reduction order.
 *
 * Errors: every argument check runs on the host before anything is enqueued.
 * On error nothing is launched and a nonzero status is returned; no exception
 * crosses the ABI. T == 0 returns MFR_OK without launching (pointers are then
 * not examined). A failed launch returns MFR_ERR_HIP; if it was not the first
 * dispatch of a split call, the dispatches before it stay enqueued.
 */
#ifndef MOE_FINALIZE_RMSNORM_H
#define MOE_FINALIZE_RMSNORM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

enum mfr_status {
    MFR_OK = 0,
    MFR_ERR_NULL = 1,   /* a required pointer is NULL (T > 0) */
    MFR_ERR_SHAPE = 2,  /* T, H or K outside the limits above */
    MFR_ERR_ALIGN = 3,  /* a pointer is not aligned as required */
    MFR_ERR_ALIAS = 4,  /* outputs overlap inputs or each other (other than residual_out == residual) */
    MFR_ERR_SCALAR = 5, /* eps < 0, or eps or scale not finite */
    MFR_ERR_HIP = 6,    /* the HIP runtime refused the launch */
    MFR_ERR_ARG = 7     /* an invalid launch override (the library's tuning interface) */
};

/* Launch paths. The token and stream paths launch one workgroup per token
 * (grid = T) and differ in workgroup shape and store policy; the persistent
 * path launches a grid sized to the GPU, each workgroup walking many tokens
 * with the next token's loads in flight while it finishes the current one.
 * All give bit-identical residual_out; normed_out can differ in the last bit
 * between workgroup shapes (their reduction trees differ). */
enum mfr_path {
    MFR_PATH_UNSUPPORTED = 0,
    MFR_PATH_TOKEN = 1,   /* small T, latency: widest workgroup per token (768 threads at H = 6144),
                             write-through bf16 stores up to T = 64 */
    MFR_PATH_STREAM = 2,  /* large T, bandwidth: 256 threads per token, write-through stores once
                             the outputs pass 12 MiB */
    MFR_PATH_PERSIST = 3  /* large T, bandwidth: persistent multi-token workgroups, two tokens in
                             flight each (H <= 6144, K <= 8; not the checked calls with FP8
                             output, which take the automatic path) */
};

/* The fused op. Definition, layouts, limits and errors: see above. */
int moe_finalize_rmsnorm(const uint16_t* expert_out, const int32_t* perm_idx,
                         const float* topk_w, const uint16_t* shared_out,
                         const uint16_t* residual, const uint16_t* gamma,
                         float eps, float scale,
                         uint16_t* residual_out, uint16_t* normed_out,
                         int64_t T, int64_t H, int64_t K, hipStream_t stream);

/* The fused op told the row count R of expert_out. A slot whose index is at
 * or past R is treated as masked: its row is not read and its weight is
 * ignored, so a wrong index cannot read outside expert_out. If bad_index is
 * not NULL, the kernel sets *bad_index (int32, device memory, 4-byte
 * aligned) to 1 when any token holds such an index. It never writes 0, so
 * clear the flag before the call and read it after the stream has passed
 * the kernel. The caller chooses between failing, retrying or accepting the
 * masked result. R above 2^31 means the same as 2^31, because int32 indices
 * address no more. With R known, the overlap check covers all of
 * expert_out. Otherwise as moe_finalize_rmsnorm: for in-range indices the
 * outputs are bit-identical to it. The operation is the one defined above
 * (vLLM pull request #62174, Details). The row bound is this library's
 * addition, for callers that cannot vouch for their indices. */
int moe_finalize_rmsnorm_checked(const uint16_t* expert_out, int64_t R,
                                 const int32_t* perm_idx, const float* topk_w,
                                 const uint16_t* shared_out, const uint16_t* residual,
                                 const uint16_t* gamma, float eps, float scale,
                                 uint16_t* residual_out, uint16_t* normed_out,
                                 int32_t* bad_index,
                                 int64_t T, int64_t H, int64_t K, hipStream_t stream);

/* The fused op with the normalised output also (or only) produced as dynamic
 * per-token FP8, the activation format of the FP8 projection that consumes it
 * ("Port the validated GLM-5.2 H200 production path to latest vLLM", Prepared
 * experiment branches: the attention projections run FP8 GEMMs with static
 * per-tensor weight scales and dynamic per-token activation scales). With y the
 * fp32 normalised row (before any bf16 rounding):
 *
 *   amax             = max_h |y[h]|
 *   fp8_scale[t]     = amax / 448                (1 for an all-zero row)
 *   normed_fp8[t,h]  = E4M3(y[h] * 448 / amax)   (OCP E4M3: bias 7, 3 mantissa
 *                      bits, round to nearest even, saturated to +-448)
 *
 * so y[h] ~= value(normed_fp8[t,h]) * fp8_scale[t]. The library forms the two
 * quotients with the hardware reciprocal, each within 2^-20 relative, the
 * factor 448 / amax rounded low, so that no code passes 448: a code can then
 * differ from that of the exact quotient only where y[h] * 448 / amax lies
 * within that distance of the midpoint between two codes. Arguments as for
 * moe_finalize_rmsnorm, plus:
 *   normed_out   [T, H] bf16   optional: NULL skips the bf16 normed output
 *   normed_fp8   [T, H] uint8  E4M3 codes, 8-byte aligned
 *   fp8_scale    [T]    fp32   per-token scale, 4-byte aligned
 * No output may overlap another output or any input (residual_out ==
 * residual excepted). residual_out, and normed_out when given, are
 * bit-identical to those of moe_finalize_rmsnorm with the same arguments. */
int moe_finalize_rmsnorm_fp8(const uint16_t* expert_out, const int32_t* perm_idx,
                             const float* topk_w, const uint16_t* shared_out,
                             const uint16_t* residual, const uint16_t* gamma,
                             float eps, float scale,
                             uint16_t* residual_out, uint16_t* normed_out,
                             uint8_t* normed_fp8, float* fp8_scale,
                             int64_t T, int64_t H, int64_t K, hipStream_t stream);

/* The FP8-output op told the row count R of expert_out: the row bound and
 * the flag of moe_finalize_rmsnorm_checked, the outputs of
 * moe_finalize_rmsnorm_fp8. An index at or past R is treated as masked and
 * sets *bad_index to 1 when bad_index is not NULL (the flag is never cleared
 * by the library). For in-range indices every output is bit-identical to
 * that of moe_finalize_rmsnorm_fp8 with the same arguments; with the flag
 * raised they are those of moe_finalize_rmsnorm_fp8 with the offending slots
 * masked. Limits, alignment, aliasing and errors as for the two calls it
 * combines; the overlap check covers all R rows of expert_out. */
int moe_finalize_rmsnorm_fp8_checked(const uint16_t* expert_out, int64_t R,
                                     const int32_t* perm_idx, const float* topk_w,
                                     const uint16_t* shared_out, const uint16_t* residual,
                                     const uint16_t* gamma, float eps, float scale,
                                     uint16_t* residual_out, uint16_t* normed_out,
                                     uint8_t* normed_fp8, float* fp8_scale, int32_t* bad_index,
                                     int64_t T, int64_t H, int64_t K, hipStream_t stream);

/* Dense residual add + RMSNorm: the same tail with no routed part, for the
 * layers whose row-parallel attention / MLP outputs, or the final main-model
 * and MTP norms, feed the residual stream ("Port the validated GLM-5.2 H200
 * production path to latest vLLM", Ported behavior: those outputs are fused
 * with the all-reduce, the residual add and RMSNorm; on one GPU the all-reduce
 * is the identity). For each token t and hidden index h:
 *
 *   s[h]              = x[t,h] + residual[t,h]            (fp32)
 *   residual_out[t,h] = bf16(s[h])
 *   normed_out[t,h]   = bf16(s[h] / sqrt(mean_h(s^2) + eps) * gamma[h])
 *
 *   x, residual, residual_out, normed_out  [T, H] bf16;  gamma [H] bf16.
 * Limits, alignment (16 bytes for every pointer), ownership, stream ordering
 * and errors as for moe_finalize_rmsnorm; residual_out may be exactly
 * residual, and no other output may overlap an input or the other output.
 * The launch shape follows the same rule of T as moe_finalize_rmsnorm_path. */
int residual_add_rmsnorm(const uint16_t* x, const uint16_t* residual, const uint16_t* gamma,
                         float eps, uint16_t* residual_out, uint16_t* normed_out,
                         int64_t T, int64_t H, hipStream_t stream);

/* The dense residual add + RMSNorm with the normalised output also (or only)
 * produced as dynamic per-token FP8, for a dense tail whose output feeds an
 * FP8 projection (the page's attention projections take dynamic per-token
 * activation scales: "Port the validated GLM-5.2 H200 production path to
 * latest vLLM", Prepared experiment branches). The FP8 rule is the one of
 * moe_finalize_rmsnorm_fp8, applied to the fp32 normalised row of
 * residual_add_rmsnorm. Arguments as for residual_add_rmsnorm, plus:
 *   normed_out   [T, H] bf16   optional: NULL skips the bf16 normed output
 *   normed_fp8   [T, H] uint8  E4M3 codes, 8-byte aligned
 *   fp8_scale    [T]    fp32   per-token scale, 4-byte aligned
 * No output may overlap another output or any input (residual_out ==
 * residual excepted). residual_out, and normed_out when given, are
 * bit-identical to those of residual_add_rmsnorm with the same arguments. */
int residual_add_rmsnorm_fp8(const uint16_t* x, const uint16_t* residual, const uint16_t* gamma,
                             float eps, uint16_t* residual_out, uint16_t* normed_out,
                             uint8_t* normed_fp8, float* fp8_scale,
                             int64_t T, int64_t H, hipStream_t stream);

/* Which path moe_finalize_rmsnorm would take for this shape from the calling
 * thread (the MFR_PATH environment variable, read once at load, and a launch
 * override of the library's tuning interface are taken into account);
 * MFR_PATH_UNSUPPORTED if the shape is outside the limits. Pure host function: no HIP call. A
 * caller can use it to decide, before deferring its finalize, that the fused
 * op will accept the shape (the page's layers defer only when the fused kernel
 * will run: Details). T == 0 reports the path a nonzero T would take. */
int moe_finalize_rmsnorm_path(int64_t T, int64_t H, int64_t K);

/* Static, NUL-terminated description of a status code. Never NULL. */
const char* moe_finalize_rmsnorm_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FINALIZE_RMSNORM_H */
