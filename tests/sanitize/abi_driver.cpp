// Drives the host side of the C ABI (path query, strerror, the launch
// override and every argument check) for a build under AddressSanitizer and
// UndefinedBehaviorSanitizer. Nothing reaches a kernel launch: every call
// either returns an error status or has T = 0, so no GPU is needed. The run
// must finish without a sanitizer report and exit 0.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "mfr_tuning.h"
#include "moe_finalize_rmsnorm.h"

static int failures = 0;
static void expect(int got, int want, const char* what) {
    if (got != want) {
        std::fprintf(stderr, "FAIL: %s: got %d, want %d\n", what, got, want);
        ++failures;
    }
}

template <class T>
static T* at(uintptr_t a) { return reinterpret_cast<T*>(a); }  // never dereferenced

int main() {
    const int64_t T = 4, H = 2048, K = 8;
    const uintptr_t A = 1u << 20, step = 1u << 24;  // disjoint fake buffers
    const uint16_t* E = at<const uint16_t>(A);
    const int32_t* P = at<const int32_t>(A + step);
    const float* W = at<const float>(A + 2 * step);
    const uint16_t* S = at<const uint16_t>(A + 3 * step);
    const uint16_t* R = at<const uint16_t>(A + 4 * step);
    const uint16_t* G = at<const uint16_t>(A + 5 * step);
    uint16_t* RO = at<uint16_t>(A + 6 * step);
    uint16_t* NO = at<uint16_t>(A + 7 * step);
    uint8_t* Q = at<uint8_t>(A + 8 * step);
    float* SC = at<float>(A + 9 * step);
    const float nan = std::numeric_limits<float>::quiet_NaN();
    const float inf = std::numeric_limits<float>::infinity();

    expect(moe_finalize_rmsnorm_path(8, 6144, 8), MFR_PATH_TOKEN, "path small T");
    expect(moe_finalize_rmsnorm_path(8192, 6144, 8), MFR_PATH_STREAM, "path large T");
    expect(moe_finalize_rmsnorm_path(0, 6144, 8), MFR_PATH_TOKEN, "path T = 0");
    expect(moe_finalize_rmsnorm_path(8, 6145, 8), MFR_PATH_UNSUPPORTED, "path ragged H");
    expect(moe_finalize_rmsnorm_path(8, 6144, 17), MFR_PATH_UNSUPPORTED, "path K > 16");
    expect(moe_finalize_rmsnorm_path(-1, 6144, 8), MFR_PATH_UNSUPPORTED, "path T < 0");
    for (int c = -1; c <= 8; ++c)
        if (!moe_finalize_rmsnorm_strerror(c)) expect(0, 1, "strerror returns text");
    expect(mfr_tuning_force_launch(4, 0, 0), MFR_ERR_ARG, "force bad path");
    expect(mfr_tuning_force_launch(0, 5, 0), MFR_ERR_ARG, "force bad vpt");
    expect(mfr_tuning_force_launch(0, 0, 5), MFR_ERR_ARG, "force bad store");
    expect(mfr_tuning_force_token_order(2), MFR_ERR_ARG, "force bad token order");
    expect(mfr_tuning_force_residency(-1), MFR_ERR_ARG, "force bad residency");
    expect(mfr_tuning_force_token_order(MFR_ORDER_XCD_RANGES), MFR_OK, "force token order");
    expect(mfr_tuning_force_token_order(MFR_ORDER_DEFAULT), MFR_OK, "token order reset");
    expect(mfr_tuning_force_launch(MFR_PATH_STREAM, 2, MFR_STORE_WRITE_THROUGH), MFR_OK, "force");
    expect(moe_finalize_rmsnorm_path(1, 6144, 8), MFR_PATH_STREAM, "forced path");
    expect(mfr_tuning_force_launch(0, 0, 0), MFR_OK, "force reset");

    // the fused op
    expect(moe_finalize_rmsnorm(E, P, W, S, R, G, 1e-6f, 1.f, RO, NO, 0, H, K, nullptr), MFR_OK,
           "T = 0");
    expect(moe_finalize_rmsnorm(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 1e-6f, 1.f,
                                nullptr, nullptr, 0, H, K, nullptr), MFR_OK, "T = 0, null pointers");
    expect(moe_finalize_rmsnorm(E, P, W, S, R, G, 1e-6f, 1.f, RO, NO, T, 2044, K, nullptr),
           MFR_ERR_SHAPE, "H % 8");
    expect(moe_finalize_rmsnorm(E, P, W, S, R, G, 1e-6f, 1.f, RO, NO, T, H, 0, nullptr),
           MFR_ERR_SHAPE, "K = 0");
    expect(moe_finalize_rmsnorm(E, P, W, S, R, G, 1e-6f, 1.f, RO, NO, INT64_MAX, H, K, nullptr),
           MFR_ERR_SHAPE, "T too large");
    expect(moe_finalize_rmsnorm(E, P, W, S, R, G, -1e-6f, 1.f, RO, NO, T, H, K, nullptr),
           MFR_ERR_SCALAR, "eps < 0");
    expect(moe_finalize_rmsnorm(E, P, W, S, R, G, nan, 1.f, RO, NO, T, H, K, nullptr),
           MFR_ERR_SCALAR, "eps NaN");
    expect(moe_finalize_rmsnorm(E, P, W, S, R, G, 1e-6f, inf, RO, NO, T, H, K, nullptr),
           MFR_ERR_SCALAR, "scale inf");
    expect(moe_finalize_rmsnorm(E, P, W, S, R, nullptr, 1e-6f, 1.f, RO, NO, T, H, K, nullptr),
           MFR_ERR_NULL, "null gamma");
    expect(moe_finalize_rmsnorm(E, P, W, S, R, G, 1e-6f, 1.f, RO + 1, NO, T, H, K, nullptr),
           MFR_ERR_ALIGN, "misaligned residual_out");
    expect(moe_finalize_rmsnorm(E, at<const int32_t>(A + step + 2), W, S, R, G, 1e-6f, 1.f, RO, NO,
                                T, H, K, nullptr), MFR_ERR_ALIGN, "misaligned perm_idx");
    expect(moe_finalize_rmsnorm(E, P, W, S, R, G, 1e-6f, 1.f, RO, RO + 64, T, H, K, nullptr),
           MFR_ERR_ALIAS, "outputs overlap");
    expect(moe_finalize_rmsnorm(E, P, W, S, R, G, 1e-6f, 1.f, RO, at<uint16_t>(A + 3 * step), T, H,
                                K, nullptr), MFR_ERR_ALIAS, "normed_out == shared_out");
    expect(moe_finalize_rmsnorm(E, P, W, S, R, G, 1e-6f, 1.f, at<uint16_t>(A + 4 * step + 16), NO,
                                T, H, K, nullptr), MFR_ERR_ALIAS, "residual_out overlaps residual");

    // the op told R: its own checks, and the overlap check over all R rows
    int32_t* FLAG = at<int32_t>(A + 10 * step);
    expect(moe_finalize_rmsnorm_checked(E, -1, P, W, S, R, G, 1e-6f, 1.f, RO, NO, FLAG, T, H, K,
                                        nullptr), MFR_ERR_SHAPE, "checked R < 0");
    expect(moe_finalize_rmsnorm_checked(E, T * K, P, W, S, R, G, 1e-6f, 1.f, RO, NO, FLAG + 0, 0,
                                        H, K, nullptr), MFR_OK, "checked T = 0");
    expect(moe_finalize_rmsnorm_checked(nullptr, T * K, P, W, S, R, G, 1e-6f, 1.f, RO, NO, FLAG, T,
                                        H, K, nullptr), MFR_ERR_NULL, "checked null rows");
    expect(moe_finalize_rmsnorm_checked(E, T * K, P, W, S, R, G, 1e-6f, 1.f, RO, NO,
                                        at<int32_t>(A + 10 * step + 2), T, H, K, nullptr),
           MFR_ERR_ALIGN, "checked misaligned flag");
    expect(moe_finalize_rmsnorm_checked(E, T * K, P, W, S, R, G, 1e-6f, 1.f, RO,
                                        at<uint16_t>(A + 16 * H), FLAG, T, H, K, nullptr),
           MFR_ERR_ALIAS, "checked output inside the rows");
    expect(moe_finalize_rmsnorm_checked(E, (int64_t{1} << 40), P, W, S, R, G, 1e-6f, 1.f, RO, NO,
                                        at<int32_t>(A + 3 * step), T, H, K, nullptr),
           MFR_ERR_ALIAS, "checked huge R: the declared rows cover the outputs");

    // FP8 output
    expect(moe_finalize_rmsnorm_fp8(E, P, W, S, R, G, 1e-6f, 1.f, RO, nullptr, nullptr, SC, T, H, K,
                                    nullptr), MFR_ERR_NULL, "fp8 null codes");
    expect(moe_finalize_rmsnorm_fp8(E, P, W, S, R, G, 1e-6f, 1.f, RO, nullptr, Q + 4, SC, T, H, K,
                                    nullptr), MFR_ERR_ALIGN, "fp8 misaligned codes");
    expect(moe_finalize_rmsnorm_fp8(E, P, W, S, R, G, 1e-6f, 1.f, RO, nullptr, Q, at<float>(A + 8 * step + 64),
                                    T, H, K, nullptr), MFR_ERR_ALIAS, "fp8 scale inside codes");
    expect(moe_finalize_rmsnorm_fp8(E, P, W, S, R, G, 1e-6f, 1.f, RO, NO, Q, SC, 0, H, K, nullptr),
           MFR_OK, "fp8 T = 0");

    // dense tail
    expect(residual_add_rmsnorm(S, R, G, 1e-6f, RO, NO, T, 7, nullptr), MFR_ERR_SHAPE, "dense H");
    expect(residual_add_rmsnorm(S, R, G, nan, RO, NO, T, H, nullptr), MFR_ERR_SCALAR, "dense eps");
    expect(residual_add_rmsnorm(S, R, nullptr, 1e-6f, RO, NO, T, H, nullptr), MFR_ERR_NULL,
           "dense null gamma");
    expect(residual_add_rmsnorm(S, R, G, 1e-6f, RO, RO, T, H, nullptr), MFR_ERR_ALIAS,
           "dense outputs alias");
    expect(residual_add_rmsnorm(S, R, G, 1e-6f, RO, NO, 0, H, nullptr), MFR_OK, "dense T = 0");

    // FP8 output with the row bound
    expect(moe_finalize_rmsnorm_fp8_checked(E, -1, P, W, S, R, G, 1e-6f, 1.f, RO, nullptr, Q, SC,
                                            FLAG, T, H, K, nullptr),
           MFR_ERR_SHAPE, "fp8 checked negative R");
    expect(moe_finalize_rmsnorm_fp8_checked(E, T * K, P, W, S, R, G, 1e-6f, 1.f, RO, nullptr, Q,
                                            reinterpret_cast<float*>(FLAG), FLAG, T, H, K, nullptr),
           MFR_ERR_ALIAS, "fp8 checked flag on the scales");
    expect(moe_finalize_rmsnorm_fp8_checked(E, T * K, P, W, S, R, G, 1e-6f, 1.f, RO, nullptr,
                                            nullptr, SC, FLAG, T, H, K, nullptr),
           MFR_ERR_NULL, "fp8 checked null codes");
    expect(moe_finalize_rmsnorm_fp8_checked(E, T * K, P, W, S, R, G, 1e-6f, 1.f, RO, nullptr, Q, SC,
                                            FLAG, 0, H, K, nullptr),
           MFR_OK, "fp8 checked T = 0");

    // dense tail with FP8 output
    expect(residual_add_rmsnorm_fp8(S, R, G, 1e-6f, RO, nullptr, nullptr, SC, T, H, nullptr),
           MFR_ERR_NULL, "dense fp8 null codes");
    expect(residual_add_rmsnorm_fp8(S, R, G, 1e-6f, RO, nullptr, Q + 4, SC, T, H, nullptr),
           MFR_ERR_ALIGN, "dense fp8 misaligned codes");
    expect(residual_add_rmsnorm_fp8(S, R, G, -1.f, RO, nullptr, Q, SC, T, H, nullptr),
           MFR_ERR_SCALAR, "dense fp8 eps");
    expect(residual_add_rmsnorm_fp8(S, R, G, 1e-6f, RO, NO, reinterpret_cast<uint8_t*>(NO), SC, T,
                                    H, nullptr),
           MFR_ERR_ALIAS, "dense fp8 codes on the bf16 normed output");
    expect(residual_add_rmsnorm_fp8(S, R, G, 1e-6f, RO, NO, Q, SC, 0, H, nullptr), MFR_OK,
           "dense fp8 T = 0");

    if (failures) return 1;
    std::printf("abi driver: ok\n");
    return 0;
}
