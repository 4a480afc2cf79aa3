// Oracle for the fused MoE finalize + residual add + RMSNorm.
//
// TEST INFRASTRUCTURE ONLY. This file is the slow, plain, obviously-correct
// CPU definition that the GPU library is checked against. Only the test
// suite, the smoke check and the CPU-baseline leg of the benchmark load it.
// It shares no code, header, table or helper with the HIP library and must
// never be reached from the product path.
//
// What it computes (vLLM pull request #62174, where a decode MoE layer leaves
// its top-k reduction to the next layer's fused norm):
//   * Details: the fused kernel takes the top-k sum of the GEMM2 rows, applies
//     the routed scaling factor, adds the shared-expert output, all-reduces
//     (the identity on one GPU), adds the residual and applies RMSNorm.
//   * Validation: its result is checked against the separate steps (the
//     finalize, the shared add, and RMSNorm of the all-reduced sum), and the
//     page notes that outputs moved because intermediate roundings are gone:
//     the sum is rounded a single time.
//   * Claims: the kernel keeps its sums in FP32.
// Written here as that plain definition, in fp64, with exactly one rounding
// to bf16 at each output (residual_out and normed_out).
//
// Readings taken where the page is silent:
//   * RMSNorm is x / sqrt(mean_h(x^2) + eps) * gamma (eps inside the root,
//     mean over the hidden size, gamma multiplies).
//   * The norm's input is the unrounded sum (the residual stream is rounded
//     to bf16 only for the residual output).
//   * A negative permutation index marks a masked slot: its weight is
//     ignored and its row is never read. An all-masked token has a routed
//     part of exactly zero.
//   * Order of adds: (scale * routed + shared) + residual. In fp64 the order
//     is immaterial for the inputs used here.
//
// Rounding: bf16 values widen to double exactly. The only narrowing is
// rne_bf16_from_f64(), which rounds the double straight to bf16 (no fp32
// intermediate, which would round twice), ties to even, with bf16
// subnormals, overflow to infinity and NaN handled.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

// bf16 bit pattern -> double. bf16 is the upper half of an IEEE binary32,
// so the widening is exact.
double bf16_bits_to_double(uint16_t b) {
    uint32_t u = static_cast<uint32_t>(b) << 16;
    float f;
    std::memcpy(&f, &u, sizeof f);
    return static_cast<double>(f);
}

// Round a double to the nearest bf16 (8 significant bits, exponent range of
// binary32), ties to even.
uint16_t rne_bf16_from_f64(double x) {
    const bool neg = std::signbit(x);
    const uint16_t sign = neg ? 0x8000u : 0x0000u;
    if (std::isnan(x)) return static_cast<uint16_t>(sign | 0x7FC0u);
    double a = std::fabs(x);
    if (std::isinf(a)) return static_cast<uint16_t>(sign | 0x7F80u);
    if (a == 0.0) return sign;

    // a = m * 2^ex with m in [0.5, 1): the leading bit has weight 2^(ex-1).
    int ex = 0;
    (void)std::frexp(a, &ex);
    int lead = ex - 1;
    // bf16 normals have leading weight >= 2^-126; below that the spacing is
    // fixed at the subnormal quantum 2^-133.
    if (lead < -126) lead = -126;
    const int qexp = lead - 7;  // spacing of bf16 values near a

    // n = a / 2^qexp is exact (power-of-two scaling of a normal result).
    const double n = std::ldexp(a, -qexp);
    double fl = std::floor(n);
    const double frac = n - fl;  // exact: n < 2^9 here
    double r;
    if (frac > 0.5) {
        r = fl + 1.0;
    } else if (frac < 0.5) {
        r = fl;
    } else {
        r = (std::fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;  // tie: to even
    }
    const double y = std::ldexp(r, qexp);  // a bf16 value, or 2^128
    if (y >= 0x1p128) return static_cast<uint16_t>(sign | 0x7F80u);
    // y is exactly representable in binary32; its top half is the bf16.
    const float yf = static_cast<float>(y);
    uint32_t u;
    std::memcpy(&u, &yf, sizeof u);
    return static_cast<uint16_t>(sign | static_cast<uint16_t>(u >> 16));
}

// Round a double to OCP FP8 E4M3 ("e4m3fn": 1 sign bit, 4 exponent bits with
// bias 7, 3 mantissa bits, largest finite value 448, no infinities), ties to
// even, saturating: magnitudes at or above 448 give +-448. Returns the code.
uint8_t rne_e4m3_sat_from_f64(double v) {
    const uint8_t sign = std::signbit(v) ? 0x80u : 0x00u;
    if (std::isnan(v)) return static_cast<uint8_t>(sign | 0x7Fu);
    const double a = std::fabs(v);
    if (a >= 448.0) return static_cast<uint8_t>(sign | 0x7Eu);
    if (a == 0.0) return sign;
    int ex = 0;
    (void)std::frexp(a, &ex);
    int lead = ex - 1;          // a in [2^lead, 2^(lead+1))
    if (lead < -6) lead = -6;   // below the smallest normal 2^-6 the spacing is 2^-9
    const int qexp = lead - 3;  // spacing of E4M3 values near a
    const double n = std::ldexp(a, -qexp);
    const double fl = std::floor(n);
    const double frac = n - fl;
    double r;
    if (frac > 0.5) {
        r = fl + 1.0;
    } else if (frac < 0.5) {
        r = fl;
    } else {
        r = (std::fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    }
    const double y = std::ldexp(r, qexp);  // an E4M3 value (at most 448 here)
    if (y == 0.0) return sign;
    int ey = 0;
    (void)std::frexp(y, &ey);
    const int e = ey - 1;
    if (e < -6) {  // subnormal: y = m * 2^-9
        const int m = static_cast<int>(std::ldexp(y, 9));
        return static_cast<uint8_t>(sign | m);
    }
    const int m = static_cast<int>((std::ldexp(y, -e) - 1.0) * 8.0);
    return static_cast<uint8_t>(sign | ((e + 7) << 3) | m);
}

}  // namespace

extern "C" {

enum {
    MFR_ORACLE_OK = 0,
    MFR_ORACLE_ERR_SHAPE = 1,
    MFR_ORACLE_ERR_INDEX = 2,
};

// Plain per-token evaluation.
//   expert_out   [R, H]  bf16 bits  (GEMM2 output rows)
//   perm_idx     [T, K]  int32      (row of expert_out for token t, slot k; <0 = masked)
//   topk_w       [T, K]  fp32       (routing weight of the slot)
//   shared_out   [T, H]  bf16 bits
//   residual     [T, H]  bf16 bits
//   gamma        [H]     bf16 bits
//   residual_out [T, H]  bf16 bits  (out) RNE(s)
//   normed_out   [T, H]  bf16 bits  (out) RNE(s / sqrt(mean(s^2) + eps) * gamma)
//   s_exact      [T, H]  double     (out, optional) unrounded s
//   normed_exact [T, H]  double     (out, optional) unrounded normed value
// Returns MFR_ORACLE_ERR_INDEX if a non-negative index is >= R; outputs of
// tokens before the failing one are written, later ones are not.
int mfr_oracle_finalize_rmsnorm(const uint16_t* expert_out, int64_t R,
                                const int32_t* perm_idx, const float* topk_w,
                                const uint16_t* shared_out, const uint16_t* residual,
                                const uint16_t* gamma, float eps, float scale,
                                int64_t T, int64_t H, int64_t K,
                                uint16_t* residual_out, uint16_t* normed_out,
                                double* s_exact, double* normed_exact) {
    if (T < 0 || H <= 0 || K < 0 || R < 0) return MFR_ORACLE_ERR_SHAPE;
    std::vector<double> routed(static_cast<size_t>(H));
    std::vector<double> s(static_cast<size_t>(H));
    const double scale_d = static_cast<double>(scale);
    const double eps_d = static_cast<double>(eps);

    for (int64_t t = 0; t < T; ++t) {
        // Top-k sum of the token's routed rows (masked slots skipped).
        for (int64_t h = 0; h < H; ++h) routed[h] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const int64_t idx = perm_idx[t * K + k];
            if (idx < 0) continue;
            if (idx >= R) return MFR_ORACLE_ERR_INDEX;
            const double w = static_cast<double>(topk_w[t * K + k]);
            const uint16_t* row = expert_out + idx * H;
            for (int64_t h = 0; h < H; ++h) routed[h] += w * bf16_bits_to_double(row[h]);
        }
        // Routed scaling, shared add, (all-reduce = identity), residual add.
        for (int64_t h = 0; h < H; ++h) {
            s[h] = scale_d * routed[h] + bf16_bits_to_double(shared_out[t * H + h]) +
                   bf16_bits_to_double(residual[t * H + h]);
        }
        // RMSNorm of the unrounded sum.
        double sumsq = 0.0;
        for (int64_t h = 0; h < H; ++h) sumsq += s[h] * s[h];
        const double mean_sq = sumsq / static_cast<double>(H);
        const double denom = std::sqrt(mean_sq + eps_d);
        for (int64_t h = 0; h < H; ++h) {
            const double y = s[h] / denom * bf16_bits_to_double(gamma[h]);
            residual_out[t * H + h] = rne_bf16_from_f64(s[h]);
            normed_out[t * H + h] = rne_bf16_from_f64(y);
            if (s_exact) s_exact[t * H + h] = s[h];
            if (normed_exact) normed_exact[t * H + h] = y;
        }
    }
    return MFR_ORACLE_OK;
}

// Dense residual add + RMSNorm: the same tail with no routed part.
// ("Port the validated GLM-5.2 H200 production path to latest vLLM", Ported
// behavior: the attention and MLP row-parallel partial outputs are fused with
// the all-reduce, the residual add and RMSNorm, and so are the final
// main-model norm and the MTP final norm; on one GPU the all-reduce is the
// identity.) Per token: s = x + residual in fp64, residual_out = RNE(s),
// normed_out = RNE(s / sqrt(mean(s^2) + eps) * gamma).
//   x, residual  [T, H] bf16 bits;  gamma [H] bf16 bits
//   s_exact / normed_exact: optional unrounded outputs, as above.
int mfr_oracle_residual_rmsnorm(const uint16_t* x, const uint16_t* residual,
                                const uint16_t* gamma, float eps, int64_t T, int64_t H,
                                uint16_t* residual_out, uint16_t* normed_out,
                                double* s_exact, double* normed_exact) {
    if (T < 0 || H <= 0) return MFR_ORACLE_ERR_SHAPE;
    std::vector<double> s(static_cast<size_t>(H));
    const double eps_d = static_cast<double>(eps);
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h)
            s[h] = bf16_bits_to_double(x[t * H + h]) + bf16_bits_to_double(residual[t * H + h]);
        double sumsq = 0.0;
        for (int64_t h = 0; h < H; ++h) sumsq += s[h] * s[h];
        const double denom = std::sqrt(sumsq / static_cast<double>(H) + eps_d);
        for (int64_t h = 0; h < H; ++h) {
            const double y = s[h] / denom * bf16_bits_to_double(gamma[h]);
            residual_out[t * H + h] = rne_bf16_from_f64(s[h]);
            normed_out[t * H + h] = rne_bf16_from_f64(y);
            if (s_exact) s_exact[t * H + h] = s[h];
            if (normed_exact) normed_exact[t * H + h] = y;
        }
    }
    return MFR_ORACLE_OK;
}

// Dynamic per-token FP8 quantisation of rows of (unrounded) values: the
// activation format of an FP8 GEMM with dynamic per-token activation scales
// ("Port the validated GLM-5.2 H200 production path to latest vLLM", Prepared
// experiment branches: the attention projections whose input is this norm's
// output run FP8 GEMMs with static per-tensor weight scales and dynamic
// per-token activation scales). Per row: amax = max |y|, scale = amax / 448
// (1 when amax is 0), code = E4M3(y / scale) rounded to nearest even.
//   y       [T, H] double   values to quantise (e.g. normed_exact)
//   codes   [T, H] uint8    (out) E4M3 codes
//   scales  [T]    double   (out) per-row scale; y ~= E4M3 value * scale
//   scaled  [T, H] double   (out, optional) y / scale before rounding
void mfr_oracle_fp8_quantize_rows(const double* y, int64_t T, int64_t H, uint8_t* codes,
                                  double* scales, double* scaled) {
    for (int64_t t = 0; t < T; ++t) {
        double amax = 0.0;
        for (int64_t h = 0; h < H; ++h) amax = std::fmax(amax, std::fabs(y[t * H + h]));
        const double sc = amax > 0.0 ? amax / 448.0 : 1.0;
        scales[t] = sc;
        for (int64_t h = 0; h < H; ++h) {
            const double v = y[t * H + h] / sc;
            codes[t * H + h] = rne_e4m3_sat_from_f64(v);
            if (scaled) scaled[t * H + h] = v;
        }
    }
}

// Elementwise double -> E4M3 rounding (saturating), exported for the pins.
void mfr_oracle_rne_e4m3_from_f64(const double* x, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = rne_e4m3_sat_from_f64(x[i]);
}

// Elementwise double -> bf16 rounding, exported so the rounding itself can be
// pinned by the tests.
void mfr_oracle_rne_bf16_from_f64(const double* x, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = rne_bf16_from_f64(x[i]);
}

}  // extern "C"
