// Drives every exported oracle function over ordinary, degenerate and
// erroneous inputs, for a build under AddressSanitizer and
// UndefinedBehaviorSanitizer. Values are not checked here (the pins do
// that); the run must finish without a sanitizer report and exit 0.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <random>
#include <vector>

extern "C" {
int mfr_oracle_finalize_rmsnorm(const uint16_t* expert_out, int64_t R, const int32_t* perm_idx,
                                const float* topk_w, const uint16_t* shared_out,
                                const uint16_t* residual, const uint16_t* gamma, float eps,
                                float scale, int64_t T, int64_t H, int64_t K,
                                uint16_t* residual_out, uint16_t* normed_out, double* s_exact,
                                double* normed_exact);
int mfr_oracle_residual_rmsnorm(const uint16_t* x, const uint16_t* residual, const uint16_t* gamma,
                                float eps, int64_t T, int64_t H, uint16_t* residual_out,
                                uint16_t* normed_out, double* s_exact, double* normed_exact);
void mfr_oracle_fp8_quantize_rows(const double* y, int64_t T, int64_t H, uint8_t* codes,
                                  double* scales, double* scaled);
void mfr_oracle_rne_e4m3_from_f64(const double* x, int64_t n, uint8_t* out);
void mfr_oracle_rne_bf16_from_f64(const double* x, int64_t n, uint16_t* out);
}

static int failures = 0;
static void expect(bool ok, const char* what) {
    if (!ok) {
        std::fprintf(stderr, "FAIL: %s\n", what);
        ++failures;
    }
}

int main() {
    std::mt19937 gen(12345);
    std::uniform_int_distribution<int> bits(0, 0xFFFF);
    const int64_t T = 5, H = 24, K = 3, R = T * K + 2;
    std::vector<uint16_t> E(R * H), sh(T * H), rs(T * H), g(H), ro(T * H), no(T * H);
    for (auto& v : E) v = static_cast<uint16_t>(bits(gen) & 0x3FFF);  // finite values
    for (auto& v : sh) v = static_cast<uint16_t>(bits(gen) & 0xBFFF);
    for (auto& v : rs) v = static_cast<uint16_t>(bits(gen) & 0xBFFF);
    for (auto& v : g) v = static_cast<uint16_t>(0x3F80 | (bits(gen) & 0x7F));
    std::vector<int32_t> idx(T * K);
    std::vector<float> w(T * K, 0.25f);
    for (int64_t i = 0; i < T * K; ++i) idx[i] = (i % 4 == 3) ? -1 : static_cast<int32_t>(i);
    std::vector<double> s(T * H), ne(T * H);

    expect(mfr_oracle_finalize_rmsnorm(E.data(), R, idx.data(), w.data(), sh.data(), rs.data(),
                                       g.data(), 1e-6f, 2.5f, T, H, K, ro.data(), no.data(),
                                       s.data(), ne.data()) == 0, "finalize");
    expect(mfr_oracle_finalize_rmsnorm(E.data(), R, idx.data(), w.data(), sh.data(), rs.data(),
                                       g.data(), 0.0f, 1.0f, T, H, K, ro.data(), no.data(),
                                       nullptr, nullptr) == 0, "finalize without exact outputs");
    expect(mfr_oracle_finalize_rmsnorm(E.data(), R, idx.data(), w.data(), sh.data(), rs.data(),
                                       g.data(), 1e-6f, 1.0f, 0, H, K, ro.data(), no.data(),
                                       s.data(), ne.data()) == 0, "zero tokens");
    std::vector<int32_t> bad = idx;
    bad[T * K - 1] = static_cast<int32_t>(R);
    expect(mfr_oracle_finalize_rmsnorm(E.data(), R, bad.data(), w.data(), sh.data(), rs.data(),
                                       g.data(), 1e-6f, 1.0f, T, H, K, ro.data(), no.data(),
                                       s.data(), ne.data()) == 2, "index >= R is an error");
    expect(mfr_oracle_finalize_rmsnorm(E.data(), R, idx.data(), w.data(), sh.data(), rs.data(),
                                       g.data(), 1e-6f, 1.0f, T, 0, K, ro.data(), no.data(),
                                       s.data(), ne.data()) == 1, "H = 0 is a shape error");
    // an all-zero row with eps = 0: 0 / sqrt(0) gives NaN on purpose
    std::vector<uint16_t> z(H, 0), zo(H), zn(H);
    expect(mfr_oracle_residual_rmsnorm(z.data(), z.data(), g.data(), 0.0f, 1, H, zo.data(),
                                       zn.data(), nullptr, nullptr) == 0, "zero row");
    expect(mfr_oracle_residual_rmsnorm(sh.data(), rs.data(), g.data(), 1e-6f, T, H, ro.data(),
                                       no.data(), s.data(), ne.data()) == 0, "dense");

    // FP8 rows: ordinary, all zero, a NaN element, an infinite element, tiny values
    const double inf = std::numeric_limits<double>::infinity();
    const double nan = std::numeric_limits<double>::quiet_NaN();
    std::vector<double> y = {1.0, -0.5, 0.25, 2.0, 0.0, 7.0, -3.5, 0.1,
                             0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0,
                             1.0, nan, 2.0, -3.0, 0.5, 0.0, 1e-3, -1.0,
                             1.0, inf, 2.0, -3.0, 0.5, 0.0, 1e-3, -1.0,
                             1e-300, -2e-300, 3e-310, 0.0, 5e-324, -1e-305, 1e-299, 0.0};
    std::vector<uint8_t> codes(y.size());
    std::vector<double> scales(5), scaled(y.size());
    mfr_oracle_fp8_quantize_rows(y.data(), 5, 8, codes.data(), scales.data(), scaled.data());
    mfr_oracle_fp8_quantize_rows(y.data(), 5, 8, codes.data(), scales.data(), nullptr);
    expect(scales[1] == 1.0, "zero row scale");

    // elementwise roundings over special and boundary values
    std::vector<double> x = {0.0, -0.0, nan, -nan, inf, -inf, 448.0, 464.0, 480.0, -1e9,
                             std::ldexp(1.0, -9), std::ldexp(1.0, -10), std::ldexp(3.0, -11),
                             std::ldexp(1.0, -133), std::ldexp(1.0, -134), std::ldexp(3.0, -135),
                             std::ldexp(1.0, -150), 3.3895313892515355e38, 3.4e38, 1e308,
                             5e-324, 1.0 + std::ldexp(1.0, -8), 1.0 + std::ldexp(3.0, -9)};
    std::vector<uint8_t> e8(x.size());
    std::vector<uint16_t> b16(x.size());
    mfr_oracle_rne_e4m3_from_f64(x.data(), static_cast<int64_t>(x.size()), e8.data());
    mfr_oracle_rne_bf16_from_f64(x.data(), static_cast<int64_t>(x.size()), b16.data());
    expect(b16[0] == 0x0000 && b16[1] == 0x8000, "signed zeros");
    expect(e8[6] == 0x7E, "448 is the largest finite E4M3");

    if (failures) return 1;
    std::printf("oracle driver: ok\n");
    return 0;
}
