"""Plant plausible mistakes in copies of the oracle source (on the CPU) and
check that the pins catch every one of them."""
import os

import pytest

import oracle
from oracle import build as oracle_build
from tests import oracle_pins

# (name, text in mfr_oracle.cpp, replacement)
MUTANTS = [
    ("drop_shared", "bf16_bits_to_double(shared_out[t * H + h]) +", ""),
    ("residual_sign", "bf16_bits_to_double(residual[t * H + h]);",
     "(-bf16_bits_to_double(residual[t * H + h]));"),
    ("perm_transposed", "perm_idx[t * K + k]", "perm_idx[k * T + t]"),
    ("weight_slot_reversed", "topk_w[t * K + k]", "topk_w[t * K + (K - 1 - k)]"),
    ("eps_outside_root", "std::sqrt(mean_sq + eps_d)", "(std::sqrt(mean_sq) + eps_d)"),
    ("sum_not_mean", "sumsq / static_cast<double>(H)", "sumsq"),
    ("gamma_plus_one", "* bf16_bits_to_double(gamma[h])", "* (1.0 + bf16_bits_to_double(gamma[h]))"),
    ("scale_dropped", "scale_d * routed[h]", "routed[h]"),
    ("norm_of_rounded_numerator", "s[h] / denom", "bf16_bits_to_double(rne_bf16_from_f64(s[h])) / denom"),
    ("norm_of_rounded_sumsq", "sumsq += s[h] * s[h];",
     "{ const double q = bf16_bits_to_double(rne_bf16_from_f64(s[h])); sumsq += q * q; }"),
    ("round_after_shared_add",
     "s[h] = scale_d * routed[h] + bf16_bits_to_double(shared_out[t * H + h]) +",
     "s[h] = bf16_bits_to_double(rne_bf16_from_f64(scale_d * routed[h] + "
     "bf16_bits_to_double(shared_out[t * H + h]))) +"),
    ("zero_index_masked", "if (idx < 0) continue;", "if (idx <= 0) continue;"),
    ("ties_up", "r = (std::fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "r = fl + 1.0;"),
    ("subnormals_flushed", "if (lead < -126) lead = -126;", "if (lead < -126) return sign;"),
    ("truncate_not_round", "if (frac > 0.5) {", "if (frac > 2.0) {"),
    ("dense_drop_residual",
     "bf16_bits_to_double(x[t * H + h]) + bf16_bits_to_double(residual[t * H + h]);",
     "bf16_bits_to_double(x[t * H + h]);"),
    ("dense_eps_outside_root", "std::sqrt(sumsq / static_cast<double>(H) + eps_d)",
     "(std::sqrt(sumsq / static_cast<double>(H)) + eps_d)"),
    ("dense_sum_not_mean", "sumsq / static_cast<double>(H) + eps_d", "sumsq + eps_d"),
    ("dense_gamma_dropped",
     "const double denom = std::sqrt(sumsq / static_cast<double>(H) + eps_d);\n"
     "        for (int64_t h = 0; h < H; ++h) {\n"
     "            const double y = s[h] / denom * bf16_bits_to_double(gamma[h]);",
     "const double denom = std::sqrt(sumsq / static_cast<double>(H) + eps_d);\n"
     "        for (int64_t h = 0; h < H; ++h) {\n"
     "            const double y = s[h] / denom;"),
    ("e4m3_ties_up",
     "r = (std::fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;\n    }\n    const double y = std::ldexp(r, qexp);  // an E4M3 value",
     "r = fl + 1.0;\n    }\n    const double y = std::ldexp(r, qexp);  // an E4M3 value"),
    ("e4m3_no_saturation", "if (a >= 448.0) return static_cast<uint8_t>(sign | 0x7Eu);", ""),
    ("e4m3_fnuz_max", "amax > 0.0 ? amax / 448.0 : 1.0", "amax > 0.0 ? amax / 240.0 : 1.0"),
    ("e4m3_bias_8", "((e + 7) << 3)", "((e + 8) << 3)"),
    ("e4m3_subnormal_spacing", "if (lead < -6) lead = -6;", "if (lead < -7) lead = -7;"),
    ("fp8_scale_from_first_element", "amax = std::fmax(amax, std::fabs(y[t * H + h]));",
     "amax = std::fabs(y[t * H]);"),
    ("masked_slot_reads_row0", "if (idx < 0) continue;", "const int64_t r0 = idx < 0 ? 0 : idx;\n"
     "            if (r0 >= R) return MFR_ORACLE_ERR_INDEX;\n"
     "            const double w0 = static_cast<double>(topk_w[t * K + k]);\n"
     "            for (int64_t h = 0; h < H; ++h) routed[h] += w0 * bf16_bits_to_double(expert_out[r0 * H + h]);\n"
     "            continue;"),
    ("last_slot_dropped", "for (int64_t k = 0; k < K; ++k) {\n            const int64_t idx",
     "for (int64_t k = 0; k < K - 1; ++k) {\n            const int64_t idx"),
    ("bf16_nan_to_zero", "if (std::isnan(x)) return static_cast<uint16_t>(sign | 0x7FC0u);",
     "if (std::isnan(x)) return sign;"),
    ("bf16_overflow_to_max_finite", "if (y >= 0x1p128) return static_cast<uint16_t>(sign | 0x7F80u);",
     "if (y >= 0x1p128) return static_cast<uint16_t>(sign | 0x7F7Fu);"),
    ("e4m3_nan_to_zero", "if (std::isnan(v)) return static_cast<uint8_t>(sign | 0x7Fu);",
     "if (std::isnan(v)) return sign;"),
    ("fp8_zero_row_scale_zero", "amax > 0.0 ? amax / 448.0 : 1.0", "amax > 0.0 ? amax / 448.0 : 0.0"),
    ("fp8_amax_signed", "amax = std::fmax(amax, std::fabs(y[t * H + h]));",
     "amax = std::fmax(amax, y[t * H + h]);"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    with open(oracle_build.SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new)
    path = os.path.join(tmp_path, f"{name}.cpp")
    with open(path, "w") as f:
        f.write(mutated)
    lib = oracle_build.compile_source(path, os.path.join(tmp_path, f"lib{name}.so"))
    o = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            caught.append(pin.__name__)
            break
    assert caught, f"no pin caught the mutant {name}"
