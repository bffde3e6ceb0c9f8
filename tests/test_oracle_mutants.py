"""Plants plausible mistakes in copies of the oracle (on the CPU) and checks that
at least one pin catches each. The copies are built in a temporary directory;
the oracle itself is never modified."""
import os

import pytest

import oracle
import oracle_pins

# (name, text in bca_oracle.c, replacement)
MUTANTS = [
    ("window_lower_bound_off_by_one", "return (c >= t - (int64_t)W) && (c <= t - 1);",
     "return (c >= t - (int64_t)W - 1) && (c <= t - 1);"),
    ("window_admits_own_id", "return (c >= t - (int64_t)W) && (c <= t - 1);",
     "return (c >= t - (int64_t)W) && (c <= t);"),
    ("reference_not_always_visible", "if (c == ORACLE_CUR_ID || c == ORACLE_REF_ID) return 1;",
     "if (c == ORACLE_CUR_ID) return 1;"),
    ("scale_dropped", "s[j] = scale * acc;", "s[j] = acc;"),
    ("exp_sign_flipped", "double p = exp(s[j] - shift);", "double p = exp(shift - s[j]);"),
    ("lse_without_shift", "lse[(size_t)h * nq + i] = shift + log(l);",
     "lse[(size_t)h * nq + i] = log(l);"),
    ("no_max_subtraction", "double shift = literal ? 0.0 : m;", "double shift = 0.0;"),
    ("head_index_dropped_in_keys", "const double* kj = k + ((size_t)j * H + h) * d;",
     "const double* kj = k + ((size_t)j * H + 0) * d;"),
    ("dot_product_short", "for (int c = 0; c < d; ++c) acc += qi[c] * kj[c];",
     "for (int c = 0; c + 1 < d; ++c) acc += qi[c] * kj[c];"),
    ("values_not_normalised", "for (int c = 0; c < d; ++c) oi[c] /= l;", ""),
    ("merge_weight_sign", "double w = (x == -INFINITY) ? 0.0 : exp(x - M);",
     "double w = (x == -INFINITY) ? 0.0 : exp(M - x);"),
    ("merge_lse_without_max", "lse[r] = M + log(wsum);", "lse[r] = log(wsum);"),
    ("e4m3_ties_away", "pick = (lo & 1) ? up : lo;", "pick = up;"),
    ("e4m3_subnormal_exponent", "mag = ldexp((double)m / 8.0, -6);",
     "mag = ldexp((double)m / 8.0, -7);"),
    ("e4m3_bias_wrong", "mag = ldexp(1.0 + (double)m / 8.0, e - 7);",
     "mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    ("e4m3_no_saturation", "if (a >= 448.0) return (uint8_t)(sign | 0x7E);",
     "if (a >= 464.0) return (uint8_t)(sign | 0x7F);"),
    ("rope_second_sign", "yi[2 * i + 1] = x0 * s + x1 * c;", "yi[2 * i + 1] = -x0 * s + x1 * c;"),
    ("rope_frequency_exponent", "pow(base, -2.0 * i / d)", "pow(base, -1.0 * i / d)"),
    ("rope_position_off_by_one", "const double pos = (double)(pos0 + r);",
     "const double pos = (double)(pos0 + r + 1);"),
    ("rope_pairs_split_halves", "const double x0 = xi[2 * i], x1 = xi[2 * i + 1];",
     "const double x0 = xi[i], x1 = xi[i + d / 2];"),
    ("sequence_window_off_by_one", "admit = (cj >= ci - W) && (cj <= ci);",
     "admit = (cj >= ci - W - 1) && (cj <= ci);"),
    ("sequence_next_chunk_visible", "admit = (cj >= ci - W) && (cj <= ci);",
     "admit = (cj >= ci - W) && (cj <= ci + 1);"),
    ("sequence_prefix_dropped", "        admit = 1;\n      } else {", "        admit = 0;\n      } else {"),
    ("sequence_chunk_of_key_ignores_prefix", "int cj = (j - P) / n;", "int cj = j / n;"),
    ("block_scale_fixed_code", "? a / qmax : 1.0f;", "? a / 448.0f : 1.0f;"),
    ("block_scale_over_all_heads", "float v = fabsf(x[((size_t)r * H + h) * d + j]);",
     "float v = fabsf(x[((size_t)r * H + 0) * d + j]);"),
    ("int8_ties_away", "if (rem > 0.5 || (rem == 0.5 && (q & 1))) q += 1;",
     "if (rem >= 0.5) q += 1;"),
    ("int8_truncates", "if (rem > 0.5 || (rem == 0.5 && (q & 1))) q += 1;", ""),
    ("int8_clamp_128", "if (y > 127.0f) y = 127.0f;", "if (y > 128.0f) y = 128.0f;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(oracle.SRC_PATH).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    so = oracle.compile_oracle(path, os.path.join(tmp_path, "libmutant.so"))
    lib = oracle.OracleLib(so)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {name}"
