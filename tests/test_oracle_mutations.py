"""Plant plausible mistakes in a copy of the oracle (CPU only) and check that
the pin suite fails for each one. Guards the pins themselves: a pin set that
still passes on a broken oracle would prove nothing."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "tq1_oracle.c")

MUTATIONS = {
    "digit_order_reversed": ("*digit = e / 32;", "*digit = 4 - e / 32;"),
    "qh_byte_digit_swapped": ("*byte_index = 48 + (e - 240) % 4;\n        *digit = (e - 240) / 4;",
                              "*byte_index = 48 + (e - 240) / 4;\n        *digit = (e - 240) % 4;"),
    "round_half_even": ("float r = roundf(xb[i] * id);", "float r = rintf(xb[i] * id);"),
    "divide_instead_of_reciprocal": ("float r = roundf(xb[i] * id);", "float r = roundf(xb[i] / dq);"),
    "activation_scale_index": ("q81_scale(a, nblk, t, j));", "q81_scale(a, nblk, t, j / 8));"),
    "weight_scale_block": ("int64_t B = j / 8;", "int64_t B = j / 4;"),
    "sum_field_unscaled": ("oracle_f32_to_f16(dq * (float)sum);", "oracle_f32_to_f16((float)sum);"),
    "trit_sign_flipped": ("(int8_t)(oracle_base3_digit(blk[p], c) - 1);",
                          "(int8_t)(1 - oracle_base3_digit(blk[p], c));"),
    "byte_walk_drops_sum_q": ("= su[b] - sq;", "= su[b];"),
    "f16_ties_up": ("if (rem > half || (rem == half && (n & 1)))", "if (rem >= half)"),
    "clamp_126": ("if (q > 127)\n                    q = 127;", "if (q > 126)\n                    q = 126;"),
    "dequant_scale_of_next_block": ("oracle_f16_to_f32(dd[k / TQ1_BLOCK_ELEMS])",
                                    "oracle_f16_to_f32(dd[(k / TQ1_BLOCK_ELEMS + 1) % nb])"),
    "bf16_truncates": ("if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))",
                       "if (0)"),
    "residual_subtracted": ("y64[t * N + n] = y64[t * N + n] + rv;",
                            "y64[t * N + n] = y64[t * N + n] - rv;"),
    "residual_transposed": ("double rv = (double)r[t * N + n];",
                            "double rv = (double)r[(n * T + t) % (N * T)];"),
    "tq2_field_and_byte_swapped": ("*byte_index = 32 * (e / 128) + e % 32;\n    *field = (e % 128) / 32;",
                                   "*byte_index = 32 * (e / 128) + (e % 128) / 4;\n    *field = e % 4;"),
    "tq2_field_weight_4_to_2": ("value[p] += (t + 1) << (2 * f);", "value[p] += (t + 1) << f;"),
    "tq2_trit_sign_flipped": ("(int8_t)(u - 1);", "(int8_t)(1 - u);"),
    "tq2_byte_walk_drops_sum_q": ("= su[b] - sumq;", "= su[b];"),
    "tq2_scale_of_next_block": ("oracle_f16_to_f32(dd[j / 8]);",
                                "oracle_f16_to_f32(dd[(j / 8 + 1) % nb]);"),
    "slots_read_token_column": ("int64_t col = column_per_pair ? ts : ts / n_used;",
                                "int64_t col = ts / n_used;"),
    "glu_sigmoid_without_its_argument": ("double silu = g / (1.0 + exp(-g));",
                                         "double silu = 1.0 / (1.0 + exp(-g));"),
    "glu_gate_and_up_swapped": ("oracle_mmvq(wg, a, NULL, g64, absg, N, K, T) || oracle_mmvq(wu, a, NULL, u64, absu, N, K, T)",
                                "oracle_mmvq(wu, a, NULL, g64, absg, N, K, T) || oracle_mmvq(wg, a, NULL, u64, absu, N, K, T)"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTATIONS[name]
    text = open(SRC).read()
    assert before in text, "mutation anchor vanished: " + name
    src = tmp_path / "mut.c"
    src.write_text(text.replace(before, after))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-std=c99", "-O1", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    str(src), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, TQ1_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    assert r.returncode == 1, "pins did not catch mutation %s:\n%s" % (name, r.stdout[-2000:])
