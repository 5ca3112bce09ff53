"""The pins must catch plausible mistakes in the oracle.

Each case copies the oracle's C source, plants one mistake in the copy, builds
it with gcc in a temporary directory and runs the pin suite against it in a
subprocess; the suite must fail.  The committed oracle is never modified.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "fp8bs_oracle.c")

MUTANTS = {
    "dropped_last_chunk": ("for (c = 0; c < K / 128; ++c)", "for (c = 0; c + 1 < K / 128; ++c)"),
    "lost_sign": ("return s ? -v : v;", "return v;"),
    "subnormal_scale": ("v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    "exponent_bias": ("v = ldexp((double)(8 + m), e - 10);", "v = ldexp((double)(8 + m), e - 9);"),
    "first_chunk_scale_only": ("s = (double)sa[c * sa_step] * (double)sb[c * sb_step];",
                               "s = (double)sa[0] * (double)sb[c * sb_step];"),
    "b_scale_block_index": ("SB + (g * nb + n / 128) * kb", "SB + (g * nb + (n / 128 + 1) % nb) * kb"),
    "b_row_as_column_block": ("B + (g * N + n) * K", "B + (g * N + (n ^ 1) % N) * K"),
    "truncating_round": ("r = rint(n);", "r = floor(n);"),
    "rounds_through_fp32": ("uint16_t sign = signbit(x) ? 0x8000u : 0u;",
                            "uint16_t sign = signbit(x) ? 0x8000u : 0u; x = (double)(float)x;"),
    "masked_off_by_one": ("if (r >= valid) continue;", "if (r > valid) continue;"),
    "padding_written": ("if (g < 0 || g >= G) continue;", "if (g >= G) continue; if (g < 0) g = 0;"),
    # quantiser
    "enc_ties_to_odd": ("(d == best_d && (code & 1) == 0)", "(d == best_d && (code & 1) == 1)"),
    "enc_truncates": ("double d = fabs(a - fp8bs_oracle_dec_e4m3((uint8_t)code));",
                      "double d = a - fp8bs_oracle_dec_e4m3((uint8_t)code); if (d < 0) continue;"),
    "scale_from_inverse": ("return a / 448.0f;", "return 1.0f / *inv;"),
    "no_scale_floor": ("const float a = amax < 1e-4f ? 1e-4f : amax;", "const float a = amax;"),
    "addend_dropped": ("fp8bs_oracle_bf16_rne((double)C[i * N + n] +",
                       "fp8bs_oracle_bf16_rne(0.0 * (double)C[i * N + n] +"),
    "addend_masked_slot_rows": ("if (i % rows >= valid) continue;", "if (i % rows > valid) continue;"),
    "weight_block_skips_last_row": ("int64_t n1 = 128 * i + 128 < N ? 128 * i + 128 : N;",
                                    "int64_t n1 = 128 * i + 127 < N ? 128 * i + 127 : N;"),
    # stored forms and the K-grouped product
    "layout_a_step_k": ("const ptrdiff_t a_step = a_transposed ? M : 1;",
                        "const ptrdiff_t a_step = a_transposed ? K : 1;"),
    "layout_b_forms_swapped": ("const uint8_t* b = b_transposed ? B + n * K : B + n;",
                               "const uint8_t* b = b_transposed ? B + n : B + n * K;"),
    "layout_addend_dropped": ("if (C) v += (double)C[r * N + n];", "(void)C;"),
    "kgrouped_group_offset": ("for (j = 0; j < gg; ++j) k0 += ks[j];",
                              "for (j = 0; j + 1 < gg; ++j) k0 += ks[j];"),
    "kgrouped_b_scale_per_block": ("SB + n * kbt + k0 / 128", "SB + (n / 128) * kbt + k0 / 128"),
    "kgrouped_a_scale_from_chunk0": ("SA + m * kbt + k0 / 128", "SA + m * kbt"),
    "kgrouped_truncates": ("D[i * N + n] = (float)v;",
                           "{ float f = (float)v; if (fabs((double)f) > fabs(v)) "
                           "f = nextafterf(f, 0.0f); D[i * N + n] = f; }"),
    "kgrouped_addend_dropped": ("if (C) v += (double)C[i * N + n];", "(void)C;"),
}
PIN_FILES = ["test_oracle_pins.py", "test_oracle_quant_pins.py", "test_oracle_layout_pins.py"]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mut_c = tmp_path / "mutant.c"
    mut_c.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                    "-o", str(so), str(mut_c), "-lm"], check=True)
    env = dict(os.environ, FP8BS_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] +
                       [os.path.join(ROOT, "tests", f) for f in PIN_FILES],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
