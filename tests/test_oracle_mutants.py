"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies ``oracle/oracle.c``, applies one plausible mistake (a dropped
term, a wrong sign, index or bit order, a transposed operand, a wrong tie
rule), compiles the mutant into a temporary directory, swaps it in for the
real oracle library, and runs the pin tests of ``test_oracle.py`` against it.
At least one pin must fail for every mutant.  The real library is restored
afterwards; nothing here touches the GPU path.
"""
import os
import subprocess

import pytest

import oracle
import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "unpack_drops_straddle": ("v |= row[w + 1] << (32 - s);", "v |= 0;"),
    "unpack_msb_first": ("uint32_t v = row[w] >> s;", "uint32_t v = row[w] >> (32 - bits - s);"),
    "pack_msb_first": ("row[j >> 5] |= 1u << (j & 31);", "row[j >> 5] |= 1u << (31 - (j & 31));"),
    "dequant_drops_bias": ("return s * (double)q + b;", "return s * (double)q;"),
    "dequant_bias_sign": ("return s * (double)q + b;", "return s * (double)q - b;"),
    "dequant_wrong_group": ("row_scales[k / 64]", "row_scales[0]"),
    "dequant_zero_point_form": ("return s * (double)q + b;", "return s * ((double)q - b);"),
    "affine_x_row_fixed": ("oracle_bf16_to_double(x[m * K + k]);\n                acc += p;",
                           "oracle_bf16_to_double(x[k]);\n                acc += p;"),
    "dense_transposed_W": ("double w = oracle_bf16_to_double(W[n * K + k]);",
                           "double w = oracle_bf16_to_double(W[k * N + n]);"),
    "dense_sign": ("double p = w * xv;\n                acc += p;", "double p = w * xv;\n                acc -= p;"),
    "abs_sum_signed": ("                aacc += fabs(p);\n            }\n            y[m * N + n] = acc;",
                       "                aacc += p;\n            }\n            y[m * N + n] = acc;"),
    "swiglu_exp_sign": ("exp(-ga)", "exp(ga)"),
    "swiglu_gate_up_swapped": ("out[i] = silu * ua;", "out[i] = (ua / (1.0 + exp(-ua))) * ga;"),
    "argmax_highest_tie": ("if (y[m * N + n] > y[m * N + best])", "if (y[m * N + n] >= y[m * N + best])"),
    "bf16_round_half_up": ("u += 0x7FFFu + lsb;", "u += 0x8000u + 0u * lsb;"),
    "bf16_truncate": ("u += 0x7FFFu + lsb;", "u += 0u * lsb;"),
    "swiglu_gate_abs_sum_signed": ("gaa += fabs(pg);\n                uaa += fabs(pu);\n            }\n            double silu = ga / (1.0 + exp(-ga));\n            int64_t i = m * N + n;\n            out[i] = silu * ua;\n            if (g) g[i] = ga;\n            if (u) u[i] = ua;\n            if (Ag) Ag[i] = gaa;\n            if (Au) Au[i] = uaa;\n        }\n    }\n}",
                                   "gaa += pg;\n                uaa += fabs(pu);\n            }\n            double silu = ga / (1.0 + exp(-ga));\n            int64_t i = m * N + n;\n            out[i] = silu * ua;\n            if (g) g[i] = ga;\n            if (u) u[i] = ua;\n            if (Ag) Ag[i] = gaa;\n            if (Au) Au[i] = uaa;\n        }\n    }\n}"),
    "swiglu_up_abs_sum_from_gate": ("                uaa += fabs(pu);\n            }\n            double silu = ga / (1.0 + exp(-ga));\n            int64_t i = m * N + n;\n            out[i] = silu * ua;\n            if (g) g[i] = ga;\n            if (u) u[i] = ua;\n            if (Ag) Ag[i] = gaa;\n            if (Au) Au[i] = uaa;\n        }\n    }\n}",
                                    "                uaa += fabs(pg);\n            }\n            double silu = ga / (1.0 + exp(-ga));\n            int64_t i = m * N + n;\n            out[i] = silu * ua;\n            if (g) g[i] = ga;\n            if (u) u[i] = ua;\n            if (Ag) Ag[i] = gaa;\n            if (Au) Au[i] = uaa;\n        }\n    }\n}"),
    "swiglu_abs_sums_swapped": ("            if (Ag) Ag[i] = gaa;\n            if (Au) Au[i] = uaa;\n        }\n    }\n}\n\n/* Unfused SwiGLU chain over two affine",
                                "            if (Ag) Ag[i] = uaa;\n            if (Au) Au[i] = gaa;\n        }\n    }\n}\n\n/* Unfused SwiGLU chain over two affine"),
    "swiglu_affine_up_uses_gate_scales": ("dequant(bits, Wuq + n * wpr, su + n * gpr", "dequant(bits, Wuq + n * wpr, sg + n * gpr"),
    "swiglu_affine_gate_drops_bias": ("dequant(bits, Wgq + n * wpr, sg + n * gpr, bg + n * gpr, k)",
                                      "dequant(bits, Wgq + n * wpr, sg + n * gpr, bg + n * gpr, k) - oracle_bf16_to_double(bg[n * gpr + k / 64])"),
    "swiglu_affine_gate_up_swapped": ("double silu = ga / (1.0 + exp(-ga));\n            int64_t i = m * N + n;\n            out[i] = silu * ua;\n            if (g) g[i] = ga;\n            if (u) u[i] = ua;\n            if (Ag) Ag[i] = gaa;\n            if (Au) Au[i] = uaa;\n        }\n    }\n    return 0;",
                                      "double silu = ua / (1.0 + exp(-ua));\n            int64_t i = m * N + n;\n            out[i] = silu * ga;\n            if (g) g[i] = ga;\n            if (u) u[i] = ua;\n            if (Ag) Ag[i] = gaa;\n            if (Au) Au[i] = uaa;\n        }\n    }\n    return 0;"),
}

# Pin tests to run against each mutant (all CPU, seconds in total).
PINS = [
    (pins.test_bf16_decode_all_patterns_match_torch, {}),
    (pins.test_f32_to_bf16_ties_to_even_by_hand, {}),
    (pins.test_affine_closed_form_all_equal_codes_exact, {}),
    (pins.test_dense_matches_numpy_matmul_and_abs_sum, {}),
    (pins.test_dense_one_hot_returns_weight_exactly, {}),
    (pins.test_swiglu_matches_numpy_chain, {}),
    (pins.test_swiglu_special_cases, {}),
    (pins.test_argmax_lowest_index_wins_ties_and_matches_numpy, {}),
    (pins.test_affine_scale_and_bias_are_per_group_and_per_row, {}),
    (pins.test_dense_matches_exact_brute_force, {}),
    (pins.test_swiglu_abs_sums_pinned, {}),
    (pins.test_swiglu_tolerance_covers_admissible_perturbations, {}),
]
for _b in (2, 3, 4, 5, 6, 7, 8):
    PINS += [
        (pins.test_pack_unpack_roundtrip_random_and_patterns, {"bits": _b}),
        (pins.test_unpack_of_random_words_matches_bigint_stream, {"bits": _b}),
        (pins.test_affine_zero_codes_give_bias_times_group_sums, {"bits": _b}),
        (pins.test_affine_unit_scale_zero_bias_is_integer_dot, {"bits": _b}),
        (pins.test_affine_matches_exact_brute_force_on_tiny_exact_inputs, {"bits": _b}),
        (pins.test_swiglu_affine_equals_dense_chain_on_exact_weights, {"bits": _b}),
    ]
for _b in (3, 4, 8):
    PINS.append((pins.test_swiglu_affine_streams_and_special_cases, {"bits": _b}))
for _row in pins._golden_rows():
    PINS.append((pins.test_pack_worked_vectors, {"row": _row}))


def _build_mutant(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) >= 1, "mutation anchor not found: %s" % name
    mutated = text.replace(old, new)
    src = tmp_path / ("%s.c" % name)
    src.write_text(mutated)
    lib = tmp_path / ("lib%s.so" % name)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-w",
                    "-o", str(lib), str(src), "-lm"], check=True)
    return str(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    lib = oracle.bind(_build_mutant(tmp_path, name, old, new))
    monkeypatch.setattr(oracle, "_lib", lib)
    caught = []
    for fn, kwargs in PINS:
        try:
            fn(**kwargs)
        except AssertionError:
            caught.append(fn.__name__)
    assert caught, "no pin caught mutant %s" % name


# Planted mistakes in the propagated SwiGLU bound (oracle/__init__.py): each
# loosens or drops a term of swiglu_tolerance; the soundness pin must fail.
TOL_MUTANTS = {
    "slope_1_0": ("1.1 * tg", "1.0 * tg"),
    "gate_term_missing_tu": ("(np.abs(u) + tu)", "(np.abs(u))"),
    "up_term_dropped": ("np.abs(silu) * tu +", ""),
    "gate_term_dropped": ("1.1 * tg * (np.abs(u) + tu) +", ""),
    "up_term_uses_g": ("np.abs(silu) * tu", "np.abs(silu) * tg"),
}


@pytest.mark.parametrize("name", sorted(TOL_MUTANTS))
def test_bound_pin_catches_planted_mistake(name, monkeypatch):
    import inspect
    old, new = TOL_MUTANTS[name]
    src = inspect.getsource(oracle.swiglu_tolerance)
    assert src.count(old) == 1, "mutation anchor not found: %s" % name
    ns = {"np": oracle.np, "tolerance": oracle.tolerance}
    exec(src.replace(old, new), ns)
    monkeypatch.setattr(oracle, "swiglu_tolerance", ns["swiglu_tolerance"])
    with pytest.raises(AssertionError):
        pins.test_swiglu_tolerance_covers_admissible_perturbations()
