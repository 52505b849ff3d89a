"""Mutation check of the oracle's pins (no GPU).

Each mutant is a copy of ``oracle/oracle.c`` with one plausible mistake planted
in it (a dropped term, a flipped order or tie rule, a transposed operand, an
overflowing int32 comparison, fp32 accumulation, lost value bits, four cosine-norm
mistakes).  The copy is
compiled in a temporary directory; at least one pin must fail against it.  The
real oracle is never modified.
"""
import os

import pytest

import oracle
from oracle import build as oracle_build
import oracle_pins

MUTANTS = {
    "drop_last_term": ("for (int64_t c = 0; c < d; ++c)", "for (int64_t c = 0; c < d - 1; ++c)"),
    "ascending_scores": ("if (a->score != b->score) return (a->score > b->score) ? -1 : 1;",
                         "if (a->score != b->score) return (a->score < b->score) ? -1 : 1;"),
    "tie_to_higher_index": ("    if (a->index != b->index) return (a->index < b->index) ? -1 : 1;\n    return 0;\n}\n\nstatic int better_first_int",
                            "    if (a->index != b->index) return (a->index > b->index) ? -1 : 1;\n    return 0;\n}\n\nstatic int better_first_int"),
    "transposed_corpus": ("acc += (double)row[c] * (double)query[c];",
                          "acc += (double)corpus[c * n + i] * (double)query[c];"),
    "int32_subtraction_compare": ("if (a->value != b->value) return (a->value > b->value) ? -1 : 1;\n    if (a->index != b->index) return (a->index < b->index) ? -1 : 1;\n    return 0;\n}\n\nstatic int better_first_float",
                                  "if (a->value != b->value) return ((int32_t)((uint32_t)(int32_t)b->value - (uint32_t)(int32_t)a->value) < 0) ? -1 : 1;\n    if (a->index != b->index) return (a->index < b->index) ? -1 : 1;\n    return 0;\n}\n\nstatic int better_first_float"),
    "fp32_accumulator": ("double acc = 0.0;", "float acc = 0.0f;"),
    "value_bits_lost": ("memcpy(&out_val[r], &values[items[r].index], sizeof(float));",
                        "out_val[r] = items[r].value + 0.0f;"),
    "wrong_query_index": ("(double)query[c]", "(double)query[d - 1 - c]"),
    "cosine_no_query_norm": ("const double denom = q_norm * sqrt(r_sq);", "const double denom = sqrt(r_sq);"),
    "cosine_squared_norms": ("const double q_norm = sqrt(q_sq);", "const double q_norm = q_sq;"),
    "cosine_zero_norm_scores_zero": ("scores[i] / denom : -INFINITY;", "scores[i] / denom : 0.0;"),
    "cosine_row_norm_uses_query": ("r_sq += (double)row[c] * (double)row[c];",
                                   "r_sq += (double)row[c] * (double)query[c];"),
}


def _build_mutant(tmp_path, name):
    src = open(oracle_build.SOURCE).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new, 1)
    path = os.path.join(tmp_path, f"oracle_{name}.c")
    with open(path, "w") as f:
        f.write(mutated)
    out = os.path.join(tmp_path, f"liboracle_{name}.so")
    oracle_build.build(source=path, out=out, extra_cflags=("-w",), quiet=True)
    return oracle.Oracle(out)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    mutant = _build_mutant(str(tmp_path), name)
    failures = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, RuntimeError, ValueError, IndexError):
            failures.append(pin.__name__)
    assert failures, f"no pin caught mutant {name}"
