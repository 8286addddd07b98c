"""Mutation check of the oracle's pins.

Each case plants one plausible mistake in a temporary copy of the oracle's C
source (a dropped term, a wrong sign or lag, a wrong index, a transposed
operand), compiles it on the CPU, and asserts that at least one pin from
test_oracle_pins.py rejects it.  The committed oracle is never modified.
"""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import HEADWISE, LOWRANK, Shape
from tests import test_oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "dynconv_oracle.c")

# (name, text in the oracle source, replacement)
MUTANTS = [
    ("fwd_drops_residual", "double acc = x[row * D + c];", "double acc = 0.0;"),
    ("fwd_flips_taps", "acc += wt[c * k + j] * x[(row - j) * D + c];",
     "acc += wt[c * k + (k - 1 - j)] * x[(row - j) * D + c];"),
    ("fwd_drops_lag0_history", "if (t - j < 0 || !same_doc(s, row, row - j)) break;\n          acc += wt",
     "if ((t - j < 1 && j > 0) || !same_doc(s, row, row - j)) break;\n          acc += wt"),
    # packed documents: the window crosses a document start
    ("packed_fwd_ignores_documents", "if (t - j < 0 || !same_doc(s, row, row - j)) break;",
     "if (t - j < 0) break;"),
    ("packed_dx_ignores_documents", "if (t + j > T - 1 || !same_doc(s, row, row + j)) break;",
     "if (t + j > T - 1) break;"),
    ("packed_G_ignores_documents", "(((t_) - (j_) < 0 || !same_doc(s, (b_) * T + (t_), (b_) * T + (t_) - (j_)))",
     "(((t_) - (j_) < 0)"),
    ("packed_doc_off_by_one", "return s->doc == NULL || s->doc[r1] == s->doc[r2];",
     "return s->doc == NULL || s->doc[r1] == s->doc[r2 > 0 ? r2 - 1 : r2];"),
    # the producing projection: a transposed weight, a dropped row
    ("proj_transposed", "acc += h[t * d + i] * Wp[i * D + c];", "acc += h[t * d + i] * Wp[(c % d) * D + (i % D)];"),
    ("proj_drops_last_row", "for (int64_t i = 0; i < d; ++i) acc += h[t * d + i] * Wp",
     "for (int64_t i = 0; i < d - 1; ++i) acc += h[t * d + i] * Wp"),
    ("head_index_interleaved", "const int64_t e = c / hd;", "const int64_t e = c % s->n_heads;"),
    ("lowrank_U_transposed", "for (int64_t m = 0; m < D * k; ++m) wt[m] += zq * Uq[m];",
     "for (int64_t m = 0; m < D * k; ++m) wt[m] += zq * U[m * N + q];"),
    ("bias_dropped", "wt[m] += w0[m];", "wt[m] += 0.0 * w0[m];"),
    ("dx_uses_wrong_token_filter", "acc += w[(row + j) * D * k + c * k + j] * dy[(row + j) * D + c];",
     "acc += w[row * D * k + c * k + j] * dy[(row + j) * D + c];"),
    ("dx_drops_residual", "double acc = dy[row * D + c];", "double acc = 0.0;"),
    ("G_drops_lag", "x[((b_) * T + (t_) - (j_)) * D + (c_)])",
     "x[((b_) * T + (t_)) * D + (c_)])"),
    ("dW_wrong_row", "const double hi = h[t * d + i];\n          const double *gt",
     "const double hi = h[t * d + (d - 1 - i)];\n          const double *gt"),
    ("dz_flips_taps", "acc += G_AT(b, t, c, j) * U[q * D * k + c * k + j];",
     "acc += G_AT(b, t, c, j) * U[q * D * k + c * k + (k - 1 - j)];"),
    ("dU_wrong_rank_index", "const double zq = z[row * N + q];",
     "const double zq = z[row * N + (N - 1 - q)];"),
    ("dA_uses_z_for_dz", "for (int64_t q = 0; q < N; ++q) dAi[q] += hi * g[t * N + q];",
     "for (int64_t q = 0; q < N; ++q) dAi[q] += hi * z[t * N + q];"),
    ("dh_transposed", "acc += g[t * N + n] * M[i * N + n];",
     "acc += g[t * N + n] * M[(d - 1 - i) * N + n];"),
    ("dw0_sign", "for (int64_t t = 0; t < T; ++t) acc += G_AT(b, t, c, j);\n        dw0",
     "for (int64_t t = 0; t < T; ++t) acc -= G_AT(b, t, c, j);\n        dw0"),
]


def _battery(orc):
    """Run pins; return the names of those that fail."""
    failed = []

    def run(name, fn, *args):
        try:
            fn(orc, *args)
        except AssertionError:
            failed.append(name)

    for f in ("worked_headwise.json", "worked_lowrank.json"):
        run(f"golden:{f}", P.test_golden_worked_example, f)
    for s in P.SHAPES:
        run(f"static:{s}", P.test_zero_generator_is_static_conv, s)
        run(f"dense:{s}", P.test_dense_matrix_form, s)
        run(f"autograd:{s}", P.test_grads_match_torch_autograd, s)
        run(f"causal:{s}", P.test_causality, s)
    run("hw==lr", P.test_headwise_equals_lowrank)
    for base, lens in P.PACKED:
        run(f"packed:{lens}", P.test_packed_equals_documents_run_alone, base, lens)
    for s in P.SHAPES:
        run(f"proj:{s}", P.test_proj_is_matmul, s)
    return failed


@pytest.fixture(scope="module")
def src_text():
    return open(SRC).read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, src_text, name, old, new):
    assert src_text.count(old) == 1, f"mutation site for {name} not unique/present"
    mutated = src_text.replace(old, new)
    csrc = tmp_path / "mutant.c"
    csrc.write_text(mutated)
    lib = tmp_path / f"lib_{name}.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-w", "-o", str(lib),
                    str(csrc)], check=True)
    failed = _battery(oracle.OracleLib(str(lib)))
    assert failed, f"no pin caught mutant {name}"


def test_unmutated_oracle_passes_battery(orc):
    assert _battery(orc) == []
