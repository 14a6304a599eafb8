"""Plant mistakes in copies of the oracle and show the pins catch every one.

Each mutant is ``oracle/oracle.c`` with one plausible slip (a dropped decay, a
wrong exponent, a transposed operand, reading before writing, a misplaced
eps, a wrong feature map branch, an over-decayed ragged tail ...), built with
gcc into a temporary directory.  The whole pin battery then runs against it
and at least one pin must fail.  Mutants are CPU-only and never leave the
temporary directory.
"""
import os
import subprocess

import pytest

import oracle
from tests import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text to find -- must occur exactly once, replacement)
MUTANTS = [
    ("recurrent_drops_gamma",
     "S[i * dv + j] = g * S[i * dv + j] + kt[i] * vt[j];",
     "S[i * dv + j] = S[i * dv + j] + kt[i] * vt[j];"),
    ("recurrent_reads_before_write",
     "acc += qt[i] * S[i * dv + j];",
     "acc += qt[i] * (S[i * dv + j] - kt[i] * vt[j]);"),
    ("recurrent_transposed_outer_product",
     "S[i * dv + j] = g * S[i * dv + j] + kt[i] * vt[j];",
     "S[i * dv + j] = g * S[i * dv + j] + kt[j % dk] * vt[i % dv];"),
    ("recurrent_ignores_initial_state",
     "        if (init_state)\n",
     "        if (0 && init_state)\n"),
    ("parallel_exponent_off_by_one",
     "const double d_nm = pow(g, (double)(n - m));",
     "const double d_nm = pow(g, (double)(n - m + 1));"),
    ("parallel_mask_excludes_diagonal",
     "for (long m = 0; m <= n; ++m) {",
     "for (long m = 0; m < n; ++m) {"),
    ("rows_exponent_sign",
     "const double w = score * pow(g, (double)(t - s));",
     "const double w = score * pow(g, (double)(s - t));"),
    ("chunk_inter_decay_off_by_one",
     "const double xi = pow(g, (double)(i + 1));",
     "const double xi = pow(g, (double)i);"),
    ("chunk_state_zeta_off_by_one",
     "const double zeta = pow(g, (double)(c - 1 - j));",
     "const double zeta = pow(g, (double)(c - j));"),
    ("chunk_state_decay_off_by_one",
     "const double gc = pow(g, (double)c);",
     "const double gc = pow(g, (double)(c - 1));"),
    ("chunk_tail_over_decayed",
     "const double gc = pow(g, (double)c);",
     "const double gc = pow(g, (double)chunk);"),
    ("chunk_intra_decay_transposed",
     "const double w = score * pow(g, (double)(i - j));",
     "const double w = score * pow(g, (double)(j - i));"),
    ("decode_drops_gamma",
     "S[i * dv + j] = g * S[i * dv + j] + kn[i] * vn[j];",
     "S[i * dv + j] = S[i * dv + j] + kn[i] * vn[j];"),
    ("decode_reads_before_write",
     "acc += qn[i] * S[i * dv + j];",
     "acc += qn[i] * (S[i * dv + j] - kn[i] * vn[j]);"),
    ("phi_negative_branch_is_elu",
     "return x > 0.0 ? x + 1.0 : exp(x);",
     "return x > 0.0 ? x + 1.0 : exp(x) - 1.0;"),
    ("phi_forgets_plus_one",
     "return x > 0.0 ? x + 1.0 : exp(x);",
     "return x > 0.0 ? x : exp(x);"),
    ("linattn_drops_eps",
     "den += eps;",
     "den += 0.0;"),
    ("linattn_z_not_accumulated",
     "z[i] += pk[i];",
     "z[i] = pk[i];"),
    ("linattn_reads_before_write",
     "num += S[i * dv + j] * pq[i];",
     "num += (S[i * dv + j] - pk[i] * vt[j]) * pq[i];"),
    ("linattn_parallel_drops_eps",
     "ot[j] /= (rowsum + eps);",
     "ot[j] /= rowsum;"),
    ("linattn_ignores_initial_state",
     "        if (init_S)\n",
     "        if (0 && init_S)\n"),
    ("linattn_ignores_initial_normaliser",
     "        if (init_z)\n",
     "        if (0 && init_z)\n"),
    ("linattn_decode_reads_before_write",
     "num += Sn[i * dv + j] * fq[i];",
     "num += (Sn[i * dv + j] - fk[i] * vn[j]) * fq[i];"),
    ("linattn_decode_z_not_accumulated",
     "zn[i] += fk[i];",
     "zn[i] = fk[i];"),
    ("linattn_decode_drops_eps",
     "double den = eps;",
     "double den = 0.0;"),
    ("linattn_decode_raw_query",
     "fq[i] = phi_elu1(qn[i]);",
     "fq[i] = qn[i];"),
    ("linattn_decode_transposed_outer_product",
     "Sn[i * dv + j] += fk[i] * vn[j];",
     "Sn[i * dv + j] += fk[j % dk] * vn[i % dv];"),
    ("bwd_reverse_state_drops_gamma",
     "U[i * dv + j] = g * U[i * dv + j] + qt[i] * dot[j];",
     "U[i * dv + j] = U[i * dv + j] + qt[i] * dot[j];"),
    ("bwd_reverse_state_excludes_own_token",
     "acc += U[i * dv + j] * vt[j];",
     "acc += (U[i * dv + j] - qt[i] * dot[j]) * vt[j];"),
    ("bwd_dv_reads_transposed_state",
     "acc += U[i * dv + j] * kt[i];",
     "acc += U[(i * dv + j) % (dk * dv)] * kt[(i + 1) % dk];"),
    ("bwd_dq_uses_state_before_token",
     "acc += Sf[i * dv + j] * dot[j];",
     "acc += (Sf[i * dv + j] - kt[i] * vt[j]) * dot[j];"),
    ("bwd_forward_state_drops_gamma",
     "Sf[i * dv + j] = g * Sf[i * dv + j] + kt[i] * vt[j];",
     "Sf[i * dv + j] = Sf[i * dv + j] + kt[i] * vt[j];"),
    ("norm_floor_missing",
     "const double den = fabs(r) > 1.0 ? fabs(r) : 1.0;",
     "const double den = fabs(r) > 0.0 ? fabs(r) : 1.0;"),
    ("norm_sign_kept",
     "const double den = fabs(r) > 1.0 ? fabs(r) : 1.0;",
     "const double den = fabs(r) > 1.0 ? r : 1.0;"),
    ("norm_sum_not_decayed",
     "n[i] = g * n[i] + kt[i];",
     "n[i] = n[i] + kt[i];"),
    ("norm_groupnorm_sample_variance",
     "var /= (double)dv;",
     "var /= (double)(dv - 1);"),
    ("norm_groupnorm_eps_outside_sqrt",
     "const double rstd = 1.0 / sqrt(var + eps);",
     "const double rstd = 1.0 / (sqrt(var) + eps);"),
    ("gla_gate_on_value_axis",
     "const double a = exp(gt[i]);\n                for (long j = 0; j < dv; ++j)\n                    Sg[i * dv + j] = a * Sg[i * dv + j] + kt[i] * vt[j];",
     "for (long j = 0; j < dv; ++j)\n                    Sg[i * dv + j] = exp(gt[j % dk]) * Sg[i * dv + j] + kt[i] * vt[j];"),
    ("gla_gate_applied_after_write",
     "Sg[i * dv + j] = a * Sg[i * dv + j] + kt[i] * vt[j];",
     "Sg[i * dv + j] = a * (Sg[i * dv + j] + kt[i] * vt[j]);"),
    ("gla_gate_not_exponentiated",
     "const double a = exp(gt[i]);",
     "const double a = 1.0 + gt[i];"),
    ("linattn_rows_doubles_eps",
     "o[j] /= (rowsum + eps);",
     "o[j] /= (rowsum + 2.0 * eps);"),
]


def _build_mutant(tmp_path, name, find, repl):
    src = open(SRC).read()
    assert src.count(find) == 1, f"mutation {name}: pattern occurs {src.count(find)} times"
    mutated = src.replace(find, repl)
    c = tmp_path / f"{name}.c"
    c.write_text(mutated)
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", str(so),
                    str(c), "-lm"], check=True, capture_output=True)
    return str(so)


@pytest.mark.parametrize("name,find,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, find, repl):
    so = _build_mutant(tmp_path, name, find, repl)
    caught = []
    with oracle.using_library(so):
        for pin in pins.ALL_PINS:
            try:
                pin()
            except (AssertionError, RuntimeError, FloatingPointError, ValueError):
                caught.append(pin.__name__)
                break
    assert caught, f"no pin caught the planted mistake {name!r}"
