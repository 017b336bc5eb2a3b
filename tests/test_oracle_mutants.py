"""Plants plausible mistakes in copies of the oracle and checks the pins catch every one.

Each mutant is a one-line text substitution in oracle/fwa_oracle.c (a dropped term, a wrong
sign or index, a swapped operand, a wrong constant).  The copy is compiled into a temporary
directory and every pin of tests/oracle_pins.py runs against it; at least one must fail.  The
substituted text must occur exactly once in the real source, so the list stays in step with it.
CPU only; the real oracle is never modified.
"""
import os

import pytest

import oracle
from oracle import build as obuild
from oracle_pins import ALL_PINS

MUTANTS = {
    "roll_direction_literal_formula": (
        "double p = x[j] * x[src];", "double p = x[j] * x[(j + i) % two_dk];"),
    "concat_k_k_instead_of_k_minus_k": (
        "x[d_k + j] = -k[j] > 0.0 ? -k[j] : 0.0;", "x[d_k + j] = k[j] > 0.0 ? k[j] : 0.0;"),
    "eps_as_max": (
        "phi[d] = phi[d] / (sum + ORACLE_DPFP_EPS);",
        "phi[d] = phi[d] / (sum > ORACLE_DPFP_EPS ? sum : ORACLE_DPFP_EPS);"),
    "eps_dropped": ("phi[d] = phi[d] / (sum + ORACLE_DPFP_EPS);", "phi[d] = phi[d] / sum;"),
    "eps_value": ("#define ORACLE_DPFP_EPS 1e-6", "#define ORACLE_DPFP_EPS 1e-5"),
    "blocks_interleaved": ("phi[(i - 1) * two_dk + j] = p;", "phi[j * nu + (i - 1)] = p;"),
    "read_before_write": (
        "for (int d = 0; d < D; ++d) s += W[(size_t)r * D + d] * phi_q[d];",
        "for (int d = 0; d < D; ++d) s += (W[(size_t)r * D + d] - beta * (v[r] - vbar[r]) * phi_k[d]) * phi_q[d];"),
    "delta_sign_flipped": (
        "double c = beta * (v[r] - vbar[r]);", "double c = beta * (vbar[r] - v[r]);"),
    "delta_term_dropped": ("double c = beta * (v[r] - vbar[r]);", "double c = beta * v[r];"),
    "beta_not_squashed": (
        "double beta = oracle_sigmoid(beta_logit[row]);", "double beta = beta_logit[row];"),
    "sigmoid_sign": ("if (l >= 0.0) return 1.0 / (1.0 + exp(-l));",
                     "if (l >= 0.0) return 1.0 / (1.0 + exp(l));"),
    "sigmoid_negative_branch": ("return e / (1.0 + e);", "return 1.0 / (1.0 + e);"),
    "retrieve_with_query": (
        "for (int d = 0; d < D; ++d) s += W[(size_t)r * D + d] * phi_k[d];",
        "for (int d = 0; d < D; ++d) s += W[(size_t)r * D + d] * phi_q[d];"),
    "initial_state_ignored": (
        "if (W0) memcpy(W, W0 + s * d_v * D", "if (0) memcpy(W, W0 + s * d_v * D"),
    "key_from_query": (
        "dpfp_one(k + row * d_k, pk, d_k, nu, work);", "dpfp_one(q + row * d_k, pk, d_k, nu, work);"),
    "value_time_shift": (
        "v + row * d_v, beta, y + row * d_v",
        "v + (s * T + (t + 1) % T) * d_v, beta, y + row * d_v"),
    "mask_predicate_sign": (
        "int pos_s = src < d_k ? (k[src] > 0.0) : (k[src - d_k] < 0.0);",
        "int pos_s = src < d_k ? (k[src] > 0.0) : (k[src - d_k] > 0.0);"),
    "step_beta_not_squashed": (
        "double beta = oracle_sigmoid(beta_logit[s]);", "double beta = beta_logit[s];"),
    # the reverse pass
    "bwd_retrieval_term_dropped": (
        "for (int d = 0; d < D; ++d) G[(size_t)r * D + d] += dvb * pk[d];",
        "for (int d = 0; d < D; ++d) G[(size_t)r * D + d] += 0.0 * pk[d];"),
    "bwd_key_grad_from_new_memory": (
        "sacc += P[(size_t)r * D + d] * (-beta * du[r]);",
        "sacc += N[(size_t)r * D + d] * (-beta * du[r]);"),
    "bwd_query_grad_from_old_memory": (
        "sacc += N[(size_t)r * D + d] * dyt[r];", "sacc += P[(size_t)r * D + d] * dyt[r];"),
    "bwd_dpfp_normaliser_term_dropped": (
        "double draw = (dphi[(i - 1) * two_dk + j] - dot) / den;",
        "double draw = dphi[(i - 1) * two_dk + j] / den;"),
    "bwd_dpfp_negative_half_sign": (
        "if (k[j] < 0.0) g -= dx[d_k + j];", "if (k[j] < 0.0) g += dx[d_k + j];"),
    "bwd_dpfp_rolled_factor": ("dx[src] += draw * x[j];", "dx[src] += draw * x[src];"),
    "bwd_sigmoid_derivative_dropped": (
        "dbeta_logit[row] = dbeta * beta * (1.0 - beta);", "dbeta_logit[row] = dbeta;"),
    "bwd_dv_missing_beta": ("dv[row * d_v + r] = beta * du[r];", "dv[row * d_v + r] = du[r];"),
    "bwd_dbeta_sign": ("dbeta += du[r] * (vt[r] - vbar[r]);", "dbeta += du[r] * (vbar[r] - vt[r]);"),
    "bwd_checkpoint_stale": (
        "memcpy(ck + (size_t)(t / ORACLE_CHECKPOINT) * WS, W, sizeof(double) * WS);",
        "if (t == 0) memcpy(ck + (size_t)(t / ORACLE_CHECKPOINT) * WS, W, sizeof(double) * WS);"),
    # sum-update linear attention
    "sum_normaliser_dropped": ("y[row * d_v + r] = den != 0.0 ? num / den : 0.0;",
                               "y[row * d_v + r] = num;"),
    "sum_z_not_updated": ("for (int d = 0; d < D; ++d) z[d] += pk[d];",
                          "for (int d = 0; d < D; ++d) z[d] += 0.0 * pk[d];"),
    "sum_z_from_query": ("for (int d = 0; d < D; ++d) z[d] += pk[d];",
                         "for (int d = 0; d < D; ++d) z[d] += pq[d];"),
    "sum_denominator_with_key": ("for (int d = 0; d < D; ++d) den += z[d] * pq[d];",
                                 "for (int d = 0; d < D; ++d) den += z[d] * pk[d];"),
    "sum_value_outer_query": ("for (int d = 0; d < D; ++d) W[(size_t)r * D + d] += vt[r] * pk[d];",
                              "for (int d = 0; d < D; ++d) W[(size_t)r * D + d] += vt[r] * pq[d];"),
    "sum_initial_z_ignored": ("if (z0) memcpy(z, z0 + s * D", "if (0) memcpy(z, z0 + s * D"),
    "sum_initial_state_ignored": ("if (W0) memcpy(W, W0 + (size_t)s * d_v * D",
                                  "if (0) memcpy(W, W0 + (size_t)s * d_v * D"),
    # projections
    "proj_head_split_transposed": (
        "q[((b * H + n / d_k) * T + t) * d_k + n % d_k] = s;",
        "q[((b * H + n % H) * T + t) * d_k + n / H] = s;"),
    "proj_key_block_offset": ("const int m = n - nq;", "const int m = n - nq + 1 < nq ? n - nq + 1 : n - nq;"),
    "proj_output_bias_dropped": ("if (bo) s += bo[n];", "if (0) s += bo[n];"),
    "proj_output_head_order": (
        "s += y[((b * H + kk / d_v) * T + t) * d_v + kk % d_v] * Wo[(int64_t)n * Kc + kk];",
        "s += y[((b * H + kk % H) * T + t) * d_v + kk / H] * Wo[(int64_t)n * Kc + kk];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/present"
    mpath = tmp_path / f"mutant_{name}.c"
    mpath.write_text(src.replace(old, new))
    lib = obuild.build(str(mpath), str(tmp_path / f"libmutant_{name}.so"), extra_flags=("-w",))
    O = oracle.Oracle(lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(O)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin detects mutant {name}"


def test_real_oracle_passes_all_pins():
    O = oracle.default()
    for pin in ALL_PINS:
        pin(O)
    assert os.path.exists(obuild.LIB)
