"""Plausible mistakes planted in copies of the oracle (on the CPU) must each be
caught by at least one pin.  This shows the pins constrain every part of the
oracle: the gate, the decay, the delta correction, the read-out, the head and
sequence indexing, the chunkwise solve, the bf16 rounding and the backward."""
import os
import shutil

import pytest

import oracle
from tests import oracle_pins

MUTANTS = {
    "gate_sign": ("g_min / (1.0 + exp(-x))", "g_min / (1.0 + exp(x))"),
    "gate_no_exp_A": ("const double s = exp(A[h]);", "const double s = A[h];"),
    "gate_exp_neg_A": ("const double s = exp(A[h]);", "const double s = exp(-A[h]);"),
    "gate_A_of_head_0": ("const double s = exp(A[h]);", "const double s = exp(A[0]);"),
    "decay_sign": ("const double a = exp(g[c]);", "const double a = exp(-g[c]);"),
    "decay_dropped": ("for (int j = 0; j < dv; ++j) row[j] *= a;",
                      "for (int j = 0; j < dv; ++j) row[j] *= 1.0;"),
    "delta_sign": ("u[j] = beta * (v[j] - u[j]);", "u[j] = beta * (v[j] + u[j]);"),
    "beta_dropped": ("u[j] = beta * (v[j] - u[j]);", "u[j] = (v[j] - u[j]);"),
    "erase_dropped": ("u[j] = beta * (v[j] - u[j]);", "u[j] = beta * v[j];"),
    "read_key_not_query": ("const double qc = q[c];", "const double qc = k[c];"),
    "head_index": ("const int n = (int)(w / H), h = (int)(w % H);\n        double* S = (double*)malloc(sizeof(double) * (size_t)(ssz + dv));",
                   "const int n = (int)(w / H), h = 0;\n        double* S = (double*)malloc(sizeof(double) * (size_t)(ssz + dv));"),
    "state_of_first_seq": ("if (S0) memcpy(S, S0 + w * ssz, sizeof(double) * (size_t)ssz);\n        else memset(S, 0, sizeof(double) * (size_t)ssz);\n        for (int64_t t = cu[n];",
                           "if (S0) memcpy(S, S0 + (w % H) * ssz, sizeof(double) * (size_t)ssz);\n        else memset(S, 0, sizeof(double) * (size_t)ssz);\n        for (int64_t t = cu[n];"),
    "wy_no_beta": ("double x = (r == j) ? beta[j * bstride] : 0.0;", "double x = (r == j) ? 1.0 : 0.0;"),
    "wy_decay_sign": ("s += k[r * ld + c] * k[i * ld + c] * exp(G[r * dk + c] - G[i * dk + c]);",
                      "s += k[r * ld + c] * k[i * ld + c] * exp(G[i * dk + c] - G[r * dk + c]);"),
    "chunk_P_no_diag": ("for (int i = 0; i <= r; ++i) s += P[r * L + i] * U[i * dv + jv];",
                        "for (int i = 0; i < r; ++i) s += P[r * L + i] * U[i * dv + jv];"),
    "chunk_state_no_decay": ("double s = exp(gl) * S[c * dv + jv];", "double s = S[c * dv + jv];"),
    "bf16_one_bit_short": ("int sc = e - 8;", "int sc = e - 7;"),
    "bwd_dk_no_erase_term": ("s += dS[c * dv + j] * u[j] + Sp[c * dv + j] * dw[j];",
                             "s += dS[c * dv + j] * u[j];"),
    "bwd_dw_sign": ("dw[j] = -bt * du[j];", "dw[j] = bt * du[j];"),
    "bwd_dbeta_uses_u": ("db += du[j] * r[j];", "db += du[j] * u[j];"),
    "bwd_no_decay_of_dS": ("dS[c * dv + j] = a[c] * dsp;", "dS[c * dv + j] = dsp;"),
    "bwd_dg_without_a": ("dg[th * dk + c] = a[c] * s;", "dg[th * dk + c] = s;"),
    "bwd_dq_before_update": ("s += Sc[c * dv + j] * dOt[j];", "s += Sp[c * dv + j] * dOt[j];"),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not unique in the oracle source"
    src = tmp_path / "mutant.c"
    src.write_text(source.replace(old, new))
    lib_path = str(tmp_path / "libmutant.so")
    oracle.build(str(src), lib_path)
    lib = oracle.load(lib_path)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
