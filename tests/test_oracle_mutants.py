"""Plant plausible mistakes in a copy of the oracle and make sure the pins
catch every one of them.  Runs on the CPU only; the real oracle is untouched.
"""
import ctypes
import subprocess
from pathlib import Path

import pytest

import oracle
from tests import oracle_pins

SRC = Path(oracle.__file__).resolve().parent / "gdr_oracle.c"

# (name, text in gdr_oracle.c, replacement): each is a mistake someone could
# plausibly make when writing the recurrence from the pages.
MUTANTS = [
    ("no_decay", "S[i * dv + j] *= a;", "S[i * dv + j] *= 1.0;"),
    ("predict_from_undecayed", "acc += S[i * dv + j] * k[i];",
     "acc += S[i * dv + j] * k[i] / exp(g[i]);"),
    ("delta_sign", "(v[j] - vhat[j])", "(v[j] + vhat[j])"),
    ("beta_dropped", "beta * k[i] * (v[j] - vhat[j])", "k[i] * (v[j] - vhat[j])"),
    ("read_pre_update", "acc += S[i * dv + j] * q[i];",
     "acc += (S[i * dv + j] - beta * k[i] * (v[j] - vhat[j])) * q[i];"),
    ("transposed_state_predict", "acc += S[i * dv + j] * k[i];", "acc += S[j * dv + i] * k[i];"),
    ("transposed_state_read", "acc += S[i * dv + j] * q[i];", "acc += S[j * dv + i] * q[i];"),
    ("scale_dropped", "o[j] = scale * acc;", "o[j] = acc;"),
    ("head_repeat_tiled", "const int hq = h / rep;", "const int hq = h % Hqk;"),
    ("v_head_index", "(bt * Hv + h) * dv", "(bt * Hv + hq) * dv"),
    ("q_normalised_by_k", "orc_l2norm(qt, dk, qn);", "orc_l2norm(kt, dk, qn);"),
    ("l2_eps_dropped", "sqrt(ss + ORC_L2_EPS)", "sqrt(ss)"),
    ("sigmoid_sign", "1.0 / (1.0 + exp(-x))", "1.0 / (1.0 + exp(x))"),
    ("softplus_branch", "log1p(exp(-z))", "log1p(exp(z))"),
    ("fused_gate_sign", "double g = -exp(A_log_h)", "double g = exp(A_log_h)"),
    ("fused_gate_no_exp", "double g = -exp(A_log_h)", "double g = -(A_log_h)"),
    ("qk_split_swapped", "const double* qt = qkv + b * row + (size_t)hq * dk;",
     "const double* qt = qkv + b * row + (size_t)Hqk * dk + (size_t)hq * dk;"),
    ("scalar_gate_as_zero", "for (int i = 0; i < dk; ++i) g_out[i] = gate_sc;",
     "for (int i = 0; i < dk; ++i) g_out[i] = 0.0;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, tmp_path, monkeypatch):
    text = SRC.read_text()
    assert text.count(old) >= 1, f"mutation site for {name} not found"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(text.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", str(mutant),
                    "-o", str(so), "-lm"], check=True)
    monkeypatch.setattr(oracle, "_lib", oracle._bind(ctypes.CDLL(str(so))))
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check()
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(check.__name__)
    assert caught, f"no pin caught mutant {name}"
