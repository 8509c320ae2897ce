"""The pins are strong enough: each plausible mistake planted in a copy of the
oracle's source (on the CPU, in a temporary directory) is caught by at least
one pin.  The real oracle is never modified."""
import os

import pytest

import oracle
from tests import pins

# (name, exact source text, replacement)
MUTANTS = [
    ("input_gate_dropped", "row[b] = fp * row[b] + ip * kt[a] * vt[b];",
     "row[b] = fp * row[b] + kt[a] * vt[b];"),
    ("forget_dropped_in_n", "n[a] = fp * n[a] + ip * kt[a];", "n[a] = n[a] + ip * kt[a];"),
    ("stabilizer_forgets_past", "double m_new = fmax(fg[t] + m, ig[t]);",
     "double m_new = fmax(fg[t], ig[t]);"),
    ("floor_one_on_stabilized", "double den = fmax(fabs(nq), exp(-m));",
     "double den = fmax(fabs(nq), 1.0);"),
    ("abs_dropped", "double den = fmax(fabs(nq), exp(-m));", "double den = fmax(nq, exp(-m));"),
    ("key_read_out", "num[b] += row[b] * qt[a];", "num[b] += row[b] * kt[a];"),
    ("memory_transposed", "num[b] += row[b] * qt[a];", "num[b] += C[b * dk + a] * qt[a];"),
    ("output_gate_exp", "ht[b] = sigmoid(ot[b]) * num[b] / den;", "ht[b] = exp(ot[b]) * num[b] / den;"),
    ("forget_sigmoid", "double fp = exp(fg[t] + m - m_new);",
     "double fp = sigmoid(fg[t] + m - m_new);"),
    ("stabilizer_not_carried", "m = m_new;", "m = 0.0;"),
    ("input_gate_off_by_one", "double ip = exp(ig[t] - m_new);",
     "double ip = exp(ig[t > 0 ? t - 1 : 0] - m_new);"),
    ("initial_m_ignored", "m = m0[p];", "m = 0.0 * m0[p];"),
    ("normalizer_half", "nq += n[a] * qt[a];", "nq += 0.5 * n[a] * qt[a];"),
    ("forget_sign", "double fp = exp(fg[t] + m - m_new);", "double fp = exp(-fg[t] + m - m_new);"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    with open(oracle.SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mpath = os.path.join(tmp_path, "mutant.c")
    with open(mpath, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.build(src=mpath, out=os.path.join(tmp_path, f"libmut_{name}.so"),
                       extra_flags=("-Wno-error", "-w"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, FloatingPointError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
