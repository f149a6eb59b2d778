"""The CPU oracle checked against facts fixed outside itself (CPU only).

The pins live in tests/oracle_pins.py.  The mutation test below plants one
plausible mistake at a time into a copy of oracle.c (a dropped term, a wrong
sign, a wrong index, a swapped operand, a wrong exponent bias...), builds it,
and requires that at least one pin rejects every such build.
"""
import os
import subprocess

import pytest

import oracle
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# (text in oracle.c, replacement, what the mistake is)
MUTANTS = [
    ("p_out[j] = scale * acc;", "p_out[j] = acc;", "scale dropped"),
    ("p_out[j] = exp(p_out[j] - m);", "p_out[j] = exp(p_out[j] + m);", "wrong sign of max shift"),
    ("if (p_out[j] > m)", "if (p_out[j] < m)", "row min instead of row max"),
    ("acc += qrow[t] * kr[t];", "acc += qrow[t] * kr[d - 1 - t];", "wrong K column index"),
    ("p_out[j] /= z;", "p_out[j] /= 1.0;", "softmax normalisation dropped"),
    ("o_out[t] += pj * vr[t];", "o_out[t] += pj * vr[0];", "wrong V column index"),
    ("*lse_out = m + log(z);", "*lse_out = log(z);", "row max dropped from LSE"),
    ("Vd[j * d + t] = elem(v, dtype, (head * N + j) * d + t);",
     "Vd[j * d + t] = elem(v, dtype, (head * N + (N - 1 - j)) * d + t);", "V rows not paired with K rows"),
    ("mag = ldexp((double)(f | 0x400), e - 25);", "mag = ldexp((double)(f | 0x400), e - 24);",
     "binary16 exponent bias off by one"),
    ("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;", "bfloat16 widening shift"),
    ("mag = ldexp((double)f, -24);", "mag = ldexp((double)f, -23);", "binary16 subnormals doubled"),
    ("                int64_t g = rows ? rows[r] : r;",
     "                int64_t g = rows ? rows[r0] : r;", "selected rows all take the group's first query"),
    ("double alpha = exp(m - m_ij);", "double alpha = exp(m_ij - m);", "online rescale sign"),
    ("Oi[t] *= alpha;", "Oi[t] *= 1.0;", "online O rescale dropped"),
    ("l = alpha * l + rowsum;", "l = l + rowsum;", "online l rescale dropped"),
    # backward (oracle_attention_bwd)
    ("const double ds = prow[j] * (dprow[j] - Di);", "const double ds = prow[j] * dprow[j];",
     "softmax Jacobian row term dropped"),
    ("const double ds = prow[j] * (dprow[j] - Di);", "const double ds = prow[j] * (Di - dprow[j]);",
     "dS sign flipped"),
    ("Di += prow[j] * acc;", "Di += acc;", "row term not weighted by P"),
    ("acc += gi[t] * vj[t];", "acc += gi[t] * vj[d - 1 - t];", "wrong V column in dP"),
    ("dQh[i * d + t] += scale * ds * kj[t];", "dQh[i * d + t] += scale * ds * qi[t];",
     "dQ built from Q instead of K"),
    ("dkj[t] += scale * ds * qi[t];", "dkj[t] += ds * qi[t];", "scale dropped from dK"),
    ("dvj[t] += prow[j] * gi[t];", "dvj[t] += ds * gi[t];", "dV built from dS instead of P"),
    ("dOd[t] = (double)dout[head * N * d + t];", "dOd[t] = (double)dout[t];",
     "dO of head 0 used for every head"),
]


def _pins_reject():
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, RuntimeError, FloatingPointError, ValueError) as e:
            failed.append(f"{pin.__name__}: {str(e)[:80]}")
    return failed


@pytest.mark.parametrize("needle,repl,what", MUTANTS, ids=[m[2] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, needle, repl, what):
    src = open(oracle._SRC).read()
    assert src.count(needle) == 1, f"mutation site for '{what}' not found exactly once"
    mutant_c = tmp_path / "mutant.c"
    mutant_c.write_text(src.replace(needle, repl))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(mutant_c), "-o",
                    str(so), "-lm"], check=True)
    prev = oracle.use_library(str(so))
    try:
        failed = _pins_reject()
    finally:
        oracle.restore_library(prev)
    assert failed, f"no pin caught the planted mistake: {what}"
