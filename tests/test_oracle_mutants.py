"""Planted mistakes in a copy of the oracle must each be caught by at least one pin (CPU only).

Each mutation edits one expression of oracle.c in a temporary copy (the kinds of slip a
reader checking the oracle against the definition would look for: a dropped term, a wrong
sign, an off-by-one mask, a wrong index, a swapped operand), compiles it with gcc and runs
the pins of ``oracle_pins`` on it.
"""
import os

import pytest

import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTATIONS = [
    ("drop scale in scores", "s[j] = J->scale * dot(qi, Kh + j * J->d, J->d);", "s[j] = dot(qi, Kh + j * J->d, J->d);"),
    ("causal mask excludes the diagonal", "return J->causal ? i + 1 : J->N;", "return J->causal ? (i > 0 ? i : 1) : J->N;"),
    ("causal mask lets one future key in", "return J->causal ? i + 1 : J->N;", "return J->causal ? (i + 2 < J->N ? i + 2 : J->N) : J->N;"),
    ("no softmax normalisation", "o[c] = acc[c] / l;", "o[c] = acc[c];"),
    ("LSE without the max", "J->out1[slice * J->nrows + r] = m + log(l);", "J->out1[slice * J->nrows + r] = log(l);"),
    ("LSE in base 2", "J->out1[slice * J->nrows + r] = m + log(l);", "J->out1[slice * J->nrows + r] = m + log2(l);"),
    ("max subtracted with wrong sign", "for (int64_t j = j0; j < nvis; ++j) {\n    s[j] = exp(s[j] - m);",
     "for (int64_t j = j0; j < nvis; ++j) {\n    s[j] = exp(s[j] + m);"),
    ("decode max subtracted with wrong sign", "for (int64_t j = 0; j < nvis; ++j) {\n          s[j] = exp(s[j] - m);",
     "for (int64_t j = 0; j < nvis; ++j) {\n          s[j] = exp(s[j] + m);"),
    ("value columns reversed", "acc[c] += s[j] * Vh[j * d + c];", "acc[c] += s[j] * Vh[j * d + (d - 1 - c)];"),
    ("GQA heads interleaved", "int64_t b = slice / J->Hq, hq = slice % J->Hq, g = hq / group;\n    int64_t i = J->rows",
     "int64_t b = slice / J->Hq, hq = slice % J->Hq, g = hq % J->Hkv;\n    int64_t i = J->rows"),
    ("dQ missing scale", "dq[c] = J->scale * acc[c];", "dq[c] = acc[c];"),
    ("dS with + D", "double dS = P * (dP - Di);", "double dS = P * (dP + Di);"),
    ("dQ uses V instead of K", "acc[c] += dS * Kh[j * d + c];", "acc[c] += dS * Vh[j * d + c];"),
    ("row statistics ignore the chosen rows",
     "int64_t i = J->rows[slice * J->nrows + r];\n    int64_t b = slice / J->Hq, hq = slice % J->Hq, g = hq / group;\n    const double* qi = J->q + (slice * N + i) * d;\n    const double* dOi",
     "int64_t i = r;\n    int64_t b = slice / J->Hq, hq = slice % J->Hq, g = hq / group;\n    const double* qi = J->q + (slice * N + i) * d;\n    const double* dOi"),
    ("D without 1/l", "D += (s[j] / l) * dot(dOi, Vh + j * d, d);", "D += s[j] * dot(dOi, Vh + j * d, d);"),
    ("dK uses dO instead of Q", "dk[c] += dS * qi[c];", "dk[c] += dS * dOi[c];"),
    ("dV uses Q instead of dO", "dv[c] += P * dOi[c];", "dv[c] += P * qi[c];"),
    ("dV from dS instead of P", "dv[c] += P * dOi[c];", "dv[c] += dS * dOi[c];"),
    ("dK/dV causal start off by one", "int64_t i0 = J->causal ? j : 0;", "int64_t i0 = J->causal ? j + 1 : 0;"),
    ("dK missing scale", "odk[c] = J->scale * dk[c];", "odk[c] = dk[c];"),
    ("dK/dV only first head of the group", "for (int64_t hq = g * group; hq < (g + 1) * group; ++hq) {",
     "for (int64_t hq = g * group; hq < g * group + 1; ++hq) {"),
    ("P without the row max", "double P = exp(sij - J->m[slice * N + i]) / J->l[slice * N + i];",
     "double P = exp(sij) / J->l[slice * N + i];"),
    ("window start one key late", "return (J->window >= 0 && i > J->window) ? i - J->window : 0;",
     "return (J->window >= 0 && i >= J->window) ? i - J->window + 1 : 0;"),
    ("window start one key early", "return (J->window >= 0 && i > J->window) ? i - J->window : 0;",
     "return (J->window >= 0 && i > J->window + 1) ? i - J->window - 1 : 0;"),
    ("window ignored by dK/dV", "int64_t i1 = last_query(J, j);", "int64_t i1 = N;"),
    ("dK/dV window end one row short", "? j + J->window + 1 : J->N;", "? j + J->window : J->N;"),
    ("decode causal aligned to the start", "const int64_t nvis = causal ? Nk - Nq + i + 1 : Nk;",
     "const int64_t nvis = causal ? i + 1 : Nk;"),
    ("decode causal one key short", "const int64_t nvis = causal ? Nk - Nq + i + 1 : Nk;",
     "const int64_t nvis = causal ? Nk - Nq + i : Nk;"),
    ("decode without normalisation", "oi[c] = acc / l;", "oi[c] = acc;"),
    ("decode GQA head mapping", "const int64_t g = hq / group;\n      const double* Kh = k + (b * Hkv + g) * Nk * d;",
     "const int64_t g = hq % Hkv;\n      const double* Kh = k + (b * Hkv + g) * Nk * d;"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor not unique/not found: " + name
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = oracle.compile_library(str(path), str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            if pin is oracle_pins.pin_finite_differences:
                pin(orc, shapes=[(1, 2, 1, 5, 2), (1, 2, 2, 3, 4)])
            else:
                pin(orc)
        except (AssertionError, FloatingPointError, ValueError, RuntimeError):
            caught.append(pin.__name__)
    assert caught, "planted mistake not caught by any pin: " + name
