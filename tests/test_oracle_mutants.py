"""Planted mistakes in the oracle must be caught by its pins (CPU).

Each mutant is a copy of ``oracle/lion_oracle.c`` with one plausible mistake (a dropped term, a
wrong sign, a shifted index, a swapped operand), built into a temporary library.  The test
requires at least one pin in ``oracle_pins.py`` to fail on every mutant, so that a passing pin
set says something about the oracle rather than about itself.  The mistakes live only in these
temporary copies; the oracle source is never modified.
"""
import os
import tempfile

import pytest

import oracle
from tests.oracle_pins import ALL_PINS

MUTANTS = [
    ("mask forward index shifted", "causal ? 0.0 : m[j - 1] * lam[j];", "causal ? 0.0 : m[j - 1] * lam[j - 1];"),
    ("causal keeps later keys", "causal ? 0.0 : m[j - 1] * lam[j];", "m[j - 1] * lam[j];"),
    ("causal masks earlier keys", "m[j] = m[j + 1] * lam[j + 1];", "m[j] = causal ? 0.0 : m[j + 1] * lam[j + 1];"),
    ("mask backward index shifted", "m[j] = m[j + 1] * lam[j + 1];", "m[j] = m[j + 1] * lam[j];"),
    ("mask diagonal not one", "m[i] = 1.0;", "m[i] = 0.5;"),
    ("eps dropped", "div = den + eps;", "div = den;"),
    ("eps subtracted", "div = den + eps;", "div = den - eps;"),
    ("elu+1 loses the +1", "x[c] > 0.0 ? x[c] + 1.0 : exp(x[c])", "x[c] > 0.0 ? x[c] : exp(x[c])"),
    ("elu branch flipped", "x[c] > 0.0 ? x[c] + 1.0 : exp(x[c])", "x[c] < 0.0 ? x[c] + 1.0 : exp(x[c])"),
    ("silu sign", "out[c] = x[c] / (1.0 + exp(-x[c]));", "out[c] = x[c] / (1.0 + exp(x[c]));"),
    ("norm without sqrt", "nrm = sqrt(ss);\n        for (c = 0; c < d; ++c)\n            out[c]",
     "nrm = ss;\n        for (c = 0; c < d; ++c)\n            out[c]"),
    ("score uses v for k", "s += phq_i[c] * kj[c];", "s += phq_i[c] * vj[c];"),
    ("numerator uses k for v", "num[c] += p * vj[c];", "num[c] += p * kj[c];"),
    ("row sum of |P|", "den += p;", "den += pa;"),
    ("mask not applied", "p = s * m[j];", "p = s;"),
    ("per-head decay indexed by batch", "lam[t] = exp(log_lambda[bh % H]);", "lam[t] = exp(log_lambda[bh / H]);"),
    ("per-token decays reversed", "lam[t] = exp(log_lambda[(size_t)bh * L + t]);",
     "lam[t] = exp(log_lambda[(size_t)bh * L + (L - 1 - t)]);"),
    ("decay not exponentiated", "lam[t] = exp(log_lambda[(size_t)bh * L + t]);",
     "lam[t] = -log_lambda[(size_t)bh * L + t];"),
    ("keys of the query row", "phi_row(mask_kind, k + (base + j) * d, d, phk + (size_t)j * d);",
     "phi_row(mask_kind, q + (base + j) * d, d, phk + (size_t)j * d);"),
    ("absolute score drops a factor", "sa += fabs(phq_i[c]) * fabs(kj[c]);", "sa += fabs(phq_i[c]);"),
    ("abs numerator without |v|", "anum[c] += pa * fabs(vj[c]);", "anum[c] += pa * vj[c];"),
    ("bwd delta term dropped", "dp = gv - delta;", "dp = gv;"),
    ("bwd dv without the mask", "dv[(base + j) * d + c] += m[j] * s[j] * g[c];", "dv[(base + j) * d + c] += s[j] * g[c];"),
    ("bwd silu derivative wrong", "dx[c] = nrm > 0.0 ? sig * (1.0 + x[c] * (1.0 - sig))",
     "dx[c] = nrm > 0.0 ? sig * (1.0 + x[c] * sig)"),
    ("bwd norm projection dropped", "(g[c] - ph * pg) / nrm", "g[c] / nrm"),
    ("bwd elu derivative flat", "g[c] * (x[c] > 0.0 ? 1.0 : exp(x[c]))", "g[c] * 1.0"),
    ("bwd decay range off by one", "diff[lo + 1] += w;", "diff[lo] += w;"),
    ("bwd key grad from its own phi", "dphk[(size_t)j * d + c] += ds * pq[c];",
     "dphk[(size_t)j * d + c] += ds * phk[(size_t)j * d + c];"),
    ("bwd per-head decay from one batch entry", "for (b2 = 0; b2 < B; ++b2)", "for (b2 = 0; b2 < 1; ++b2)"),
    ("selectivity bias dropped", "double z = bias[h], ll, ks;", "double z = 0.0, ll, ks;"),
    ("selectivity log sigmoid sign", "ll = z >= 0.0 ? -log1p(exp(-z)) : z - log1p(exp(z));",
     "ll = z >= 0.0 ? -log1p(exp(z)) : z - log1p(exp(z));"),
    ("selectivity key scale is lambda", "ks = -1.0 / (1.0 + exp(z));", "ks = 1.0 / (1.0 + exp(-z));"),
    ("selectivity weights of the wrong head", "z += xi[c] * w[(size_t)h * Dm + c];", "z += xi[c] * w[c];"),
    ("two-order mask ignores the second order", "m[j] = 0.5 * (mb[j] + mc[pos[j]]);", "m[j] = 0.5 * (mb[j] + mb[j]);"),
    ("two-order decays not permuted", "lamc[p] = lam[order[p]];", "lamc[p] = lam[p];"),
    ("two-order key position not mapped", "m[j] = 0.5 * (mb[j] + mc[pos[j]]);", "m[j] = 0.5 * (mb[j] + mc[j]);"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, oracle_lib):
    with open(oracle.SRC) as fh:
        src = fh.read()
    assert src.count(old) == 1, f"mutation site for '{name}' not unique or missing"
    with tempfile.TemporaryDirectory() as tmp:
        msrc = os.path.join(tmp, "mutant.c")
        mlib = os.path.join(tmp, "libmutant.so")
        with open(msrc, "w") as fh:
            fh.write(src.replace(old, new))
        oracle.build(src=msrc, out=mlib)
        caught = []
        for pin in ALL_PINS:
            try:
                pin(mlib)
            except AssertionError:
                caught.append(pin.__name__)
            except (ValueError, FloatingPointError, ZeroDivisionError):
                caught.append(pin.__name__ + " (error)")
    assert caught, f"no pin caught the planted mistake '{name}'"
