"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pins catch every one of them.

Each mutant is the oracle's C source with one textual change, compiled into
a temporary library; the real oracle is untouched.
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")

MUTANTS = [
    ("scale dropped", "p[j] = scale * dot;", "p[j] = dot;"),
    ("scale squared", "p[j] = scale * dot;", "p[j] = scale * scale * dot;"),
    ("max added instead of subtracted", "p[j] = exp(p[j] - m);",
     "p[j] = exp(p[j] + m);"),
    ("no normalisation", "        p[j] /= l;", "        p[j] /= 1.0;"),
    ("causal mask off by one (j >= i)", "if (causal && j > i)",
     "if (causal && j >= i)"),
    ("causal mask missing", "if (causal && j > i)", "if (0 && j > i)"),
    ("lse in base 2", "m + log(l)", "m + log2(l)"),
    ("lse without the max", "m + log(l)", "log(l)"),
    ("last feature dropped from the dot", "for (int64_t c = 0; c < d; ++c)\n            dot",
     "for (int64_t c = 0; c + 1 < d; ++c)\n            dot"),
    ("keys read in reverse order", "const double *kj = k + j * d;",
     "const double *kj = k + (nk - 1 - j) * d;"),
    ("V rows read in reverse order", "const double *vj = v + j * d;",
     "const double *vj = v + (jend - 1 - j) * d;"),
    ("PV sum stops one key early", "int64_t jend = (causal && i + 1 < nk) ? i + 1 : nk;",
     "int64_t jend = (causal && i + 1 < nk) ? i : nk - 1;"),
    ("max taken as min", "if (p[j] > m)", "if (p[j] < m && p[j] > -INFINITY)"),
    # gradients
    ("dS without the D term", "p[j] * (dp[j] - di)", "p[j] * dp[j]"),
    ("dS sign flipped", "p[j] * (dp[j] - di)", "p[j] * (di - dp[j])"),
    ("dK accumulates K instead of Q", "dkj[c] += ds * qi[c];", "dkj[c] += ds * kj[c];"),
    ("dV accumulates dS instead of P", "dvj[c] += p[j] * gi[c];", "dvj[c] += ds * gi[c];"),
    ("dQ without the scale", "dqi[c] *= jb->scale;", "dqi[c] *= 1.0;"),
    ("dK without the scale", "dkh[e] = scale * sk;", "dkh[e] = sk;"),
    ("dP from K instead of V", "const double *vj = jb->v + j * d;",
     "const double *vj = jb->k + j * d;"),
    ("D summed without P", "di += p[j] * s;", "di += s;"),
    ("partial sums of other threads dropped",
     "for (int t = 0; t < nthreads; ++t) {\n                sk",
     "for (int t = 0; t < 1; ++t) {\n                sk"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site not unique/found: %r" % old
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(old, new))
    lib = oracle.build(src=str(mut), out=str(tmp_path / "libmutant.so"))
    orc = oracle.OracleLib(lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, RuntimeError, FloatingPointError,
                OverflowError):
            caught.append(pin.__name__)
    assert caught, "mutant %r passed every pin" % name
