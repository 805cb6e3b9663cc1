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
    ("last feature dropped from the dot",
     "for (int64_t c = 0; c < d; ++c)\n            dot += qi[c] * kj[c];\n        p[j]",
     "for (int64_t c = 0; c + 1 < d; ++c)\n            dot += qi[c] * kj[c];\n        p[j]"),
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
    ("dS without the D term (key pass)", "pij * (dpij - jb->delta[head * nq + i])",
     "pij * dpij"),
    ("dK accumulates K instead of Q", "dkj[c] += ds * qi[c];", "dkj[c] += ds * kj[c];"),
    ("dV accumulates dS instead of P", "dvj[c] += pij * gi[c];", "dvj[c] += ds * gi[c];"),
    ("dQ without the scale", "dqi[c] *= jb->scale;", "dqi[c] *= 1.0;"),
    ("dK without the scale", "dkj[c] *= jb->scale;", "dkj[c] *= 1.0;"),
    ("dP from K instead of V", "const double *vj = vh + j * d;",
     "const double *vj = kh + j * d;"),
    ("dP from K instead of V (key pass)",
     "const double *vj = jb->v + (head * nk + j) * d;",
     "const double *vj = jb->k + (head * nk + j) * d;"),
    ("D summed without P", "di += p[j] * s;", "di += s;"),
    ("key pass P not normalised", "pij /= li;", "pij /= 1.0;"),
    ("key pass skips the diagonal row", "i = jb->causal ? j : 0;",
     "i = jb->causal ? j + 1 : 0;"),
    ("key pass stops one row early", "i < nq; ++i) {\n        const double li",
     "i + 1 < nq; ++i) {\n        const double li"),
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


# Mistakes planted in the oracle's FP8 block quantiser (Python): each is a
# text change of ``quantize_fp8``'s source, executed into a copy of the
# module's namespace and patched in for the duration of the test.
FP8_MUTANTS = [
    ("one exponent per head",
     [("amax = np.abs(blocks).max(axis=(-2, -1))",
       "amax = np.broadcast_to(np.abs(blocks).max(axis=(-3, -2, -1))[..., None],"
       " blocks.shape[:-2])")]),
    ("one exponent per row, the block's largest returned",
     [("amax = np.abs(blocks).max(axis=(-2, -1))",
       "amax = np.abs(blocks).max(axis=-1)"),
      ("scaled = blocks * np.ldexp(np.float32(1), -e)[..., None, None]",
       "scaled = blocks * np.ldexp(np.float32(1), -e)[..., None]"),
      ("return codes[..., :n, :], e", "return codes[..., :n, :], e.max(axis=-1)")]),
    ("blocks interleaved (row r in block r mod nb)",
     [("blocks = yp.reshape(yp.shape[:-2] + (nb, block_rows, d))",
       "blocks = yp.reshape(yp.shape[:-2] + (block_rows, nb, d)).swapaxes(-3, -2)"),
      ("codes = to_e4m3_codes(scaled).reshape(yp.shape)",
       "codes = to_e4m3_codes(scaled).swapaxes(-3, -2).reshape(yp.shape)")]),
    ("block exponent one too large",
     [("e = block_exponent(amax)", "e = block_exponent(amax) + 1")]),
    ("rotation without the signs",
     [("y = fwht_f32(y * np.asarray(signs, dtype=np.float32))", "y = fwht_f32(y)")]),
]


@pytest.mark.parametrize("name,edits", FP8_MUTANTS, ids=[m[0] for m in FP8_MUTANTS])
def test_fp8_quantiser_mutant_is_caught(monkeypatch, name, edits):
    import inspect

    src = inspect.getsource(oracle.quantize_fp8)
    for old, new in edits:
        assert src.count(old) == 1, "mutation site not unique/found: %r" % old
        src = src.replace(old, new)
    ns = dict(vars(oracle))
    exec(compile(src, "<mutant quantize_fp8>", "exec"), ns)
    monkeypatch.setattr(oracle, "quantize_fp8", ns["quantize_fp8"])
    orc = oracle._default()
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, RuntimeError, FloatingPointError,
                OverflowError, IndexError):
            caught.append(pin.__name__)
    assert caught, "mutant %r passed every pin" % name
    print(name, "caught by", caught)
