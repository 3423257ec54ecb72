"""Plant one plausible mistake at a time in a copy of the oracle's C source,
build it on the CPU, and check that at least one pin catches it.  This is
what makes the pins a check of the oracle rather than a restatement of it."""
import os
import subprocess

import pytest

import oracle
import oracle_pins

# (what the mistake is, exact text in oracle.c, replacement)
MUTANTS = [
    ("chain: x - b1", "t[i] = (double)x[i] + (double)b1[i];", "t[i] = (double)x[i] - (double)b1[i];"),
    ("chain: relu dropped", "r[i] = (t[i] < 0.0) ? 0.0 : t[i];", "r[i] = t[i];"),
    ("chain: b1 used for b2", "y[i] = u[i] + (double)b2[i];", "y[i] = u[i] + (double)b1[i];"),
    ("chain: scale ignored", "u[i] = r[i] * s;", "u[i] = r[i];"),
    ("chain: SEQ rounding dropped", "if (seq) t[i] = r32(t[i]);", ""),
    ("10-op: bias indexed by row", "RS(t1[i * cols + j] + (double)bias[j])", "RS(t1[i * cols + j] + (double)bias[i % cols])"),
    ("10-op: mean over cols - 1", "m[i] = RS(acc / (double)cols);", "m[i] = RS(acc / (double)(cols - 1));"),
    ("10-op: q from t not a", "q[k] = RS(a[k] * cc);", "q[k] = RS(t[k] * cc);"),
    ("10-op: gamma and beta swapped", "* (double)gamma[j]);", "* (double)beta[j]);"),
    ("10-op: mean indexed by column", "RS(s[i * cols + j] - m[i])", "RS(s[i * cols + j] - m[j % rows])"),
    ("10-op: alpha rounded in exact mode", "const double al = seq ? r32(alpha) : alpha;", "const double al = r32(alpha);"),
    ("LN: unbiased variance", "var[i] = acc / (double)cols;", "var[i] = acc / (double)(cols - 1);"),
    ("LN: eps outside the root", "sqrt(var[i] + eps_used);", "(sqrt(var[i]) + eps_used);"),
    ("LN: residual dropped", "xv = xv + load_elem(dtype, residual, k);", "xv = xv + 0.0;"),
    ("LN: gamma/beta swapped", "double g = load_elem(dtype, gamma, j), b = load_elem(dtype, beta, j);",
     "double g = load_elem(dtype, beta, j), b = load_elem(dtype, gamma, j);"),
    ("LN: centring skipped in variance", "double dlt = v[i * cols + j] - mean[i];", "double dlt = v[i * cols + j];"),
    ("GeLU: u^2 for u^3", "double u3 = u * u * u;", "double u3 = u * u;"),
    ("GeLU: factor u dropped", "return 0.5 * u * (1.0 + tanh(z));", "return 0.5 * (1.0 + tanh(z));"),
    ("GeLU: wrong constant", "0.7978845608 * inner", "0.7978845 * inner"),
    ("bf16 decode shift", "uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    ("bf16 ties away from zero", "u += 0x7fffu + ((u >> 16) & 1u);", "u += 0x8000u;"),
    ("LN SEQ: mean kept in binary64", "if (seq) mean[i] = r32(mean[i]);", ""),
    ("LN SEQ: bf16 store skipped after the divide", "nrm[i * cols + j] = seq ? rstore(dtype, nv) : nv;",
     "nrm[i * cols + j] = seq ? r32(nv) : nv;"),
    ("round: truncation for nearest", "double r = ldexp(rint(ldexp(a, -q)), q);", "double r = ldexp(floor(ldexp(a, -q)), q);"),
    ("round: one significand bit short", "int q = lead - (p - 1);", "int q = lead - (p - 2);"),
    ("round: no subnormal floor", "if (lead < emin) lead = emin;", ""),
    ("round: no overflow to infinity", "if (r > maxf) r = INFINITY;", ""),
    ("f16 encode: exponent bias off by one", "(uint16_t)((e - 1 + 15) << 10)", "(uint16_t)((e + 15) << 10)"),
    ("f16 encode: subnormal scale", "(uint16_t)ldexp(a, 24)); /* zero or subnormal */", "(uint16_t)ldexp(a, 23)); /* zero or subnormal */"),
    ("softmax: maximum not subtracted", "double d = (double)x[i * cols + j] - m[i];", "double d = (double)x[i * cols + j];"),
    ("softmax: minimum for maximum", "if (v > mi) mi = v;", "if (v < mi || mi == -INFINITY) mi = v;"),
    ("softmax: sum skips the last column", "for (int64_t j = 0; j < cols; ++j) acc += e[i * cols + j];", "for (int64_t j = 0; j + 1 < cols; ++j) acc += e[i * cols + j];"),
    ("softmax: divide by cols", "const double q = e[i * cols + j] / l[i];", "const double q = e[i * cols + j] / (double)cols;"),
    ("softmax SEQ: difference not rounded", "if (seq) d = rstore(dtype, d);", ""),
    ("softmax SEQ: exponential not rounded", "e[i * cols + j] = seq ? rstore(dtype, ev) : ev;", "e[i * cols + j] = ev;"),
    ("softmax SEQ: quotient not rounded", "y[i * cols + j] = seq ? rstore(dtype, q) : q;", "y[i * cols + j] = q;"),
    ("philox: nine rounds", "for (int r = 0; r < 10; ++r) {", "for (int r = 0; r < 9; ++r) {"),
    ("philox: no key bump", "k0 += 0x9E3779B9u;", ""),
    ("philox: c1 and c3 swapped", "uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;", "uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[3] ^ k0;"),
    ("dropout: word 0 for every element", "const uint32_t w = out[(i & 7) >> 1];", "const uint32_t w = out[0];"),
    ("dropout: low half for every element", "return (i & 1) ? (w >> 16) : (w & 0xFFFFu);", "return w & 0xFFFFu;"),
    ("dropout: keep below the threshold", "const int keep = w >= threshold;", "const int keep = w < threshold;"),
    ("dropout: no rescale", "double v = keep ? y[k] * sc : 0.0;", "double v = keep ? y[k] : 0.0;"),
    ("dropout: relu dropped", "for (int64_t k = 0; k < n; ++k) y[k] = (y[k] < 0.0) ? 0.0 : y[k];", ""),
    ("LN SEQ/SEQ3: GeLU output not rounded", "if (seq || seq3) o = rstore(dtype, o);", ""),
    ("LN SEQ: GeLU output not rounded (SEQ3 still rounds)", "if (seq || seq3) o = rstore(dtype, o);",
     "if (seq3) o = rstore(dtype, o);"),
    ("LN SEQ3: u not rounded", "if (seq3) uv = rstore(dtype, uv);", ""),
    ("LN SEQ3: residual sum not rounded", "if (seq || seq3) xv = rstore(dtype, xv);",
     "if (seq) xv = rstore(dtype, xv);"),
    ("dropout: first_row ignored", "dropout_bits(seed, offset, (uint64_t)(first_row * cols + k));",
     "dropout_bits(seed, offset, (uint64_t)k);"),
    ("dropout SEQ3: output not rounded", "if (seq3) v = rstore(dtype, v);", ""),
    ("dropout SEQ3: scale kept in binary64", "const double sc = seq3 ? r32(scale) : scale;",
     "const double sc = scale;"),
]


@pytest.mark.parametrize("what,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(what, old, new, tmp_path):
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation site for '{what}' must appear exactly once"
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(src.replace(old, new))
    so = str(tmp_path / "liboracle_mutant.so")
    oracle.build(str(mutant), so)
    lib = oracle.load(so)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError) as e:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake: {what}"
