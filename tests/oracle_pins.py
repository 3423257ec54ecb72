"""Pins that tie the CPU oracle to something other than itself.

Each ``pin_*`` takes a loaded oracle library (``oracle.load()`` or a mutant
build) and raises ``AssertionError`` when the oracle disagrees with:

* the hand-derived worked examples under ``tests/golden/`` (each cites the page
  and section whose definition it works through);
* exact rational arithmetic (``fractions.Fraction``) or 40-digit ``mpmath`` on
  tiny inputs (brute force);
* closed forms and invariants that the definitions fix;
* independent library code (numpy float64 / float32, torch CPU float64
  ``layer_norm`` and tanh-``gelu``, torch's bfloat16 conversion).

The same functions run in ``test_oracle_pins.py`` (must pass) and in
``test_oracle_mutants.py`` (a planted mistake in the oracle must make at least
one of them fail).
"""
from __future__ import annotations

import math
from fractions import Fraction

import mpmath
import numpy as np

import oracle
from golden_io import read

RNG_SEED = 20241202


def _rng(k=0):
    return np.random.default_rng([RNG_SEED, k])


def _close(a, b, rtol, atol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    bad = ~(np.abs(a - b) <= atol + rtol * np.abs(b))
    bad |= np.isnan(a) != np.isnan(b)
    assert not bad.any(), f"{what}: {int(bad.sum())} mismatches, first {a[bad][:3]} vs {b[bad][:3]}"


# ----------------------------------------------------------------- chain

def pin_chain_worked(lib):
    g = read("chain_worked.txt")
    x, b1, b2 = (np.array(g[k], np.float32) for k in ("x", "b1", "b2"))
    y = oracle.pointwise_chain(x, b1, b2, g["scale"], lib=lib)
    assert np.array_equal(y, np.array(g["y"])), f"chain worked example: {y}"


def pin_chain_bruteforce(lib):
    r = _rng(1)
    x, b1, b2 = (r.standard_normal(32).astype(np.float32) for _ in range(3))
    scale = Fraction(1, 2)
    exact = []
    for i in range(32):
        t = Fraction(float(x[i])) + Fraction(float(b1[i]))
        t = t if t > 0 else Fraction(0)
        exact.append(float(t * scale + Fraction(float(b2[i]))))
    y = oracle.pointwise_chain(x, b1, b2, 0.5, lib=lib)
    _close(y, exact, 1e-15, 1e-300, "chain vs exact rationals")
    ys = oracle.pointwise_chain(x, b1, b2, 0.5, mode=oracle.SEQ, lib=lib)
    _close(ys, exact, 2.0 ** -22, 2.0 ** -40, "chain seq vs exact rationals")


def pin_chain_invariants(lib):
    r = _rng(2)
    n = 4096
    x, b1, b2 = (r.standard_normal(n).astype(np.float32) for _ in range(3))
    y = oracle.pointwise_chain(x, b1, b2, 0.5, lib=lib)
    b2d = b2.astype(np.float64)
    assert (y >= b2d).all(), "relu(.)*scale + b2 must be >= b2 for scale > 0"
    dead = (x.astype(np.float64) + b1.astype(np.float64)) <= 0
    assert dead.any() and np.array_equal(y[dead], b2d[dead]), "y == b2 exactly where x + b1 <= 0"
    y1 = oracle.pointwise_chain(x, b1, np.zeros(n, np.float32), 1.0, lib=lib)
    relu = np.maximum(x.astype(np.float64) + b1.astype(np.float64), 0.0)
    assert np.array_equal(y1, relu), "scale 1, b2 0 reduces to relu(x + b1)"
    # NaN propagates through relu (eager semantics)
    xn = x.copy()
    xn[7] = np.nan
    yn = oracle.pointwise_chain(xn, b1, b2, 0.5, lib=lib)
    assert np.isnan(yn[7]) and not np.isnan(np.delete(yn, 7)).any()


def pin_chain_numpy(lib):
    r = _rng(3)
    x, b1, b2 = (r.standard_normal(10007).astype(np.float32) for _ in range(3))
    ref = np.maximum(x.astype(np.float64) + b1, 0.0) * 0.5 + b2.astype(np.float64)
    _close(oracle.pointwise_chain(x, b1, b2, 0.5, lib=lib), ref, 1e-15, 0.0, "chain vs numpy f64")
    # SEQ mode is one correctly rounded fp32 op at a time: numpy float32 does exactly that
    t = x + b1
    u = np.where(t < 0, np.float32(0), t) * np.float32(0.5)
    ref32 = (u + b2).astype(np.float64)
    ys = oracle.pointwise_chain(x, b1, b2, 0.5, mode=oracle.SEQ, lib=lib)
    assert np.array_equal(ys, ref32), "chain SEQ must equal numpy float32 op by op"
    # a non-dyadic scale: rounding t before the multiply now matters
    u = np.where(t < 0, np.float32(0), t) * np.float32(0.3)
    ys = oracle.pointwise_chain(x, b1, b2, 0.3, mode=oracle.SEQ, lib=lib)
    assert np.array_equal(ys, (u + b2).astype(np.float64)), "chain SEQ, scale 0.3"


# ----------------------------------------------------------------- 10-op graph

def pin_tenop_worked(lib):
    g = read("tenop_worked.txt")
    x = np.array([g["x"]], np.float32)
    y = oracle.row_mean_epilogue(x, *(np.array(g[k], np.float32) for k in ("bias", "gamma", "beta")),
                                 alpha=g["alpha"], c=g["c"], lib=lib)
    _close(y[0], g["y"], 1e-13, 1e-13, "10-op worked example")


def _tenop_exact(x, bias, gamma, beta, alpha, c):
    rows, cols = x.shape
    al, cc = Fraction(alpha), Fraction(c)
    s = [[None] * cols for _ in range(rows)]
    for i in range(rows):
        for j in range(cols):
            t = Fraction(float(x[i, j])) * al + Fraction(float(bias[j]))
            a = t if t > 0 else Fraction(0)
            s[i][j] = a * a + a * cc
    y = np.empty((rows, cols))
    for i in range(rows):
        m = sum(s[i]) / cols
        for j in range(cols):
            y[i, j] = float((s[i][j] - m) * Fraction(float(gamma[j])) + Fraction(float(beta[j])))
    return y


def pin_tenop_bruteforce(lib):
    r = _rng(4)
    x = r.standard_normal((4, 8)).astype(np.float32)
    bias, gamma, beta = (r.standard_normal(8).astype(np.float32) for _ in range(3))
    ref = _tenop_exact(x, bias, gamma, beta, "1.1", "0.1")
    y = oracle.row_mean_epilogue(x, bias, gamma, beta, 1.1, 0.1, lib=lib)
    _close(y, ref, 1e-12, 1e-12, "10-op vs exact rationals (decimal 1.1, 0.1)")
    # a wide, non-square case against numpy float64 (rows and cols differ, so a
    # swapped axis or a bias indexed by row cannot pass)
    x = r.standard_normal((5, 37)).astype(np.float32)
    bias, gamma, beta = (r.standard_normal(37).astype(np.float32) for _ in range(3))
    a = np.maximum(x.astype(np.float64) * 1.1 + bias, 0.0)
    s = a * a + a * 0.1
    ref = (s - s.mean(axis=1, keepdims=True)) * gamma.astype(np.float64) + beta
    _close(oracle.row_mean_epilogue(x, bias, gamma, beta, lib=lib), ref, 1e-12, 1e-12, "10-op vs numpy f64")


def pin_tenop_invariants(lib):
    r = _rng(5)
    rows, cols = 6, 40
    x = r.standard_normal((rows, cols)).astype(np.float32)
    bias, beta = (r.standard_normal(cols).astype(np.float32) for _ in range(2))
    k = np.float32(1.75)
    y = oracle.row_mean_epilogue(x, bias, np.full(cols, k, np.float32), beta, lib=lib)
    # constant gamma: every row of y has mean(beta) as its mean
    _close(y.mean(axis=1), np.full(rows, beta.astype(np.float64).mean()), 0, 1e-12, "row mean = mean(beta)")
    y = oracle.row_mean_epilogue(x, bias, np.ones(cols, np.float32), np.zeros(cols, np.float32), lib=lib)
    _close(y.mean(axis=1), np.zeros(rows), 0, 1e-12, "gamma 1, beta 0: row mean 0")
    # every t <= 0: s = 0, m = 0, so y == beta exactly
    xn = -np.abs(x) - 1
    y = oracle.row_mean_epilogue(xn, -np.abs(bias), r.standard_normal(cols).astype(np.float32), beta, lib=lib)
    assert np.array_equal(y, np.broadcast_to(beta.astype(np.float64), y.shape)), "all-dead rows give beta"
    # s >= 0, so y - beta has the sign pattern of (s - m) * gamma; with gamma = 1
    # the row minimum sits at the smallest s, which is >= 0 - m
    y = oracle.row_mean_epilogue(x, bias, np.ones(cols, np.float32), np.zeros(cols, np.float32), lib=lib)
    a = np.maximum(x.astype(np.float64) * 1.1 + bias, 0)
    m = (a * a + 0.1 * a).mean(axis=1)
    assert (y.min(axis=1) >= -m - 1e-12).all(), "s >= 0 bounds y below by -m"


def pin_tenop_seq(lib):
    # rows of 8 values of moderate size: the row sums of the fp32 s values are
    # exact in binary64, so the SEQ mean is RN32 of the exact mean, and every
    # other op is one correctly rounded fp32 op (numpy float32)
    r = _rng(6)
    x = r.standard_normal((16, 8)).astype(np.float32)
    bias, gamma, beta = (r.standard_normal(8).astype(np.float32) for _ in range(3))
    t = x * np.float32(1.1) + bias
    a = np.where(t < 0, np.float32(0), t)
    s = a * a + a * np.float32(0.1)
    m = np.array([np.float32(math.fsum(map(float, row)) / 8) for row in s], np.float32)[:, None]
    ref = ((s - m) * gamma + beta).astype(np.float64)
    y = oracle.row_mean_epilogue(x, bias, gamma, beta, mode=oracle.SEQ, lib=lib)
    assert np.array_equal(y, ref), "10-op SEQ must equal numpy float32 op by op"


# ----------------------------------------------------------------- LayerNorm (+ residual, GeLU)

def _ln_mp(v, gamma, beta, eps, act):
    """40-digit mpmath LayerNorm (+ tanh-GeLU) of one row of exact inputs."""
    mpmath.mp.dps = 40
    vv = [mpmath.mpf(float(t)) for t in v]
    n = len(vv)
    mu = mpmath.fsum(vv) / n
    var = mpmath.fsum([(t - mu) ** 2 for t in vv]) / n
    sd = mpmath.sqrt(var + mpmath.mpf(eps))
    out = []
    for j, t in enumerate(vv):
        u = (t - mu) / sd * mpmath.mpf(float(gamma[j])) + mpmath.mpf(float(beta[j]))
        if act:
            z = mpmath.mpf("0.7978845608") * (u + mpmath.mpf("0.044715") * u ** 3)
            u = mpmath.mpf("0.5") * u * (1 + mpmath.tanh(z))
        out.append(float(u))
    return out


def pin_ln_worked(lib):
    g = read("layernorm_worked.txt")
    y = oracle.add_layernorm_gelu(np.array([g["x"]], np.float32), None,
                                  np.array(g["gamma"], np.float32), np.array(g["beta"], np.float32),
                                  eps=g["eps"], act=oracle.ACT_NONE, lib=lib)
    _close(y[0], g["y"], 1e-15, 0, "LayerNorm worked example")
    mpmath.mp.dps = 30
    inv = float(1 / mpmath.sqrt(mpmath.mpf("1.00001")))
    _close(np.abs(y[0]), np.full(8, inv), 1e-15, 0, "1/sqrt(1 + eps)")


def pin_ln_closed_forms(lib):
    r = _rng(7)
    # two-valued row a, b alternating: +-(|a - b|/2) / sqrt(((a - b)/2)^2 + eps)
    a, b = 1.25, -3.5
    x = np.array([[a, b] * 6], np.float32)
    y = oracle.add_layernorm_gelu(x, None, np.ones(12, np.float32), np.zeros(12, np.float32),
                                  eps=1e-5, act=oracle.ACT_NONE, lib=lib)
    h = abs(a - b) / 2
    mag = h / math.sqrt(h * h + 1e-5)
    _close(y[0], np.array([mag, -mag] * 6), 1e-14, 0, "two-valued row")
    # constant rows give beta exactly
    cols = 33
    xc = np.repeat(r.standard_normal((4, 1)).astype(np.float32) * 50, cols, axis=1)
    gamma = r.standard_normal(cols).astype(np.float32)
    beta = r.standard_normal(cols).astype(np.float32)
    y = oracle.add_layernorm_gelu(xc, None, gamma, beta, act=oracle.ACT_NONE, lib=lib)
    assert np.array_equal(y, np.broadcast_to(beta.astype(np.float64), y.shape)), "constant row -> beta"
    # gamma 1, beta 0: row mean 0, biased variance var/(var + eps)
    x = (r.standard_normal((5, 64)) * np.array([[1e-3], [0.01], [1], [10], [100]])).astype(np.float32)
    y = oracle.add_layernorm_gelu(x, None, np.ones(64, np.float32), np.zeros(64, np.float32),
                                  act=oracle.ACT_NONE, lib=lib)
    mpmath.mp.dps = 40
    for i in range(5):
        vv = [mpmath.mpf(float(t)) for t in x[i]]
        mu = mpmath.fsum(vv) / 64
        var = mpmath.fsum([(t - mu) ** 2 for t in vv]) / 64
        want = float(var / (var + mpmath.mpf(1e-5)))
        _close(y[i].mean(), 0.0, 0, 1e-13, "normalised row mean")
        _close(np.mean(y[i] ** 2) - y[i].mean() ** 2, want, 1e-12, 0, "normalised biased variance")
    # shift invariance: LN(x + c) == LN(x) (dyadic values, so x + 64 is exact in fp32)
    xs = (np.round(r.standard_normal((3, 16)) * 8) / 8).astype(np.float32)
    g1 = r.standard_normal(16).astype(np.float32)
    b1 = r.standard_normal(16).astype(np.float32)
    y0 = oracle.add_layernorm_gelu(xs, None, g1, b1, act=oracle.ACT_GELU_TANH, lib=lib)
    y1 = oracle.add_layernorm_gelu(xs + np.float32(64), None, g1, b1, act=oracle.ACT_GELU_TANH, lib=lib)
    _close(y1, y0, 1e-12, 1e-12, "shift invariance")


def pin_ln_bruteforce(lib):
    r = _rng(8)
    for dt in ("f32", "bf16"):
        x = r.standard_normal((4, 8)).astype(np.float32) * 3 + 1
        res = r.standard_normal((4, 8)).astype(np.float32)
        gamma = (1 + 0.1 * r.standard_normal(8)).astype(np.float32)
        beta = (0.1 * r.standard_normal(8)).astype(np.float32)
        if dt == "bf16":
            args = [_torch_bf16_bits(a) for a in (x, res, gamma, beta)]
            vals = [a.astype(np.uint32) << 16 for a in args]
            x, res, gamma, beta = (v.view(np.float32) for v in vals)
        else:
            args = [x, res, gamma, beta]
        for act in (oracle.ACT_NONE, oracle.ACT_GELU_TANH):
            for with_res in (False, True):
                y = oracle.add_layernorm_gelu(args[0], args[1] if with_res else None, args[2], args[3],
                                              eps=1e-5, act=act, lib=lib)
                for i in range(4):
                    v = x[i].astype(np.float64) + (res[i] if with_res else 0)
                    ref = _ln_mp(v, gamma, beta, 1e-5, act == oracle.ACT_GELU_TANH)
                    _close(y[i], ref, 1e-12, 1e-13, f"LN {dt} act={act} res={with_res} vs mpmath")


def pin_ln_torch(lib):
    import torch
    import torch.nn.functional as F
    r = _rng(9)
    rows, cols = 7, 301
    x = (r.standard_normal((rows, cols)) * 2 + r.uniform(-100, 100, (rows, 1))).astype(np.float32)
    res = r.standard_normal((rows, cols)).astype(np.float32)
    gamma = (1 + 0.1 * r.standard_normal(cols)).astype(np.float32)
    beta = (0.1 * r.standard_normal(cols)).astype(np.float32)
    tx, tr = torch.from_numpy(x).double(), torch.from_numpy(res).double()
    tg, tb = torch.from_numpy(gamma).double(), torch.from_numpy(beta).double()
    ln = F.layer_norm(tx + tr, (cols,), tg, tb, eps=1e-5)
    y = oracle.add_layernorm_gelu(x, res, gamma, beta, act=oracle.ACT_NONE, lib=lib)
    _close(y, ln.numpy(), 1e-10, 1e-10, "LN vs torch float64 layer_norm")
    # torch's tanh-GeLU uses sqrt(2/pi) = 0.7978845608028654; the pages' literal
    # 0.7978845608 differs by 3.6e-12 relative, far inside this tolerance
    g = F.gelu(ln, approximate="tanh")
    y = oracle.add_layernorm_gelu(x, res, gamma, beta, act=oracle.ACT_GELU_TANH, lib=lib)
    _close(y, g.numpy(), 1e-9, 1e-10, "LN + GeLU vs torch float64")


def pin_gelu(lib):
    g = read("gelu_values.txt")
    got = oracle.gelu_tanh(np.array(g["u"]), lib=lib)
    _close(got, g["g"], 1e-13, 1e-15, "GeLU worked values")
    mpmath.mp.dps = 40
    u = _rng(10).standard_normal(200) * 4
    ref = [float(mpmath.mpf("0.5") * mpmath.mpf(t) * (1 + mpmath.tanh(
        mpmath.mpf("0.7978845608") * (mpmath.mpf(t) + mpmath.mpf("0.044715") * mpmath.mpf(t) ** 3))))
        for t in u]
    # for u << 0 the literal 1 + tanh(z) cancels, so the error is absolute
    # (about 1e-16 |u|), not relative
    _close(oracle.gelu_tanh(u, lib=lib), ref, 1e-14, 1e-14, "GeLU vs mpmath")
    # odd-part identity: g(u) - g(-u) = u
    _close(oracle.gelu_tanh(u, lib=lib) - oracle.gelu_tanh(-u, lib=lib), u, 1e-14, 1e-300, "g(u)-g(-u)=u")


def pin_residual_zero(lib):
    r = _rng(11)
    x = _torch_bf16_bits(r.standard_normal((3, 40)).astype(np.float32))
    z = np.zeros_like(x)
    g = _torch_bf16_bits((1 + 0.1 * r.standard_normal(40)).astype(np.float32))
    b = _torch_bf16_bits((0.1 * r.standard_normal(40)).astype(np.float32))
    for mode in (oracle.EXACT, oracle.SEQ, oracle.SEQ3):
        y0 = oracle.add_layernorm_gelu(x, None, g, b, mode=mode, lib=lib)
        y1 = oracle.add_layernorm_gelu(x, z, g, b, mode=mode, lib=lib)
        assert np.array_equal(y0, y1), "a zero residual changes nothing"
        y2 = oracle.add_layernorm_gelu(z, x, g, b, mode=mode, lib=lib)
        assert np.array_equal(y0, y2), "x + r is symmetric"


def _torch_bf16_bits(a):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def pin_bf16_encode(lib):
    r = _rng(12)
    bits = r.integers(0, 2 ** 32, 1 << 18, dtype=np.uint64).astype(np.uint32)
    # ties and their neighbours, both signs, subnormals, the largest finite, infinities
    ties = (r.integers(0, 2 ** 16, 4096, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    special = np.array([0, 0x80000000, 1, 0x807FFFFF, 0x7F7FFFFF, 0x7F800000, 0xFF800000,
                        0x3F808000, 0x3F818000, 0x3F807FFF, 0x3F808001], np.uint32)
    bits = np.concatenate([bits, ties, ties + 1, ties - 1, special])
    f = bits.view(np.float32)
    finite = np.isfinite(f) | np.isinf(f)
    got = oracle.to_bf16(f, lib=lib)
    want = _torch_bf16_bits(f)
    assert np.array_equal(got[finite], want[finite]), "bf16 RNE vs torch"
    nan = ~finite
    assert ((got[nan] & 0x7F80) == 0x7F80).all() and ((got[nan] & 0x7F) != 0).all(), "NaN stays NaN"


def pin_ln_seq(lib):
    """SEQ mode of LayerNorm (+ residual, GeLU) against an op-by-op emulation
    with numpy float32 arithmetic and torch's bfloat16 rounding."""
    import torch
    r = _rng(13)
    rows, cols = 6, 64

    def rb(a):  # fp32 -> bf16 -> fp32 through torch
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).float().numpy()

    x = rb(r.standard_normal((rows, cols)).astype(np.float32))
    res = rb(r.standard_normal((rows, cols)).astype(np.float32))
    gamma = rb((1 + 0.1 * r.standard_normal(cols)).astype(np.float32))
    beta = rb((0.1 * r.standard_normal(cols)).astype(np.float32))
    v = rb(x + res)
    mu = np.array([np.float32(math.fsum(map(float, row)) / cols) for row in v], np.float32)[:, None]
    var = np.array([np.float32(math.fsum((float(t) - float(m)) ** 2 for t in row) / cols)
                    for row, m in zip(v, mu[:, 0])], np.float32)[:, None]
    cen = rb(v - mu)
    sd = np.sqrt(var + np.float32(1e-5))
    nrm = rb(cen / sd)
    u = rb(nrm * gamma + beta)
    bits = _torch_bf16_bits
    y = oracle.add_layernorm_gelu(bits(x), bits(res), bits(gamma), bits(beta), act=oracle.ACT_NONE,
                                  mode=oracle.SEQ, lib=lib)
    assert np.array_equal(y, u.astype(np.float64)), "LN SEQ (bf16) must match op-by-op emulation"
    # fp32 I/O: same chain with float32 storage
    x32 = (r.standard_normal((rows, cols)) + 20).astype(np.float32)
    g32 = (1 + 0.1 * r.standard_normal(cols)).astype(np.float32)
    b32 = (0.1 * r.standard_normal(cols)).astype(np.float32)
    mu = np.array([np.float32(math.fsum(map(float, row)) / cols) for row in x32], np.float32)[:, None]
    var = np.array([np.float32(math.fsum((float(t) - float(m)) ** 2 for t in row) / cols)
                    for row, m in zip(x32, mu[:, 0])], np.float32)[:, None]
    ref = ((x32 - mu) / np.sqrt(var + np.float32(1e-5))) * g32 + b32
    y = oracle.add_layernorm_gelu(x32, None, g32, b32, act=oracle.ACT_NONE, mode=oracle.SEQ, lib=lib)
    assert np.array_equal(y, ref.astype(np.float64)), "LN SEQ (fp32) must match op-by-op emulation"


def _rb(a):
    """float32 -> bfloat16 (nearest even, torch's conversion) -> float32."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def _gelu_mp(u):
    """tanh-GeLU with the printed constants, each value evaluated in 40-digit
    mpmath and rounded once to binary64 (an evaluation independent of the
    oracle's C code)."""
    mpmath.mp.dps = 40
    out = []
    for t in np.asarray(u, np.float64).ravel():
        m = mpmath.mpf(float(t))
        z = mpmath.mpf("0.7978845608") * (m + mpmath.mpf("0.044715") * m ** 3)
        out.append(float(mpmath.mpf("0.5") * m * (1 + mpmath.tanh(z))))
    return np.array(out, np.float64).reshape(np.shape(u))


def _ln_f64_torch(v, gamma, beta, eps=1e-5):
    """LayerNorm rows in float64 with torch's CPU layer_norm (library code)."""
    import torch
    import torch.nn.functional as F
    t = torch.from_numpy(np.asarray(v, np.float64))
    g = torch.from_numpy(np.asarray(gamma, np.float64))
    b = torch.from_numpy(np.asarray(beta, np.float64))
    return F.layer_norm(t, (t.shape[1],), g, b, eps=eps).numpy()


def pin_ln_seq_gelu(lib):
    """SEQ mode with the residual and the tanh-GeLU: the seven eager launches of
    [P2] section 2.3's chain (add, mean, var, sub, div, mul-add, gelu), every
    element-wise result stored in the I/O type.  Emulated op by op with numpy
    float32 arithmetic, torch's bfloat16 rounding and a 40-digit GeLU rounded
    to the storage type at its store."""
    r = _rng(43)
    rows, cols = 5, 48
    x = _rb(r.standard_normal((rows, cols)).astype(np.float32) * 2)
    res = _rb(r.standard_normal((rows, cols)).astype(np.float32) * 2)
    gamma = _rb((1 + 0.1 * r.standard_normal(cols)).astype(np.float32))
    beta = _rb((0.1 * r.standard_normal(cols)).astype(np.float32))
    v = _rb(x + res)
    mu = np.array([np.float32(math.fsum(map(float, row)) / cols) for row in v], np.float32)[:, None]
    var = np.array([np.float32(math.fsum((float(t) - float(m)) ** 2 for t in row) / cols)
                    for row, m in zip(v, mu[:, 0])], np.float32)[:, None]
    nrm = _rb(_rb(v - mu) / np.sqrt(var + np.float32(1e-5)))
    u = _rb(nrm * gamma + beta)
    want = _rb(_gelu_mp(u).astype(np.float32)).astype(np.float64)
    bits = _torch_bf16_bits
    y = oracle.add_layernorm_gelu(bits(x), bits(res), bits(gamma), bits(beta), act=oracle.ACT_GELU_TANH,
                                  mode=oracle.SEQ, lib=lib)
    assert np.array_equal(y, want), \
        f"LN+GeLU SEQ (bf16): {int((y != want).sum())} of {y.size} differ from the op-by-op emulation"
    # fp32 I/O: the same seven ops, each stored as binary32
    x32 = r.standard_normal((rows, cols)).astype(np.float32)
    r32 = r.standard_normal((rows, cols)).astype(np.float32)
    g32 = (1 + 0.1 * r.standard_normal(cols)).astype(np.float32)
    b32 = (0.1 * r.standard_normal(cols)).astype(np.float32)
    v = x32 + r32
    mu = np.array([np.float32(math.fsum(map(float, row)) / cols) for row in v], np.float32)[:, None]
    var = np.array([np.float32(math.fsum((float(t) - float(m)) ** 2 for t in row) / cols)
                    for row, m in zip(v, mu[:, 0])], np.float32)[:, None]
    u = ((v - mu) / np.sqrt(var + np.float32(1e-5))) * g32 + b32
    want = _gelu_mp(u).astype(np.float32).astype(np.float64)
    y = oracle.add_layernorm_gelu(x32, r32, g32, b32, act=oracle.ACT_GELU_TANH, mode=oracle.SEQ, lib=lib)
    assert np.array_equal(y, want), \
        f"LN+GeLU SEQ (fp32): {int((y != want).sum())} of {y.size} differ from the op-by-op emulation"


def pin_ln_seq3(lib):
    """SEQ3 mode: the three eager launches of [P2] section 2.3's chain -- the
    residual add, one LayerNorm kernel, the GeLU -- each result stored in the
    I/O type; the LayerNorm launch itself computes in binary64.  Emulated with
    numpy float32 for the add, torch's float64 layer_norm for the middle launch,
    torch's rounding to the storage type and a 40-digit GeLU."""
    r = _rng(44)
    rows, cols = 5, 56
    x = _rb(r.standard_normal((rows, cols)).astype(np.float32) * 2 + 0.5)
    res = _rb(r.standard_normal((rows, cols)).astype(np.float32) * 2)
    gamma = _rb((1 + 0.1 * r.standard_normal(cols)).astype(np.float32))
    beta = _rb((0.1 * r.standard_normal(cols)).astype(np.float32))
    v = _rb(x + res)
    u = _rb(_ln_f64_torch(v, gamma, beta).astype(np.float32))
    bits = _torch_bf16_bits
    y = oracle.add_layernorm_gelu(bits(x), bits(res), bits(gamma), bits(beta), act=oracle.ACT_NONE,
                                  mode=oracle.SEQ3, lib=lib)
    assert np.array_equal(y, u.astype(np.float64)), \
        f"LN SEQ3 (bf16): {int((y != u).sum())} of {y.size} differ from add -> layer_norm, each stored"
    want = _rb(_gelu_mp(u).astype(np.float32)).astype(np.float64)
    y = oracle.add_layernorm_gelu(bits(x), bits(res), bits(gamma), bits(beta), act=oracle.ACT_GELU_TANH,
                                  mode=oracle.SEQ3, lib=lib)
    assert np.array_equal(y, want), \
        f"LN+GeLU SEQ3 (bf16): {int((y != want).sum())} of {y.size} differ from add -> layer_norm -> gelu"
    x32 = r.standard_normal((rows, cols)).astype(np.float32)
    r32 = r.standard_normal((rows, cols)).astype(np.float32)
    g32 = (1 + 0.1 * r.standard_normal(cols)).astype(np.float32)
    b32 = (0.1 * r.standard_normal(cols)).astype(np.float32)
    u = _ln_f64_torch(x32 + r32, g32, b32).astype(np.float32)
    want = _gelu_mp(u).astype(np.float32).astype(np.float64)
    y = oracle.add_layernorm_gelu(x32, r32, g32, b32, act=oracle.ACT_GELU_TANH, mode=oracle.SEQ3, lib=lib)
    assert np.array_equal(y, want), \
        f"LN+GeLU SEQ3 (fp32): {int((y != want).sum())} of {y.size} differ from the three launches"


def _nearest_even_bits(x, table_vals, table_bits, max_bits, inf_bits):
    """Brute force: the bit pattern of the value in `table_vals` (all finite
    non-negative values of a format, ascending, with their patterns) nearest to
    |x|, ties to the even pattern; beyond the largest finite value by half an
    ulp or more, infinity.  Exact comparisons in binary64 (every candidate and
    every midpoint used here is exact in binary64)."""
    out = np.empty(x.shape, np.uint16)
    for i, v in enumerate(x):
        a = abs(float(v))
        sign = 0x8000 if math.copysign(1.0, float(v)) < 0 else 0
        k = int(np.searchsorted(table_vals, a))
        if k == len(table_vals):
            hi_v = table_vals[-1] + (table_vals[-1] - table_vals[-2])  # next binade step past the max
            mid = (table_vals[-1] + hi_v) / 2
            b = inf_bits if a >= mid else max_bits
        elif table_vals[k] == a:
            b = table_bits[k]
        else:
            lo, hi = table_vals[k - 1], table_vals[k]
            mid = (lo + hi) / 2
            if a < mid:
                b = table_bits[k - 1]
            elif a > mid:
                b = table_bits[k]
            else:
                b = table_bits[k - 1] if table_bits[k - 1] % 2 == 0 else table_bits[k]
            if b == max_bits + 1:  # rounded up past the largest finite value
                b = inf_bits
        out[i] = sign | b
    return out


def _round_cases(r, emin, emax, p):
    """Random doubles over the format's range (subnormals to overflow), exact
    ties, ties nudged by less than binary32 can hold, and edge values."""
    e = r.integers(emin - p - 2, emax + 2, 4000)
    vals = r.uniform(1.0, 2.0, 4000) * np.exp2(e.astype(np.float64))
    sig = r.integers(0, 2 ** p, 2000)
    ex = r.integers(emin, emax + 1, 2000)
    ties = (1.0 + (2 * sig + 1) * 2.0 ** (-p)) * np.exp2(ex.astype(np.float64))
    nudged = ties * (1 + 2.0 ** -40)
    vals = np.concatenate([vals, -vals[:500], ties, ties * (1 - 2.0 ** -40), nudged])
    return vals


def pin_round_f16(lib):
    """binary16: against numpy's float64 -> float16 conversion (a direct,
    correctly rounded library routine) and against brute force."""
    r = _rng(20)
    x = _round_cases(r, -14, 15, 11)
    x = np.concatenate([x, [0.0, -0.0, 65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
                            1 + 2.0 ** -11 + 2.0 ** -40, np.inf, -np.inf]])
    got = oracle.round_bits(x, "f16", lib=lib)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want), f"f16 rounding vs numpy: {int((got != want).sum())} mismatches"
    allbits = np.arange(0, 0x7C00, dtype=np.uint16)
    vals = allbits.view(np.float16).astype(np.float64)
    sub = r.choice(len(x), 1500, replace=False)
    fin = x[sub][np.isfinite(x[sub])]
    bf = _nearest_even_bits(fin, vals, allbits, 0x7BFF, 0x7C00)
    assert np.array_equal(oracle.round_bits(fin, "f16", lib=lib), bf), "f16 rounding vs brute force"
    nan = oracle.round_bits(np.array([np.nan]), "f16", lib=lib)[0]
    assert (nan & 0x7C00) == 0x7C00 and (nan & 0x3FF) != 0, "NaN stays NaN"


def pin_round_bf16(lib):
    """bfloat16 directly from binary64: brute force over every finite pattern,
    agreement with the binary32 encoder (pinned against torch) on values that
    are binary32, and the double-rounding trap that a conversion through
    binary32 gets wrong."""
    r = _rng(21)
    x = _round_cases(r, -126, 127, 8)
    allbits = np.arange(0, 0x7F80, dtype=np.uint32)
    vals = (allbits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    sub = r.choice(len(x), 3000, replace=False)
    fin = x[sub][np.isfinite(x[sub])]
    bf = _nearest_even_bits(fin, vals, allbits.astype(np.uint16), 0x7F7F, 0x7F80)
    assert np.array_equal(oracle.round_bits(fin, "bf16", lib=lib), bf), "bf16 rounding vs brute force"
    f32 = r.standard_normal(20000).astype(np.float32)
    assert np.array_equal(oracle.round_bits(f32.astype(np.float64), "bf16", lib=lib),
                          oracle.to_bf16(f32, lib=lib)), "bf16 from binary64 vs from binary32 on binary32 values"
    trap = np.array([1 + 2.0 ** -8 + 2.0 ** -40, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 3.4e38, -3.0e38])
    assert list(oracle.round_bits(trap, "bf16", lib=lib)) == [0x3F81, 0x3F80, 0x3F82, 0x7F80, 0xFF62], \
        "bf16 rounding edge cases"


def pin_softmax_worked(lib):
    g = read("softmax_worked.txt")
    for k in range(3):
        x = np.array([g[f"x{k}"]], np.float32)
        y = oracle.softmax(x, lib=lib)[0]
        want = np.array(g[f"y{k}"])
        assert np.all(np.abs(y - want) <= g["tol"]), f"softmax worked row {k}: {y}"
        assert np.array_equal(y == 0, want == 0), "masked entries must be exactly 0"


def pin_softmax_closed_forms(lib):
    r = _rng(30)
    # equal entries: 1/n, correctly rounded (exp(0) = 1 exactly, n exactly, one division)
    for n in (1, 3, 7, 64, 1000):
        y = oracle.softmax(np.full((2, n), -1.25, np.float32), lib=lib)
        assert np.all(y == 1.0 / n), f"uniform row of {n}"
    # two entries: the logistic function of the difference (40-digit mpmath)
    a = r.standard_normal((50, 2)).astype(np.float32) * 4
    y = oracle.softmax(a, lib=lib)
    mpmath.mp.dps = 40
    want = np.array([[float(1 / (1 + mpmath.exp(mpmath.mpf(float(b)) - mpmath.mpf(float(c)))))
                      for c, b in ((row[0], row[1]), (row[1], row[0]))] for row in a])
    _close(y, want, 1e-14, 0, "two-entry softmax vs logistic")
    # large entries: exact only if the maximum is subtracted before exp
    big = np.array([[1000.0, 1000.0 + math.log(3.0)], [-1000.0, -1000.0]], np.float32)
    y = oracle.softmax(big, lib=lib)
    _close(y[1], [0.5, 0.5], 0, 0, "equal large negative entries")
    assert np.all(np.isfinite(y)) and abs(y[0].sum() - 1) < 1e-12, f"no overflow: {y[0]}"


def pin_softmax_bruteforce(lib):
    r = _rng(31)
    x = (r.standard_normal((6, 17)) * 3).astype(np.float32)
    x[2, 5] = -np.inf
    x[4, :] = x[4, 0]
    y = oracle.softmax(x, lib=lib)
    mpmath.mp.dps = 40
    for i in range(x.shape[0]):
        row = [mpmath.mpf(float(v)) if np.isfinite(v) else mpmath.mpf("-inf") for v in x[i]]
        m = max(row)
        ex = [mpmath.exp(v - m) for v in row]
        tot = mpmath.fsum(ex)
        want = np.array([float(e / tot) for e in ex])
        _close(y[i], want, 1e-14, 0, f"softmax row {i} vs 40-digit mpmath")


def pin_softmax_torch(lib):
    """torch.softmax on CPU float64 (an independent implementation), with
    masked (-inf) entries and rows of very different scales."""
    import torch
    r = _rng(32)
    x = (r.standard_normal((40, 300)) * np.exp2(r.integers(-4, 6, (40, 1)))).astype(np.float32)
    x[r.random(x.shape) < 0.1] = -np.inf
    x[:, 0] = r.standard_normal(40).astype(np.float32)  # no row fully masked
    y = oracle.softmax(x, lib=lib)
    want = torch.softmax(torch.from_numpy(x.astype(np.float64)), dim=-1).numpy()
    _close(y, want, 1e-13, 1e-300, "softmax vs torch float64")
    assert np.array_equal(y == 0, np.isneginf(x)), "exactly the masked entries are 0"
    s = y.sum(axis=1)
    assert np.all(np.abs(s - 1) < 1e-13), "rows sum to 1"


def _f32_ordered(a):
    i = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    return np.where(i < 0, -(i & 0x7FFFFFFF), i)


def pin_softmax_seq(lib):
    """The eager (SEQ) softmax against the same op sequence evaluated by
    independent libraries -- numpy float32 operations for binary32 storage,
    torch CPU bfloat16 tensors for bfloat16 storage (each op's result stored
    in the I/O type, the row sum taken in float64 and kept as float32) --
    which may differ only where their exponentials round differently; and
    rows whose every intermediate is exact."""
    import torch

    def rn(v, dt):
        v32 = np.float32(v)
        return float(torch.tensor(v32).to(torch.bfloat16).float()) if dt == "bf16" else float(v32)

    for dt in ("f32", "bf16"):
        x = np.full((3, 9), -np.inf, np.float32)
        x[0, 4] = 2.5                      # one finite entry: 1 there, 0 elsewhere
        x[1, [1, 3, 7]] = -1.0             # three equal maxima: 1/3 rounded to the I/O type
        x[2, :] = 0.75                     # nine equal entries
        y = oracle.softmax(x, mode=oracle.SEQ, dtype=dt, lib=lib)
        assert np.array_equal(y[0], np.eye(9)[4]), f"{dt}: one-hot row {y[0]}"
        assert np.all(y[1, [1, 3, 7]] == rn(1 / 3, dt)) and np.all(np.delete(y[1], [1, 3, 7]) == 0), \
            f"{dt}: three maxima {y[1]}"
        assert np.all(y[2] == rn(1 / 9, dt)), f"{dt}: uniform row {y[2]}"

    r = _rng(33)
    x = (r.standard_normal((64, 257)) * np.exp2(r.integers(0, 5, (64, 1)))).astype(np.float32)
    # binary32 storage: numpy float32
    y = oracle.softmax(x, mode=oracle.SEQ, dtype="f32", lib=lib)
    assert np.array_equal(y, y.astype(np.float32).astype(np.float64)), "f32 SEQ results must be binary32 values"
    d = (x - x.max(axis=1, keepdims=True)).astype(np.float32)
    e = np.exp(d).astype(np.float32)
    l = e.astype(np.float64).sum(axis=1, keepdims=True).astype(np.float32)
    want = (e / l).astype(np.float32)
    # numpy's float32 exp is itself up to 2 ulp from the correctly rounded value
    ulp = np.abs(_f32_ordered(y) - _f32_ordered(want))
    assert ulp.max() <= 4 and (ulp > 2).mean() <= 0.01, \
        f"f32 SEQ vs numpy float32: max {ulp.max()} ulp, {(ulp > 2).mean():.3%} beyond 2 ulp"
    # bfloat16 storage: torch CPU bfloat16 tensors
    xb = torch.from_numpy(x).to(torch.bfloat16)
    y = oracle.softmax(xb.float().numpy(), mode=oracle.SEQ, dtype="bf16", lib=lib)
    yb = torch.from_numpy(y).to(torch.bfloat16)
    assert np.array_equal(yb.double().numpy(), y), "bf16 SEQ results must be bfloat16 values"
    eb = torch.exp(xb - xb.max(dim=1, keepdim=True).values)
    lb = eb.double().sum(dim=1, keepdim=True).float()
    wb = (eb.float() / lb).to(torch.bfloat16)
    o = lambda t: (lambda i: np.where(i < 0, -(i & 0x7FFF), i))(t.view(torch.int16).numpy().astype(np.int64))
    ulp = np.abs(o(yb) - o(wb))
    assert ulp.max() <= 1 and (ulp > 0).mean() <= 0.05, \
        f"bf16 SEQ vs torch bfloat16: max {ulp.max()} ulp, {(ulp > 0).mean():.2%} differ"
    # a large common offset: no overflow
    y = oracle.softmax(x[:4] + np.float32(1000), mode=oracle.SEQ, dtype="f32", lib=lib)
    assert np.all(np.isfinite(y)) and np.all(np.abs(y.sum(axis=1) - 1) < 1e-4), "SEQ with an offset of 1000"


def pin_philox_kat(lib):
    g = read("philox_kat.txt")
    for k in range(3):
        ctr = np.array([g[f"ctr{k}"]], np.uint32)
        key = np.array([g[f"key{k}"]], np.uint32)
        out = oracle.philox4x32_10(ctr, key, lib=lib)[0]
        assert list(out) == g[f"out{k}"], f"Philox4x32-10 known answer {k}: {[hex(v) for v in out]}"


def _ln_case_pin(r, rows, cols, dtype="f32"):
    x = (r.standard_normal((rows, cols)) * 2 + 0.3).astype(np.float32)
    g = (1 + 0.1 * r.standard_normal(cols)).astype(np.float32)
    b = (0.1 * r.standard_normal(cols)).astype(np.float32)
    if dtype == "bf16":
        to = lambda a: oracle.to_bf16(a, lib=None)
        return to(x), to(g), to(b)
    return x, g, b


def pin_dropout(lib):
    r = _rng(40)
    x, g, b = _ln_case_pin(r, 64, 1000)
    relu_ln = np.maximum(oracle.add_layernorm_gelu(x, None, g, b, act=oracle.ACT_NONE, lib=lib), 0.0)
    # p = 0 keeps everything unscaled; p = 1 drops everything
    assert np.array_equal(oracle.ln_relu_dropout(x, g, b, p=0.0, seed=5, lib=lib), relu_ln), "p = 0"
    assert not oracle.ln_relu_dropout(x, g, b, p=1.0, seed=5, lib=lib).any(), "p = 1"
    # p = 0.1: kept values are relu * 1/(1 - p) exactly, dropped ones 0, and
    # the kept set is bits >= round(p 2^16) for half i mod 8 of block (i div 8, offset)
    p, seed, offset = 0.1, 0x123456789ABC, 7
    y = oracle.ln_relu_dropout(x, g, b, p=p, seed=seed, offset=offset, lib=lib)
    n = x.size
    q = np.arange((n + 7) // 8, dtype=np.uint64)
    ctr = np.stack([q & 0xFFFFFFFF, q >> 32, np.full_like(q, offset & 0xFFFFFFFF),
                    np.full_like(q, offset >> 32)], axis=1).astype(np.uint32)
    key = np.tile(np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint32), (len(q), 1))
    words = oracle.philox4x32_10(ctr, key, lib=lib).reshape(-1)
    halves = np.stack([words & 0xFFFF, words >> 16], axis=1).reshape(-1)[:n].reshape(x.shape)
    keep = halves >= round(p * 65536)
    assert np.array_equal(y[keep], relu_ln[keep] * (1.0 / (1.0 - p))), "kept values"
    assert not y[~keep].any(), "dropped values are 0"
    # the drop fraction is p within 5 binomial standard deviations
    frac = 1.0 - keep.mean()
    assert abs(frac - p) < 5 * math.sqrt(p * (1 - p) / n), f"drop fraction {frac}"
    # the mask does not depend on the data; another offset or seed gives another mask
    x2, _, _ = _ln_case_pin(_rng(41), 64, 1000)
    y2 = oracle.ln_relu_dropout(x2, g, b, p=p, seed=seed, offset=offset, lib=lib)
    pos = (relu_ln > 0) & (np.maximum(oracle.add_layernorm_gelu(x2, None, g, b, act=oracle.ACT_NONE, lib=lib), 0) > 0)
    assert np.array_equal((y != 0)[pos], (y2 != 0)[pos]), "mask independent of the data"
    # rows [r0, r1) evaluated on their own with first_row = r0: those rows of the whole call
    for r0, r1 in ((0, 5), (17, 40), (63, 64)):
        part = oracle.ln_relu_dropout(x[r0:r1], g, b, p=p, seed=seed, offset=offset, first_row=r0, lib=lib)
        assert np.array_equal(part, y[r0:r1]), f"rows {r0}..{r1} evaluated with first_row"
    for s2, o2 in ((seed, offset + 1), (seed + 1, offset)):
        y3 = oracle.ln_relu_dropout(x, g, b, p=p, seed=s2, offset=o2, lib=lib)
        agree = ((y3 != 0) == (y != 0))[relu_ln > 0].mean()
        assert abs(agree - (p * p + (1 - p) ** 2)) < 0.02, f"masks of other (seed, offset) agree {agree}"


def _dropout_keep(shape, p, seed, offset, lib):
    """Kept-element mask of [P2] section 2.1's dropout under the Philox
    reading: half k mod 8 of block (k div 8, offset) keyed by seed, kept iff
    it is >= round(p 2^16).  Blocks from the oracle's generator, which the
    published known answers pin."""
    n = int(np.prod(shape))
    q = np.arange((n + 7) // 8, dtype=np.uint64)
    ctr = np.stack([q & 0xFFFFFFFF, q >> 32, np.full_like(q, offset & 0xFFFFFFFF),
                    np.full_like(q, offset >> 32)], axis=1).astype(np.uint32)
    key = np.tile(np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint32), (len(q), 1))
    words = oracle.philox4x32_10(ctr, key, lib=lib).reshape(-1)
    halves = np.stack([words & 0xFFFF, words >> 16], axis=1).reshape(-1)[:n].reshape(shape)
    return halves >= round(p * 65536)


def pin_dropout_seq3(lib):
    """SEQ3 mode of LayerNorm -> ReLU -> Dropout: the three eager launches of
    [P2] section 2.1 (layer_norm, relu, dropout), each result stored in the I/O
    type.  The layer_norm launch: torch's float64 layer_norm, stored; relu of a
    stored value is exact; the dropout launch an fp32 kernel: the kept value
    times the scale 1/(1 - p) rounded to binary32 (numpy float32 product),
    stored; dropped elements 0."""
    r = _rng(45)
    p, seed, offset = 0.1, 0x2545F4914F6CDD1D, 3
    for dt in ("f32", "bf16"):
        x, g, b = _ln_case_pin(r, 12, 200, dtype=dt)
        if dt == "bf16":
            xv, gv, bv = ((a.astype(np.uint32) << 16).view(np.float32) for a in (x, g, b))
            store = _rb
        else:
            xv, gv, bv = x, g, b
            store = lambda a: np.asarray(a, np.float32)
        u = store(_ln_f64_torch(xv, gv, bv).astype(np.float32))
        relu = np.maximum(u, np.float32(0))
        keep = _dropout_keep(x.shape, p, seed, offset, lib)
        kept = store(relu * np.float32(1.0 / (1.0 - p)))
        want = np.where(keep, kept, np.float32(0)).astype(np.float64)
        y = oracle.ln_relu_dropout(x, g, b, p=p, seed=seed, offset=offset, mode=oracle.SEQ3, lib=lib)
        assert np.array_equal(y, want), \
            f"LN-ReLU-dropout SEQ3 ({dt}): {int((y != want).sum())} of {y.size} differ from the three launches"


ALL_PINS = [
    pin_chain_worked, pin_chain_bruteforce, pin_chain_invariants, pin_chain_numpy,
    pin_tenop_worked, pin_tenop_bruteforce, pin_tenop_invariants, pin_tenop_seq,
    pin_ln_worked, pin_ln_closed_forms, pin_ln_bruteforce, pin_ln_torch, pin_gelu,
    pin_residual_zero, pin_bf16_encode, pin_ln_seq, pin_ln_seq_gelu, pin_ln_seq3,
    pin_round_f16, pin_round_bf16,
    pin_softmax_worked, pin_softmax_closed_forms, pin_softmax_bruteforce, pin_softmax_torch, pin_softmax_seq,
    pin_philox_kat, pin_dropout, pin_dropout_seq3,
]
