"""Full-output parity at the full workload sizes, in the launch configurations
the bench times: every output element of every row workload is compared with
the oracle, fused kernels against its binary64 result (EXACT), unfused ones
against its op-by-op evaluation (SEQ / SEQ3).

The oracle is plain single-threaded C; here it runs on chunks of about 2^20
elements of whole rows, the chunks spread over up to 16 threads (its C code
releases the GIL), and each chunk is gated as soon as it is done.  Rows are
independent, so a chunk is computed exactly as in one call over the whole
tensor (dropout takes the chunk's first row, since an element's index picks
its random bits).  Each test prints the number of elements compared, which
must equal rows x cols.

Unfused variants: besides the gates of the fused kernels, at least 99.9% of
their elements must equal the oracle's stored value bit for bit.  Each of
their element-wise ops is one correctly rounded fp32 operation stored in the
I/O type, as in SEQ; they differ only where a row statistic (binary64 sums in
another order) rounds to another fp32 value -- about 1e-5 of the rows -- or
where the GPU's fp32 exponential or GeLU moves a 16-bit rounding, about 1e-4
of the elements.  A rounding missing from any op changes most elements.  The
bf16 three-launch variants, whose middle launch is the fp32 LayerNorm kernel,
are held to the interval gate described below instead of the absolute one.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import as_f64, bits16, check_bf16, check_f32, check_ulp16, ordered, to_dev, to_host

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
CHUNK_ELEMS = 1 << 20


@pytest.fixture(scope="module")
def mbp():
    import memory_bound_pointwise_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def compare_rows(rows, cols, ref_fn, gate_fn):
    """Run ref_fn(a, b) -> float64 [b - a, cols] (the oracle on rows [a, b))
    over row chunks on THREADS threads and gate_fn(a, b, ref) on each; returns
    (the gate results, the number of elements compared)."""
    step = max(1, CHUNK_ELEMS // cols)
    spans = [(a, min(a + step, rows)) for a in range(0, rows, step)]

    def one(span):
        a, b = span
        ref = ref_fn(a, b)
        assert ref.shape == (b - a, cols)
        return gate_fn(a, b, ref), ref.size

    with ThreadPoolExecutor(THREADS) as ex:
        res = list(ex.map(one, spans))
    n = sum(r[1] for r in res)
    assert n == rows * cols, f"compared {n} of {rows * cols} elements"
    return [r[0] for r in res], n


def _iview(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _stored_equal(y, ref):
    """elements of the host output y (bf16 bits or fp32) equal to the oracle's
    stored value (exactly representable in y's type)"""
    return int((as_f64(y) == ref).sum() + (np.isnan(as_f64(y)) & np.isnan(ref)).sum())


def _abs_gate(dtype):
    return check_bf16 if dtype == "bf16" else check_f32


# ------------------------------------------------------------------ the middle LayerNorm launch, bf16
#
# The three-launch variants store the LayerNorm launch's result u in bf16, and
# that launch computes in fp32 (fp32 accumulation for bf16 I/O) where the
# oracle's SEQ3 evaluates it in binary64.  The fp32 launch is within
# E = 3e-5 (1 + |u|) of the exact u (its mean and variance sums, rstd and the
# affine step, about 3x a worst-case estimate), so its stored u is a bf16
# value in [bf16(u - E), bf16(u + E)] (rounding is monotone): for |u| above
# about 0.1 that is the nearest value c0 (SEQ3's stored u) or, near a
# midpoint, its neighbour; close to 0 it spans several values, all within E.
# The later launches (GeLU; relu and dropout) are checked exactly as the
# oracle's SEQ3 runs them: y within 1 bf16 ulp of the smallest and largest
# of their results at c_lo, c0, c_hi (the functions are monotone on so short
# an interval, or flat where GeLU has its minimum).

def _bf16_of(v64):
    """binary64 -> bit patterns of the value stored as SEQ3 stores it (binary32,
    then bfloat16 nearest even)"""
    return oracle.to_bf16(np.asarray(v64, np.float64).astype(np.float32))


def _ord16(bits):
    b = np.asarray(bits).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def _u_interval(u):
    """(c_lo, c0, c_hi): the bf16 values an fp32 launch within E of the exact
    u may store, c0 the nearest one"""
    e = 3e-5 * (1.0 + np.abs(u))
    return as_f64(_bf16_of(u - e)), as_f64(_bf16_of(u)), as_f64(_bf16_of(u + e))


def _check_interval(y_bits, later, u, what):
    """y (bf16 bits) within 1 ulp of later(c) over the stored u's interval;
    returns the number of elements off later(c0) by more than 1 ulp"""
    c_lo, c0, c_hi = _u_interval(u)
    o = [_ord16(_bf16_of(later(c))) for c in (c_lo, c0, c_hi)]
    lo, hi = np.minimum(np.minimum(o[0], o[1]), o[2]), np.maximum(np.maximum(o[0], o[1]), o[2])
    oy = _ord16(y_bits)
    ok = (oy >= lo - 1) & (oy <= hi + 1)
    if not ok.all():
        bad = [tuple(i) for i in np.argwhere(~ok)[:4]]
        rows = [f"at {i}: y {as_f64(y_bits)[i]!r} u {u[i]!r} c {c_lo[i]!r} {c0[i]!r} {c_hi[i]!r}" for i in bad]
        raise AssertionError(f"{what}: {int((~ok).sum())} elements outside the interval:\n" + "\n".join(rows))
    return int((np.abs(oy - o[1]) > 1).sum())


def _stored_sum_bits(x_bits, r_bits):
    """the add launch: x + residual in fp32 (correctly rounded), stored as bf16"""
    return oracle.to_bf16(as_f64(x_bits).astype(np.float32) + as_f64(r_bits).astype(np.float32))


def _keep_mask(a, b, cols, p, seed, offset):
    """dropout's kept elements of rows [a, b): half k mod 8 of the Philox4x32-10
    block (k div 8, offset) keyed by seed, k = row * cols + col, kept iff
    >= round(p 2^16)"""
    k0, k1 = a * cols, b * cols
    q = np.arange(k0 >> 3, ((k1 - 1) >> 3) + 1, dtype=np.uint64)
    ctr = np.stack([q & 0xFFFFFFFF, q >> 32, np.full_like(q, offset & 0xFFFFFFFF),
                    np.full_like(q, offset >> 32)], axis=1).astype(np.uint32)
    key = np.tile(np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint32), (len(q), 1))
    words = oracle.philox4x32_10(ctr, key).reshape(-1)
    halves = np.stack([words & 0xFFFF, words >> 16], axis=1).reshape(-1)
    first = k0 - ((k0 >> 3) << 3)
    return (halves[first:first + (k1 - k0)] >= round(p * 65536)).reshape(b - a, cols)


# ------------------------------------------------------------------ residual + LayerNorm (+ GeLU)

LN_FULL = ["ln_8192x4096_f32", "addln_gelu_16384x8192_bf16", "addln_gelu_262144x768_bf16",
           "addln_gelu_32768x4095_bf16", "addln_gelu_16384x12288_bf16"]


def _act_code(act):
    return oracle.ACT_GELU_TANH if act == "gelu_tanh" else oracle.ACT_NONE


def _ln_ref_fn(d, act, mode):
    r = d.get("residual")
    return lambda a, b: oracle.add_layernorm_gelu(d["x"][a:b], None if r is None else r[a:b], d["gamma"],
                                                  d["beta"], eps=1e-5, act=_act_code(act), mode=mode)


@pytest.mark.parametrize("name", LN_FULL)
def test_ln_full_output(mbp, name):
    w = W.BY_NAME[name]
    d = W.generate(w)
    print(f"{name}: fused, every element vs EXACT", flush=True)
    args = [to_dev(d["x"]), to_dev(d.get("residual")), to_dev(d["gamma"]), to_dev(d["beta"])]
    y1 = mbp.fused_add_layernorm_gelu(*args, eps=1e-5, act=w.act)
    y2 = mbp.fused_add_layernorm_gelu(*args, eps=1e-5, act=w.act)
    assert torch.equal(_iview(y1), _iview(y2)), "not deterministic"
    y = to_host(y1)
    chk = _abs_gate(w.dtype)
    res, n = compare_rows(w.rows, w.cols, _ln_ref_fn(d, w.act, oracle.EXACT),
                          lambda a, b, ref: chk(y[a:b], ref, f"{name} rows {a}..{b}"))
    err = max(r[0] for r in res)
    relaxed = sum(r[1] for r in res)
    print(f"{name}: compared {n} elements (= {w.rows} x {w.cols}), max abs err {err:.3g}, "
          f"half-ulp-gated elements {relaxed}")


@pytest.mark.parametrize("name", LN_FULL)
@pytest.mark.parametrize("gran", [0, 1])
def test_unfused_ln_full_output(mbp, name, gran):
    """The unfused variants at the sizes whose times are the bench's speedup
    denominators: 7 (5) launches against SEQ, 3 (1) against SEQ3."""
    w = W.BY_NAME[name]
    d = W.generate(w)
    mode = oracle.SEQ if gran == 0 else oracle.SEQ3
    print(f"{name}: unfused granularity {gran}, every element vs {'SEQ' if gran == 0 else 'SEQ3'}", flush=True)
    y = to_host(mbp.unfused_add_layernorm_gelu(to_dev(d["x"]), to_dev(d.get("residual")), to_dev(d["gamma"]),
                                               to_dev(d["beta"]), eps=1e-5, act=w.act, granularity=gran))
    chk = _abs_gate(w.dtype)
    two = gran == 1 and w.dtype == "bf16" and w.act == "gelu_tanh"

    def gate(a, b, ref):
        what = f"unfused {name} granularity {gran} rows {a}..{b}"
        other = 0
        if two:
            v = _stored_sum_bits(d["x"][a:b], d["residual"][a:b])
            u = oracle.add_layernorm_gelu(v, None, d["gamma"], d["beta"], act=oracle.ACT_NONE)
            seq3_u = oracle.add_layernorm_gelu(v, None, d["gamma"], d["beta"], act=oracle.ACT_NONE,
                                               mode=oracle.SEQ3)
            assert np.array_equal(_u_interval(u)[1], seq3_u), "c0 is SEQ3's stored u"
            other = _check_interval(y[a:b], oracle.gelu_tanh, u, what)
            err = float(np.nanmax(np.abs(as_f64(y[a:b]) - ref)))
        else:
            err, _ = chk(y[a:b], ref, what)
        return err, _stored_equal(y[a:b], ref), other

    res, n = compare_rows(w.rows, w.cols, _ln_ref_fn(d, w.act, mode), gate)
    same, other = sum(r[1] for r in res), sum(r[2] for r in res)
    print(f"{name} unfused granularity {gran}: compared {n} elements, max abs err "
          f"{max(r[0] for r in res):.3g}, bit-identical to the oracle {same} ({same / n:.6%}), "
          f"more than 1 ulp from the later launches at SEQ3's u (inside the interval) {other}")
    assert same >= 0.999 * n, f"only {same / n:.4%} of the elements are the oracle's stored value"


@pytest.mark.parametrize("name", ["addln_gelu_16384x8192_bf16_ld8320", "addln_gelu_16384x8192_bf16_ld8195"])
def test_ln_strided_full_output(mbp, name):
    """The padded-row workloads the bench times: x, residual and y are views
    into buffers of rows of `ld` elements; every element vs EXACT, and the
    padding left untouched."""
    w = W.NEXT_BY_NAME[name]
    d = W.generate(w)
    ld = w.params["ld"]

    def padded(a, fill):
        t = to_dev(a)
        buf = torch.full((w.rows, ld), fill, dtype=t.dtype, device="cuda")
        v = buf[:, :w.cols]
        v.copy_(t)
        return v, buf

    x, _ = padded(d["x"], 0.0)
    r, _ = padded(d["residual"], 0.0)
    y, yb = padded(np.zeros_like(d["x"]), 3.0)
    print(f"{name}: fused on rows of {ld} elements, every element vs EXACT", flush=True)
    mbp.fused_add_layernorm_gelu(x, r, to_dev(d["gamma"]), to_dev(d["beta"]), eps=1e-5, act=w.act, out=y)
    assert bool((yb[:, w.cols:].float() == 3.0).all()), "wrote into the row padding"
    yh = to_host(y.contiguous())
    res, n = compare_rows(w.rows, w.cols, _ln_ref_fn(d, w.act, oracle.EXACT),
                          lambda a, b, ref: check_bf16(yh[a:b], ref, f"{name} rows {a}..{b}"))
    print(f"{name}: compared {n} elements, max abs err {max(r_[0] for r_ in res):.3g}")


# ------------------------------------------------------------------ LayerNorm -> ReLU -> Dropout

def _dropout_gate(y, d, dtype, p, seed, offset, mode, what):
    """kept / dropped pattern exactly wherever relu(LN) > 1e-3 (closer to 0 the
    fp32 rounding of the normalised value may move an element across the
    relu), values within the LayerNorm gates"""
    chk = _abs_gate(dtype)

    def ref_fn(a, b):
        return oracle.ln_relu_dropout(d["x"][a:b], d["gamma"], d["beta"], p=p, seed=seed, offset=offset,
                                      mode=mode, first_row=a)

    two = mode == oracle.SEQ3 and dtype == "bf16"

    def gate(a, b, ref):
        u = oracle.add_layernorm_gelu(d["x"][a:b], None, d["gamma"], d["beta"], act=oracle.ACT_NONE)
        relu_ln = np.maximum(u, 0)
        yc = y[a:b]
        clear = relu_ln > 1e-3
        kept_y, kept_ref = (as_f64(yc) != 0)[clear], (ref != 0)[clear]
        assert np.array_equal(kept_y, kept_ref), \
            f"{what} rows {a}..{b}: dropout mask differs at {int((kept_y != kept_ref).sum())} elements"
        if two:
            keep = _keep_mask(a, b, u.shape[1], p, seed, offset)
            sc = np.float32(1.0 / (1.0 - p))
            later = lambda c: np.where(keep, (np.maximum(c, 0).astype(np.float32) * sc).astype(np.float64), 0.0)
            _check_interval(yc, later, u, f"{what} rows {a}..{b}")
            err = float(np.nanmax(np.abs(as_f64(yc) - ref)))
        else:
            err, _ = chk(yc, ref, f"{what} rows {a}..{b}")
        return err, int(clear.sum()), int((~kept_ref).sum()), _stored_equal(yc, ref)

    return ref_fn, gate


@pytest.mark.parametrize("variant", ["fused", "fused_misaligned_8191", "unfused"])
def test_ln_relu_dropout_full_output(mbp, variant):
    w = W.NEXT_BY_NAME["ln_relu_dropout_16384x8192_bf16"]
    pr = w.params
    cols = 8191 if variant == "fused_misaligned_8191" else w.cols
    d = W.generate(w, cols=cols)
    print(f"ln_relu_dropout {w.rows}x{cols} {variant}", flush=True)
    g, b = to_dev(d["gamma"]), to_dev(d["beta"])
    xd = to_dev(d["x"])
    if variant == "fused_misaligned_8191":
        # x and y one element past a 128-byte line: rows of 16382 bytes off 16-byte boundaries
        buf = torch.zeros(xd.numel() + 64, dtype=xd.dtype, device="cuda")
        xd_m = buf[1:1 + xd.numel()].view(xd.shape)
        xd_m.copy_(xd)
        ybuf = torch.zeros_like(buf)
        yd = ybuf[1:1 + xd.numel()].view(xd.shape)
        mbp.fused_layernorm_relu_dropout(xd_m, g, b, pr["p"], pr["seed"], pr["offset"], pr["eps"], out=yd)
        mode = oracle.EXACT
    elif variant == "fused":
        yd = mbp.fused_layernorm_relu_dropout(xd, g, b, pr["p"], pr["seed"], pr["offset"], pr["eps"])
        y2 = mbp.fused_layernorm_relu_dropout(xd, g, b, pr["p"], pr["seed"], pr["offset"], pr["eps"])
        assert torch.equal(_iview(yd), _iview(y2)), "not deterministic"
        mode = oracle.EXACT
    else:
        yd = mbp.unfused_layernorm_relu_dropout(xd, g, b, pr["p"], pr["seed"], pr["offset"], pr["eps"])
        mode = oracle.SEQ3
    y = to_host(yd)
    ref_fn, gate = _dropout_gate(y, d, w.dtype, pr["p"], pr["seed"], pr["offset"], mode,
                                 f"ln_relu_dropout {cols} {variant}")
    res, n = compare_rows(w.rows, cols, ref_fn, gate)
    clear, dropped, same = (sum(r[i] for r in res) for i in (1, 2, 3))
    print(f"ln_relu_dropout {w.rows}x{cols} {variant}: compared {n} elements, mask checked on {clear} "
          f"(dropped {dropped / clear:.4f} of them, p = {pr['p']}), max abs err {max(r[0] for r in res):.3g}, "
          f"bit-identical {same / n:.4%}")
    assert abs(dropped / clear - pr["p"]) < 5 * np.sqrt(pr["p"] * (1 - pr["p"]) / clear)
    if variant == "unfused":
        assert same >= 0.999 * n, f"only {same / n:.4%} of the elements are the oracle's stored value"


# ------------------------------------------------------------------ softmax, two-dimensional forms

def _as_f32(a):
    if a.dtype == np.uint16:
        return W.bf16_bits_to_f32(a)
    return a.astype(np.float32)


@pytest.mark.parametrize("variant", ["fused", "unfused"])
def test_softmax_full_output(mbp, variant):
    w = W.NEXT_BY_NAME["softmax_131072x4096_bf16"]
    d = W.generate(w)
    print(f"softmax {w.rows}x{w.cols} {variant}", flush=True)
    x = to_dev(d["x"])
    if variant == "fused":
        y1 = mbp.fused_softmax(x)
        assert torch.equal(_iview(y1), _iview(mbp.fused_softmax(x))), "not deterministic"
        mode = oracle.EXACT
    else:
        y1 = mbp.unfused_softmax(x)
        mode = oracle.SEQ
    y = bits16(y1)
    xf = _as_f32(d["x"])
    del y1
    res, n = compare_rows(w.rows, w.cols, lambda a, b: oracle.softmax(xf[a:b], mode=mode, dtype="bf16"),
                          lambda a, b, ref: check_ulp16(y[a:b], ref, "bf16", f"softmax {variant} rows {a}..{b}"))
    off = sum(r[1] for r in res)
    print(f"softmax {variant}: compared {n} elements, max {max(r[0] for r in res)} ulp, {off} elements 1 ulp off "
          f"({off / n:.5%})")
    if variant == "unfused":
        assert off <= 0.001 * n


def test_chain2d_full_output(mbp):
    w = W.NEXT_BY_NAME["chain2d_16384x4096_bf16_bcast"]
    d = W.generate(w)
    x, b1, b2 = (to_dev(d[k]) for k in ("x", "b1", "b2"))
    y1 = mbp.fused_pointwise_chain_2d(x, b1, b2, w.params["scale"])
    assert torch.equal(_iview(y1), _iview(mbp.fused_pointwise_chain_2d(x, b1, b2, w.params["scale"])))
    y = bits16(y1)
    xf, b1f, b2f = (_as_f32(d[k]) for k in ("x", "b1", "b2"))

    def ref_fn(a, b):
        row = np.ascontiguousarray(np.broadcast_to(b1f, (b - a, w.cols)))
        return oracle.pointwise_chain(xf[a:b], row, b2f[a:b], w.params["scale"])

    res, n = compare_rows(w.rows, w.cols, ref_fn,
                          lambda a, b, ref: check_ulp16(y[a:b], ref, w.dtype, f"chain2d rows {a}..{b}"))
    print(f"{w.name}: compared {n} elements, max {max(r[0] for r in res)} ulp, "
          f"{sum(r[1] for r in res)} elements 1 ulp off")


def test_tenop2d_full_output(mbp):
    w = W.NEXT_BY_NAME["tenop2d_8192x1024_f16_ld1056"]
    d = W.generate(w)
    ld = w.params["ld"]
    xd = to_dev(d["x"])
    xb = torch.zeros((w.rows, ld), dtype=xd.dtype, device="cuda")
    x = xb[:, :w.cols]
    x.copy_(xd)
    vec = [to_dev(d[k]) for k in ("bias", "gamma", "beta")]
    outs = []
    for _ in range(2):
        yb = torch.full((w.rows, ld), 3.0, dtype=xd.dtype, device="cuda")
        mbp.fused_row_mean_epilogue_2d(x, *vec, alpha=w.params["alpha"], c=w.params["c"], out=yb[:, :w.cols])
        assert (yb[:, w.cols:].float() == 3.0).all(), "wrote into the row padding"
        outs.append(yb[:, :w.cols])
    assert torch.equal(_iview(outs[0].contiguous()), _iview(outs[1].contiguous())), "not deterministic"
    y = bits16(outs[0])
    xf = _as_f32(d["x"])
    vf = [_as_f32(d[k]) for k in ("bias", "gamma", "beta")]
    res, n = compare_rows(w.rows, w.cols,
                          lambda a, b: oracle.row_mean_epilogue(xf[a:b], *vf, w.params["alpha"], w.params["c"]),
                          lambda a, b, ref: check_ulp16(y[a:b], ref, w.dtype, f"tenop2d rows {a}..{b}"))
    print(f"{w.name}: compared {n} elements, max {max(r[0] for r in res)} ulp, "
          f"{sum(r[1] for r in res)} elements 1 ulp off")


# ------------------------------------------------------------------ the chain and the 10-op graph, unfused

def test_unfused_tenop_full_output(mbp):
    w = W.BY_NAME["tenop_1024x1024_f32"]
    d = W.generate(w)
    args = [to_dev(d[k]) for k in ("x", "bias", "gamma", "beta")]
    ref = oracle.row_mean_epilogue(d["x"], d["bias"], d["gamma"], d["beta"], mode=oracle.SEQ)
    for fn in (mbp.unfused_row_mean_epilogue, mbp.grouped_row_mean_epilogue):
        y = to_host(fn(*args))
        err, _ = check_f32(y, ref, f"{fn.__name__} full")
        same = _stored_equal(y, ref)
        print(f"{fn.__name__} {w.rows}x{w.cols}: max abs err {err:.3g}, bit-identical {same / y.size:.4%}")
        assert same >= 0.999 * y.size
