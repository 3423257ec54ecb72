"""GPU parity: every entry point of the C ABI (through the Python binding, which
calls it via ctypes) against the CPU oracle on the same seeded inputs.

Small and ragged sizes are compared element by element in full; so are the
chain and the 10-op graph at their full workload sizes.  The other full
workload sizes (the launch configurations the bench times) are compared
element by element in test_gpu_full.py.  Row kernels are also checked for
bitwise determinism.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import (as_f64, check_bf16, check_chain, check_f32, check_softmax_f32, sample_rows,
                         to_dev, to_host, bits16, check_ulp16, ordered)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mbp():
    import memory_bound_pointwise_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _chain_inputs(n, seed_sub=0):
    w = W.scaled(W.BY_NAME["chain_4M_f32"], n=n)
    return W.generate(w)


# ------------------------------------------------------------------ pointwise chain

@pytest.mark.parametrize("n", list(range(1, 34)) + [255, 256, 257, 1000, 4099, 65537, 1 << 20])
def test_chain_sizes(mbp, n):
    d = _chain_inputs(n)
    y = mbp.fused_pointwise_chain(to_dev(d["x"]), to_dev(d["b1"]), to_dev(d["b2"]), 0.5)
    check_chain(to_host(y), oracle.pointwise_chain(d["x"], d["b1"], d["b2"], 0.5), f"n={n}")


@pytest.mark.parametrize("offs", [(1, 1, 1, 1), (2, 2, 2, 2), (3, 3, 3, 3), (0, 1, 2, 3), (1, 0, 0, 0),
                                  (0, 0, 0, 2)])
def test_chain_misaligned(mbp, offs):
    n = 10007
    d = _chain_inputs(n)
    bufs = []
    for k, name in enumerate(("x", "b1", "b2")):
        b = torch.zeros(n + 8, device="cuda")
        b[offs[k]:offs[k] + n] = to_dev(d[name])
        bufs.append(b[offs[k]:offs[k] + n])
    out = torch.full((n + 8,), 7.0, device="cuda")
    y = out[offs[3]:offs[3] + n]
    mbp.fused_pointwise_chain(*bufs, 0.5, out=y)
    check_chain(to_host(y), oracle.pointwise_chain(d["x"], d["b1"], d["b2"], 0.5), f"offsets {offs}")
    host = to_host(out)
    assert (host[:offs[3]] == 7.0).all() and (host[offs[3] + n:] == 7.0).all(), "wrote outside y"


def test_chain_in_place_and_scale(mbp):
    d = _chain_inputs(4099)
    x = to_dev(d["x"])
    mbp.fused_pointwise_chain(x, to_dev(d["b1"]), to_dev(d["b2"]), 0.3, out=x)
    check_chain(to_host(x), oracle.pointwise_chain(d["x"], d["b1"], d["b2"], 0.3), "in place, scale 0.3")


def test_chain_special_values(mbp):
    x = np.array([np.nan, np.inf, -np.inf, -0.0, 0.0, 3e38, -3e38, 1e-45, -1e-45, 1.0, -1.0, 2.0],
                 np.float32)
    b1 = np.array([0, 0, 0, 0, -0.0, 3e38, 0, -1e-45, 1e-45, -1.0, 1.0, -2.0], np.float32)
    b2 = np.array([1, 1, 1, -0.0, -0.0, 0, 5, 0, 0, 1e-30, -1e-30, 0.5], np.float32)
    y = to_host(mbp.fused_pointwise_chain(to_dev(x), to_dev(b1), to_dev(b2), 0.5))
    ref = oracle.pointwise_chain(x, b1, b2, 0.5)
    check_chain(y, ref, "special values")


def test_chain_full_workload(mbp):
    w = W.BY_NAME["chain_4M_f32"]
    d = W.generate(w)
    args = [to_dev(d[k]) for k in ("x", "b1", "b2")]
    y1 = to_host(mbp.fused_pointwise_chain(*args, 0.5))
    y2 = to_host(mbp.fused_pointwise_chain(*args, 0.5))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    worst = check_chain(y1, oracle.pointwise_chain(d["x"], d["b1"], d["b2"], 0.5), w.name)
    print(f"{w.name}: max ulp {worst}")


# ------------------------------------------------------------------ 10-op graph

# fp32 rows of up to 256 vectors take one vector per lane in 16- to 256-lane
# groups (4, 64, 100, 200, 500, 1000, 1024); wider rows the layout table;
# widths that are not whole vectors the element path
@pytest.mark.parametrize("rows,cols", [(1, 1), (1, 4), (3, 7), (2, 1024), (5, 1000), (33, 1024),
                                       (4, 4096), (3, 4093), (2, 16384), (7, 16383), (300, 64),
                                       (9, 100), (17, 200), (5, 500), (40, 1020)])
def test_tenop_shapes(mbp, rows, cols):
    w = W.scaled(W.BY_NAME["tenop_1024x1024_f32"], rows=rows)
    d = W.generate(w, cols=cols)
    y = mbp.fused_row_mean_epilogue(*(to_dev(d[k]) for k in ("x", "bias", "gamma", "beta")))
    ref = oracle.row_mean_epilogue(d["x"], d["bias"], d["gamma"], d["beta"])
    check_f32(to_host(y), ref, f"10-op {rows}x{cols}")


def test_tenop_in_place_and_misaligned(mbp):
    w = W.scaled(W.BY_NAME["tenop_1024x1024_f32"], rows=6)
    d = W.generate(w, cols=1024)
    ref = oracle.row_mean_epilogue(d["x"], d["bias"], d["gamma"], d["beta"])
    x = to_dev(d["x"])
    mbp.fused_row_mean_epilogue(x, *(to_dev(d[k]) for k in ("bias", "gamma", "beta")), out=x)
    check_f32(to_host(x), ref, "in place")
    buf = torch.zeros(6 * 1024 + 1, device="cuda")
    xs = buf[1:].view(6, 1024)
    xs.copy_(to_dev(d["x"]))
    y = mbp.fused_row_mean_epilogue(xs, *(to_dev(d[k]) for k in ("bias", "gamma", "beta")))
    check_f32(to_host(y), ref, "misaligned x (scalar path)")


@pytest.mark.parametrize("cols", [1024, 1000, 64, 4096])
def test_tenop_special_values(mbp, cols):
    """NaN and infinities in x: a NaN makes its whole row NaN (relu passes it
    on, the row sum carries it); +inf gives inf in s and in the row sum, so
    its element is inf - inf = NaN and the others -inf * gamma + beta; -inf
    is cut by the relu.  Positions of NaN and of each signed infinity must
    match the oracle, the finite elements the fp32 gate."""
    w = W.scaled(W.BY_NAME["tenop_1024x1024_f32"], rows=6)
    d = W.generate(w, cols=cols)
    x = d["x"].copy()
    x[0, 3] = np.nan
    x[1, cols // 2] = np.inf
    x[2, 0] = -np.inf
    x[3, cols - 1] = -np.inf
    x[3, 1] = np.nan
    g = d["gamma"].copy()
    g[5 % cols] = 0.0  # 0 * inf = NaN in row 1
    y = to_host(mbp.fused_row_mean_epilogue(to_dev(x), to_dev(d["bias"]), to_dev(g), to_dev(d["beta"])))
    ref = oracle.row_mean_epilogue(x, d["bias"], g, d["beta"])
    assert np.array_equal(np.isnan(y), np.isnan(ref)), "NaN positions"
    assert np.array_equal(np.isposinf(y), np.isposinf(ref)) and np.array_equal(np.isneginf(y), np.isneginf(ref)), \
        "infinity positions"
    fin = np.isfinite(ref)
    check_f32(y[fin], ref[fin], f"10-op special values, {cols} columns")
    assert np.isnan(y[0]).all() and np.isnan(y[1, cols // 2]) and np.isfinite(y[2]).all()


def test_tenop_full_workload(mbp):
    w = W.BY_NAME["tenop_1024x1024_f32"]
    d = W.generate(w)
    args = [to_dev(d[k]) for k in ("x", "bias", "gamma", "beta")]
    y1 = to_host(mbp.fused_row_mean_epilogue(*args, alpha=1.1, c=0.1))
    y2 = to_host(mbp.fused_row_mean_epilogue(*args, alpha=1.1, c=0.1))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), "not deterministic"
    err, relaxed = check_f32(y1, oracle.row_mean_epilogue(d["x"], d["bias"], d["gamma"], d["beta"]), w.name)
    print(f"{w.name}: max abs err {err:.3g}, elements with |y| >= 256: {relaxed}")
    # constant gamma: each output row has mean(beta) as its mean
    g = torch.full_like(args[2], 1.5)
    y = mbp.fused_row_mean_epilogue(args[0], args[1], g, args[3]).double()
    assert torch.allclose(y.mean(dim=1), args[3].double().mean().expand(1024), atol=1e-4)


# ------------------------------------------------------------------ LayerNorm family

def _ln_case(name, rows, cols, residual=None, act=None):
    w = W.scaled(W.BY_NAME[name], rows=rows)
    d = W.generate(w, cols=cols)
    if residual is True and d.get("residual") is None:
        # the fp32 workload has no residual: take N(0, 1) rows of the 10-op workload's x
        d["residual"] = W.generate(W.scaled(W.BY_NAME["tenop_1024x1024_f32"], rows=rows), cols=cols)["x"]
    if residual is False:
        d["residual"] = None
    act = w.act if act is None else act
    return w, d, act


def _ln_run(mbp, d, act, out=None):
    return mbp.fused_add_layernorm_gelu(to_dev(d["x"]), to_dev(d.get("residual")), to_dev(d["gamma"]),
                                        to_dev(d["beta"]), eps=1e-5, act=act, out=out)


def _ln_ref(d, act, rows=None, mode=oracle.EXACT):
    pick = (lambda a: a) if rows is None else (lambda a: None if a is None else a[rows])
    code = oracle.ACT_GELU_TANH if act == "gelu_tanh" else oracle.ACT_NONE
    return oracle.add_layernorm_gelu(pick(d["x"]), pick(d.get("residual")), d["gamma"], d["beta"],
                                     eps=1e-5, act=code, mode=mode)


F32_COLS = [1, 3, 4, 5, 64, 255, 256, 257, 1000, 1024, 4095, 4096, 8192, 10001, 12288, 16383, 16384]
BF16_COLS = [1, 7, 8, 9, 33, 255, 256, 257, 768, 1023, 1024, 4095, 4096, 8192, 12288, 16384]


@pytest.mark.parametrize("cols", F32_COLS)
@pytest.mark.parametrize("residual,act", [(False, "none"), (True, "none"), (True, "gelu_tanh")])
def test_ln_f32_shapes(mbp, cols, residual, act):
    w, d, act = _ln_case("ln_8192x4096_f32", 5, cols, residual, act)
    y = to_host(_ln_run(mbp, d, act))
    check_f32(y, _ln_ref(d, act), f"fp32 {cols} residual={residual} act={act}")


@pytest.mark.parametrize("cols", BF16_COLS)
@pytest.mark.parametrize("residual,act", [(True, "gelu_tanh"), (False, "none"), (False, "gelu_tanh")])
def test_ln_bf16_shapes(mbp, cols, residual, act):
    w, d, act = _ln_case("addln_gelu_16384x8192_bf16", 5, cols, residual, act)
    y = to_host(_ln_run(mbp, d, act))
    check_bf16(y, _ln_ref(d, act), f"bf16 {cols} residual={residual} act={act}")


@pytest.mark.parametrize("dtype_name", ["ln_8192x4096_f32", "addln_gelu_16384x8192_bf16"])
def test_ln_misaligned_and_in_place(mbp, dtype_name):
    w, d, act = _ln_case(dtype_name, 7, 1024)
    ref = _ln_ref(d, act)
    chk = check_bf16 if w.dtype == "bf16" else check_f32
    x = to_dev(d["x"])
    buf = torch.zeros(x.numel() + 1, dtype=x.dtype, device="cuda")
    xs = buf[1:].view(x.shape)
    xs.copy_(x)
    y = mbp.fused_add_layernorm_gelu(xs, to_dev(d.get("residual")), to_dev(d["gamma"]),
                                     to_dev(d["beta"]), act=act)
    chk(to_host(y), ref, "misaligned x (scalar path)")
    mbp.fused_add_layernorm_gelu(x, to_dev(d.get("residual")), to_dev(d["gamma"]), to_dev(d["beta"]),
                                 act=act, out=x)
    chk(to_host(x), ref, "in place")


@pytest.mark.parametrize("dtype_name,cols,shift,rows", [
    ("addln_gelu_16384x8192_bf16", 4095, 1, 9), ("addln_gelu_16384x8192_bf16", 4095, 0, 33),
    ("addln_gelu_16384x8192_bf16", 4095, 5, 1), ("addln_gelu_16384x8192_bf16", 4095, 3, 2),
    ("addln_gelu_16384x8192_bf16", 768, 3, 9), ("addln_gelu_16384x8192_bf16", 8192, 7, 9),
    ("addln_gelu_16384x8192_bf16", 3, 5, 40), ("addln_gelu_16384x8192_bf16", 1, 7, 21),
    ("addln_gelu_16384x8192_bf16", 13, 2, 300), ("addln_gelu_16384x8192_bf16", 12290, 1, 5),
    # 512-lane class layout with eight row groups a block (several per class)
    ("addln_gelu_16384x8192_bf16", 8191, 1, 600), ("addln_gelu_16384x8192_bf16", 6145, 0, 530),
    # 256-lane class layout, several row groups a block
    ("addln_gelu_16384x8192_bf16", 3501, 3, 300),
    ("ln_8192x4096_f32", 4093, 1, 9), ("ln_8192x4096_f32", 1024, 2, 9), ("ln_8192x4096_f32", 5, 3, 40),
    ("ln_8192x4096_f32", 6, 0, 17)])
def test_ln_common_misalignment(mbp, dtype_name, cols, shift, rows):
    """x, residual and y all start `shift` elements past a 16-byte boundary:
    the windowed path (rows off 16-byte boundaries, residue classes of the row
    shift), including the edge rows whose windows would leave the tensor."""
    w, d, act = _ln_case(dtype_name, rows, cols, residual=True)
    ref = _ln_ref(d, act)
    chk = check_bf16 if w.dtype == "bf16" else check_f32

    def place(a):
        t = to_dev(a)
        buf = torch.zeros(t.numel() + 16, dtype=t.dtype, device="cuda")
        v = buf[shift:shift + t.numel()].view(t.shape)
        v.copy_(t)
        return v, buf

    x, xb = place(d["x"])
    r, rb = place(d["residual"])
    yb = torch.full((x.numel() + 16,), 3.0, dtype=x.dtype, device="cuda")
    y = yb[shift:shift + x.numel()].view(x.shape)
    mbp.fused_add_layernorm_gelu(x, r, to_dev(d["gamma"]), to_dev(d["beta"]), act=act, out=y)
    chk(to_host(y), ref, f"common misalignment {shift}")
    host = to_host(yb).astype(np.float64) if yb.dtype != torch.bfloat16 else as_f64(to_host(yb))
    assert (host[:shift] == 3.0).all() and (host[shift + x.numel():] == 3.0).all(), "wrote outside y"


@pytest.mark.parametrize("dtype_name,cols,offs,rows", [
    ("addln_gelu_16384x8192_bf16", 4095, (1, 2, 3, 0, 0), 9),
    ("addln_gelu_16384x8192_bf16", 4096, (0, 1, 0, 0, 0), 5),
    ("addln_gelu_16384x8192_bf16", 1023, (3, 0, 7, 1, 2), 17),
    ("addln_gelu_16384x8192_bf16", 7, (1, 3, 0, 0, 0), 40),
    ("addln_gelu_16384x8192_bf16", 33, (2, 5, 1, 0, 0), 33),
    ("addln_gelu_16384x8192_bf16", 300, (0, 6, 6, 0, 0), 21),
    ("addln_gelu_16384x8192_bf16", 12288, (0, 0, 1, 0, 0), 3),
    ("addln_gelu_16384x8192_bf16", 8192, (0, 0, 0, 1, 3), 9),
    ("addln_gelu_16384x8192_bf16", 4095, (2, 2, 2, 5, 1), 11),
    ("ln_8192x4096_f32", 4093, (1, 2, 0, 0, 0), 9),
    ("ln_8192x4096_f32", 5, (0, 1, 2, 0, 0), 40),
    ("ln_8192x4096_f32", 1024, (0, 0, 3, 1, 1), 9),
    ("ln_8192x4096_f32", 130, (3, 1, 2, 2, 0), 19)])
def test_ln_independent_misalignment(mbp, dtype_name, cols, offs, rows):
    """x, residual, y, gamma and beta each `offs` elements past a 16-byte
    boundary.  Different offsets of x, residual and y take the lane-shift
    path; equal ones the per-class window path, here with gamma and beta off
    their boundaries."""
    w, d, act = _ln_case(dtype_name, rows, cols, residual=True)
    ref = _ln_ref(d, act)
    chk = check_bf16 if w.dtype == "bf16" else check_f32

    def place(a, off, fill=0.0):
        t = to_dev(a)
        buf = torch.full((t.numel() + 16,), fill, dtype=t.dtype, device="cuda")
        v = buf[off:off + t.numel()].view(t.shape)
        v.copy_(t)
        return v

    x, r = place(d["x"], offs[0]), place(d["residual"], offs[1])
    g, b = place(d["gamma"], offs[3]), place(d["beta"], offs[4])
    yb = torch.full((x.numel() + 16,), 3.0, dtype=x.dtype, device="cuda")
    y = yb[offs[2]:offs[2] + x.numel()].view(x.shape)
    mbp.fused_add_layernorm_gelu(x, r, g, b, act=act, out=y)
    chk(to_host(y), ref, f"offsets {offs}")
    host = to_host(yb).astype(np.float64) if yb.dtype != torch.bfloat16 else as_f64(to_host(yb))
    assert (host[:offs[2]] == 3.0).all() and (host[offs[2] + x.numel():] == 3.0).all(), "wrote outside y"



@pytest.mark.parametrize("name,cols,rows", [
    ("addln_gelu_16384x8192_bf16", 4095, 130), ("addln_gelu_16384x8192_bf16", 768 + 1, 70),
    ("addln_gelu_16384x8192_bf16", 1023, 33), ("addln_gelu_16384x8192_bf16", 12290, 9),
    ("ln_8192x4096_f32", 4093, 70), ("ln_8192x4096_f32", 1021, 40), ("ln_8192x4096_f32", 12289, 9),
    ("addln_gelu_16384x8192_bf16", 16383, 5)])
@pytest.mark.parametrize("bytes_off", [(4, 4, 4), (20, 20, 20), (124, 124, 124), (64, 64, 64),
                                       (4, 20, 4), (12, 12, 124)])
def test_ln_line_classes(mbp, name, cols, rows, bytes_off):
    """Rows off 16-byte boundaries, x, residual and y starting `bytes_off`
    bytes past a 128-byte line.  Equal offsets take the per-class window path
    with classes modulo a line (the rows cover every class, so every window
    offset in the line and every ring shift of gamma / beta appears); offsets
    equal only modulo 16 take it with classes modulo 16 bytes.  fp32 rows of
    12289 (over 2048 slots) take gamma / beta funnelled into registers instead
    of the LDS ring."""
    w, d, act = _ln_case(name, rows, cols, residual=True)
    ref = _ln_ref(d, act)
    chk = check_bf16 if w.dtype == "bf16" else check_f32
    es = 2 if w.dtype == "bf16" else 4

    def place(a, off_b, fill=0.0):
        t = to_dev(a)
        buf = torch.full((t.numel() + 128,), fill, dtype=t.dtype, device="cuda")
        assert buf.data_ptr() % 128 == 0
        v = buf[off_b // es:off_b // es + t.numel()].view(t.shape)
        v.copy_(t)
        return v, buf

    x, _ = place(d["x"], bytes_off[0])
    r, _ = place(d["residual"], bytes_off[1])
    y, yb = place(np.zeros_like(d["x"]), bytes_off[2], fill=3.0)
    mbp.fused_add_layernorm_gelu(x, r, to_dev(d["gamma"]), to_dev(d["beta"]), act=act, out=y)
    chk(to_host(y), ref, f"{name} {rows}x{cols} byte offsets {bytes_off}")
    host = to_host(yb).astype(np.float64) if yb.dtype != torch.bfloat16 else as_f64(to_host(yb))
    o = bytes_off[2] // es
    assert (host[:o] == 3.0).all() and (host[o + x.numel():] == 3.0).all(), "wrote outside y"


@pytest.mark.parametrize("name", ["ln_8192x4096_f32", "addln_gelu_16384x8192_bf16"])
@pytest.mark.parametrize("cols", [4096, 4095])
@pytest.mark.parametrize("eps", [0.0, 1e-12, 1.0, 100.0])
def test_ln_eps(mbp, name, cols, eps):
    """eps from 0 to far above the row variance (the output tends to beta),
    on the aligned and the per-class window kernels; rows of small spread
    (1e-3 around 5) where eps = 1e-12 and eps = 0 still differ from 1e-5"""
    w, d, act = _ln_case(name, 17, cols, residual=False)
    rng = np.random.default_rng([31, cols, int(eps * 1000)])
    x = d["x"]
    if w.dtype == "f32":
        x[3] = (5.0 + 1e-3 * rng.standard_normal(cols)).astype(np.float32)
    y = mbp.fused_add_layernorm_gelu(to_dev(x), None, to_dev(d["gamma"]), to_dev(d["beta"]), eps=eps, act=act)
    ref = oracle.add_layernorm_gelu(x, None, d["gamma"], d["beta"], eps=eps, act=(
        oracle.ACT_GELU_TANH if act == "gelu_tanh" else oracle.ACT_NONE))
    chk = check_bf16 if w.dtype == "bf16" else check_f32
    chk(to_host(y), ref, f"{name} {cols} eps={eps}")

@pytest.mark.parametrize("cols", [4095, 4096, 1001, 12287])
@pytest.mark.parametrize("offset", [3.0e3, -3.0e4, 1.0e5])
def test_ln_bf16_rows_far_from_zero(mbp, cols, offset):
    """bf16 x + residual rows with a large common offset, where the fp32
    statistics cancel unless every term is centred before it is squared:
    rows on 16-byte boundaries (vector kernel), x, residual and y at one
    offset off them (class kernel, whose windows carry elements of the
    neighbouring rows) and at different offsets (shift kernel)."""
    rng = np.random.default_rng([43, cols, int(abs(offset)), int(offset < 0)])
    rows = 37

    def bf(a):
        return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)

    x = bf(offset + 2 * rng.standard_normal((rows, cols)))
    r = bf(2 * rng.standard_normal((rows, cols)))
    g = bf(1 + 0.1 * rng.standard_normal(cols))
    b = bf(0.1 * rng.standard_normal(cols))
    bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    ref = oracle.add_layernorm_gelu(bits(x), bits(r), bits(g), bits(b), act=oracle.ACT_GELU_TANH)

    def place(t, off):
        buf = torch.zeros(t.numel() + 16, dtype=torch.bfloat16, device="cuda")
        v = buf[off:off + t.numel()].view(t.shape)
        v.copy_(t.cuda())
        return v

    for offs in ((0, 0, 0), (1, 1, 1), (3, 3, 3), (1, 2, 4)):
        xs, rs, ys = place(x, offs[0]), place(r, offs[1]), place(torch.zeros_like(x), offs[2])
        mbp.fused_add_layernorm_gelu(xs, rs, g.cuda(), b.cuda(), act="gelu_tanh", out=ys)
        err, _ = check_bf16(to_host(ys), ref, f"bf16 {rows}x{cols} offset {offset} element offsets {offs}")
        print(f"bf16 {rows}x{cols} rows around {offset}, element offsets {offs}: max abs err {err:.3g}")


@pytest.mark.parametrize("cols", [4096, 4095, 1001, 768, 12287])
def test_ln_constant_rows_give_beta(mbp, cols):
    """A row of equal values has mean exactly that value and variance 0, so the
    output is beta exactly.  Row lengths that are not powers of two catch a
    mean taken as sum * (1 / cols) without correction: one ulp off, and that
    ulp over a zero spread is scaled up by 1 / sqrt(eps).  Values of several
    magnitudes (x 1, x 1000) in every row layout kernel."""
    for name in ("ln_8192x4096_f32", "addln_gelu_16384x8192_bf16"):
        w, d, _ = _ln_case(name, 6, cols, residual=False)
        col = d["x"][:, :1]
        if w.dtype == "bf16":
            f = W.bf16_bits_to_f32(col)
            col = np.concatenate([col[:3], W.f32_to_bf16_bits(f[3:] * np.float32(1000.0))])
        else:
            col = np.concatenate([col[:3], col[3:] * np.float32(1000.0)]).astype(np.float32)
        d["x"] = np.ascontiguousarray(np.repeat(col, cols, axis=1))
        y = to_host(_ln_run(mbp, d, "none"))
        assert np.array_equal(y, np.broadcast_to(d["beta"], y.shape)), f"{name} {cols}: constant row != beta"


def test_ln_f32_two_groups_per_block(mbp):
    """fp32 rows with thousands of row groups run two groups per block (a
    grid-stride loop); an odd count leaves the last block one group."""
    w, d, act = _ln_case("ln_8192x4096_f32", 4097, 4096, residual=True, act="gelu_tanh")
    y = mbp.fused_add_layernorm_gelu(to_dev(d["x"]), to_dev(d["residual"]), to_dev(d["gamma"]),
                                     to_dev(d["beta"]), eps=1e-5, act=act)
    rows = np.unique(np.concatenate([sample_rows(4097), [2047, 2048, 2049, 4095, 4096]]))
    check_f32(to_host(y)[rows], _ln_ref(d, act, rows), "fp32 LN 4097 x 4096, two groups per block")


@pytest.mark.parametrize("rows,cols", [(1031, 3500), (517, 4096), (3, 4096), (2049, 3073)])
def test_ln_f32_persistent_loop(mbp, rows, cols):
    """Plain fp32 LayerNorm rows of 3073-4096 columns run as a loop of two
    blocks per compute unit over the rows, each block issuing its next row's
    loads ahead: row counts that leave the blocks uneven shares.  Every output
    element is checked."""
    w, d, act = _ln_case("ln_8192x4096_f32", rows, cols, residual=False, act="none")
    y = to_host(_ln_run(mbp, d, act))
    check_f32(y, _ln_ref(d, act), f"fp32 LN {rows} x {cols}, persistent loop")


@pytest.mark.parametrize("cols,residual,act", [(8192, True, "gelu_tanh"), (6144, True, "gelu_tanh"),
                                              (8192, False, "none"), (7000, False, "gelu_tanh")])
def test_ln_bf16_loads_ahead(mbp, cols, residual, act):
    """16-bit rows in 256-lane groups run two row groups per block when there
    are thousands, the second group's loads issued while the first is
    computed; an odd count leaves the last block one group.  Every element of
    the output is checked."""
    w, d, act = _ln_case("addln_gelu_16384x8192_bf16", 4097, cols, residual, act)
    y = to_host(_ln_run(mbp, d, act))
    check_bf16(y, _ln_ref(d, act), f"bf16 4097 x {cols} residual={residual} act={act}, loads ahead")


# ------------------------------------------------------------------ row strides of the row kernels

# (rows, cols, x (pad, offset), residual (pad, offset) or None, y (pad, offset) or "x")
# pads and offsets in elements: row i of an operand starts at offset + i * (cols + pad)
LN_STRIDED = [
    (37, 4096, (64, 0), (64, 0), (64, 0)),        # pitches of whole 16-byte vectors: aligned kernel
    (37, 4096, (3, 0), (3, 0), (3, 0)),           # one pitch off 16 bytes: per-class windows
    (37, 4096, (3, 5), (3, 5), (3, 5)),           # the same, bases off 16 bytes (sliced columns)
    (37, 4096, (3, 0), (5, 0), (0, 0)),           # different pitches: lane-shift kernel
    (40, 4095, (1, 0), (1, 0), "x"),              # in place on a padded buffer
    (520, 8192, (3, 0), (3, 0), "x"),             # 512 x 2 class layout, in place, several groups a block
    (300, 3600, (5, 2), (5, 2), (5, 2)),          # 256 x 2 class layout, bases off 16 bytes
    (41, 768, (8, 2), None, (9, 1)),              # narrow rows, sub-wave groups
    (9, 12288, (16, 0), (7, 3), (16, 0)),
    (5, 16384, (2, 1), (2, 1), (2, 1)),           # the widest rows, per-class windows
    (300, 64, (4, 0), (4, 0), (4, 0)),
    (33, 1000, (24, 8), (24, 8), (24, 8)),
]


def _strided(host, pad, off, fill):
    """a [rows, cols] view into a padded buffer (rows at offset + i * (cols + pad)),
    the padding holding `fill`; returns (view, whole buffer)"""
    rows, cols = host.shape
    ld = cols + pad
    buf = torch.full((off + rows * ld + 8,), fill, dtype=host.dtype, device="cuda")
    v = buf[off:off + rows * ld].view(rows, ld)[:, :cols]
    v.copy_(host.cuda())
    return v, buf


def _outside(buf, view, fill):
    """elements of buf outside the view still equal to fill"""
    mask = torch.ones(buf.numel(), dtype=torch.bool, device="cuda")
    idx = (torch.arange(view.shape[0], device="cuda")[:, None] * view.stride(0) +
           torch.arange(view.shape[1], device="cuda")[None, :] + view.storage_offset())
    mask[idx.reshape(-1)] = False
    return bool((buf[mask].float() == fill).all())


@pytest.mark.parametrize("fmt,dtype", [("f32", torch.float32), ("bf16", torch.bfloat16)], ids=["f32", "bf16"])
@pytest.mark.parametrize("rows,cols,xs,rs,ys", LN_STRIDED)
def test_ln_strided(mbp, fmt, dtype, rows, cols, xs, rs, ys):
    """Residual + LayerNorm + GeLU (and plain LayerNorm, and dropout) on
    padded and sliced rows through the row strides ([P1] section 6.2: no
    hidden .contiguous() copy): the result equals the oracle on the rows'
    values and nothing outside the output rows is written."""
    rng = np.random.default_rng([51, rows, cols, xs[0], xs[1]])
    xh = torch.from_numpy(rng.standard_normal((rows, cols)) * 2 + 0.5).to(dtype)
    rh = torch.from_numpy(rng.standard_normal((rows, cols)) * 2).to(dtype)
    g = torch.from_numpy(1 + 0.1 * rng.standard_normal(cols)).to(dtype)
    b = torch.from_numpy(0.1 * rng.standard_normal(cols)).to(dtype)
    host = (lambda t: t.view(torch.int16).numpy().view(np.uint16)) if fmt == "bf16" else (lambda t: t.numpy())
    chk = check_bf16 if fmt == "bf16" else check_f32
    fill = 7.0
    x, xbuf = _strided(xh, *xs, fill)
    r, rbuf = _strided(rh, *rs, fill) if rs is not None else (None, None)
    if ys == "x":
        y, ybuf = x, xbuf
    else:
        y, ybuf = _strided(torch.zeros_like(xh), *ys, fill)
    ref = oracle.add_layernorm_gelu(host(xh), None if r is None else host(rh), host(g), host(b),
                                    act=oracle.ACT_GELU_TANH)
    mbp.fused_add_layernorm_gelu(x, r, g.cuda(), b.cuda(), act="gelu_tanh", out=y)
    what = f"{fmt} {rows}x{cols} x{xs} r{rs} y{ys}"
    chk(to_host(y.contiguous()), ref, f"strided LN+GeLU {what}")
    assert _outside(ybuf, y, fill), f"{what}: wrote outside the output rows"
    if ys != "x":
        # plain LayerNorm and LN-ReLU-dropout on the same strided views
        ref = oracle.add_layernorm_gelu(host(xh), None, host(g), host(b), act=oracle.ACT_NONE)
        mbp.fused_add_layernorm_gelu(x, None, g.cuda(), b.cuda(), act="none", out=y)
        chk(to_host(y.contiguous()), ref, f"strided LN {what}")
        d = {"x": host(xh), "gamma": host(g), "beta": host(b)}
        w = W.scaled(W.BY_NAME["ln_8192x4096_f32" if fmt == "f32" else "addln_gelu_16384x8192_bf16"], rows=rows)
        mbp.fused_layernorm_relu_dropout(x, g.cuda(), b.cuda(), p=0.25, seed=77, offset=2, out=y)
        _check_dropout(y.contiguous(), d, w, 0.25, 77, 2, f"strided LN-ReLU-dropout {what}")
        assert _outside(ybuf, y, fill), f"{what}: dropout wrote outside the output rows"


def test_ln_strided_views(mbp):
    """Views the binding accepts (a 3-D slice whose leading dimensions collapse
    to one row stride, a residual row expanded over the rows) and one it must
    refuse (leading dimensions that do not collapse)."""
    rng = np.random.default_rng(52)
    B, S, W_, H = 3, 5, 800, 768
    big = torch.from_numpy(rng.standard_normal((B, S, W_))).to(torch.bfloat16).cuda()
    x = big[:, :, 16:16 + H]                       # strides (S*W, W, 1): row stride W
    rrow = torch.from_numpy(rng.standard_normal(H)).to(torch.bfloat16).cuda()
    r = rrow.expand(B, S, H)                       # row stride 0
    g = torch.ones(H, dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(H, dtype=torch.bfloat16, device="cuda")
    y = mbp.fused_add_layernorm_gelu(x, r, g, b, act="gelu_tanh")
    assert y.shape == x.shape and y.is_contiguous()
    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1, H)
    vbits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.add_layernorm_gelu(bits(x), bits(r), vbits(g), vbits(b), act=oracle.ACT_GELU_TANH)
    check_bf16(bits(y), ref, "3-D slice with an expanded residual row")
    with pytest.raises(ValueError):
        mbp.fused_add_layernorm_gelu(big[:, :S - 1, :H], None, g, b)   # strides (S*W, W) over sizes (B, S-1)
    with pytest.raises(ValueError):
        mbp.fused_softmax(big[:, :S - 1, :H])


SM_STRIDED = [  # rows, cols, x (pad, off), y (pad, off) or "x"
    (37, 4096, (64, 0), (0, 0)),      # padded x, dense y: both on 16-byte boundaries
    (37, 4096, (3, 0), (3, 0)),       # one pitch off 16 bytes: windows
    (37, 4096, (3, 0), (11, 0)),      # pitches 16 bytes apart (bf16/fp16: 8 elements): windows
    (37, 4095, (2, 1), (7, 4)),       # rows that never agree modulo 16: element path
    (30, 4095, (1, 0), "x"),          # in place on a padded buffer
    (64, 768, (8, 2), (8, 2)),
    (5, 16384, (2, 0), (2, 0)),
]


@pytest.mark.parametrize("fmt,dtype", [("f32", torch.float32), ("bf16", torch.bfloat16), ("f16", torch.float16)],
                         ids=["f32", "bf16", "f16"])
@pytest.mark.parametrize("rows,cols,xs,ys", SM_STRIDED)
def test_softmax_strided(mbp, fmt, dtype, rows, cols, xs, ys):
    rng = np.random.default_rng([53, rows, cols, xs[0]])
    xh, xf = _stored(rng, (rows, cols), dtype, 3.0)
    fill = 5.0
    x, xbuf = _strided(xh, *xs, fill)
    if ys == "x":
        y, ybuf = x, xbuf
    else:
        y, ybuf = _strided(torch.zeros_like(xh), *ys, fill)
    mbp.fused_softmax(x, out=y)
    _softmax_gate(y.contiguous(), oracle.softmax(xf), fmt, f"strided softmax {fmt} {rows}x{cols} x{xs} y{ys}", xf)
    assert _outside(ybuf, y, fill), "wrote outside the output rows"


# ------------------------------------------------------------------ two-dimensional forms

DT2D = [("f32", torch.float32), ("bf16", torch.bfloat16), ("f16", torch.float16)]


def _stored(rng, shape, dtype, scale=1.0):
    """seeded N(0, scale^2) values stored in `dtype`: (host tensor, float32 copy of the stored values)"""
    t = torch.from_numpy(rng.standard_normal(shape) * scale).to(dtype)
    return t, t.float().numpy()


def _padded(host, pad, sentinel=None):
    """a device view of `host` [rows, cols] inside a [rows, cols + pad] buffer"""
    rows, cols = host.shape
    fill = 0.0 if sentinel is None else sentinel
    big = torch.full((rows, cols + pad), fill, dtype=host.dtype, device="cuda")
    v = big[:, :cols]
    v.copy_(host.cuda())
    return v, big


def _bias_operand(rng, rows, cols, dtype, mode):
    """b as a dense [rows, cols] tensor, a 1-D row, or a row expanded over rows
    (stride 0); returns (device operand, float32 [rows, cols] of its values)"""
    if mode == "full":
        t, f = _stored(rng, (rows, cols), dtype)
        return t.cuda(), f
    t, f = _stored(rng, (cols,), dtype)
    d = t.cuda()
    full = np.ascontiguousarray(np.broadcast_to(f, (rows, cols)))
    return (d if mode == "row" else d.expand(rows, cols)), full


def _gate_2d(y, exact, fmt, what, row_kernel=False):
    if fmt == "f32":
        return check_f32(to_host(y), exact, what) if row_kernel else check_chain(to_host(y), exact, what)
    return check_ulp16(bits16(y), exact, fmt, what)


CHAIN_2D = [  # rows, cols, x pad, y pad, b1, b2
    (37, 1000, 0, 0, "full", "full"), (37, 1003, 0, 0, "full", "full"),
    (19, 512, 8, 24, "row", "full"), (19, 515, 3, 5, "expand", "row"),
    (1, 4099, 0, 0, "row", "row"), (64, 8, 0, 0, "expand", "expand"), (300, 24, 8, 0, "row", "expand"),
    (23, 4095, 1, 3, "full", "row"), (9, 1024, 5, 0, "expand", "full"), (5, 20001, 3, 1, "row", "full")]


@pytest.mark.parametrize("fmt,dtype", DT2D, ids=[d[0] for d in DT2D])
@pytest.mark.parametrize("rows,cols,xpad,ypad,m1,m2", CHAIN_2D)
def test_chain_2d(mbp, fmt, dtype, rows, cols, xpad, ypad, m1, m2):
    rng = np.random.default_rng([11, rows, cols, xpad])
    xh, xf = _stored(rng, (rows, cols), dtype)
    x, _ = _padded(xh, xpad)
    b1, b1f = _bias_operand(rng, rows, cols, dtype, m1)
    b2, b2f = _bias_operand(rng, rows, cols, dtype, m2)
    y, ybig = _padded(torch.zeros((rows, cols), dtype=dtype), ypad, sentinel=3.0)
    mbp.fused_pointwise_chain_2d(x, b1, b2, 0.5, out=y)
    exact = oracle.pointwise_chain(xf, b1f, b2f, 0.5)
    _gate_2d(y, exact, fmt, f"chain 2d {fmt} {rows}x{cols} pads {xpad},{ypad} {m1},{m2}")
    if ypad:
        assert (ybig[:, cols:].float() == 3.0).all(), "wrote outside the output rows"


def _halfway_cases(fmt):
    """(x, b1, b2, scale) lists whose exact chain result relu(x + b1)*scale + b2
    lies closer to a halfway point of the 16-bit format than half a binary32
    ulp, on both sides, for even and odd neighbours, both signs, and (set B,
    scale 0.5 +- 2^-40 on odd subnormals) below the normal range."""
    p = 8 if fmt == "bf16" else 11                 # significand bits
    exps = [-100, -20, -1, 0, 7, 100] if fmt == "bf16" else [1, 5, 10, 15]
    tiny = (lambda e: 2.0 ** (e - 30)) if fmt == "bf16" else (lambda e: 2.0 ** -24)
    A = []
    for e in exps:
        for k in range(0, 2 ** (p - 1), 1 if fmt == "bf16" else 7):
            v = (1 + k / 2 ** (p - 1)) * 2.0 ** e
            h = 2.0 ** (e - p)                      # half an ulp of v
            for sc in (1.0, -1.0):
                for t in (tiny(e), -tiny(e)):
                    A.append((v, h, t, sc))
    sub_lsb = 2.0 ** -133 if fmt == "bf16" else 2.0 ** -24
    norm_min = 2.0 ** -126 if fmt == "bf16" else 2.0 ** -14
    B = [k * sub_lsb for k in range(1, 2 ** (p - 1), 2)]
    B += [(1 + k / 2 ** (p - 1)) * norm_min for k in range(1, 2 ** (p - 1), 2)]
    return A, B


@pytest.mark.parametrize("fmt,dtype", DT2D[1:], ids=[d[0] for d in DT2D[1:]])
def test_narrowing_exact_near_halfway(mbp, fmt, dtype):
    """16-bit results are rounded once from binary64: inputs built so that the
    exact result sits within a binary32 rounding of a 16-bit halfway point
    (where rounding first to binary32 and then to 16 bits goes wrong), and odd
    values halved into the subnormal range; every output must equal the exact
    result rounded once (0 ulp), not merely lie within the 1-ulp gate."""
    A, B = _halfway_cases(fmt)
    cases = [(np.array([a[i] for a in A]) for i in range(4))]
    xa, b1a, b2a, sca = cases[0]
    xb = np.array(B)
    for scale in (1.0, -1.0, 0.5 + 2.0 ** -40, 0.5 - 2.0 ** -40):
        if abs(scale) == 1.0:
            sel = sca == scale
            x, b1, b2 = xa[sel], b1a[sel], b2a[sel]
        else:
            x, b1, b2 = xb, np.zeros_like(xb), np.zeros_like(xb)
        n = x.size
        cols = 64
        rows = -(-n // cols)
        pad = rows * cols - n
        host = [np.concatenate([a, np.zeros(pad)]).reshape(rows, cols) for a in (x, b1, b2)]
        dev = [torch.from_numpy(h).to(dtype).cuda() for h in host]
        stored = [d.float().cpu().numpy() for d in dev]
        for h, st in zip(host, stored):
            assert np.array_equal(h.astype(np.float32), st), "a test input is not exact in the 16-bit type"
        y = mbp.fused_pointwise_chain_2d(*dev, scale)
        exact = oracle.pointwise_chain(*stored, scale)
        want = oracle.round_bits(exact, fmt)
        got = bits16(y)
        bad = np.argwhere(got != want)
        assert bad.size == 0, (f"{fmt} scale {scale}: {len(bad)} of {n} not rounded once, first at {bad[0]}: "
                               f"exact {exact[tuple(bad[0])]!r} got {got[tuple(bad[0])]:#06x} "
                               f"want {want[tuple(bad[0])]:#06x}")


def test_chain_2d_in_place(mbp):
    rng = np.random.default_rng(12)
    for dtype, fmt in ((torch.bfloat16, "bf16"), (torch.float16, "f16")):
        xh, xf = _stored(rng, (16, 264), dtype)
        x, _ = _padded(xh, 8)
        b1, b1f = _bias_operand(rng, 16, 264, dtype, "row")
        b2, b2f = _bias_operand(rng, 16, 264, dtype, "full")
        mbp.fused_pointwise_chain_2d(x, b1, b2, 0.5, out=x)
        _gate_2d(x, oracle.pointwise_chain(xf, b1f, b2f, 0.5), fmt, f"chain 2d in place {fmt}")


# 16-bit rows that are whole 16-byte vectors on 16-byte boundaries take the
# 8-element kernel (1024, 512, 4096, 4000, 16384, 12288 with pads that keep the
# boundaries); 1020 takes the 4-element one; 1001 and 515 the element one.
TENOP_2D = [(64, 1024, 0, 0), (33, 1001, 0, 0), (40, 512, 8, 16), (21, 515, 5, 3), (1, 4096, 0, 0),
            (9, 4000, 0, 8), (12, 1020, 4, 4), (3, 16384, 0, 8), (5, 12288, 8, 0), (17, 24, 0, 0),
            (4, 13001, 3, 1), (3, 14000, 5, 0), (6, 10000, 0, 4)]


# The looping 10-op kernels run on a few blocks per compute unit (two for
# fp32, four for 16-bit), each taking many row groups in turn (its LDS
# reduction buffers alternating): row counts that give every block several
# groups and the last ones uneven shares, on each looping path -- fp32 with
# 4-element accesses and one element at a time, 16-bit with 8-element (rows
# up to 64 and past 512 vectors), 4-element and single-element accesses.
TENOP_LOOP = [("f32", 4099, 2048, 0), ("f32", 4101, 1001, 1), ("bf16", 4097, 4104, 0), ("f16", 40003, 256, 0),
              ("f16", 6001, 1028, 4), ("bf16", 8003, 1001, 1)]


@pytest.mark.parametrize("fmt,rows,cols,off", TENOP_LOOP)
def test_tenop_persistent_loop(mbp, fmt, rows, cols, off):
    dtype = dict(DT2D)[fmt]
    rng = np.random.default_rng([89, rows, cols])
    xh, xf = _stored(rng, (rows, cols), dtype)
    vecs = [_stored(rng, (cols,), dtype) for _ in range(3)]
    buf = torch.zeros(rows * cols + 8, dtype=dtype, device="cuda")
    x = buf[off:off + rows * cols].view(rows, cols)
    x.copy_(xh.cuda())
    ybuf = torch.full((rows * cols + 8,), 3.0, dtype=dtype, device="cuda")
    y = ybuf[off:off + rows * cols].view(rows, cols)
    mbp.fused_row_mean_epilogue_2d(x, *(v[0].cuda() for v in vecs), alpha=1.1, c=0.1, out=y)
    exact = oracle.row_mean_epilogue(xf, *(v[1] for v in vecs), 1.1, 0.1)
    _gate_2d(y, exact, fmt, f"10-op {fmt} {rows}x{cols} at +{off}, persistent loop", row_kernel=True)
    rest = torch.cat([ybuf[:off], ybuf[off + rows * cols:]]).float()
    assert (rest == 3.0).all(), "wrote outside y"


@pytest.mark.parametrize("fmt,dtype", DT2D, ids=[d[0] for d in DT2D])
@pytest.mark.parametrize("rows,cols,xpad,ypad", TENOP_2D)
def test_tenop_2d(mbp, fmt, dtype, rows, cols, xpad, ypad):
    rng = np.random.default_rng([13, rows, cols, xpad])
    xh, xf = _stored(rng, (rows, cols), dtype)
    x, _ = _padded(xh, xpad)
    vecs = [_stored(rng, (cols,), dtype) for _ in range(3)]
    y, ybig = _padded(torch.zeros((rows, cols), dtype=dtype), ypad, sentinel=3.0)
    mbp.fused_row_mean_epilogue_2d(x, *(v[0].cuda() for v in vecs), alpha=1.1, c=0.1, out=y)
    exact = oracle.row_mean_epilogue(xf, *(v[1] for v in vecs), 1.1, 0.1)
    _gate_2d(y, exact, fmt, f"10-op 2d {fmt} {rows}x{cols} pads {xpad},{ypad}", row_kernel=True)
    if ypad:
        assert (ybig[:, cols:].float() == 3.0).all(), "wrote outside the output rows"
    # in place, on the padded x
    mbp.fused_row_mean_epilogue_2d(x, *(v[0].cuda() for v in vecs), alpha=1.1, c=0.1, out=x)
    _gate_2d(x, exact, fmt, f"10-op 2d in place {fmt} {rows}x{cols}", row_kernel=True)


def _as_f32(a):
    """host storage array (bf16 bit patterns, float16 or float32) -> float32 values"""
    if a.dtype == np.uint16:
        return W.bf16_bits_to_f32(a)
    return a.astype(np.float32)


# ------------------------------------------------------------------ LayerNorm -> ReLU -> Dropout

def _drop_case(name, rows, cols):
    w, d, _ = _ln_case(name, rows, cols, residual=False)
    return w, d


def _check_dropout(y_dev, d, w, p, seed, offset, what, mode=oracle.EXACT):
    """the kept / dropped pattern exactly (where relu(LN) is clearly positive,
    so that rounding cannot move an element across 0), and the values within
    the LayerNorm gates"""
    exact = oracle.ln_relu_dropout(d["x"], d["gamma"], d["beta"], p=p, seed=seed, offset=offset, mode=mode)
    relu_ln = np.maximum(oracle.add_layernorm_gelu(d["x"], None, d["gamma"], d["beta"], act=oracle.ACT_NONE), 0)
    y = to_host(y_dev)
    yf = as_f64(y)
    clear = relu_ln > 1e-3
    assert np.array_equal((yf != 0)[clear], (exact != 0)[clear]), f"{what}: dropout mask differs"
    chk = check_bf16 if w.dtype == "bf16" else check_f32
    chk(y, exact, what)
    return (exact == 0)[clear].mean() if clear.any() else 0.0


@pytest.mark.parametrize("name", ["ln_8192x4096_f32", "addln_gelu_16384x8192_bf16"])
@pytest.mark.parametrize("cols", [8, 768, 1001, 1024, 4095, 4096, 8192])
@pytest.mark.parametrize("p", [0.0, 0.1, 0.5, 1.0])
def test_ln_relu_dropout(mbp, name, cols, p):
    w, d = _drop_case(name, 23, cols)
    seed, offset = 0x5EED0000DEADBEEF, 3
    args = (to_dev(d["x"]), to_dev(d["gamma"]), to_dev(d["beta"]))
    y = mbp.fused_layernorm_relu_dropout(*args, p=p, seed=seed, offset=offset)
    frac = _check_dropout(y, d, w, p, seed, offset, f"ln-relu-dropout {w.dtype} {cols} p={p}")
    if p in (0.0, 1.0):
        assert frac == p
    y2 = mbp.fused_layernorm_relu_dropout(*args, p=p, seed=seed, offset=offset)
    assert torch.equal(y, y2), "not deterministic"



@pytest.mark.parametrize("name", ["ln_8192x4096_f32", "addln_gelu_16384x8192_bf16"])
@pytest.mark.parametrize("cols,rows", [(4095, 70), (1001, 40), (7, 50), (8191, 9), (12287, 5),
                                       (8191, 200), (4500, 100)])
@pytest.mark.parametrize("off_b", [0, 4, 20, 124])
def test_ln_relu_dropout_windows(mbp, name, cols, rows, off_b):
    """x and y both `off_b` bytes past a 128-byte line, rows off 16-byte
    boundaries: the relu + dropout epilogue on vectors that straddle two
    generator blocks (the blocks shared through LDS, and for the widest rows
    computed in every slot), the rows at an unaligned start, and in place.
    8191 x 200 and 4500 x 100 (bf16: the 256 x 4 and 128 x 5 layouts, whose
    generator blocks share one LDS buffer) give each block several row groups
    of its class, so every refill of that buffer waits for the previous
    group's readers."""
    w, d = _drop_case(name, rows, cols)
    es = 4 if w.dtype == "f32" else 2
    seed, offset, p = 0x0123456789ABCDEF, 5, 0.25

    def place(t, fill):
        buf = torch.full((t.numel() + 256 // es,), fill, dtype=t.dtype, device="cuda")
        assert buf.data_ptr() % 128 == 0
        v = buf[off_b // es:off_b // es + t.numel()].view(t.shape)
        v.copy_(t)
        return v, buf

    x, _ = place(to_dev(d["x"]), 0.0)
    y, yb = place(torch.zeros_like(to_dev(d["x"])), 3.0)
    g, b = to_dev(d["gamma"]), to_dev(d["beta"])
    mbp.fused_layernorm_relu_dropout(x, g, b, p=p, seed=seed, offset=offset, out=y)
    _check_dropout(y, d, w, p, seed, offset, f"ln-relu-dropout {w.dtype} {rows}x{cols} at +{off_b} bytes")
    host = yb.float().cpu().numpy()
    o = off_b // es
    assert (host[:o] == 3.0).all() and (host[o + x.numel():] == 3.0).all(), "wrote outside y"
    mbp.fused_layernorm_relu_dropout(x, g, b, p=p, seed=seed, offset=offset, out=x)
    iv = torch.int32 if es == 4 else torch.int16
    assert torch.equal(x.view(iv), y.view(iv)), "in place differs"

def test_ln_relu_dropout_in_place_offset_misaligned_unfused(mbp):
    for name in ("ln_8192x4096_f32", "addln_gelu_16384x8192_bf16"):
        w, d = _drop_case(name, 33, 1024)
        g, b = to_dev(d["gamma"]), to_dev(d["beta"])
        x = to_dev(d["x"])
        y = mbp.fused_layernorm_relu_dropout(x, g, b, p=0.1, seed=9, offset=0)
        # in place
        xi = x.clone()
        mbp.fused_layernorm_relu_dropout(xi, g, b, p=0.1, seed=9, offset=0, out=xi)
        assert torch.equal(xi, y), "in place differs"
        # another offset: another mask (of the clearly positive elements, about p(1-p)*2 differ)
        y3 = mbp.fused_layernorm_relu_dropout(x, g, b, p=0.1, seed=9, offset=1)
        _check_dropout(y3, d, w, 0.1, 9, 1, f"{name} offset 1")
        assert not torch.equal(y3, y)
        # x one element past a 16-byte boundary: the lane-shift kernel, same result
        buf = torch.zeros(x.numel() + 8, dtype=x.dtype, device="cuda")
        xs = buf[1:1 + x.numel()].view(x.shape)
        xs.copy_(x)
        ys = mbp.fused_layernorm_relu_dropout(xs, g, b, p=0.1, seed=9, offset=0)
        _check_dropout(ys, d, w, 0.1, 9, 0, f"{name} misaligned")
        # the three eager launches, against the oracle's three-stage mode
        yu = mbp.unfused_layernorm_relu_dropout(x, g, b, p=0.1, seed=9, offset=0)
        _check_dropout(yu, d, w, 0.1, 9, 0, f"{name} unfused", mode=oracle.SEQ3)


# ------------------------------------------------------------------ row softmax

SM_COLS = [1, 7, 8, 33, 255, 256, 1000, 1024, 4095, 4096, 8192, 12288, 16384]


def _softmax_gate(y, exact, fmt, what, x):
    """x: the float32 values of the rows of y (for the fp32 bound)"""
    if fmt == "f32":
        worst, ratio = check_softmax_f32(to_host(y), exact, x, what)
        print(f"{what}: max error {worst:.1f} x 2^-24 relative, {ratio:.2f} of the bound")
        return worst, ratio
    return check_ulp16(bits16(y), exact, fmt, what)


@pytest.mark.parametrize("fmt,dtype", DT2D, ids=[d[0] for d in DT2D])
@pytest.mark.parametrize("cols", SM_COLS)
@pytest.mark.parametrize("scale", [1.0, 8.0])
def test_softmax_shapes(mbp, fmt, dtype, cols, scale):
    rng = np.random.default_rng([21, cols, int(scale)])
    rows = 9 if cols > 4096 else 37
    xh, xf = _stored(rng, (rows, cols), dtype, scale)
    y = mbp.fused_softmax(xh.cuda())
    _softmax_gate(y, oracle.softmax(xf), fmt, f"softmax {fmt} {rows}x{cols} scale {scale}", xf)



@pytest.mark.parametrize("fmt,dtype", DT2D, ids=[d[0] for d in DT2D])
@pytest.mark.parametrize("shift", [-3.0e4, 3.0e4, -60000.0])
def test_softmax_large_offsets(mbp, fmt, dtype, shift):
    """rows far from 0 (exp(x) alone would overflow or underflow): the
    running maximum keeps every exponent <= 0; aligned and windowed rows"""
    if fmt == "f16" and abs(shift) > 6.0e4:
        pytest.skip("beyond the fp16 range")
    rng = np.random.default_rng([24, abs(int(shift)), int(shift < 0)])
    for cols in (4096, 4095):
        xh, _ = _stored(rng, (9, cols), dtype, 3.0)
        xh = (xh.float() + shift).to(dtype)
        xf = xh.float().numpy()
        y = mbp.fused_softmax(xh.cuda())
        _softmax_gate(y, oracle.softmax(xf), fmt, f"softmax {fmt} 9x{cols} shifted by {shift}", xf)

@pytest.mark.parametrize("fmt,dtype", DT2D, ids=[d[0] for d in DT2D])
def test_softmax_masks_in_place_and_misaligned(mbp, fmt, dtype):
    rng = np.random.default_rng(22)
    rows, cols = 24, 1024
    xh, xf = _stored(rng, (rows, cols), dtype, 3.0)
    mask = rng.random((rows, cols)) < 0.3
    mask[5, :] = True                  # a fully masked row: 0/0 = NaN
    mask[6, :] = True
    mask[6, 777] = False               # a single surviving entry: 1 there, 0 elsewhere
    xh[torch.from_numpy(mask)] = float("-inf")
    xf = xh.float().numpy()
    exact = oracle.softmax(xf)
    assert np.isnan(exact[5]).all() and exact[6, 777] == 1.0
    y = mbp.fused_softmax(xh.cuda())
    yh = y.float().cpu().numpy()
    assert np.isnan(yh[5]).all(), "a fully masked row must be NaN"
    ok = np.ones(rows, bool)
    ok[5] = False
    # masked entries are exactly 0 (unmasked ones may round to 0 too in fp16:
    # the gate below compares them with the exact value rounded once)
    assert (yh[ok][mask[ok]] == 0).all(), "masked entries must be exactly 0"
    assert yh[6, 777] == 1.0
    _softmax_gate(y[torch.from_numpy(ok).cuda()], exact[ok], fmt, f"softmax masked {fmt}", xf[ok])
    # in place
    xd = xh.cuda()
    mbp.fused_softmax(xd, out=xd)
    assert torch.equal(xd.view(torch.int16) if xd.element_size() == 2 else xd.view(torch.int32),
                       y.view(torch.int16) if y.element_size() == 2 else y.view(torch.int32)), "in place differs"
    # x one element past a 16-byte boundary: the element path, same results
    buf = torch.zeros(rows * cols + 8, dtype=dtype, device="cuda")
    xs = buf[1:1 + rows * cols].view(rows, cols)
    xs.copy_(xh.cuda())
    y2 = mbp.fused_softmax(xs)
    _softmax_gate(y2[torch.from_numpy(ok).cuda()], exact[ok], fmt, f"softmax misaligned {fmt}", xf[ok])



@pytest.mark.parametrize("fmt,dtype", DT2D, ids=[d[0] for d in DT2D])
@pytest.mark.parametrize("cols,rows", [(4095, 70), (4088, 20), (1000, 40), (769, 70), (33, 90), (16383, 5),
                                       (12287, 9)])
@pytest.mark.parametrize("offs", [(0, 0), (4, 4), (20, 20), (124, 124), (4, 20), (12, 124), (0, 16)])
def test_softmax_windows(mbp, fmt, dtype, cols, rows, offs):
    """x and y starting offs[0] and offs[1] bytes past a 128-byte line.  Equal
    offsets modulo 16 take the windowed path (rows off 16-byte boundaries, or
    on them but not on lines), rotated onto lines when the offsets agree
    modulo 128, with the rows at an unaligned start or end done element by
    element; masked (-inf) entries fall in the shared and folded windows too."""
    es = torch.empty(0, dtype=dtype).element_size()
    if offs[0] % es or offs[1] % es:
        pytest.skip("offset not a whole element")
    rng = np.random.default_rng([23, cols, rows, offs[0], offs[1]])
    xh, _ = _stored(rng, (rows, cols), dtype, 4.0)
    mask = rng.random((rows, cols)) < 0.05
    mask[:, 0] = mask[:, -1] = True    # the first and last column of every row
    mask[1, :] = True                  # a fully masked row: NaN
    xh[torch.from_numpy(mask)] = float("-inf")
    xf = xh.float().numpy()
    exact = oracle.softmax(xf)

    def place(t, off_b, fill):
        buf = torch.full((t.numel() + 256 // es,), fill, dtype=dtype, device="cuda")
        assert buf.data_ptr() % 128 == 0
        v = buf[off_b // es:off_b // es + t.numel()].view(t.shape)
        v.copy_(t)
        return v, buf

    x, _ = place(xh.cuda(), offs[0], 0.0)
    y, yb = place(torch.zeros_like(xh).cuda(), offs[1], 3.0)
    mbp.fused_softmax(x, out=y)
    yh = y.float().cpu().numpy()
    assert np.isnan(yh[1]).all(), "a fully masked row must be NaN"
    ok = np.ones(rows, bool)
    ok[1] = False
    assert (yh[ok][mask[ok]] == 0).all(), "masked entries must be exactly 0"
    _softmax_gate(y[torch.from_numpy(ok).cuda()], exact[ok], fmt, f"softmax {fmt} {rows}x{cols} offsets {offs}", xf[ok])
    host = yb.float().cpu().numpy()
    o = offs[1] // es
    assert (host[:o] == 3.0).all() and (host[o + x.numel():] == 3.0).all(), "wrote outside y"
    if offs[0] == offs[1]:  # in place: a shared window may already hold a neighbour's outputs, in elements the row masks
        mbp.fused_softmax(x, out=x)
        iv = torch.int32 if es == 4 else torch.int16
        assert torch.equal(x.view(iv), y.view(iv)), "in place differs"

# ------------------------------------------------------------------ unfused variants

def test_unfused_chain_bit_exact(mbp):
    for n in (1, 7, 4099, 4 * 1024 * 1024):
        d = _chain_inputs(n)
        y = to_host(mbp.unfused_pointwise_chain(to_dev(d["x"]), to_dev(d["b1"]), to_dev(d["b2"]), 0.5))
        ref = oracle.pointwise_chain(d["x"], d["b1"], d["b2"], 0.5, mode=oracle.SEQ)
        assert np.array_equal(y.astype(np.float64), ref), f"unfused chain n={n} not bit-exact vs SEQ"


@pytest.mark.parametrize("rows,cols", [(3, 7), (33, 1000), (1024, 1024)])
def test_unfused_tenop(mbp, rows, cols):
    d = W.generate(W.scaled(W.BY_NAME["tenop_1024x1024_f32"], rows=rows), cols=cols)
    y = to_host(mbp.unfused_row_mean_epilogue(*(to_dev(d[k]) for k in ("x", "bias", "gamma", "beta"))))
    ref = oracle.row_mean_epilogue(d["x"], d["bias"], d["gamma"], d["beta"], mode=oracle.SEQ)
    check_f32(y, ref, f"unfused 10-op {rows}x{cols} vs SEQ")


@pytest.mark.parametrize("rows,cols,off", [(1, 1, 0), (3, 7, 1), (5, 3, 0), (33, 1000, 2),
                                           (1024, 1024, 0), (1024, 1024, 1), (4, 16384, 3), (7, 4093, 0)])
def test_grouped_tenop(mbp, rows, cols, off):
    """TVM's three-group partition of the 10-op graph: every op rounds as its
    eager kernel does, so the output equals the ten-launch variant's bit for
    bit (and the oracle's sequential fp32 evaluation within the gate); x and y
    `off` elements past a 16-byte boundary take the element-wise path."""
    d = W.generate(W.scaled(W.BY_NAME["tenop_1024x1024_f32"], rows=rows), cols=cols)

    def place(a):
        t = to_dev(a)
        buf = torch.zeros(t.numel() + 4, dtype=t.dtype, device="cuda")
        v = buf[off:off + t.numel()].view(t.shape)
        v.copy_(t)
        return v

    x = place(d["x"])
    vecs = [to_dev(d[k]) for k in ("bias", "gamma", "beta")]
    y = place(np.zeros_like(d["x"]))
    mbp.grouped_row_mean_epilogue(x, *vecs, out=y)
    y_g = to_host(y)
    y_u = to_host(mbp.unfused_row_mean_epilogue(x, *vecs))
    assert np.array_equal(y_g.view(np.uint32), y_u.view(np.uint32)), "grouped != ten launches"
    ref = oracle.row_mean_epilogue(d["x"], d["bias"], d["gamma"], d["beta"], mode=oracle.SEQ)
    check_f32(y_g, ref, f"grouped 10-op {rows}x{cols} offset {off} vs SEQ")


@pytest.mark.parametrize("name,rows", [("ln_8192x4096_f32", 64), ("addln_gelu_16384x8192_bf16", 16),
                                       ("addln_gelu_32768x4095_bf16", 16), ("addln_gelu_262144x768_bf16", 64)])
@pytest.mark.parametrize("gran", [0, 1])
def test_unfused_layernorm(mbp, name, rows, gran):
    w = W.scaled(W.BY_NAME[name], rows=rows)
    d = W.generate(w)
    y = mbp.unfused_add_layernorm_gelu(to_dev(d["x"]), to_dev(d["residual"]), to_dev(d["gamma"]),
                                       to_dev(d["beta"]), eps=1e-5, act=w.act, granularity=gran)
    mode = oracle.SEQ if gran == 0 else oracle.SEQ3
    ref = _ln_ref(d, w.act, mode=mode)
    chk = check_bf16 if w.dtype == "bf16" else check_f32
    chk(to_host(y), ref, f"unfused {name} granularity {gran}")


@pytest.mark.parametrize("name,cols,rows,off", [
    ("addln_gelu_16384x8192_bf16", 5, 9, 0), ("addln_gelu_16384x8192_bf16", 33, 7, 0),
    ("addln_gelu_16384x8192_bf16", 1023, 5, 3), ("addln_gelu_16384x8192_bf16", 4095, 3, 1),
    ("ln_8192x4096_f32", 3, 11, 0), ("ln_8192x4096_f32", 7, 11, 1), ("ln_8192x4096_f32", 1001, 3, 2)])
@pytest.mark.parametrize("gran", [0, 1])
def test_unfused_layernorm_shapes(mbp, name, cols, rows, off, gran):
    """Rows narrower than a vector, odd widths, and x and residual `off`
    elements past a 16-byte boundary: the element-wise fallback, vectors
    wrapping into the next row, and row windows at the tensor's ends."""
    w, d, act = _ln_case(name, rows, cols, residual=True)

    def place(a):
        t = to_dev(a)
        buf = torch.zeros(t.numel() + 16, dtype=t.dtype, device="cuda")
        v = buf[off:off + t.numel()].view(t.shape)
        v.copy_(t)
        return v

    y = mbp.unfused_add_layernorm_gelu(place(d["x"]), place(d["residual"]), to_dev(d["gamma"]),
                                       to_dev(d["beta"]), eps=1e-5, act=act, granularity=gran)
    ref = _ln_ref(d, act, mode=oracle.SEQ if gran == 0 else oracle.SEQ3)
    chk = check_bf16 if w.dtype == "bf16" else check_f32
    chk(to_host(y), ref, f"unfused {name} {rows}x{cols} offset {off} granularity {gran}")


SM_UNFUSED = [(3, 1), (5, 7), (33, 1000), (7, 4096), (2, 16384), (64, 768), (9, 4095)]


@pytest.mark.parametrize("fmt,dtype", DT2D[:2], ids=[d[0] for d in DT2D[:2]])
@pytest.mark.parametrize("rows,cols", SM_UNFUSED)
def test_unfused_softmax(mbp, fmt, dtype, rows, cols):
    """The five eager launches (max, x - m, exp, sum, divide) against the
    oracle's SEQ softmax (each element-wise result rounded to binary32 and to
    the I/O type, the row sum kept as binary32).  The GPU's expf is within an
    ulp of the exact exponential the oracle rounds, so bf16 results may differ
    by 1 ulp where a rounding flips and fp32 results by a few ulps.  Masked
    entries (-inf) give exactly 0; an all-masked row gives NaN."""
    rng = np.random.default_rng([17, rows, cols])
    xh = torch.from_numpy(rng.standard_normal((rows, cols)) * 3).to(dtype)
    xh[torch.from_numpy(rng.random((rows, cols)) < 0.1)] = float("-inf")
    xh[:, 0] = torch.from_numpy(rng.standard_normal(rows)).to(dtype)
    if rows > 2:
        xh[2, :] = float("-inf")
    xf = xh.float().numpy()
    y = mbp.unfused_softmax(xh.cuda())
    want = oracle.softmax(xf, mode=oracle.SEQ, dtype=fmt)
    what = f"unfused softmax {fmt} {rows}x{cols}"
    if fmt == "bf16":
        check_ulp16(bits16(y), want, fmt, what)
    else:
        got = to_host(y)
        assert np.array_equal(np.isnan(got), np.isnan(want)), f"{what}: NaN mismatch"
        d = np.where(np.isnan(want), 0, np.abs(ordered(got) - ordered(want.astype(np.float32))))
        assert d.max(initial=0) <= 4, f"{what}: max {d.max()} ulp"
    masked = np.isneginf(xf) & ~np.isnan(want)
    assert np.all(to_host(y.float())[masked] == 0), f"{what}: masked entries must be exactly 0"
    # the same result from a misaligned input (element paths of every launch)
    buf = torch.zeros(rows * cols + 1, dtype=dtype, device="cuda")
    xm = buf[1:].view(rows, cols)
    xm.copy_(xh.cuda())
    ym = mbp.unfused_softmax(xm)
    assert torch.equal(ym.view(torch.int16 if fmt == "bf16" else torch.int32),
                       y.view(torch.int16 if fmt == "bf16" else torch.int32)), f"{what}: misaligned differs"


# ------------------------------------------------------------------ misc

@pytest.mark.parametrize("nsrc", [1, 2, 3, 4])
def test_stream_rw(mbp, nsrc):
    """The calibration stream: dst = the bytewise XOR of its sources."""
    rng = np.random.default_rng([61, nsrc])
    n = (1 << 20) + 48
    srcs = [rng.integers(0, 256, n, dtype=np.uint8) for _ in range(nsrc)]
    dst = torch.zeros(n, dtype=torch.uint8, device="cuda")
    mbp.stream_rw([torch.from_numpy(a).cuda() for a in srcs], dst)
    want = srcs[0].copy()
    for a in srcs[1:]:
        want ^= a
    assert np.array_equal(dst.cpu().numpy(), want)


def test_empty_inputs(mbp):
    """rows == 0 (n == 0) is a no-op for every entry point, fused and unfused."""
    e = torch.empty(0, device="cuda")
    assert mbp.fused_pointwise_chain(e, e, e).numel() == 0
    assert mbp.unfused_pointwise_chain(e, e, e).numel() == 0
    assert mbp.convert_f32_to_bf16(e).numel() == 0
    x = torch.empty(0, 64, device="cuda")
    v = torch.zeros(64, device="cuda")
    for f in (mbp.fused_row_mean_epilogue, mbp.unfused_row_mean_epilogue, mbp.grouped_row_mean_epilogue):
        assert f(x, v, v, v).numel() == 0
    assert mbp.fused_add_layernorm_gelu(x, None, v, v).numel() == 0
    assert mbp.unfused_add_layernorm_gelu(x, None, v, v).numel() == 0
    assert mbp.fused_layernorm_relu_dropout(x, v, v).numel() == 0
    assert mbp.unfused_layernorm_relu_dropout(x, v, v).numel() == 0
    for dt in (torch.float32, torch.bfloat16, torch.float16):
        xd = torch.empty(0, 64, dtype=dt, device="cuda")
        vd = torch.zeros(64, dtype=dt, device="cuda")
        assert mbp.fused_softmax(xd).numel() == 0
        assert mbp.fused_pointwise_chain_2d(xd, vd, vd).numel() == 0
        assert mbp.fused_row_mean_epilogue_2d(xd, vd, vd, vd).numel() == 0
    assert mbp.unfused_softmax(torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")).numel() == 0
    torch.cuda.synchronize()


def test_bf16_store_conversion_exhaustive(mbp):
    """Every binary32 bit pattern through the bf16 store conversion that the
    kernels use, against round-to-nearest-even written in integer arithmetic
    (torch int64 operations on the GPU, no float conversion involved): a
    non-NaN input u gives (u + 0x7FFF + bit 16 of u) >> 16 -- carries move a
    rounded-up mantissa into the exponent and past the largest finite value
    to infinity, subnormals included; a NaN gives a NaN of the same sign."""
    chunk = 1 << 28
    x = torch.empty(chunk, dtype=torch.float32, device="cuda")
    y = torch.empty(chunk, dtype=torch.bfloat16, device="cuda")
    for c in range(1 << 4):
        u = torch.arange(c * chunk, (c + 1) * chunk, dtype=torch.int64, device="cuda")
        x.view(torch.int32).copy_(torch.where(u >= 1 << 31, u - (1 << 32), u).to(torch.int32))
        mbp.convert_f32_to_bf16(x, out=y)
        got = y.view(torch.int16).to(torch.int64) & 0xFFFF
        nan = (u & 0x7FFFFFFF) > 0x7F800000
        rne = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        bad = (got != rne) & ~nan
        assert not bad.any(), f"chunk {c}: {int(bad.sum())} patterns not rounded to nearest even, " \
                              f"first input {int(u[bad][0]):#010x} -> {int(got[bad][0]):#06x}"
        gn, un = got[nan], u[nan]
        assert (((gn & 0x7F80) == 0x7F80) & ((gn & 0x7F) != 0) & ((gn >> 15) == (un >> 31))).all(), \
            f"chunk {c}: a NaN input did not give a NaN of the same sign"
        del u, got, nan, rne, bad, gn, un


def test_stream_copy(mbp):
    src = torch.arange(1 << 20, dtype=torch.float32, device="cuda")
    dst = torch.zeros_like(src)
    mbp.stream_copy(src, dst)
    assert torch.equal(src, dst)


def test_error_is_raised(mbp):
    x = torch.zeros(4, 8, device="cuda")
    with pytest.raises(mbp.MbpError):
        mbp.fused_add_layernorm_gelu(x, None, torch.zeros(8, device="cuda"), torch.zeros(8, device="cuda"),
                                     eps=-1.0)
