"""Every row layout of the LayerNorm kernels, in each access path, under each
epilogue, against the CPU oracle on every element.

A row is held as lanes x 16-byte windows a lane; the layout is picked from the
row's number of windows (ranges ending at 32, 64, 96, 128, 256, 512, 640, 1024,
1536, 2048, 3072 and 4096 windows), and the kernel from where the rows start:
rows of whole windows on 16-byte boundaries take the aligned kernel, rows with
one common offset in their windows (x, residual and y congruent) the
window-class kernel, and anything else the lane-shift kernel.  For each range,
the narrowest and the widest row run through each path -- all three tensors
on a 16-byte boundary, all three one element past it, and x, residual and y at
three different offsets -- with and without a residual, with and without
tanh-GeLU, and with the ReLU + dropout epilogue.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import as_f64, check_bf16, check_f32, to_dev, to_host

pytestmark = pytest.mark.gpu

WINDOW_RANGES = [32, 64, 96, 128, 256, 512, 640, 1024, 1536, 2048, 3072, 4096]

# element offsets of (x, residual, y) from a 16-byte boundary
PATHS = {"aligned": (0, 0, 0), "congruent": (1, 1, 1), "independent": (1, 0, 2)}

CASES = {"f32": ("ln_8192x4096_f32", 4), "bf16": ("addln_gelu_16384x8192_bf16", 8)}

# fp32 rows past 4096 windows (16384 columns) take the two-pass kernel, up to
# the 32768-column limit
F32_WIDE = [16385, 32768]


@pytest.fixture(scope="module")
def mbp():
    import memory_bound_pointwise_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _cols(v):
    """the narrowest and the widest row of each window range (v elements a window)"""
    out, lo = [], 0
    for hi in WINDOW_RANGES:
        out += [lo * v + 1, hi * v]
        lo = hi
    return out + (F32_WIDE if v == 4 else [])


def _rows(cols):
    # several row groups a block for the narrow layouts, a few rows for the wide ones
    return max(5, min(67, 200_000 // cols))


def _inputs(name, rows, cols, residual):
    w = W.scaled(W.BY_NAME[name], rows=rows)
    d = W.generate(w, cols=cols)
    if residual and d.get("residual") is None:
        # the fp32 workload has none: N(0, 1) rows of the 10-op workload's x
        d["residual"] = W.generate(W.scaled(W.BY_NAME["tenop_1024x1024_f32"], rows=rows), cols=cols)["x"]
    if not residual:
        d["residual"] = None
    return w, d


def _place(t, off, fill):
    """t copied `off` elements past the start of a fresh (256-byte aligned) buffer"""
    buf = torch.full((t.numel() + 16,), fill, dtype=t.dtype, device="cuda")
    v = buf[off:off + t.numel()].view(t.shape)
    v.copy_(t)
    return v, buf


def _untouched(buf, off, n):
    host = as_f64(to_host(buf))
    return (host[:off] == 3.0).all() and (host[off + n:] == 3.0).all()


@pytest.mark.parametrize("fmt", ["f32", "bf16"])
@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("residual,act", [(False, "none"), (True, "none"), (False, "gelu_tanh"),
                                          (True, "gelu_tanh")])
def test_ln_every_layout(mbp, fmt, path, residual, act):
    name, v = CASES[fmt]
    ox, orr, oy = PATHS[path]
    chk = check_f32 if fmt == "f32" else check_bf16
    code = oracle.ACT_GELU_TANH if act == "gelu_tanh" else oracle.ACT_NONE
    for cols in _cols(v):
        rows = _rows(cols)
        w, d = _inputs(name, rows, cols, residual)
        what = f"{fmt} {path} {rows}x{cols} residual={residual} act={act}"
        print(what, flush=True)
        x, _ = _place(to_dev(d["x"]), ox, 0.0)
        r = _place(to_dev(d["residual"]), orr, 0.0)[0] if residual else None
        y, yb = _place(torch.zeros_like(x), oy, 3.0)
        mbp.fused_add_layernorm_gelu(x, r, to_dev(d["gamma"]), to_dev(d["beta"]), eps=1e-5, act=act, out=y)
        exact = oracle.add_layernorm_gelu(d["x"], d["residual"], d["gamma"], d["beta"], eps=1e-5, act=code)
        chk(to_host(y), exact, what)
        assert _untouched(yb, oy, y.numel()), f"{what}: wrote outside y"
    print(f"{fmt} {path} residual={residual} act={act}: {len(_cols(v))} row widths")


@pytest.mark.parametrize("fmt", ["f32", "bf16"])
@pytest.mark.parametrize("path", list(PATHS))
def test_ln_relu_dropout_every_layout(mbp, fmt, path):
    name, v = CASES[fmt]
    ox, _, oy = PATHS[path]
    chk = check_f32 if fmt == "f32" else check_bf16
    seed, offset, p = 0x243F6A8885A308D3, 7, 0.25
    for cols in _cols(v):
        rows = _rows(cols)
        w, d = _inputs(name, rows, cols, False)
        what = f"ln-relu-dropout {fmt} {path} {rows}x{cols}"
        print(what, flush=True)
        x, _ = _place(to_dev(d["x"]), ox, 0.0)
        y, yb = _place(torch.zeros_like(x), oy, 3.0)
        mbp.fused_layernorm_relu_dropout(x, to_dev(d["gamma"]), to_dev(d["beta"]), p=p, seed=seed,
                                         offset=offset, out=y)
        exact = oracle.ln_relu_dropout(d["x"], d["gamma"], d["beta"], p=p, seed=seed, offset=offset)
        relu_ln = np.maximum(oracle.add_layernorm_gelu(d["x"], None, d["gamma"], d["beta"],
                                                       act=oracle.ACT_NONE), 0)
        got = to_host(y)
        clear = relu_ln > 1e-3  # rounding cannot move these across 0
        assert np.array_equal((as_f64(got) != 0)[clear], (exact != 0)[clear]), f"{what}: mask differs"
        chk(got, exact, what)
        assert _untouched(yb, oy, y.numel()), f"{what}: wrote outside y"


# ------------------------------------------------------------------ 10-op graph, softmax, unfused ops

from test_gpu_parity import _gate_2d, _ln_ref, _softmax_gate, _stored  # noqa: E402
from parity_util import bits16, check_ulp16, ordered  # noqa: E402

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _place_dev(t, off, fill=0.0):
    """device copy of host tensor t, `off` elements past a fresh buffer's (256-byte aligned) start"""
    return _place(t.cuda(), off, fill)


# 10-op access paths: 16-byte vectors of 8 elements (16-bit rows on 16-byte
# boundaries), 4-element accesses (fp32 rows on 16-byte boundaries; 16-bit
# rows 8 bytes past one), and single elements (rows one element off)
TENOP_PATHS = {"vec8": (8, 0), "vec4": (4, 4), "elem": (4, 1)}


def _rounded_once(y, exact, fmt, what):
    """16-bit outputs must be the exact value rounded once to nearest even,
    bit for bit, wherever that rounding is stable under a relative change of
    2^-40 (binary64 arithmetic in another order moves the result far less; a
    double rounding through binary32 would be off by one ulp near halfway
    points, which the 1-ulp gate alone lets through)."""
    got = bits16(y)
    want = oracle.round_bits(exact, fmt)
    lo = oracle.round_bits(exact * (1 - 2.0 ** -40), fmt)
    hi = oracle.round_bits(exact * (1 + 2.0 ** -40), fmt)
    stable = (lo == hi) & ~np.isnan(exact)
    bad = np.argwhere(stable & (got != want))
    assert bad.size == 0, (f"{what}: {len(bad)} outputs not rounded once, first at {tuple(bad[0])}: "
                           f"got {got[tuple(bad[0])]:#06x} want {want[tuple(bad[0])]:#06x}")
    return int(stable.size - stable.sum())


def _tenop_cols(fmt, path):
    w, _ = TENOP_PATHS[path]
    out, lo = [], 0
    for hi in WINDOW_RANGES:
        first = lo * w + (1 if path == "elem" else w)
        out += [first, hi * w]
        lo = hi
    # rows past 16384 columns (any type), fp32 rows of 4-element accesses past
    # 12288 and element-path rows past 12288 take the two-pass kernel
    return sorted({c for c in out if c <= 16384} | {12289, 16385, 20000})


# fp32 rows have no 8-element path
TENOP_CASES = [(f, p) for f in ("f32", "bf16", "f16") for p in TENOP_PATHS if not (f == "f32" and p == "vec8")]


@pytest.mark.parametrize("fmt,path", TENOP_CASES)
def test_tenop_every_layout(mbp, fmt, path):
    dtype = DT[fmt]
    _, off = TENOP_PATHS[path]
    if fmt == "f32" and path == "vec4":
        off = 0
    for cols in _tenop_cols(fmt, path):
        rows = max(3, min(40, 150_000 // cols))
        rng = np.random.default_rng([71, cols, off])
        xh, xf = _stored(rng, (rows, cols), dtype)
        vecs = [_stored(rng, (cols,), dtype) for _ in range(3)]
        what = f"10-op {fmt} {path} {rows}x{cols} at +{off} elements"
        print(what, flush=True)
        x, _ = _place_dev(xh, off)
        y, yb = _place_dev(torch.zeros_like(xh), off, 3.0)
        mbp.fused_row_mean_epilogue_2d(x, *(v[0].cuda() for v in vecs), alpha=1.1, c=0.1, out=y)
        exact = oracle.row_mean_epilogue(xf, *(v[1] for v in vecs), 1.1, 0.1)
        _gate_2d(y, exact, fmt, what, row_kernel=True)
        if fmt != "f32":
            _rounded_once(y, exact, fmt, what)
        assert _untouched(yb, off, y.numel()), f"{what}: wrote outside y"


def _softmax_cols(v, fmt):
    out, lo = [], 0
    for hi in WINDOW_RANGES:
        out += [lo * v + 1, hi * v]
        if hi >= 64:
            out.append(hi * v - v)  # whole vectors, pitch off 128 bytes: rotated windows
        lo = hi
    if fmt == "f32":
        out += [16385, 32768]  # the multi-pass kernel
    return out


@pytest.mark.parametrize("fmt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("path", ["aligned", "congruent", "independent"])
def test_softmax_every_layout(mbp, fmt, path):
    dtype = DT[fmt]
    v = 4 if fmt == "f32" else 8
    ox, _, oy = PATHS[path]
    for cols in _softmax_cols(v, fmt):
        rows = max(3, min(40, 150_000 // cols))
        rng = np.random.default_rng([73, cols])
        xh, xf = _stored(rng, (rows, cols), dtype, 4.0)
        what = f"softmax {fmt} {path} {rows}x{cols}"
        print(what, flush=True)
        x, _ = _place_dev(xh, ox)
        y, yb = _place_dev(torch.zeros_like(xh), oy, 3.0)
        mbp.fused_softmax(x, out=y)
        _softmax_gate(y, oracle.softmax(xf), fmt, what, xf)
        assert _untouched(yb, oy, y.numel()), f"{what}: wrote outside y"


@pytest.mark.parametrize("fmt", ["f32", "bf16"])
@pytest.mark.parametrize("offs", [(0, 0, 0), (1, 1, 1), (1, 0, 2), (0, 0, 1)])
@pytest.mark.parametrize("gran", [0, 1])
def test_unfused_every_path(mbp, fmt, offs, gran):
    """The unfused LayerNorm forms (with and without residual and GeLU) with x,
    residual and y on or off 16-byte boundaries: each launch takes its 16-byte
    or its element path by the alignment of its own operands."""
    name, _ = CASES[fmt]
    chk = check_f32 if fmt == "f32" else check_bf16
    for cols, residual, act in [(1000, True, "gelu_tanh"), (1000, False, "gelu_tanh"), (4095, True, "none"),
                                (4096, False, "none"), (24, True, "gelu_tanh")]:
        rows = 9
        w, d = _inputs(name, rows, cols, residual)
        what = f"unfused {fmt} {rows}x{cols} residual={residual} act={act} offsets {offs} granularity {gran}"
        print(what, flush=True)
        x, _ = _place(to_dev(d["x"]), offs[0], 0.0)
        r = _place(to_dev(d["residual"]), offs[1], 0.0)[0] if residual else None
        y, yb = _place(torch.zeros_like(x), offs[2], 3.0)
        mbp.unfused_add_layernorm_gelu(x, r, to_dev(d["gamma"]), to_dev(d["beta"]), eps=1e-5, act=act,
                                       granularity=gran, out=y)
        chk(to_host(y), _ln_ref(d, act, mode=oracle.SEQ if gran == 0 else oracle.SEQ3), what)
        assert _untouched(yb, offs[2], y.numel()), f"{what}: wrote outside y"


@pytest.mark.parametrize("fmt", ["f32", "bf16"])
@pytest.mark.parametrize("offs", [(0, 0), (1, 1), (0, 1), (1, 0)])
def test_unfused_dropout_and_softmax_paths(mbp, fmt, offs):
    """The unfused LayerNorm -> ReLU -> dropout and softmax launches with x and
    y on or off 16-byte boundaries."""
    name, _ = CASES[fmt]
    chk = check_f32 if fmt == "f32" else check_bf16
    for cols in (1000, 4095, 24):
        rows = 9
        w, d = _inputs(name, rows, cols, False)
        what = f"unfused dropout {fmt} {rows}x{cols} offsets {offs}"
        print(what, flush=True)
        x, _ = _place(to_dev(d["x"]), offs[0], 0.0)
        y, yb = _place(torch.zeros_like(x), offs[1], 3.0)
        seed, offset, p = 0x9E3779B97F4A7C15, 11, 0.3
        mbp.unfused_layernorm_relu_dropout(x, to_dev(d["gamma"]), to_dev(d["beta"]), p=p, seed=seed,
                                           offset=offset, out=y)
        want = oracle.ln_relu_dropout(d["x"], d["gamma"], d["beta"], p=p, seed=seed, offset=offset,
                                      mode=oracle.SEQ3)
        chk(to_host(y), want, what)
        assert _untouched(yb, offs[1], y.numel()), f"{what}: wrote outside y"

        rng = np.random.default_rng([79, cols])
        xh = torch.from_numpy(rng.standard_normal((rows, cols)) * 3).to(DT[fmt])
        xf = xh.float().numpy()
        what = f"unfused softmax {fmt} {rows}x{cols} offsets {offs}"
        print(what, flush=True)
        xs, _ = _place_dev(xh, offs[0])
        ys, ysb = _place_dev(torch.zeros_like(xh), offs[1], 3.0)
        mbp.unfused_softmax(xs, out=ys)
        want = oracle.softmax(xf, mode=oracle.SEQ, dtype=fmt)
        if fmt == "bf16":
            check_ulp16(bits16(ys), want, fmt, what)
        else:
            dd = np.abs(ordered(to_host(ys)) - ordered(want.astype(np.float32)))
            assert dd.max(initial=0) <= 4, f"{what}: max {dd.max()} ulp"
        assert _untouched(ysb, offs[1], ys.numel()), f"{what}: wrote outside y"


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("cols,off", [(4096, 0), (4092, 4), (4095, 1)])
def test_chain_2d_rounded_once(mbp, fmt, cols, off):
    """The 16-bit chain on random inputs, every output the exact value rounded
    once (16-byte, 4-element and single-element paths)."""
    dtype = DT[fmt]
    rows = 64
    rng = np.random.default_rng([83, cols, off])
    ops = [_stored(rng, (rows, cols), dtype) for _ in range(3)]
    devs = [_place_dev(o[0], off)[0] for o in ops]
    y = mbp.fused_pointwise_chain_2d(*devs, 0.5)
    exact = oracle.pointwise_chain(*(o[1] for o in ops), 0.5)
    _rounded_once(y, exact, fmt, f"chain 2d {fmt} {rows}x{cols} at +{off}")
