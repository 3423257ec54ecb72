"""GPU parity of rows of 16385 to 32768 columns: fp32 LayerNorm (+ residual,
GeLU), LayerNorm -> ReLU -> Dropout, softmax and the 10-op graph take their
multi-pass kernels there; 16-bit LayerNorm, dropout and softmax rows stay in
512-lane register layouts.  Every output element is compared with the oracle;
strided, misaligned and in-place operands included.
"""
import numpy as np
import pytest
import torch

import oracle
from parity_util import check_bf16, check_f32, ordered, to_dev, to_host
from test_gpu_parity import (DT2D, _check_dropout, _drop_case, _gate_2d, _ln_case, _ln_ref, _ln_run, _padded,
                             _softmax_gate, _stored)

pytestmark = pytest.mark.gpu

WIDE = [16385, 24576, 32768]


@pytest.fixture(scope="module")
def mbp():
    import memory_bound_pointwise_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert m.MAX_COLS == 32768
    return m


@pytest.mark.parametrize("name", ["ln_8192x4096_f32", "addln_gelu_16384x8192_bf16"])
@pytest.mark.parametrize("cols", WIDE)
@pytest.mark.parametrize("residual,act", [(False, "none"), (True, "gelu_tanh")])
def test_ln_wide(mbp, name, cols, residual, act):
    w, d, act = _ln_case(name, 3, cols, residual, act)
    chk = check_bf16 if w.dtype == "bf16" else check_f32
    y = _ln_run(mbp, d, act)
    chk(to_host(y), _ln_ref(d, act), f"{w.dtype} 3x{cols} residual={residual} act={act}")
    assert torch.equal(y, _ln_run(mbp, d, act)), "not deterministic"


@pytest.mark.parametrize("name", ["ln_8192x4096_f32", "addln_gelu_16384x8192_bf16"])
def test_ln_wide_strided_misaligned_in_place(mbp, name):
    cols = 20001
    w, d, act = _ln_case(name, 4, cols, True, "gelu_tanh")
    ref = _ln_ref(d, act)
    chk = check_bf16 if w.dtype == "bf16" else check_f32
    x = to_dev(d["x"])
    r = to_dev(d["residual"])
    g, b = to_dev(d["gamma"]), to_dev(d["beta"])
    # x one element off its allocation's start, rows 7 elements apart from the
    # next; the residual dense; y with its own pad
    xbuf = torch.zeros(x.shape[0] * (cols + 7) + 1, dtype=x.dtype, device="cuda")
    xs = xbuf[1:1 + x.shape[0] * (cols + 7)].view(x.shape[0], cols + 7)[:, :cols]
    xs.copy_(x)
    y, ybig = _padded(torch.zeros(x.shape, dtype=x.dtype), 5, sentinel=3.0)
    mbp.fused_add_layernorm_gelu(xs, r, g, b, act=act, out=y)
    chk(to_host(y), ref, f"{w.dtype} 4x{cols} strided, misaligned")
    assert (ybig[:, cols:].float() == 3.0).all(), "wrote outside the output rows"
    mbp.fused_add_layernorm_gelu(xs, r, g, b, act=act, out=xs)
    chk(to_host(xs), ref, f"{w.dtype} 4x{cols} in place")


@pytest.mark.parametrize("name", ["ln_8192x4096_f32", "addln_gelu_16384x8192_bf16"])
@pytest.mark.parametrize("cols", [16385, 32768])
@pytest.mark.parametrize("p", [0.1, 0.5])
def test_ln_relu_dropout_wide(mbp, name, cols, p):
    w, d = _drop_case(name, 3, cols)
    seed, offset = 0x5EED0000DEADBEEF, 3
    args = (to_dev(d["x"]), to_dev(d["gamma"]), to_dev(d["beta"]))
    y = mbp.fused_layernorm_relu_dropout(*args, p=p, seed=seed, offset=offset)
    frac = _check_dropout(y, d, w, p, seed, offset, f"ln-relu-dropout {w.dtype} 3x{cols} p={p}")
    assert abs(frac - p) < 0.02, f"dropped fraction {frac} for p={p}"
    assert torch.equal(y, mbp.fused_layernorm_relu_dropout(*args, p=p, seed=seed, offset=offset)), \
        "not deterministic"


@pytest.mark.parametrize("fmt,dtype", DT2D, ids=[d[0] for d in DT2D])
@pytest.mark.parametrize("cols", WIDE)
def test_softmax_wide(mbp, fmt, dtype, cols):
    rng = np.random.default_rng([29, cols])
    xh, xf = _stored(rng, (3, cols), dtype, 4.0)
    x = xh.cuda()
    y = mbp.fused_softmax(x)
    _softmax_gate(y, oracle.softmax(xf), fmt, f"softmax {fmt} 3x{cols}", xf)
    assert torch.equal(y, mbp.fused_softmax(x)), "not deterministic"


@pytest.mark.parametrize("fmt,dtype", DT2D, ids=[d[0] for d in DT2D])
def test_softmax_wide_masks_strided_in_place(mbp, fmt, dtype):
    cols = 24577
    rng = np.random.default_rng([31, cols])
    xh, xf = _stored(rng, (4, cols), dtype, 2.0)
    xh[1, ::3] = float("-inf")        # masked entries: exactly 0
    xh[2, :] = float("-inf")          # a fully masked row: NaN
    xh[3, 100] = float("nan")         # a NaN: its row NaN
    xf = xh.float().numpy()
    x, _ = _padded(xh, 3)
    y = mbp.fused_softmax(x)
    yh = to_host(y).astype(np.float64) if fmt == "f32" else y.float().cpu().numpy().astype(np.float64)
    assert np.all(yh[1, ::3] == 0.0), "masked entries not exactly 0"
    assert np.isnan(yh[2]).all() and np.isnan(yh[3]).all(), "degenerate rows not NaN"
    _softmax_gate(y[:2], oracle.softmax(xf[:2]), fmt, f"softmax {fmt} 2x{cols} strided", xf[:2])
    # y in x's layout (same pad): the same kernel as in place, so the same bits;
    # y above (dense rows, pitch unlike x's modulo 16) took the element kernel,
    # whose sums run in another order
    y2, _ = _padded(torch.zeros_like(xh), 3)
    mbp.fused_softmax(x, out=y2)
    mbp.fused_softmax(x, out=x)
    iv = torch.int32 if x.element_size() == 4 else torch.int16   # NaN rows compare as bits
    assert torch.equal(x.contiguous().view(iv), y2.contiguous().view(iv)), "in place differs"
    _softmax_gate(x[:2], oracle.softmax(xf[:2]), fmt, f"softmax {fmt} 2x{cols} in place", xf[:2])


@pytest.mark.parametrize("fmt,dtype", DT2D, ids=[d[0] for d in DT2D])
@pytest.mark.parametrize("cols,xpad,ypad", [(16385, 0, 0), (24576, 8, 3), (32768, 0, 8)])
def test_tenop_wide(mbp, fmt, dtype, cols, xpad, ypad):
    rows = 3
    rng = np.random.default_rng([37, cols, xpad])
    xh, xf = _stored(rng, (rows, cols), dtype)
    x, _ = _padded(xh, xpad)
    vecs = [_stored(rng, (cols,), dtype) for _ in range(3)]
    y, ybig = _padded(torch.zeros((rows, cols), dtype=dtype), ypad, sentinel=3.0)
    mbp.fused_row_mean_epilogue_2d(x, *(v[0].cuda() for v in vecs), alpha=1.1, c=0.1, out=y)
    exact = oracle.row_mean_epilogue(xf, *(v[1] for v in vecs), 1.1, 0.1)
    _gate_2d(y, exact, fmt, f"10-op {fmt} {rows}x{cols} pads {xpad},{ypad}", row_kernel=True)
    if ypad:
        assert (ybig[:, cols:].float() == 3.0).all(), "wrote outside the output rows"


def test_unfused_wide(mbp):
    """the unfused variants loop over any row length: LayerNorm (7 launches)
    and softmax at 24576 columns against the oracle's eager-op roundings"""
    cols = 24576
    w, d, act = _ln_case("addln_gelu_16384x8192_bf16", 3, cols, True, "gelu_tanh")
    y = mbp.unfused_add_layernorm_gelu(to_dev(d["x"]), to_dev(d["residual"]), to_dev(d["gamma"]),
                                       to_dev(d["beta"]), act=act, granularity=0)
    check_bf16(to_host(y), _ln_ref(d, act, mode=oracle.SEQ), f"unfused bf16 3x{cols}")
    rng = np.random.default_rng([41, cols])
    xh, xf = _stored(rng, (3, cols), torch.float32, 3.0)
    got = to_host(mbp.unfused_softmax(xh.cuda()))
    want = oracle.softmax(xf, mode=oracle.SEQ, dtype="f32")
    d = np.abs(ordered(got) - ordered(want.astype(np.float32)))
    assert d.max() <= 4, f"unfused softmax f32 3x{cols}: max {d.max()} ulp"


def test_cols_past_the_maximum_rejected(mbp):
    x = torch.zeros(2, mbp.MAX_COLS + 1, device="cuda")
    g = torch.ones(mbp.MAX_COLS + 1, device="cuda")
    with pytest.raises(Exception):
        mbp.fused_add_layernorm_gelu(x, None, g, g)
    with pytest.raises(Exception):
        mbp.fused_softmax(x)
