"""Tensors of more than 2^31 elements: every flat index, row offset and
dropout counter is 64-bit.  Inputs are drawn on the GPU (seeded); the oracle
checks sampled rows or elements -- the first, the last, and those on both
sides of element 2^31 -- at the same gates as the other parity tests.  Each
test holds at most ~35 GB of device memory and frees it at the end."""
import numpy as np
import pytest
import torch

import oracle
from parity_util import bits16, check_bf16, check_chain, check_f32, to_host

pytestmark = pytest.mark.gpu

BIG = 1 << 31


@pytest.fixture(scope="module")
def mbp():
    import memory_bound_pointwise_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _randn(shape, dtype, seed, std=1.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return (torch.randn(shape, generator=g, device="cuda", dtype=torch.float32) * std).to(dtype)


def _rows_around(rows, cols):
    """rows holding the first elements, the last ones, and element 2^31"""
    r = BIG // cols
    return np.array(sorted({0, 1, r - 1, r, r + 1, rows - 2, rows - 1}))


def _host16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def test_chain_past_2_31(mbp):
    n = BIG + (1 << 20) + 3
    x, b1, b2 = (_randn((n,), torch.float32, s) for s in (1, 2, 3))
    y = mbp.fused_pointwise_chain(x, b1, b2, 0.5)
    idx = np.unique(np.concatenate([np.arange(64), np.arange(BIG - 64, BIG + 64), np.arange(n - 64, n),
                                    np.random.default_rng(5).integers(0, n, 4096)]))
    ti = torch.from_numpy(idx).cuda()
    pick = lambda t: t[ti].cpu().numpy()
    ref = oracle.pointwise_chain(pick(x), pick(b1), pick(b2), 0.5)
    check_chain(pick(y), ref, f"chain n={n}, sampled elements")


@pytest.mark.parametrize("cols", [8192, 4095])
def test_layernorm_bf16_past_2_31(mbp, cols):
    rows = BIG // cols + 5
    x, r = _randn((rows, cols), torch.bfloat16, 11), _randn((rows, cols), torch.bfloat16, 12)
    g = (1 + 0.1 * _randn((cols,), torch.float32, 13)).to(torch.bfloat16)
    b = (0.1 * _randn((cols,), torch.float32, 14)).to(torch.bfloat16)
    y = mbp.fused_add_layernorm_gelu(x, r, g, b, eps=1e-5, act="gelu_tanh")
    rs = _rows_around(rows, cols)
    ti = torch.from_numpy(rs).cuda()
    ref = oracle.add_layernorm_gelu(_host16(x[ti]), _host16(r[ti]), _host16(g), _host16(b), eps=1e-5,
                                    act=oracle.ACT_GELU_TANH)
    check_bf16(to_host(y[ti]), ref, f"residual+LN+GeLU {rows}x{cols} bf16, rows around element 2^31")


@pytest.mark.parametrize("cols", [4096, 4095])
def test_softmax_bf16_past_2_31(mbp, cols):
    """4096: 16-byte accesses; 4095: the windowed path (rows off 16-byte boundaries)"""
    rows = BIG // cols + 3
    x = _randn((rows, cols), torch.bfloat16, 21, std=3.0)
    y = mbp.fused_softmax(x)
    rs = _rows_around(rows, cols)
    ti = torch.from_numpy(rs).cuda()
    from parity_util import check_ulp16
    check_ulp16(bits16(y[ti]), oracle.softmax(x[ti].float().cpu().numpy()), "bf16",
                f"softmax {rows}x{cols} bf16, rows around element 2^31")


def test_tenop_f32_past_2_31(mbp):
    rows, cols = BIG // 1024 + 3, 1024
    x = _randn((rows, cols), torch.float32, 31)
    bias, gamma, beta = (_randn((cols,), torch.float32, s) for s in (32, 33, 34))
    y = mbp.fused_row_mean_epilogue(x, bias, gamma, beta)
    rs = _rows_around(rows, cols)
    ti = torch.from_numpy(rs).cuda()
    ref = oracle.row_mean_epilogue(x[ti].cpu().numpy(), *(t.cpu().numpy() for t in (bias, gamma, beta)))
    check_f32(to_host(y[ti]), ref, f"10-op {rows}x{cols} fp32, rows around element 2^31")


# ------------------------------------------------------------------ more row groups than one dispatch holds
#
# A dispatch addresses at most 2^32 - 1 work-items, 2^24 - 1 blocks of 256
# threads; the narrowest layouts hold 16 rows a block, so 2^28 + 37 rows need
# more blocks than that.  Kernels that loop over row groups run on a capped
# grid; those with one block per row group are launched on chunks of 2^21 rows.

MANY = (1 << 28) + 37
CHUNK = 1 << 21


def _rows_many(rows):
    """first and last rows, both sides of every 2^21-row chunk boundary in the
    first few and the last, around 16 x (2^24 - 1) rows (a full 256-thread
    dispatch of 16-row groups), and a seeded random sample"""
    near = [0, 1, 2, rows - 3, rows - 2, rows - 1, 16 * ((1 << 24) - 1) - 1, 16 * ((1 << 24) - 1),
            16 * ((1 << 24) - 1) + 1]
    for k in (1, 2, 3, rows // CHUNK - 1, rows // CHUNK):
        near += [k * CHUNK - 1, k * CHUNK, k * CHUNK + 1]
    sample = np.random.default_rng(41).integers(0, rows, 2000)
    return np.unique(np.clip(np.array(near + list(sample)), 0, rows - 1))


@pytest.mark.parametrize("cols", [8, 7])
def test_layernorm_bf16_many_rows(mbp, cols):
    """8: 16-byte accesses (16 rows a block, a capped grid); 7: rows off
    16-byte boundaries (the window-class kernel, its class blocks capped)"""
    rows = MANY
    x, r = _randn((rows, cols), torch.bfloat16, 51), _randn((rows, cols), torch.bfloat16, 52)
    g = (1 + 0.1 * _randn((cols,), torch.float32, 53)).to(torch.bfloat16)
    b = (0.1 * _randn((cols,), torch.float32, 54)).to(torch.bfloat16)
    y = torch.full_like(x, 3.0)
    mbp.fused_add_layernorm_gelu(x, r, g, b, eps=1e-5, act="gelu_tanh", out=y)
    ti = torch.from_numpy(_rows_many(rows)).cuda()
    ref = oracle.add_layernorm_gelu(_host16(x[ti]), _host16(r[ti]), _host16(g), _host16(b), eps=1e-5,
                                    act=oracle.ACT_GELU_TANH)
    check_bf16(to_host(y[ti]), ref, f"residual+LN+GeLU {rows}x{cols} bf16, sampled rows")
    assert not (y == 3.0).all(dim=1).any().item(), "a row was not written"


@pytest.mark.parametrize("cols", [4, 5])
def test_softmax_f32_many_rows(mbp, cols):
    """4: 16-byte accesses; 5: rows off 16-byte boundaries (windows); both in
    2^21-row chunks"""
    rows = MANY
    x = _randn((rows, cols), torch.float32, 61, std=3.0)
    y = torch.full_like(x, 3.0)
    mbp.fused_softmax(x, out=y)
    ti = torch.from_numpy(_rows_many(rows)).cuda()
    from parity_util import check_softmax_f32
    xs = x[ti].cpu().numpy()
    check_softmax_f32(to_host(y[ti]), oracle.softmax(xs), xs, f"softmax {rows}x{cols} fp32, sampled rows")
    assert not (y == 3.0).all(dim=1).any().item(), "a row was not written"


def test_tenop_f32_many_rows(mbp):
    """one 16-lane group a row, 16 rows a block, no loop: 2^21-row chunks"""
    rows, cols = MANY, 4
    x = _randn((rows, cols), torch.float32, 71)
    bias, gamma, beta = (_randn((cols,), torch.float32, s) for s in (72, 73, 74))
    y = torch.full_like(x, 3.0)
    mbp.fused_row_mean_epilogue(x, bias, gamma, beta, out=y)
    ti = torch.from_numpy(_rows_many(rows)).cuda()
    ref = oracle.row_mean_epilogue(x[ti].cpu().numpy(), *(t.cpu().numpy() for t in (bias, gamma, beta)))
    check_f32(to_host(y[ti]), ref, f"10-op {rows}x{cols} fp32, sampled rows")
    assert not (y == 3.0).all(dim=1).any().item(), "a row was not written"


def test_tenop_f16_wave_many_rows(mbp):
    """the wave-per-row kernel (rows of 65-128 vectors) on more rows than one
    chunk: 2^21-row chunks of 16-row blocks"""
    rows, cols = 2 * CHUNK + 21, 520
    x = _randn((rows, cols), torch.float16, 81)
    bias, gamma, beta = (_randn((cols,), torch.float16, s) for s in (82, 83, 84))
    y = mbp.fused_row_mean_epilogue_2d(x, bias, gamma, beta, 1.1, 0.1)
    rs = _rows_many(rows)
    ti = torch.from_numpy(rs).cuda()
    ref = oracle.row_mean_epilogue(x[ti].float().cpu().numpy(), *(t.float().cpu().numpy() for t in (bias, gamma, beta)),
                                   1.1, 0.1)
    from parity_util import check_ulp16
    check_ulp16(bits16(y[ti]), ref, "f16", f"10-op {rows}x{cols} fp16, sampled rows")
