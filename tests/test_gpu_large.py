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
