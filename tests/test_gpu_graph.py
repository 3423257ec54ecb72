"""HIP graph capture of library calls (the mbp_graph_* entry points).

A captured sequence -- the unfused variants' several launches, or one fused
launch -- must replay to exactly what the same calls give eagerly.  Each case
is replayed several times, with ordinary eager work (new input values written
by torch) and synchronisations between the replays, and every replay is
compared with an eager run on the same inputs.  The graphs hold kernel nodes
only (no memset nodes): the node count equals the launches per call.
"""
import numpy as np
import pytest
import torch

import workloads as W
from parity_util import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mbp():
    import memory_bound_pointwise_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _tenop(mbp, rows, cols):
    d = W.generate(W.scaled(W.BY_NAME["tenop_1024x1024_f32"], rows=rows), cols=cols)
    return to_dev(d["x"]), [to_dev(d[k]) for k in ("bias", "gamma", "beta")]


def _case(mbp, name):
    """(x to rewrite between replays, call(out, ws), out template, workspace
    bytes, launches per call)."""
    m = mbp
    if name == "chain_unfused":
        d = W.generate(W.scaled(W.BY_NAME["chain_4M_f32"], n=(1 << 20) + 3))
        x, b1, b2 = (to_dev(d[k]) for k in ("x", "b1", "b2"))
        nb = m.workspace_bytes(m.OP_CHAIN, m.F32, 1, x.numel())
        return x, lambda y, ws: m.unfused_pointwise_chain(x, b1, b2, 0.5, out=y, workspace=ws), nb, 4
    if name == "chain_fused":
        d = W.generate(W.scaled(W.BY_NAME["chain_4M_f32"], n=(1 << 20) + 3))
        x, b1, b2 = (to_dev(d[k]) for k in ("x", "b1", "b2"))
        return x, lambda y, ws: m.fused_pointwise_chain(x, b1, b2, 0.5, out=y), 0, 1
    if name in ("tenop_unfused", "tenop_grouped", "tenop_fused"):
        x, v = _tenop(mbp, 1024, 1000)
        if name == "tenop_unfused":
            nb = m.workspace_bytes(m.OP_ROW_MEAN, m.F32, 1024, 1000)
            return x, lambda y, ws: m.unfused_row_mean_epilogue(x, *v, out=y, workspace=ws), nb, 10
        if name == "tenop_grouped":
            nb = m.workspace_bytes(m.OP_ROW_MEAN, m.F32, 1024, 1000, granularity=m.UNFUSED_GROUPED)
            return x, lambda y, ws: m.grouped_row_mean_epilogue(x, *v, out=y, workspace=ws), nb, 3
        return x, lambda y, ws: m.fused_row_mean_epilogue(x, *v, out=y), 0, 1
    if name in ("ln_unfused", "ln_fused"):
        w = W.scaled(W.BY_NAME["addln_gelu_16384x8192_bf16"], rows=64)
        d = W.generate(w, cols=4095)
        x, r, g, b = (to_dev(d[k]) for k in ("x", "residual", "gamma", "beta"))
        if name == "ln_unfused":
            nb = m.workspace_bytes(m.OP_LAYERNORM, m.BF16, 64, 4095, True, "gelu_tanh")
            return x, (lambda y, ws: m.unfused_add_layernorm_gelu(x, r, g, b, act="gelu_tanh", out=y,
                                                                  workspace=ws)), nb, 7
        return x, lambda y, ws: m.fused_add_layernorm_gelu(x, r, g, b, act="gelu_tanh", out=y), 0, 1
    if name in ("lnrd_unfused", "lnrd_fused", "lnrd_fused_4095"):
        w = W.scaled(W.BY_NAME["addln_gelu_16384x8192_bf16"], rows=32)
        d = W.generate(w, cols=4095 if name == "lnrd_fused_4095" else 8192)
        x, g, b = (to_dev(d[k]) for k in ("x", "gamma", "beta"))
        kw = dict(p=0.1, seed=0x5EED, offset=12345)
        if name == "lnrd_unfused":
            nb = m.workspace_bytes(m.OP_LN_RELU_DROPOUT, m.BF16, 32, 8192)
            return x, (lambda y, ws: m.unfused_layernorm_relu_dropout(x, g, b, out=y, workspace=ws,
                                                                      **kw)), nb, 3
        return x, lambda y, ws: m.fused_layernorm_relu_dropout(x, g, b, out=y, **kw), 0, 1
    if name == "softmax":
        x = torch.randn(257, 1000, device="cuda", dtype=torch.bfloat16)
        return x, lambda y, ws: m.fused_softmax(x, out=y), 0, 1
    if name == "softmax_unfused":
        x = torch.randn(257, 1000, device="cuda", dtype=torch.bfloat16)
        nb = m.workspace_bytes(m.OP_SOFTMAX, m.BF16, 257, 1000)
        return x, lambda y, ws: m.unfused_softmax(x, out=y, workspace=ws), nb, 5
    raise KeyError(name)


CASES = ["chain_unfused", "chain_fused", "tenop_unfused", "tenop_grouped", "tenop_fused",
         "ln_unfused", "ln_fused", "lnrd_unfused", "lnrd_fused", "lnrd_fused_4095", "softmax", "softmax_unfused"]


@pytest.mark.parametrize("name", CASES)
def test_graph_replays_match_eager(mbp, name):
    x, call, nb, launches = _case(mbp, name)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    y_graph = torch.empty_like(x)
    y_eager = torch.empty_like(x)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with mbp.capture(side) as cap:
        call(y_graph, ws)
    g = cap.graph
    assert g.nodes == launches, f"{name}: {g.nodes} graph nodes, expected {launches} launches"
    gen = torch.Generator(device="cuda").manual_seed(7)
    for rep in range(4):
        if rep:  # eager work between the replays: new input values
            x.copy_(torch.randn(x.shape, generator=gen, device="cuda", dtype=torch.float32).to(x.dtype))
        y_graph.fill_(float("nan"))
        torch.cuda.synchronize()
        if rep % 2:
            g.launch(side)
            side.synchronize()
        else:
            g.launch()  # the current (default) stream
            torch.cuda.synchronize()
        call(y_eager, ws)
        torch.cuda.synchronize()
        a = y_graph.view(torch.int16 if x.element_size() == 2 else torch.int32)
        b = y_eager.view(a.dtype)
        assert torch.equal(a, b), f"{name}: replay {rep} differs from the eager call"
    g.close()
    g.close()  # a second close is a no-op
    with pytest.raises(ValueError):
        g.launch()


def test_graph_capture_errors(mbp):
    x, v = _tenop(mbp, 8, 64)
    y = torch.empty_like(x)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    # a call that fails validation while recording records nothing
    with mbp.capture(side) as cap:
        with pytest.raises(mbp.MbpError):
            mbp.fused_row_mean_epilogue(x, *v, alpha=float("inf"), out=y)
        mbp.fused_row_mean_epilogue(x, *v, out=y)
    assert cap.graph.nodes == 1
    cap.graph.close()
    # an empty capture is an error, and the stream is usable afterwards
    with pytest.raises(mbp.MbpError) as e:
        with mbp.capture(side):
            pass
    assert e.value.status == 8
    # an exception inside the block ends the capture and propagates
    with pytest.raises(RuntimeError, match="inside"):
        with mbp.capture(side):
            mbp.fused_row_mean_epilogue(x, *v, out=y)
            raise RuntimeError("inside")
    with mbp.capture(side) as cap:
        mbp.fused_row_mean_epilogue(x, *v, out=y)
        mbp.fused_row_mean_epilogue(y, *v, out=y)
    assert cap.graph.nodes == 2
    cap.graph.launch(side)
    side.synchronize()
    ref = mbp.fused_row_mean_epilogue(mbp.fused_row_mean_epilogue(x, *v), *v)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
    cap.graph.close()
    with pytest.raises(ValueError):
        mbp.capture(torch.cuda.default_stream())
