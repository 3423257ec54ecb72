"""grouped_row_mean_epilogue_noalloc -- the entry point that allocates nothing
(its intermediates s and m live in the library's static scratch array) --
called through the C ABI and compared with grouped_row_mean_epilogue, which
runs the same three kernels on a caller's workspace: the outputs must be equal
bit for bit, call after call, whatever the previous call left in the scratch.
Both are also held to the oracle's sequential fp32 evaluation (SEQ) within the
fp32 gate."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import check_f32, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mbp():
    import memory_bound_pointwise_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _inputs(rows, cols, sub):
    from dataclasses import replace
    w = replace(W.scaled(W.BY_NAME["tenop_1024x1024_f32"], rows=rows), sub=sub)
    return W.generate(w, cols=cols)


def _call_noalloc(mbp, x, vecs, y):
    rows, cols = x.shape
    stream = torch.cuda.current_stream().cuda_stream
    return mbp.lib.grouped_row_mean_epilogue_noalloc(
        x.data_ptr(), *(v.data_ptr() for v in vecs), y.data_ptr(), rows, cols, 1.1, 0.1, stream)


def _call_grouped(mbp, x, vecs, y, ws):
    rows, cols = x.shape
    stream = torch.cuda.current_stream().cuda_stream
    return mbp.lib.grouped_row_mean_epilogue(
        x.data_ptr(), *(v.data_ptr() for v in vecs), y.data_ptr(), rows, cols, 1.1, 0.1,
        ws.data_ptr(), ws.numel(), stream)


def test_noalloc_matches_grouped_call_after_call(mbp):
    # largest first (4080 x 1024 fills the 16 MiB array to within 48 KiB),
    # then smaller inputs that find the earlier contents in the scratch
    for k, (rows, cols) in enumerate([(4080, 1024), (333, 700), (1024, 1024), (7, 9)]):
        d = _inputs(rows, cols, sub=k + 1)
        print(f"noalloc call {k}: {rows}x{cols}", flush=True)
        x = to_dev(d["x"])
        vecs = [to_dev(d[n]) for n in ("bias", "gamma", "beta")]
        nb = mbp.workspace_bytes(mbp.OP_ROW_MEAN, mbp.F32, rows, cols, granularity=mbp.UNFUSED_GROUPED)
        assert nb <= 16 << 20
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        y_ref = torch.full_like(x, float("nan"))
        y_na = torch.full_like(x, float("nan"))
        assert _call_grouped(mbp, x, vecs, y_ref, ws) == 0, mbp.lib.mbp_last_error()
        assert _call_noalloc(mbp, x, vecs, y_na) == 0, mbp.lib.mbp_last_error()
        torch.cuda.synchronize()
        a, b = to_host(y_na), to_host(y_ref)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), \
            f"{rows}x{cols}: noalloc differs from grouped at {int((a != b).sum())} elements"
        ref = oracle.row_mean_epilogue(d["x"], d["bias"], d["gamma"], d["beta"], mode=oracle.SEQ)
        check_f32(a, ref, f"noalloc {rows}x{cols} vs SEQ")


def test_noalloc_rejects_inputs_beyond_the_scratch(mbp):
    # 4096 x 1024 needs 16 MiB + 16 KiB: refused on the host, nothing launched
    x = torch.zeros((4096, 1024), dtype=torch.float32, device="cuda")
    v = torch.zeros(1024, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    st = _call_noalloc(mbp, x, [v, v, v], y)
    assert st == 6, f"status {st}"  # MBP_ERR_WORKSPACE
    assert b"static scratch" in mbp.lib.mbp_last_error()
    assert _call_noalloc(mbp, x[:0], [v, v, v], y) == 0  # rows == 0: no-op
