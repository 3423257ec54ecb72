"""The C-ABI library on the host: it loads, exports every function that
include/mbp.h declares, and rejects bad arguments before launching anything.
No GPU: every call here fails host validation (or is pure host bookkeeping)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mbp.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def mbp():
    import memory_bound_pointwise_amd as m
    return m


def test_header_declares_the_boundary():
    fns = header_functions()
    for name in ("fused_pointwise_chain", "fused_row_mean_epilogue", "fused_add_layernorm_gelu",
                 "fused_pointwise_chain_2d", "fused_row_mean_epilogue_2d", "fused_softmax",
                 "fused_layernorm_relu_dropout", "unfused_layernorm_relu_dropout",
                 "unfused_pointwise_chain", "unfused_row_mean_epilogue", "unfused_add_layernorm_gelu",
                 "grouped_row_mean_epilogue", "unfused_softmax", "mbp_graph_capture_begin", "mbp_graph_capture_end",
                 "fused_add_layernorm_gelu_2d", "fused_layernorm_relu_dropout_2d", "fused_softmax_2d",
                 "grouped_row_mean_epilogue_noalloc", "mbp_stream_rw",
                 "mbp_graph_launch", "mbp_graph_destroy"):
        assert name in fns


def test_library_exports_every_declared_symbol(mbp):
    out = subprocess.run(["nm", "-D", "--defined-only", mbp.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [f for f in header_functions() if f not in exported]
    assert not missing, f"declared but not exported: {missing}"
    bound = {name for name, _, _ in mbp.SIGNATURES}
    assert bound == set(header_functions()), "the binding must cover exactly the declared functions"


def test_abi_version_and_strings(mbp):
    assert mbp.lib.mbp_abi_version() == 7
    for code, name in mbp.STATUS_NAMES.items():
        assert mbp.lib.mbp_status_string(code)
    assert mbp.lib.mbp_status_string(99) == b"unknown status"


L = None  # shorthand for the ctypes library, set in each test


def st(name, *args):
    return getattr(L, name)(*args)


# Fake, never-dereferenced addresses: every call below fails validation first.
A = 0x10000000
B = 0x20000000
Y = 0x30000000


def test_chain_validation(mbp):
    global L
    L = mbp.lib
    assert st("fused_pointwise_chain", A, B, B, Y, -1, 0.5, None) == 2            # SHAPE
    assert st("fused_pointwise_chain", None, None, None, None, 0, 0.5, None) == 0  # n == 0: no-op
    assert st("fused_pointwise_chain", A, None, B, Y, 8, 0.5, None) == 1          # NULL
    assert st("fused_pointwise_chain", A + 2, B, B, Y, 8, 0.5, None) == 4         # ALIGN
    assert st("fused_pointwise_chain", A, B, B, Y, 8, float("inf"), None) == 8    # ARG
    assert st("fused_pointwise_chain", A, B, B, A + 4, 8, 0.5, None) == 5         # partial overlap
    assert b"overlaps" in L.mbp_last_error()
    # the unfused variant forbids even exact aliasing, and needs a workspace
    assert st("unfused_pointwise_chain", A, B, B, A, 8, 0.5, Y + 4096, 4096, None) == 5
    assert st("unfused_pointwise_chain", A, B, B, Y, 8, 0.5, None, 0, None) == 6
    assert st("unfused_pointwise_chain", A, B, B, Y, 8, 0.5, Y + 0x10000 + 16, 1 << 20, None) == 6
    assert st("unfused_pointwise_chain", A, B, B, Y, 8, 0.5, Y + 0x10000, 16, None) == 6
    assert st("unfused_pointwise_chain", A, B, B, Y, 1024, 0.5, A + 256, 1 << 20, None) == 5


def test_row_validation(mbp):
    global L
    L = mbp.lib
    big = mbp.MAX_COLS + 1
    assert st("fused_row_mean_epilogue", A, B, B, B, Y, 4, 0, 1.1, 0.1, None) == 2
    assert st("fused_row_mean_epilogue", A, B, B, B, Y, 4, big, 1.1, 0.1, None) == 2
    assert st("fused_row_mean_epilogue", A, B, B, B, Y, -1, 8, 1.1, 0.1, None) == 2
    assert st("fused_row_mean_epilogue", A, B, B, B, Y, 2 ** 62, 8, 1.1, 0.1, None) == 2
    assert st("fused_row_mean_epilogue", A, B, B, B, Y, 0, 8, 1.1, 0.1, None) == 0
    assert st("fused_row_mean_epilogue", A, B, B, B, Y, 4, 8, float("nan"), 0.1, None) == 8
    assert st("fused_row_mean_epilogue", A, B, Y + 8, B, Y, 4, 8, 1.1, 0.1, None) == 5  # y over gamma
    assert st("fused_add_layernorm_gelu", 7, A, None, B, B, Y, 4, 8, 1e-5, 0, None) == 3
    assert st("fused_add_layernorm_gelu", 0, A, None, B, B, Y, 4, 8, 1e-5, 9, None) == 3
    assert st("fused_add_layernorm_gelu", 0, A, None, B, B, Y, 4, 8, -1.0, 0, None) == 8
    assert st("fused_add_layernorm_gelu", 1, A + 1, None, B, B, Y, 4, 8, 1e-5, 0, None) == 4
    assert st("fused_add_layernorm_gelu", 0, A + 2, None, B, B, Y, 4, 8, 1e-5, 0, None) == 4
    assert st("fused_add_layernorm_gelu", 1, A, A + 2, B, B, A + 2, 4, 8, 1e-5, 1, None) == 5
    assert st("fused_add_layernorm_gelu", 1, None, None, B, B, Y, 4, 8, 1e-5, 1, None) == 1
    assert st("fused_add_layernorm_gelu", 1, A, None, B, B, Y, 4, big, 1e-5, 1, None) == 2
    assert st("unfused_add_layernorm_gelu", 1, A, None, B, B, Y, 4, 8, 1e-5, 1, 5, None, 0, None) == 8


def test_2d_validation(mbp):
    global L
    L = mbp.lib
    c2 = "fused_pointwise_chain_2d"
    # dtype, x, ldx, b1, ldb1, b2, ldb2, y, ldy, rows, cols, scale, stream
    assert st(c2, 5, A, 8, B, 0, B, 0, Y, 8, 4, 8, 0.5, None) == 3                # DTYPE
    assert st(c2, 2, A, 8, B, 0, B, 0, Y, 8, -1, 8, 0.5, None) == 2               # rows < 0
    assert st(c2, 2, A, 8, B, 0, B, 0, Y, 8, 0, 8, 0.5, None) == 0                # rows == 0: no-op
    assert st(c2, 2, A, 8, B, 0, B, 0, Y, 8, 4, 0, 0.5, None) == 2                # cols == 0
    assert st(c2, 2, None, 8, B, 0, B, 0, Y, 8, 4, 8, 0.5, None) == 1             # NULL
    assert st(c2, 2, A + 1, 8, B, 0, B, 0, Y, 8, 4, 8, 0.5, None) == 4            # fp16 misaligned
    assert st(c2, 0, A + 2, 8, B, 0, B, 0, Y, 8, 4, 8, 0.5, None) == 4            # fp32 misaligned
    assert st(c2, 2, A, 4, B, 0, B, 0, Y, 8, 4, 8, 0.5, None) == 2                # 0 < ldx < cols
    assert st(c2, 2, A, 8, B, 0, B, 0, Y, 4, 4, 8, 0.5, None) == 2                # ldy < cols
    assert st(c2, 2, A, 8, B, 0, B, 0, Y, 0, 4, 8, 0.5, None) == 2                # broadcast output
    assert st(c2, 2, A, 8, B, -8, B, 0, Y, 8, 4, 8, 0.5, None) == 2               # negative stride
    assert st(c2, 2, A, 8, B, 0, B, 0, Y, 8, 4, 8, float("inf"), None) == 8       # ARG
    assert st(c2, 2, A, 8, B, 0, B, 0, A + 2, 8, 4, 8, 0.5, None) == 5            # partial overlap
    assert st(c2, 2, A, 8, B, 0, B, 0, A, 16, 4, 8, 0.5, None) == 5               # y == x, other stride
    assert st(c2, 2, A, 8, Y + 4, 0, B, 0, Y, 8, 4, 8, 0.5, None) == 5            # y over a broadcast b1
    r2 = "fused_row_mean_epilogue_2d"
    # dtype, x, ldx, bias, gamma, beta, y, ldy, rows, cols, alpha, c, stream
    assert st(r2, 1, A, 8, B, B, B, Y, 8, 4, mbp.MAX_COLS + 1, 1.1, 0.1, None) == 2
    assert st(r2, 1, A, 8, B, B, B, Y, 8, 4, 8, float("nan"), 0.1, None) == 8
    assert st(r2, 1, A, 8, B, Y + 2, B, Y, 8, 4, 8, 1.1, 0.1, None) == 5          # y over gamma
    assert st(r2, 1, A, 8, None, B, B, Y, 8, 4, 8, 1.1, 0.1, None) == 1
    assert st(r2, 1, A, 8, B, B, B, A, 12, 4, 8, 1.1, 0.1, None) == 5             # y == x, other stride
    # fp16 is for the two-dimensional forms only
    assert st("fused_add_layernorm_gelu", 2, A, None, B, B, Y, 4, 8, 1e-5, 0, None) == 3


def test_dropout_validation(mbp):
    global L
    L = mbp.lib
    f = "fused_layernorm_relu_dropout"
    # dtype, x, gamma, beta, y, rows, cols, eps, p, seed, offset, stream
    assert st(f, 1, A, B, B, Y, 4, 8, 1e-5, 1.5, 0, 0, None) == 8                # p > 1
    assert st(f, 1, A, B, B, Y, 4, 8, 1e-5, float("nan"), 0, 0, None) == 8       # p NaN
    assert st(f, 1, A, B, B, Y, 4, 8, 1e-5, -0.1, 0, 0, None) == 8               # p < 0
    assert st(f, 2, A, B, B, Y, 4, 8, 1e-5, 0.1, 0, 0, None) == 3                # fp16: not here
    assert st(f, 1, A, B, B, Y, 0, 8, 1e-5, 0.1, 0, 0, None) == 0                # rows == 0
    assert st(f, 1, A, B, B, A + 2, 4, 8, 1e-5, 0.1, 0, 0, None) == 5            # partial overlap
    u = "unfused_layernorm_relu_dropout"
    assert st(u, 1, A, B, B, Y, 4, 8, 1e-5, 0.1, 0, 0, None, 0, None) == 6       # no workspace
    assert st(u, 1, A, B, B, A, 4, 8, 1e-5, 0.1, 0, 0, Y + 4096, 1 << 20, None) == 5  # in place
    m = mbp
    assert m.launches_per_call(m.OP_LN_RELU_DROPOUT, True) == 1
    assert m.launches_per_call(m.OP_LN_RELU_DROPOUT, False) == 3
    assert m.workspace_bytes(m.OP_LN_RELU_DROPOUT, m.BF16, 4, 8) == 2 * 256


def test_workspace_and_launch_counts(mbp):
    m = mbp
    assert m.launches_per_call(m.OP_CHAIN, True) == 1
    assert m.launches_per_call(m.OP_CHAIN, False) == 4
    assert m.launches_per_call(m.OP_ROW_MEAN, False) == 10
    assert m.launches_per_call(m.OP_LAYERNORM, False) == 5
    assert m.launches_per_call(m.OP_LAYERNORM, False, has_residual=True, act="gelu_tanh") == 7
    assert m.launches_per_call(m.OP_LAYERNORM, False, m.UNFUSED_EAGER, True, "gelu_tanh") == 3
    assert m.launches_per_call(m.OP_LAYERNORM, False, 7) == -1
    n = 4 * 1024 * 1024
    assert m.workspace_bytes(m.OP_CHAIN, m.F32, 1, n) == 2 * 4 * n
    assert m.workspace_bytes(m.OP_ROW_MEAN, m.F32, 1024, 1024) == 3 * 4 * 1024 * 1024 + 4096
    full = 16384 * 8192 * 2
    assert m.workspace_bytes(m.OP_LAYERNORM, m.BF16, 16384, 8192, True, "gelu_tanh") == \
        3 * full + 2 * 16384 * 4
    assert m.workspace_bytes(m.OP_LAYERNORM, m.BF16, 16384, 8192, True, "gelu_tanh",
                             m.UNFUSED_EAGER) == 2 * full
    assert m.workspace_bytes(m.OP_LAYERNORM, m.F32, 0, 8) == 0
    with pytest.raises(ValueError):
        m.workspace_bytes(m.OP_LAYERNORM, 5, 4, 8)


def test_grouped_validation(mbp):
    global L
    L = mbp.lib
    g = "grouped_row_mean_epilogue"
    # x, bias, gamma, beta, y, rows, cols, alpha, c, workspace, workspace_bytes, stream
    ws = Y + 0x100000
    assert st(g, A, B, B, B, Y, 4, 0, 1.1, 0.1, ws, 1 << 20, None) == 2               # cols == 0
    assert st(g, A, B, B, B, Y, 0, 8, 1.1, 0.1, None, 0, None) == 0                   # rows == 0
    assert st(g, A, None, B, B, Y, 4, 8, 1.1, 0.1, ws, 1 << 20, None) == 1            # NULL
    assert st(g, A, B, B, B, Y, 4, 8, float("inf"), 0.1, ws, 1 << 20, None) == 8      # ARG
    assert st(g, A, B, B, B, A, 4, 8, 1.1, 0.1, ws, 1 << 20, None) == 5               # y == x
    assert st(g, A, B, B, B, Y, 4, 8, 1.1, 0.1, None, 0, None) == 6                   # no workspace
    assert st(g, A, B, B, B, Y, 4, 8, 1.1, 0.1, ws, 16, None) == 6                    # too small
    assert st(g, A, B, B, B, Y, 4, 8, 1.1, 0.1, A, 1 << 20, None) == 5                # ws over x
    m = mbp
    assert m.launches_per_call(m.OP_ROW_MEAN, False, m.UNFUSED_GROUPED) == 3
    assert m.workspace_bytes(m.OP_ROW_MEAN, m.F32, 1024, 1024, granularity=m.UNFUSED_GROUPED) == \
        4 * 1024 * 1024 + 4096


def test_graph_host_errors(mbp):
    """Argument errors of the graph entry points, found before any HIP call."""
    L = mbp.lib
    h = ctypes.c_void_p(1234)
    assert L.mbp_graph_capture_begin(None) == 8                       # the NULL stream
    assert L.mbp_graph_capture_end(None, ctypes.byref(h)) == 8
    assert h.value is None                                           # cleared on failure
    assert L.mbp_graph_capture_end(A, None) == 1
    assert L.mbp_graph_launch(None, None) == 1
    assert L.mbp_graph_nodes(None) == -1
    assert L.mbp_graph_destroy(None) == 0
    import torch
    with pytest.raises(ValueError):
        mbp.capture(None)


def test_unfused_softmax_validation(mbp):
    global L
    L = mbp.lib
    u = "unfused_softmax"
    ws = Y + 0x100000
    # dtype, x, y, rows, cols, workspace, workspace_bytes, stream
    assert st(u, 2, A, Y, 4, 8, ws, 1 << 20, None) == 3                 # fp16: fused only
    assert st(u, 1, A, Y, 4, 0, ws, 1 << 20, None) == 2                 # cols == 0
    assert st(u, 1, A, Y, 0, 8, None, 0, None) == 0                     # rows == 0
    assert st(u, 1, A, A, 4, 8, ws, 1 << 20, None) == 5                 # y == x
    assert st(u, 1, A, Y, 4, 8, None, 0, None) == 6                     # no workspace
    assert st(u, 0, A, Y, 4, 8, ws, 16, None) == 6                      # too small
    m = mbp
    assert m.launches_per_call(m.OP_SOFTMAX, True) == 1
    assert m.launches_per_call(m.OP_SOFTMAX, False) == 5
    assert m.workspace_bytes(m.OP_SOFTMAX, m.BF16, 4, 8) == 4 * 256
    with pytest.raises(ValueError):
        m.workspace_bytes(m.OP_SOFTMAX, m.F16, 4, 8)


def test_row_2d_validation(mbp):
    """The strided forms of residual + LayerNorm + GeLU, LayerNorm-ReLU-dropout
    and softmax: stride rules, in-place only with the same stride, gamma and
    beta never overlapped."""
    global L
    L = mbp.lib
    f = "fused_add_layernorm_gelu_2d"
    # dtype, x, ldx, residual, ldr, gamma, beta, y, ldy, rows, cols, eps, act, stream
    assert st(f, 2, A, 8, None, 0, B, B, Y, 8, 4, 8, 1e-5, 0, None) == 3          # fp16: not here
    assert st(f, 1, A, 8, None, 0, B, B, Y, 8, 4, 8, 1e-5, 5, None) == 3          # unknown act
    assert st(f, 1, A, 8, None, 0, B, B, Y, 8, 4, 8, -1.0, 0, None) == 8          # eps < 0
    assert st(f, 1, A, 8, None, 0, B, B, Y, 8, 0, 8, 1e-5, 0, None) == 0          # rows == 0
    assert st(f, 1, A, 6, None, 0, B, B, Y, 8, 4, 8, 1e-5, 0, None) == 2          # 0 < ldx < cols
    assert st(f, 1, A, 8, B, 6, B + 64, B + 64, Y, 8, 4, 8, 1e-5, 0, None) == 2   # 0 < ldr < cols
    assert st(f, 1, A, 8, None, 0, B, B, Y, 6, 4, 8, 1e-5, 0, None) == 2          # ldy < cols
    assert st(f, 1, A, 8, None, 0, B, B, Y, 8, 4, mbp.MAX_COLS + 1, 1e-5, 0, None) == 2
    assert st(f, 1, A, 8, None, 0, B, B, A, 16, 4, 8, 1e-5, 0, None) == 5         # y == x, other stride
    assert st(f, 1, A, 8, None, 0, B, B, A + 2, 8, 4, 8, 1e-5, 0, None) == 5       # partial overlap
    assert st(f, 1, A, 8, None, 0, Y + 4, B, Y, 8, 4, 8, 1e-5, 0, None) == 5       # y over gamma
    assert st(f, 1, A, 8, None, 0, B, B, Y + 1, 8, 4, 8, 1e-5, 0, None) == 4       # y misaligned
    assert st(f, 1, None, 8, None, 0, B, B, Y, 8, 4, 8, 1e-5, 0, None) == 1        # NULL x
    d = "fused_layernorm_relu_dropout_2d"
    # dtype, x, ldx, gamma, beta, y, ldy, rows, cols, eps, p, seed, offset, stream
    assert st(d, 1, A, 8, B, B, Y, 8, 4, 8, 1e-5, 1.5, 0, 0, None) == 8           # p > 1
    assert st(d, 1, A, 8, B, B, A, 12, 4, 8, 1e-5, 0.1, 0, 0, None) == 5          # y == x, other stride
    assert st(d, 1, A, 5, B, B, Y, 8, 4, 8, 1e-5, 0.1, 0, 0, None) == 2           # 0 < ldx < cols
    sm = "fused_softmax_2d"
    # dtype, x, ldx, y, ldy, rows, cols, stream
    assert st(sm, 3, A, 8, Y, 8, 4, 8, None) == 3                                  # DTYPE
    assert st(sm, 1, A, 7, Y, 8, 4, 8, None) == 2                                  # 0 < ldx < cols
    assert st(sm, 1, A, 8, A, 9, 4, 8, None) == 5                                  # y == x, other stride
    assert st(sm, 1, A, 8, Y, 8, 0, 8, None) == 0                                  # rows == 0
    assert st(sm, 1, A, 8, Y, 8, 4, mbp.MAX_COLS + 1, None) == 2


def test_stream_rw_validation(mbp):
    import ctypes
    L = mbp.lib
    arr = lambda *p: (ctypes.c_void_p * len(p))(*p)
    f = L.mbp_stream_rw
    assert f(arr(A), 0, Y, 64, None) == 8                 # nsrc < 1
    assert f(arr(A, A, A, A, A), 5, Y, 64, None) == 8     # nsrc > 4
    assert f(arr(A), 1, Y, 0, None) == 0                  # bytes == 0: no-op
    assert f(arr(A, None), 2, Y, 64, None) == 1           # a NULL source
    assert f(arr(A), 1, None, 64, None) == 1              # NULL dst
    assert f(arr(A + 8), 1, Y, 64, None) == 4             # source off 16 bytes
    assert f(arr(A), 1, Y, 24, None) == 4                 # bytes not a multiple of 16
    assert f(arr(A, B), 2, B + 32, 64, None) == 5         # dst overlaps a source


def test_convert_validation(mbp):
    L = mbp.lib
    f = L.mbp_convert_f32_to_bf16
    assert f(A, Y, -1, None) == 2                 # SHAPE
    assert f(None, None, 0, None) == 0            # n == 0: no-op
    assert f(None, Y, 8, None) == 1               # NULL
    assert f(A + 2, Y, 8, None) == 4              # x not 4-byte aligned
    assert f(A, Y + 1, 8, None) == 4              # y not 2-byte aligned
    assert f(A, A + 16, 8, None) == 5             # y overlaps x


def test_binding_rejects_cpu_tensors(mbp):
    import torch
    x = torch.zeros(8)
    with pytest.raises(ValueError):
        mbp.fused_pointwise_chain(x, x, x)


def test_kernel_coverage_lists_the_kernels(tmp_path):
    """tests/kernel_coverage.py: the library's kernel stubs are found, and a
    kernel trace's names (with their argument lists) match them."""
    import sys
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import kernel_coverage as kc
    inst = kc.instantiated()
    assert "mbp::ln::ln_vec_kernel<mbp::BF16IO, 256, 4, true, 1>" in inst
    assert "mbp::chain_kernel<1>" in inst
    assert not any("shape_kernel" in n for n in inst)
    stats = tmp_path / "k.csv"
    stats.write_text('"Name","Calls"\n'
                     '"void mbp::(anonymous namespace)::chain_kernel<1>(float const*, float const*, float const*, '
                     'float*, long, long, long, double)",3\n'
                     '"__amd_rocclr_copyBuffer",2\n')
    assert kc.dispatched(str(stats)) == {"mbp::chain_kernel<1>"}
    assert kc.main(["kernel_coverage.py", str(stats)]) == 1
