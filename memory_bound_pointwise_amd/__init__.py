"""Python binding of libmbp, the gfx950 library of vertically fused memory-bound
chains (C ABI in ``include/mbp.h``).

This module only marshals arguments: it checks tensors, takes their device
pointers and the current HIP stream, and calls the C entry point of the same
name through ctypes.  Every step of the computation runs in the library's HIP
kernels.  There is no fallback: if ``libmbp.so`` has not been built the import
fails, and a non-zero status from the library raises ``MbpError``.

PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmbp.so")

F32, BF16, F16 = 0, 1, 2
ACT_NONE, ACT_GELU_TANH = 0, 1
OP_CHAIN, OP_ROW_MEAN, OP_LAYERNORM, OP_LN_RELU_DROPOUT, OP_SOFTMAX = 0, 1, 2, 3, 4
UNFUSED_PRIMITIVE, UNFUSED_EAGER, UNFUSED_GROUPED = 0, 1, 2
MAX_COLS = 32768

STATUS_NAMES = {0: "MBP_OK", 1: "MBP_ERR_NULL", 2: "MBP_ERR_SHAPE", 3: "MBP_ERR_DTYPE",
                4: "MBP_ERR_ALIGN", 5: "MBP_ERR_OVERLAP", 6: "MBP_ERR_WORKSPACE",
                7: "MBP_ERR_HIP", 8: "MBP_ERR_ARG"}

# (name, restype, argtypes) of every symbol that include/mbp.h declares
_P, _I64, _D, _I, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double, ctypes.c_int, ctypes.c_size_t
_U64 = ctypes.c_uint64
SIGNATURES = [
    ("fused_pointwise_chain", _I, [_P, _P, _P, _P, _I64, _D, _P]),
    ("fused_row_mean_epilogue", _I, [_P, _P, _P, _P, _P, _I64, _I64, _D, _D, _P]),
    ("fused_add_layernorm_gelu", _I, [_I, _P, _P, _P, _P, _P, _I64, _I64, _D, _I, _P]),
    ("fused_softmax", _I, [_I, _P, _P, _I64, _I64, _P]),
    ("fused_softmax_2d", _I, [_I, _P, _I64, _P, _I64, _I64, _I64, _P]),
    ("fused_add_layernorm_gelu_2d", _I, [_I, _P, _I64, _P, _I64, _P, _P, _P, _I64, _I64, _I64, _D, _I, _P]),
    ("fused_layernorm_relu_dropout_2d", _I, [_I, _P, _I64, _P, _P, _P, _I64, _I64, _I64, _D, _D, _U64, _U64, _P]),
    ("fused_layernorm_relu_dropout", _I, [_I, _P, _P, _P, _P, _I64, _I64, _D, _D, _U64, _U64, _P]),
    ("unfused_layernorm_relu_dropout", _I, [_I, _P, _P, _P, _P, _I64, _I64, _D, _D, _U64, _U64, _P, _SZ, _P]),
    ("unfused_softmax", _I, [_I, _P, _P, _I64, _I64, _P, _SZ, _P]),
    ("fused_pointwise_chain_2d", _I, [_I, _P, _I64, _P, _I64, _P, _I64, _P, _I64, _I64, _I64, _D, _P]),
    ("fused_row_mean_epilogue_2d", _I, [_I, _P, _I64, _P, _P, _P, _P, _I64, _I64, _I64, _D, _D, _P]),
    ("unfused_pointwise_chain", _I, [_P, _P, _P, _P, _I64, _D, _P, _SZ, _P]),
    ("unfused_row_mean_epilogue", _I, [_P, _P, _P, _P, _P, _I64, _I64, _D, _D, _P, _SZ, _P]),
    ("grouped_row_mean_epilogue", _I, [_P, _P, _P, _P, _P, _I64, _I64, _D, _D, _P, _SZ, _P]),
    ("grouped_row_mean_epilogue_noalloc", _I, [_P, _P, _P, _P, _P, _I64, _I64, _D, _D, _P]),
    ("unfused_add_layernorm_gelu", _I, [_I, _P, _P, _P, _P, _P, _I64, _I64, _D, _I, _I, _P, _SZ, _P]),
    ("mbp_unfused_workspace_bytes", _SZ, [_I, _I, _I64, _I64, _I, _I, _I]),
    ("mbp_launches_per_call", _I, [_I, _I, _I, _I, _I]),
    ("mbp_graph_capture_begin", _I, [_P]),
    ("mbp_graph_capture_end", _I, [_P, ctypes.POINTER(_P)]),
    ("mbp_graph_launch", _I, [_P, _P]),
    ("mbp_graph_nodes", _I64, [_P]),
    ("mbp_graph_destroy", _I, [_P]),
    ("mbp_stream_copy", _I, [_P, _P, _SZ, _P]),
    ("mbp_stream_rw", _I, [ctypes.POINTER(_P), _I, _P, _SZ, _P]),
    ("mbp_convert_f32_to_bf16", _I, [_P, _P, _I64, _P]),
    ("mbp_status_string", ctypes.c_char_p, [_I]),
    ("mbp_last_error", ctypes.c_char_p, []),
    ("mbp_abi_version", _I, []),
]


class MbpError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)}: {detail}")
        self.status = status


def _load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(
            f"libmbp.so not found at {path}: build it first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _call(name: str, *args) -> None:
    st = getattr(lib, name)(*args)
    if st != 0:
        raise MbpError(name, st, lib.mbp_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(t, name, dtypes, device=None, strided=False):
    """type, device and dtype checks; dense unless `strided` (then any tensor
    _row_view accepts)"""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not strided and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dtype_code(t):
    return BF16 if t.dtype == torch.bfloat16 else F32


def _act_code(act):
    if act in (None, "none", ACT_NONE):
        return ACT_NONE
    if act in ("gelu_tanh", "gelu", ACT_GELU_TANH):
        return ACT_GELU_TANH
    raise ValueError(f"unknown act {act!r}")


def _rows_cols(x):
    if x.dim() < 1:
        raise ValueError("x must have at least one dimension")
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    return rows, cols


def _row_view(t, name):
    """(rows, cols, ld) of a tensor seen as [rows, cols] rows of its last
    dimension: the last dimension must be contiguous and the leading ones must
    collapse to one row stride ld (elements; 0 for a row expanded over the
    others).  A dense tensor has ld == cols."""
    if t.dim() < 1:
        raise ValueError(f"{name} must have at least one dimension")
    rows, cols = _rows_cols(t)
    if cols > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name}: the elements of a row must be contiguous (last stride 1)")
    if t.dim() == 1 or rows <= 1:
        return rows, cols, cols
    sizes, strides = t.shape[:-1], t.stride()[:-1]
    ld = None
    for i in range(len(sizes) - 1, -1, -1):  # innermost leading dimension first
        if sizes[i] == 1:
            continue
        if ld is None:
            ld = strides[i]
            span = ld * sizes[i]
        elif strides[i] != span:
            raise ValueError(f"{name}: the leading dimensions do not collapse to one row stride")
        else:
            span *= sizes[i]
    if ld != 0 and ld < cols:
        raise ValueError(f"{name}: rows overlap (row stride {ld} < {cols})")
    return rows, cols, ld


# ------------------------------------------------------------------ fused

def fused_pointwise_chain(x, b1, b2, scale=0.5, out=None):
    """y = relu(x + b1) * scale + b2 on fp32 tensors of one shape (one launch)."""
    for t, n in ((x, "x"), (b1, "b1"), (b2, "b2"), (out, "out")):
        _check(t, n, (torch.float32,), x.device)
    if not (x.shape == b1.shape == b2.shape):
        raise ValueError("x, b1, b2 must have the same shape")
    y = torch.empty_like(x) if out is None else out
    if y.shape != x.shape:
        raise ValueError("out has the wrong shape")
    _call("fused_pointwise_chain", _ptr(x), _ptr(b1), _ptr(b2), _ptr(y), x.numel(), float(scale),
          _stream(x))
    return y


def fused_row_mean_epilogue(x, bias, gamma, beta, alpha=1.1, c=0.1, out=None):
    """The 10-op graph: s = relu(x*alpha + bias)^2 + c*relu(...), y = (s - rowmean(s))*gamma + beta."""
    for t, n in ((x, "x"), (bias, "bias"), (gamma, "gamma"), (beta, "beta"), (out, "out")):
        _check(t, n, (torch.float32,), x.device)
    rows, cols = _rows_cols(x)
    for t, n in ((bias, "bias"), (gamma, "gamma"), (beta, "beta")):
        if t.numel() != cols:
            raise ValueError(f"{n} must have {cols} elements")
    y = torch.empty_like(x) if out is None else out
    if y.shape != x.shape:
        raise ValueError("out has the wrong shape")
    _call("fused_row_mean_epilogue", _ptr(x), _ptr(bias), _ptr(gamma), _ptr(beta), _ptr(y), rows,
          cols, float(alpha), float(c), _stream(x))
    return y


def fused_add_layernorm_gelu(x, residual, gamma, beta, eps=1e-5, act="gelu_tanh", out=None):
    """gelu_tanh(LayerNorm(x + residual) * gamma + beta) over the last dimension.

    fp32 or bf16 (all tensors one dtype); residual may be None; act "none"
    gives plain LayerNorm.  x, residual and out may be strided views whose
    rows are contiguous (e.g. x[:, :cols] of a wider buffer, or an expanded
    residual row): they are read and written in place through the row
    strides, never copied."""
    dts = (torch.float32, torch.bfloat16)
    _check(x, "x", dts, strided=True)
    for t, n in ((residual, "residual"), (out, "out")):
        _check(t, n, (x.dtype,), x.device, strided=True)
    for t, n in ((gamma, "gamma"), (beta, "beta")):
        _check(t, n, (x.dtype,), x.device)
    rows, cols, ldx = _row_view(x, "x")
    ldr = cols
    if residual is not None:
        if residual.shape != x.shape:
            raise ValueError("residual must have x's shape")
        ldr = _row_view(residual, "residual")[2]
    for t, n in ((gamma, "gamma"), (beta, "beta")):
        if t.numel() != cols:
            raise ValueError(f"{n} must have {cols} elements")
    y = torch.empty(x.shape, dtype=x.dtype, device=x.device) if out is None else out
    if y.shape != x.shape:
        raise ValueError("out has the wrong shape")
    ldy = _row_view(y, "out")[2]
    if ldx == ldr == ldy == cols:
        _call("fused_add_layernorm_gelu", _dtype_code(x), _ptr(x), _ptr(residual), _ptr(gamma),
              _ptr(beta), _ptr(y), rows, cols, float(eps), _act_code(act), _stream(x))
    else:
        _call("fused_add_layernorm_gelu_2d", _dtype_code(x), _ptr(x), ldx, _ptr(residual), ldr, _ptr(gamma),
              _ptr(beta), _ptr(y), ldy, rows, cols, float(eps), _act_code(act), _stream(x))
    return y


def fused_layernorm(x, gamma, beta, eps=1e-5, out=None):
    """Plain LayerNorm (no residual, no activation) over the last dimension."""
    return fused_add_layernorm_gelu(x, None, gamma, beta, eps=eps, act="none", out=out)


def _ln_drop_args(x, gamma, beta, out):
    dts = (torch.float32, torch.bfloat16)
    _check(x, "x", dts)
    for t, n in ((gamma, "gamma"), (beta, "beta"), (out, "out")):
        _check(t, n, (x.dtype,), x.device)
    rows, cols = _rows_cols(x)
    for t, n in ((gamma, "gamma"), (beta, "beta")):
        if t.numel() != cols:
            raise ValueError(f"{n} must have {cols} elements")
    y = torch.empty_like(x) if out is None else out
    if y.shape != x.shape:
        raise ValueError("out has the wrong shape")
    return rows, cols, y


def fused_layernorm_relu_dropout(x, gamma, beta, p=0.1, seed=0, offset=0, eps=1e-5, out=None):
    """dropout(relu(LayerNorm(x) * gamma + beta), p) over the last dimension,
    training semantics, one launch.  The mask is a function of (seed, offset,
    element index): Philox4x32-10, 16 bits per element.  x and out may be
    strided views whose rows are contiguous (the mask follows the element's
    position in the result, not its address)."""
    dts = (torch.float32, torch.bfloat16)
    _check(x, "x", dts, strided=True)
    _check(out, "out", (x.dtype,), x.device, strided=True)
    for t, n in ((gamma, "gamma"), (beta, "beta")):
        _check(t, n, (x.dtype,), x.device)
    rows, cols, ldx = _row_view(x, "x")
    for t, n in ((gamma, "gamma"), (beta, "beta")):
        if t.numel() != cols:
            raise ValueError(f"{n} must have {cols} elements")
    y = torch.empty(x.shape, dtype=x.dtype, device=x.device) if out is None else out
    if y.shape != x.shape:
        raise ValueError("out has the wrong shape")
    ldy = _row_view(y, "out")[2]
    seed, offset = int(seed) & (2 ** 64 - 1), int(offset) & (2 ** 64 - 1)
    if ldx == ldy == cols:
        _call("fused_layernorm_relu_dropout", _dtype_code(x), _ptr(x), _ptr(gamma), _ptr(beta), _ptr(y),
              rows, cols, float(eps), float(p), seed, offset, _stream(x))
    else:
        _call("fused_layernorm_relu_dropout_2d", _dtype_code(x), _ptr(x), ldx, _ptr(gamma), _ptr(beta), _ptr(y),
              ldy, rows, cols, float(eps), float(p), seed, offset, _stream(x))
    return y


def unfused_layernorm_relu_dropout(x, gamma, beta, p=0.1, seed=0, offset=0, eps=1e-5, out=None,
                                   workspace=None):
    """The same as three launches (layer_norm, relu, dropout) through HBM."""
    rows, cols, y = _ln_drop_args(x, gamma, beta, out)
    nb = workspace_bytes(OP_LN_RELU_DROPOUT, _dtype_code(x), rows, cols)
    ws = _workspace(nb, x.device, workspace)
    _call("unfused_layernorm_relu_dropout", _dtype_code(x), _ptr(x), _ptr(gamma), _ptr(beta), _ptr(y),
          rows, cols, float(eps), float(p), int(seed) & (2 ** 64 - 1), int(offset) & (2 ** 64 - 1),
          _ptr(ws), ws.numel() * ws.element_size(), _stream(x))
    return y


# ------------------------------------------------------------------ two-dimensional forms

_DTYPES_2D = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}


def _matrix(t, name, rows, cols, dtype, device, broadcast_ok):
    """(pointer, row stride in elements) of a [rows, cols] operand whose rows
    are contiguous.  A 1-D [cols] tensor, or a 2-D one whose row stride is 0
    (``expand``), is one row used for every row."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.dim() == 1:
        if t.shape[0] != cols or (cols > 1 and t.stride(0) != 1):
            raise ValueError(f"{name} must be [{cols}] with unit stride or [{rows}, {cols}]")
        ld = 0
    elif t.dim() == 2:
        if tuple(t.shape) != (rows, cols):
            raise ValueError(f"{name} must be [{rows}, {cols}] (got {tuple(t.shape)})")
        if cols > 1 and t.stride(1) != 1:
            raise ValueError(f"{name}: elements of a row must be contiguous (column stride 1)")
        ld = t.stride(0) if rows > 1 else 0
    else:
        raise ValueError(f"{name} must be 1-D or 2-D")
    if ld == 0 and rows > 1 and not broadcast_ok:
        raise ValueError(f"{name} cannot be a broadcast row")
    return t.data_ptr(), ld


def _out_2d(out, rows, cols, dtype, device):
    if out is None:
        out = torch.empty((rows, cols), dtype=dtype, device=device)
    ptr, ld = _matrix(out, "out", rows, cols, dtype, device, broadcast_ok=False)
    return out, ptr, (ld if rows > 1 else cols)


def fused_pointwise_chain_2d(x, b1, b2, scale=0.5, out=None):
    """y = relu(x + b1) * scale + b2 on [rows, cols] operands with any row
    stride (x, b1, b2 may be broadcast rows: 1-D or expanded), fp32 / bf16 /
    fp16 (one dtype).  Returns out, or a new dense [rows, cols] tensor."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.device.type != "cuda":
        raise ValueError("x must be a 2-D GPU tensor")
    if x.dtype not in _DTYPES_2D:
        raise TypeError(f"unsupported dtype {x.dtype}")
    rows, cols = x.shape
    args = [_matrix(t, n, rows, cols, x.dtype, x.device, True) for t, n in ((x, "x"), (b1, "b1"), (b2, "b2"))]
    y, yp, ldy = _out_2d(out, rows, cols, x.dtype, x.device)
    (xp, ldx), (ap, lda), (bp, ldb) = args
    _call("fused_pointwise_chain_2d", _DTYPES_2D[x.dtype], xp, ldx, ap, lda, bp, ldb, yp, ldy, rows, cols,
          float(scale), _stream(x))
    return y


def fused_row_mean_epilogue_2d(x, bias, gamma, beta, alpha=1.1, c=0.1, out=None):
    """The 10-op graph on a [rows, cols] x with any row stride, fp32 / bf16 /
    fp16 (every operand one dtype); bias, gamma, beta dense [cols]."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.device.type != "cuda":
        raise ValueError("x must be a 2-D GPU tensor")
    if x.dtype not in _DTYPES_2D:
        raise TypeError(f"unsupported dtype {x.dtype}")
    rows, cols = x.shape
    xp, ldx = _matrix(x, "x", rows, cols, x.dtype, x.device, True)
    vec = []
    for t, n in ((bias, "bias"), (gamma, "gamma"), (beta, "beta")):
        if not isinstance(t, torch.Tensor) or t.dim() != 1:
            raise ValueError(f"{n} must be a 1-D tensor of {cols} elements")
        vec.append(_matrix(t, n, rows, cols, x.dtype, x.device, True)[0])
    y, yp, ldy = _out_2d(out, rows, cols, x.dtype, x.device)
    _call("fused_row_mean_epilogue_2d", _DTYPES_2D[x.dtype], xp, ldx, vec[0], vec[1], vec[2], yp, ldy, rows,
          cols, float(alpha), float(c), _stream(x))
    return y


def fused_softmax(x, out=None):
    """Row softmax over the last dimension (fp32, bf16 or fp16; one launch).
    x and out may be strided views whose rows are contiguous."""
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    if x.dtype not in _DTYPES_2D:
        raise TypeError(f"unsupported dtype {x.dtype}")
    _check(x, "x", (x.dtype,), strided=True)
    _check(out, "out", (x.dtype,), x.device, strided=True)
    rows, cols, ldx = _row_view(x, "x")
    y = torch.empty(x.shape, dtype=x.dtype, device=x.device) if out is None else out
    if y.shape != x.shape:
        raise ValueError("out has the wrong shape")
    ldy = _row_view(y, "out")[2]
    if ldx == ldy == cols:
        _call("fused_softmax", _DTYPES_2D[x.dtype], _ptr(x), _ptr(y), rows, cols, _stream(x))
    else:
        _call("fused_softmax_2d", _DTYPES_2D[x.dtype], _ptr(x), ldx, _ptr(y), ldy, rows, cols, _stream(x))
    return y


# ------------------------------------------------------------------ unfused

def workspace_bytes(op, dtype, rows, cols, has_residual=False, act=ACT_NONE,
                    granularity=UNFUSED_PRIMITIVE):
    n = lib.mbp_unfused_workspace_bytes(op, dtype, rows, cols, int(bool(has_residual)),
                                        _act_code(act), granularity)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid arguments for workspace size")
    return n


def launches_per_call(op, fused, granularity=UNFUSED_PRIMITIVE, has_residual=False, act=ACT_NONE):
    return lib.mbp_launches_per_call(op, int(bool(fused)), granularity, int(bool(has_residual)),
                                     _act_code(act))


def _workspace(nbytes, device, workspace):
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    return workspace


def unfused_pointwise_chain(x, b1, b2, scale=0.5, out=None, workspace=None):
    """The chain as four launches (add, relu, mul, add) through HBM temporaries."""
    for t, n in ((x, "x"), (b1, "b1"), (b2, "b2"), (out, "out")):
        _check(t, n, (torch.float32,), x.device)
    y = torch.empty_like(x) if out is None else out
    nb = workspace_bytes(OP_CHAIN, F32, 1, x.numel())
    ws = _workspace(nb, x.device, workspace)
    _call("unfused_pointwise_chain", _ptr(x), _ptr(b1), _ptr(b2), _ptr(y), x.numel(), float(scale),
          _ptr(ws), ws.numel() * ws.element_size(), _stream(x))
    return y


def unfused_row_mean_epilogue(x, bias, gamma, beta, alpha=1.1, c=0.1, out=None, workspace=None):
    """The 10-op graph as ten launches through HBM temporaries."""
    for t, n in ((x, "x"), (bias, "bias"), (gamma, "gamma"), (beta, "beta"), (out, "out")):
        _check(t, n, (torch.float32,), x.device)
    rows, cols = _rows_cols(x)
    y = torch.empty_like(x) if out is None else out
    nb = workspace_bytes(OP_ROW_MEAN, F32, rows, cols)
    ws = _workspace(nb, x.device, workspace)
    _call("unfused_row_mean_epilogue", _ptr(x), _ptr(bias), _ptr(gamma), _ptr(beta), _ptr(y), rows,
          cols, float(alpha), float(c), _ptr(ws), ws.numel() * ws.element_size(), _stream(x))
    return y


def grouped_row_mean_epilogue(x, bias, gamma, beta, alpha=1.1, c=0.1, out=None, workspace=None):
    """The 10-op graph as TVM's three groups: prologue (s written), row mean,
    epilogue -- three launches, s through HBM."""
    for t, n in ((x, "x"), (bias, "bias"), (gamma, "gamma"), (beta, "beta"), (out, "out")):
        _check(t, n, (torch.float32,), x.device)
    rows, cols = _rows_cols(x)
    y = torch.empty_like(x) if out is None else out
    nb = workspace_bytes(OP_ROW_MEAN, F32, rows, cols, granularity=UNFUSED_GROUPED)
    ws = _workspace(nb, x.device, workspace)
    _call("grouped_row_mean_epilogue", _ptr(x), _ptr(bias), _ptr(gamma), _ptr(beta), _ptr(y), rows,
          cols, float(alpha), float(c), _ptr(ws), ws.numel() * ws.element_size(), _stream(x))
    return y


def grouped_row_mean_epilogue_noalloc(x, bias, gamma, beta, alpha=1.1, c=0.1, out=None):
    """grouped_row_mean_epilogue with s and m in the library's static scratch
    array (no workspace; the C call allocates nothing).  Pass ``out=`` to keep
    the whole call allocation-free."""
    for t, n in ((x, "x"), (bias, "bias"), (gamma, "gamma"), (beta, "beta"), (out, "out")):
        _check(t, n, (torch.float32,), x.device)
    rows, cols = _rows_cols(x)
    y = torch.empty_like(x) if out is None else out
    _call("grouped_row_mean_epilogue_noalloc", _ptr(x), _ptr(bias), _ptr(gamma), _ptr(beta), _ptr(y),
          rows, cols, float(alpha), float(c), _stream(x))
    return y


def unfused_softmax(x, out=None, workspace=None):
    """Row softmax as five eager launches (max, subtract, exp, sum, divide)
    through HBM temporaries; fp32 or bf16."""
    _check(x, "x", (torch.float32, torch.bfloat16))
    _check(out, "out", (x.dtype,), x.device)
    rows, cols = _rows_cols(x)
    y = torch.empty_like(x) if out is None else out
    if y.shape != x.shape:
        raise ValueError("out has the wrong shape")
    code = _dtype_code(x)
    nb = workspace_bytes(OP_SOFTMAX, code, rows, cols)
    ws = _workspace(nb, x.device, workspace)
    _call("unfused_softmax", code, _ptr(x), _ptr(y), rows, cols, _ptr(ws), ws.numel() * ws.element_size(),
          _stream(x))
    return y


def unfused_add_layernorm_gelu(x, residual, gamma, beta, eps=1e-5, act="gelu_tanh",
                               granularity=UNFUSED_PRIMITIVE, out=None, workspace=None):
    """Residual + LayerNorm + GeLU as one launch per op (granularity 0) or as
    add / layernorm / gelu launches (granularity 1)."""
    dts = (torch.float32, torch.bfloat16)
    _check(x, "x", dts)
    for t, n in ((residual, "residual"), (gamma, "gamma"), (beta, "beta"), (out, "out")):
        _check(t, n, (x.dtype,), x.device)
    rows, cols = _rows_cols(x)
    y = torch.empty_like(x) if out is None else out
    code = _act_code(act)
    nb = workspace_bytes(OP_LAYERNORM, _dtype_code(x), rows, cols, residual is not None, code,
                         granularity)
    ws = _workspace(nb, x.device, workspace)
    _call("unfused_add_layernorm_gelu", _dtype_code(x), _ptr(x), _ptr(residual), _ptr(gamma),
          _ptr(beta), _ptr(y), rows, cols, float(eps), code, granularity, _ptr(ws),
          ws.numel() * ws.element_size(), _stream(x))
    return y


# ------------------------------------------------------------------ graphs

def _stream_handle(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


class Graph:
    """An instantiated HIP graph of library calls (``mbp_graph_*``): replay it
    with ``launch``; ``close`` (or garbage collection) releases it."""

    def __init__(self, handle: int):
        self._h = handle

    @property
    def nodes(self) -> int:
        return int(lib.mbp_graph_nodes(self._h))

    def launch(self, stream=None) -> None:
        if self._h is None:
            raise ValueError("graph has been closed")
        _call("mbp_graph_launch", self._h, _stream_handle(stream))

    def close(self) -> None:
        h, self._h = self._h, None
        if h is not None:
            _call("mbp_graph_destroy", h)

    def __del__(self):
        with contextlib.suppress(Exception):
            self.close()


class capture:
    """Record the library calls made on ``stream`` (a created
    ``torch.cuda.Stream``, made current inside the block) into a ``Graph``,
    available as ``.graph`` after the block.  Inside the block nothing may
    allocate device memory: pass ``out=`` and ``workspace=`` to every call."""

    def __init__(self, stream: torch.cuda.Stream):
        if not isinstance(stream, torch.cuda.Stream) or stream.cuda_stream == 0:
            raise ValueError("capture needs a created torch.cuda.Stream")
        self.stream = stream
        self.graph = None
        self._ctx = None

    def __enter__(self):
        _call("mbp_graph_capture_begin", self.stream.cuda_stream)
        self._ctx = torch.cuda.stream(self.stream)
        self._ctx.__enter__()
        return self

    def __exit__(self, et, ev, tb):
        self._ctx.__exit__(et, ev, tb)
        h = _P()
        st = lib.mbp_graph_capture_end(self.stream.cuda_stream, ctypes.byref(h))
        if et is not None:  # the capture has ended; report the original error
            if st == 0:
                lib.mbp_graph_destroy(h)
            return False
        if st != 0:
            raise MbpError("mbp_graph_capture_end", st, lib.mbp_last_error().decode())
        self.graph = Graph(h.value)
        return False


def convert_f32_to_bf16(x, out=None):
    """fp32 -> bf16 with the kernels' store conversion (round to nearest even)."""
    _check(x, "x", (torch.float32,))
    _check(out, "out", (torch.bfloat16,), x.device)
    y = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device) if out is None else out
    if y.numel() != x.numel():
        raise ValueError("out has the wrong size")
    _call("mbp_convert_f32_to_bf16", _ptr(x), _ptr(y), x.numel(), _stream(x))
    return y


def stream_rw(srcs, dst):
    """dst = srcs[0] ^ srcs[1] ^ ... over dst's bytes: the bare stream of a
    kernel reading len(srcs) tensors and writing one (bandwidth floors)."""
    nbytes = dst.numel() * dst.element_size()
    for i, t in enumerate(srcs):
        _check(t, f"srcs[{i}]", (t.dtype,), dst.device)
        if t.numel() * t.element_size() < nbytes:
            raise ValueError(f"srcs[{i}] is smaller than dst")
    _check(dst, "dst", (dst.dtype,))
    arr = (_P * len(srcs))(*[t.data_ptr() for t in srcs])
    _call("mbp_stream_rw", arr, len(srcs), _ptr(dst), nbytes, _stream(dst))
    return dst


def stream_copy(src, dst):
    """Plain 128-bit streaming copy (bandwidth calibration)."""
    _check(src, "src", (src.dtype,))
    _check(dst, "dst", (dst.dtype,), src.device)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst is smaller than src")
    _call("mbp_stream_copy", _ptr(src), _ptr(dst), nbytes, _stream(src))
    return dst
