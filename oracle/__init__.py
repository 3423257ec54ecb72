"""Python access to the CPU oracle (oracle/oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers.  The product path
(``memory_bound_pointwise_amd``) never imports this package.

The oracle is plain C built with ``gcc -O2 -fno-fast-math -ffp-contract=off``
into ``oracle/liboracle.so``; this module only marshals numpy arrays into it.
All results come back as float64 arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

EXACT, SEQ, SEQ3 = 0, 1, 2
F32, BF16 = 0, 1
ACT_NONE, ACT_GELU_TANH = 0, 1

CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared"]


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle (always; the caller decides when)."""
    cmd = ["gcc", *CFLAGS, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib = None


def load(path: str | None = None):
    """Load liboracle.so, building it only when no build exists."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        _lib = _bind(ctypes.CDLL(LIB))
    return _lib


def _bind(lib):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    D = ctypes.c_double
    I = ctypes.c_int
    lib.oracle_pointwise_chain.argtypes = [P, P, P, I64, D, I, P]
    lib.oracle_pointwise_chain.restype = I
    lib.oracle_row_mean_epilogue.argtypes = [P, P, P, P, I64, I64, D, D, I, P]
    lib.oracle_row_mean_epilogue.restype = I
    lib.oracle_add_layernorm_gelu.argtypes = [I, P, P, P, P, I64, I64, D, I, I, P]
    lib.oracle_add_layernorm_gelu.restype = I
    lib.oracle_gelu_tanh.argtypes = [P, I64, P]
    lib.oracle_gelu_tanh.restype = None
    lib.oracle_to_bf16.argtypes = [P, I64, P]
    lib.oracle_to_bf16.restype = None
    lib.oracle_round_to_f16.argtypes = [P, I64, P]
    lib.oracle_round_to_f16.restype = None
    lib.oracle_round_to_bf16.argtypes = [P, I64, P]
    lib.oracle_round_to_bf16.restype = None
    lib.oracle_softmax.argtypes = [P, I64, I64, P]
    lib.oracle_softmax.restype = I
    lib.oracle_softmax_mode.argtypes = [I, P, I64, I64, I, P]
    lib.oracle_softmax_mode.restype = I
    lib.oracle_philox4x32_10.argtypes = [P, P, I64, P]
    lib.oracle_philox4x32_10.restype = None
    U32, U64 = ctypes.c_uint32, ctypes.c_uint64
    lib.oracle_ln_relu_dropout.argtypes = [I, P, P, P, I64, I64, D, U32, D, U64, U64, I64, I, P]
    lib.oracle_ln_relu_dropout.restype = I
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what}: oracle returned {rc}")


def pointwise_chain(x, b1, b2, scale=0.5, mode=EXACT, lib=None):
    lib = lib or load()
    x, b1, b2 = _f32(x), _f32(b1), _f32(b2)
    if not (x.shape == b1.shape == b2.shape):
        raise ValueError("shape mismatch")
    y = np.empty(x.shape, dtype=np.float64)
    _check(lib.oracle_pointwise_chain(_ptr(x), _ptr(b1), _ptr(b2), x.size, scale, mode, _ptr(y)),
           "pointwise_chain")
    return y


def row_mean_epilogue(x, bias, gamma, beta, alpha=1.1, c=0.1, mode=EXACT, lib=None):
    lib = lib or load()
    x = _f32(x)
    rows, cols = x.shape
    bias, gamma, beta = _f32(bias), _f32(gamma), _f32(beta)
    for v in (bias, gamma, beta):
        if v.shape != (cols,):
            raise ValueError("vector length must equal cols")
    y = np.empty((rows, cols), dtype=np.float64)
    _check(lib.oracle_row_mean_epilogue(_ptr(x), _ptr(bias), _ptr(gamma), _ptr(beta), rows, cols,
                                        alpha, c, mode, _ptr(y)), "row_mean_epilogue")
    return y


def add_layernorm_gelu(x, residual, gamma, beta, eps=1e-5, act=ACT_GELU_TANH, mode=EXACT, lib=None):
    """x, residual: [rows, cols]; float32 arrays (fp32 I/O) or uint16 arrays holding
    bfloat16 bit patterns (bf16 I/O).  residual may be None."""
    lib = lib or load()
    if x.dtype == np.uint16:
        dt, cast = BF16, (lambda a: np.ascontiguousarray(a, dtype=np.uint16))
    elif x.dtype == np.float32:
        dt, cast = F32, _f32
    else:
        raise TypeError("x must be float32 or uint16 (bf16 bits)")
    x = cast(x)
    rows, cols = x.shape
    r = None if residual is None else cast(residual)
    if r is not None and r.shape != x.shape:
        raise ValueError("residual shape mismatch")
    g, b = cast(gamma), cast(beta)
    if g.shape != (cols,) or b.shape != (cols,):
        raise ValueError("gamma/beta length must equal cols")
    y = np.empty((rows, cols), dtype=np.float64)
    _check(lib.oracle_add_layernorm_gelu(dt, _ptr(x), _ptr(r), _ptr(g), _ptr(b), rows, cols, eps,
                                         act, mode, _ptr(y)), "add_layernorm_gelu")
    return y


def gelu_tanh(u, lib=None):
    lib = lib or load()
    u = np.ascontiguousarray(u, dtype=np.float64)
    out = np.empty_like(u)
    lib.oracle_gelu_tanh(_ptr(u), u.size, _ptr(out))
    return out


def to_bf16(x, lib=None):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    lib = lib or load()
    x = _f32(x)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.oracle_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


def round_bits(x, fmt, lib=None):
    """float64 -> bit patterns (uint16) of binary16 ("f16") or bfloat16
    ("bf16"), rounded once to nearest even directly from binary64."""
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    fn = {"f16": lib.oracle_round_to_f16, "bf16": lib.oracle_round_to_bf16}[fmt]
    fn(_ptr(x), x.size, _ptr(out))
    return out


def softmax(x, mode=EXACT, dtype="f32", lib=None):
    """Row softmax over the last dimension of a 2-D array of stored values
    (float32; 16-bit inputs widened to float32 first).  mode SEQ: as eager
    one-op kernels storing `dtype` ("f32" or "bf16") evaluate it."""
    lib = lib or load()
    x = _f32(x)
    if x.ndim != 2:
        raise ValueError("x must be 2-D")
    y = np.empty(x.shape, dtype=np.float64)
    dt = {"f32": F32, "bf16": BF16}[dtype]
    _check(lib.oracle_softmax_mode(dt, _ptr(x), x.shape[0], x.shape[1], mode, _ptr(y)), "softmax")
    return y


def philox4x32_10(ctr, key, lib=None):
    """Philox4x32-10 blocks: ctr [n, 4] uint32, key [n, 2] uint32 -> [n, 4] uint32."""
    lib = lib or load()
    ctr = np.ascontiguousarray(ctr, dtype=np.uint32).reshape(-1, 4)
    key = np.ascontiguousarray(key, dtype=np.uint32).reshape(-1, 2)
    out = np.empty_like(ctr)
    lib.oracle_philox4x32_10(_ptr(ctr), _ptr(key), ctr.shape[0], _ptr(out))
    return out


def dropout_threshold(p):
    """(threshold, scale) of drop probability p: an element is dropped when
    its 16 random bits are below round(p * 2^16); kept ones are scaled by
    1 / (1 - p)."""
    if not 0.0 <= p <= 1.0:
        raise ValueError("p must be in [0, 1]")
    t = int(round(p * 65536.0))
    scale = 0.0 if p == 1.0 else 1.0 / (1.0 - p)
    return t, scale


def ln_relu_dropout(x, gamma, beta, p=0.1, seed=0, offset=0, eps=1e-5, mode=EXACT, first_row=0, lib=None):
    """LayerNorm -> ReLU -> Dropout (training semantics) over the last dimension.
    x may be rows [first_row, first_row + len(x)) of a larger tensor: the
    element indices that pick the random bits are those of that tensor."""
    lib = lib or load()
    if x.dtype == np.uint16:
        dtype, cast = BF16, (lambda a: np.ascontiguousarray(a, dtype=np.uint16))
    elif x.dtype == np.float32:
        dtype, cast = F32, _f32
    else:
        raise TypeError("x must be float32 or uint16 (bf16 bits)")
    x, gamma, beta = cast(x), cast(gamma), cast(beta)
    rows, cols = x.shape
    if gamma.shape != (cols,) or beta.shape != (cols,):
        raise ValueError("gamma/beta length must equal cols")
    t, scale = dropout_threshold(p)
    y = np.empty((rows, cols), dtype=np.float64)
    _check(lib.oracle_ln_relu_dropout(dtype, _ptr(x), _ptr(gamma), _ptr(beta), rows, cols, eps, t,
                                      scale, seed, offset, first_row, mode, _ptr(y)), "ln_relu_dropout")
    return y
