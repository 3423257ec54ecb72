"""Seeded synthetic inputs for every workload of the fused memory-bound chains.

This module holds the workload shapes and the input recipe, and nothing of the
methods' arithmetic.  Both sides use it: the tests and the bench feed the same
arrays to the HIP library (through the binding) and to the CPU oracle.

Recipe (numpy ``PCG64`` streams keyed by ``SeedSequence``; tensor k in
argument order draws vectors from key (seed, sub, k) and each block of about
2**20 elements of whole rows from key (seed, sub, k, block), so blocks are
drawn in parallel threads with the same result as sequentially):

* standard normals are drawn as float32 (numpy's float32 ziggurat) and scaled
  by an exact power of two where the workload asks for std 2;
* parameter vectors (bias, gamma, beta) and per-row offsets are drawn in
  float64 and rounded once to the storage type;
* bfloat16 values are produced from float32 by round-to-nearest-even on the
  dropped 16 bits and handled as uint16 bit patterns; binary16 values by
  numpy's float32 -> float16 conversion (round to nearest even).

The shapes and distributions are those the pages use: ``randn`` tensors for the
pointwise chain (PyTorch operator-fusion practice post, section 3.1), the 10-op
model's f32[1024,1024] and f32[1024] (TorchInductor Pipeline 与算子融合, the
example at the top of the post), and LayerNorm rows; the LayerNorm offsets
U(-100, 100) per row, gamma ~ N(1, 0.1), beta ~ N(0, 0.1) and the hidden-size
sweep are the workload definitions this library is measured on.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "chain" | "row_mean" | "layernorm" | "chain2d" | "row_mean2d" | "softmax"
    #                      | "ln_relu_dropout" | "layernorm2d" (layernorm on padded rows)
    seed: int
    sub: int = 0
    n: int = 0           # chain: element count
    rows: int = 0
    cols: int = 0
    dtype: str = "f32"   # "f32", "bf16" (layernorm, 2-D forms) or "f16" (2-D forms)
    residual: bool = False
    act: str = "none"    # "none" | "gelu_tanh"
    std: float = 1.0     # std of x (and residual) for bf16 layernorm
    params: dict = field(default_factory=dict)

    @property
    def elems(self) -> int:
        return self.n if self.kind == "chain" else self.rows * self.cols

    @property
    def compulsory_bytes(self) -> int:
        """Bytes the fused kernel must move: each input read once, output written once."""
        if self.kind == "chain":
            return 4 * 4 * self.n                      # x, b1, b2 in; y out (fp32)
        if self.kind == "row_mean":
            return 4 * 2 * self.rows * self.cols + 4 * 3 * self.cols   # x in, y out; bias/gamma/beta
        es = 4 if self.dtype == "f32" else 2
        if self.kind == "chain2d":
            return es * (3 * self.rows * self.cols + self.cols)        # x, b2 in, y out; b1 one row
        if self.kind == "row_mean2d":
            return es * (2 * self.rows * self.cols + 3 * self.cols)    # x in, y out; bias/gamma/beta
        if self.kind == "softmax":
            return es * 2 * self.rows * self.cols                      # x in, y out
        if self.kind == "ln_relu_dropout":
            return es * (2 * self.rows * self.cols + 2 * self.cols)    # x in, y out; gamma, beta
        es = 2 if self.dtype == "bf16" else 4
        tensors = 3 if self.residual else 2           # x (+ residual) in, y out
        return es * tensors * self.rows * self.cols + es * 2 * self.cols   # + gamma, beta


WORKLOADS = [
    Workload("chain_4M_f32", "chain", seed=1, n=4 * 1024 * 1024, params=dict(scale=0.5)),
    Workload("tenop_1024x1024_f32", "row_mean", seed=2, rows=1024, cols=1024,
             params=dict(alpha=1.1, c=0.1)),
    Workload("ln_8192x4096_f32", "layernorm", seed=3, rows=8192, cols=4096, dtype="f32",
             params=dict(eps=1e-5)),
    Workload("addln_gelu_16384x8192_bf16", "layernorm", seed=4, rows=16384, cols=8192,
             dtype="bf16", residual=True, act="gelu_tanh", params=dict(eps=1e-5)),
    Workload("addln_gelu_262144x768_bf16", "layernorm", seed=5, sub=1, rows=262144, cols=768,
             dtype="bf16", residual=True, act="gelu_tanh", std=2.0, params=dict(eps=1e-5)),
    Workload("addln_gelu_32768x4095_bf16", "layernorm", seed=5, sub=2, rows=32768, cols=4095,
             dtype="bf16", residual=True, act="gelu_tanh", std=2.0, params=dict(eps=1e-5)),
    Workload("addln_gelu_16384x12288_bf16", "layernorm", seed=5, sub=3, rows=16384, cols=12288,
             dtype="bf16", residual=True, act="gelu_tanh", std=2.0, params=dict(eps=1e-5)),
]
BY_NAME = {w.name: w for w in WORKLOADS}

# The two-dimensional forms (16-bit storage, broadcast rows, row strides):
# measured beside the workloads above, not part of the headline figure.
#   chain2d: x [rows, cols] and b2 [rows, cols] dense, b1 one row [cols] used
#            for every row (stride 0), y dense; bf16.
#   row_mean2d: x and y [rows, cols] inside rows of params["ld"] elements
#            (padded rows), bias / gamma / beta [cols]; fp16.
#   softmax: x [rows, cols] ~ N(0, 1), y dense; bf16.
NEXT_WORKLOADS = [
    Workload("chain2d_16384x4096_bf16_bcast", "chain2d", seed=6, rows=16384, cols=4096, dtype="bf16",
             params=dict(scale=0.5)),
    Workload("tenop2d_8192x1024_f16_ld1056", "row_mean2d", seed=7, rows=8192, cols=1024, dtype="f16",
             params=dict(alpha=1.1, c=0.1, ld=1056)),
    # row softmax at the attention-probability shape of the PyTorch
    # operator-fusion practice post, section 4.1 (batch 1, 32 heads,
    # seq_len 4096: probs of 32 x 4096 x 4096, i.e. 131072 rows of 4096)
    Workload("softmax_131072x4096_bf16", "softmax", seed=8, rows=131072, cols=4096, dtype="bf16"),
    # LayerNorm -> ReLU -> Dropout (p = 0.1 as in "算子融合与 Kernel 优化", section
    # 2.1) at the residual-LayerNorm workload's shape, without the residual
    Workload("ln_relu_dropout_16384x8192_bf16", "ln_relu_dropout", seed=4, rows=16384, cols=8192,
             dtype="bf16", params=dict(eps=1e-5, p=0.1, seed=0x5EED, offset=0)),
    # residual + LayerNorm + GeLU on padded rows, read and written through
    # the row strides (the PyTorch operator-fusion practice post, section 6.2:
    # no hidden .contiguous() copy): the residual-LayerNorm workload's inputs
    # with x, residual and y each a [16384, 8192] view into a buffer of rows of
    # params["ld"] elements -- 8320 keeps every row on a 128-byte line, 8195
    # puts them off 16-byte boundaries (one stride for the three)
    Workload("addln_gelu_16384x8192_bf16_ld8320", "layernorm2d", seed=4, rows=16384, cols=8192,
             dtype="bf16", residual=True, act="gelu_tanh", params=dict(eps=1e-5, ld=8320)),
    Workload("addln_gelu_16384x8192_bf16_ld8195", "layernorm2d", seed=4, rows=16384, cols=8192,
             dtype="bf16", residual=True, act="gelu_tanh", params=dict(eps=1e-5, ld=8195)),
]
NEXT_BY_NAME = {w.name: w for w in NEXT_WORKLOADS}


def scaled(w: Workload, rows: int | None = None, n: int | None = None) -> Workload:
    """The same workload at another size (tests use small and ragged sizes)."""
    from dataclasses import replace
    if w.kind == "chain":
        return replace(w, name=f"{w.name}@n{n}", n=n)
    return replace(w, name=f"{w.name}@r{rows}", rows=rows)


BLOCK_ELEMS = 1 << 20
_THREADS = 8


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _blocks(rows: int, cols: int):
    """Row blocks of about BLOCK_ELEMS elements; block b covers rows [lo, hi)."""
    per = max(1, BLOCK_ELEMS // max(cols, 1))
    return [(b, lo, min(rows, lo + per)) for b, lo in enumerate(range(0, rows, per))]


def _parallel(fn, items):
    items = list(items)
    if len(items) <= 1:
        for it in items:
            fn(it)
        return
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(min(_THREADS, len(items))) as ex:
        list(ex.map(fn, items))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even (no NaNs arise here)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    flat = a.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)

    def work(span):
        lo, hi = span
        u = flat[lo:hi].view(np.uint32)
        t = u >> np.uint32(16)
        t &= np.uint32(1)
        t += np.uint32(0x7FFF)
        t += u
        t >>= np.uint32(16)
        out[lo:hi] = t

    _parallel(work, [(lo, min(flat.size, lo + BLOCK_ELEMS)) for lo in range(0, flat.size, BLOCK_ELEMS)])
    return out.reshape(a.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_f32(key, rows: int, cols: int, std: float = 1.0, offsets=None) -> np.ndarray:
    """[rows, cols] float32 standard normals (times std, plus a per-row offset),
    each row block drawn from its own stream key + (block,)."""
    out = np.empty((rows, cols), dtype=np.float32)

    def work(blk):
        b, lo, hi = blk
        g = _rng(*key, b)
        view = out[lo:hi]
        g.standard_normal(out=view, dtype=np.float32)
        if std != 1.0:
            view *= np.float32(std)
        if offsets is not None:
            view[...] = (view.astype(np.float64) + offsets[lo:hi, None]).astype(np.float32)

    _parallel(work, _blocks(rows, cols))
    return out


def store(a: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values in a storage type: bf16 as uint16 bit patterns, f16 as
    numpy float16 (both round to nearest even)."""
    if dtype == "bf16":
        return f32_to_bf16_bits(a)
    if dtype == "f16":
        return np.asarray(a, dtype=np.float32).astype(np.float16)
    return np.asarray(a, dtype=np.float32)


def generate(w: Workload, cols: int | None = None) -> dict:
    """Inputs of workload ``w`` as host numpy arrays (``cols`` overrides the width).

    Tensor k (argument order) of a workload with seed s and sub-index u uses the
    stream keys (s, u, k) for vectors and (s, u, k, block) for row blocks."""
    s, u = w.seed, w.sub
    if w.kind == "chain":
        x, b1, b2 = (_normal_f32((s, u, k), 1, w.n).reshape(-1) if w.n else np.empty(0, np.float32)
                     for k in range(3))
        return dict(x=x, b1=b1, b2=b2)
    rows, c = w.rows, cols or w.cols
    if w.kind == "chain2d":
        return dict(x=store(_normal_f32((s, u, 0), rows, c), w.dtype),
                    b1=store(_rng(s, u, 1).standard_normal(c).astype(np.float32), w.dtype),
                    b2=store(_normal_f32((s, u, 2), rows, c), w.dtype))
    if w.kind == "softmax":
        return dict(x=store(_normal_f32((s, u, 0), rows, c), w.dtype))
    if w.kind == "ln_relu_dropout":
        g64 = 1.0 + 0.1 * _rng(s, u, 2).standard_normal(c)
        b64 = 0.1 * _rng(s, u, 3).standard_normal(c)
        return dict(x=store(_normal_f32((s, u, 0), rows, c), w.dtype),
                    gamma=store(g64.astype(np.float32), w.dtype), beta=store(b64.astype(np.float32), w.dtype))
    if w.kind == "row_mean2d":
        return dict(x=store(_normal_f32((s, u, 0), rows, c), w.dtype),
                    **{k: store(_rng(s, u, i + 1).standard_normal(c).astype(np.float32), w.dtype)
                       for i, k in enumerate(("bias", "gamma", "beta"))})
    if w.kind == "row_mean":
        return dict(x=_normal_f32((s, u, 0), rows, c),
                    bias=_rng(s, u, 1).standard_normal(c).astype(np.float32),
                    gamma=_rng(s, u, 2).standard_normal(c).astype(np.float32),
                    beta=_rng(s, u, 3).standard_normal(c).astype(np.float32))
    gamma64 = 1.0 + 0.1 * _rng(s, u, 2).standard_normal(c)
    beta64 = 0.1 * _rng(s, u, 3).standard_normal(c)
    if w.dtype == "f32":
        off = _rng(s, u, 4).uniform(-100.0, 100.0, size=rows)
        x = _normal_f32((s, u, 0), rows, c, offsets=off)
        r = _normal_f32((s, u, 1), rows, c) if w.residual else None
        return dict(x=x, residual=r, gamma=gamma64.astype(np.float32), beta=beta64.astype(np.float32))
    x = f32_to_bf16_bits(_normal_f32((s, u, 0), rows, c, std=w.std))
    r = f32_to_bf16_bits(_normal_f32((s, u, 1), rows, c, std=w.std)) if w.residual else None
    return dict(x=x, residual=r,
                gamma=f32_to_bf16_bits(gamma64.astype(np.float32)),
                beta=f32_to_bf16_bits(beta64.astype(np.float32)))


def to_device(a, device="cuda"):
    """Copy a host array to a torch tensor on `device` (bf16 bit patterns become
    a bfloat16 tensor).  None passes through."""
    if a is None:
        return None
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)
