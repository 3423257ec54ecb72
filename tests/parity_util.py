"""Helpers of the GPU parity tests: moving the seeded inputs to the device,
and the comparison gates.

Gates (fused kernels against the oracle's binary64 result):
* pointwise chain: at most 2 ulp between the fp32 output and the exact result
  rounded to fp32 (ulp distance on the ordered integer line, +0 == -0);
* fp32 row kernels: |y - exact| <= max(1e-5, half an fp32 ulp of exact);
* bf16 row kernels: |y - exact| <= max(2e-2, half a bf16 ulp of exact).
The half-ulp term only matters where no output of the storage type can be
within 1e-5 (|exact| >= 256 in fp32) or 2e-2 (|exact| >= 8 in bf16) of the
exact value; those elements are counted and reported.
"""
from __future__ import annotations

import numpy as np
import torch

import workloads as W


def to_dev(a, dev="cuda"):
    return W.to_device(a, dev)


def to_host(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(a):
    if a.dtype == np.uint16:
        return W.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def ordered(a32):
    i = np.ascontiguousarray(a32, dtype=np.float32).view(np.int32).astype(np.int64)
    return np.where(i < 0, -(i & 0x7FFFFFFF), i)


def ulp_distance(a32, b32):
    return np.abs(ordered(a32) - ordered(b32))


def half_ulp(exact, mant_bits):
    _, e = np.frexp(np.abs(exact))
    return np.ldexp(1.0, e - 1 - mant_bits) / 2


def check_chain(y32, exact, what=""):
    d = ulp_distance(y32, exact.astype(np.float32))
    nan_ok = np.isnan(y32) == np.isnan(exact)
    assert nan_ok.all(), f"{what}: NaN mismatch"
    d = np.where(np.isnan(exact), 0, d)
    assert d.max(initial=0) <= 2, f"{what}: max {d.max()} ulp at {np.argmax(d)}"
    return int(d.max(initial=0))


def check_abs(y, exact, tol, mant_bits, what=""):
    y = as_f64(y)
    err = np.abs(y - exact)
    lim = np.maximum(tol, half_ulp(exact, mant_bits) * (1 + 2.0 ** -10))
    bad = ~(err <= lim)
    bad &= ~(np.isnan(y) & np.isnan(exact))
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements over the gate; max err "
                           f"{np.nanmax(err):.3g}, first at {np.argwhere(bad)[:3].tolist()}")
    relaxed = int((half_ulp(exact, mant_bits) > tol).sum())
    return float(np.nanmax(err, initial=0.0)), relaxed


def check_f32(y, exact, what=""):
    return check_abs(y, exact, 1e-5, 23, what)


def check_bf16(y, exact, what=""):
    return check_abs(y, exact, 2e-2, 7, what)


def sample_rows(rows, k=48, seed=7):
    r = np.random.default_rng(seed)
    pick = set([0, 1, rows - 1, rows - 2]) | set(r.integers(0, rows, size=k).tolist())
    return np.array(sorted(p for p in pick if 0 <= p < rows))
