"""Helpers of the GPU parity tests: moving the seeded inputs to the device,
and the comparison gates.

Gates (fused kernels against the oracle's binary64 result):
* pointwise chain: at most 2 ulp between the fp32 output and the exact result
  rounded to fp32 (ulp distance on the ordered integer line, +0 == -0);
* fp32 row kernels: |y - exact| <= max(1e-5, half an fp32 ulp of exact);
* bf16 row kernels: |y - exact| <= max(2e-2, half a bf16 ulp of exact);
* 16-bit outputs of the two-dimensional forms (binary64 inside, one rounding
  at the store): at most 1 ulp, on the ordered bit line, from the exact result
  rounded once to the format by the oracle;
* fp32 softmax: relative to the exact probability, with a bound derived from
  the kernel's fp32 arithmetic and the row's input range (check_softmax_f32).
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


def bits16(t):
    """bit patterns (uint16) of a bf16 / fp16 device tensor"""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def ordered16(b):
    i = np.asarray(b).astype(np.int64)
    return np.where(i & 0x8000, -(i & 0x7FFF), i)


def is_nan16(b, fmt):
    b = np.asarray(b).astype(np.int64)
    e, m = (0x7C00, 0x3FF) if fmt == "f16" else (0x7F80, 0x7F)
    return ((b & e) == e) & ((b & m) != 0)


def check_ulp16(bits, exact, fmt, what=""):
    import oracle
    want = oracle.round_bits(exact, fmt)
    nan_e, nan_y = np.isnan(exact), is_nan16(bits, fmt)
    assert (nan_e == nan_y).all(), f"{what}: NaN mismatch"
    d = np.where(nan_e, 0, np.abs(ordered16(bits) - ordered16(want)))
    assert d.max(initial=0) <= 1, f"{what}: max {d.max()} ulp at {np.unravel_index(np.argmax(d), d.shape)}"
    return int(d.max(initial=0)), int((d > 0).sum())


def check_softmax_f32(y, exact, x, what=""):
    """fp32 softmax: |y - e| <= (192 + 8 R) 2^-24 e + 2^-125 per element, R the
    range (max - min) of the row's finite inputs.  The kernel's output is
    exp2((x - m_lane) log2e) * (exp2((m_lane - m) log2e) / l) in fp32: rounding
    the difference and its product with log2e moves each exponential by at
    most 3 2^-24 times its argument, and along any term's chain of rescalings
    the arguments add up to m - x <= R (6 R for the element and for l
    together); each v_exp_f32 adds 2 ulp, the per-lane sum at most 64
    roundings, the (at most 21) merges 4 each, the divide and the product 2.
    Subnormal results may flush: the 2^-125 floor.  Returns the largest error
    in units of 2^-24 e and the largest error / bound."""
    yh = np.asarray(y, np.float64)
    x = np.asarray(x, np.float64)
    assert yh.shape == exact.shape == x.shape
    nan_e = np.isnan(exact)
    assert (np.isnan(yh) == nan_e).all(), f"{what}: NaN mismatch"
    fin = np.where(np.isfinite(x), x, np.nan)
    with np.errstate(all="ignore"):
        rng_ = np.nanmax(fin, axis=1, keepdims=True) - np.nanmin(fin, axis=1, keepdims=True)
    rng_ = np.where(np.isnan(rng_), 0.0, rng_)
    u = 2.0 ** -24
    err = np.where(nan_e, 0.0, np.abs(yh - exact))
    bound = (192.0 + 8.0 * rng_) * u * np.abs(np.where(nan_e, 0.0, exact)) + 2.0 ** -125
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements over the gate, first at "
                           f"{np.argwhere(bad)[:3].tolist()}: err {err[bad][:3]}, bound {bound[bad][:3]}")
    with np.errstate(all="ignore"):
        rel = np.where(exact > 0, err / (u * np.abs(exact)), 0.0)
    return float(np.nanmax(rel, initial=0.0)), float(np.max(err / bound, initial=0.0))


def sample_rows(rows, k=48, seed=7):
    r = np.random.default_rng(seed)
    pick = set([0, 1, rows - 1, rows - 2]) | set(r.integers(0, rows, size=k).tolist())
    return np.array(sorted(p for p in pick if 0 <= p < rows))
