"""CPU float64 oracle for batched weighted isotonic regression (ctypes binding).

TEST INFRASTRUCTURE ONLY: the checker, not the product.  Only the test suite,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this module.  It shares no code with the GPU library and never imports it.

The arithmetic lives in ``iso_oracle.c`` (pool adjacent violators in float64,
page "Merge Hulls Without Copying Vertices: GPU Isotonic Regression", Sec. 1
and Sec. 2.1 Eq. (1); semantics from the "torchisotonic" PyPI page, section
"Semantics").  This module only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "iso_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK = 0
EINVAL = -1
EWEIGHT = -3


def build() -> str:
    """Compile liboracle.so with gcc (plain C, no fast-math, no FMA contraction)."""
    cmd = [
        "gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared",
        "-pthread", "-o", _LIB + ".tmp", _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        bp = ctypes.POINTER(ctypes.c_uint8)
        lib.iso_oracle_fit.restype = ctypes.c_int
        lib.iso_oracle_fit.argtypes = [
            dp, dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_double,
            dp, bp, bp, bp, ctypes.c_int,
        ]
        lib.iso_oracle_vjp.restype = ctypes.c_int
        lib.iso_oracle_vjp.argtypes = [dp, bp, bp, bp, dp, ctypes.c_int64, ctypes.c_int64, dp]
        lib.iso_oracle_vjp_w.restype = ctypes.c_int
        lib.iso_oracle_vjp_w.argtypes = [dp, dp, bp, bp, bp, dp, ctypes.c_int64, ctypes.c_int64, dp]
        _lib = lib
    return _lib


def _dptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _bptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


def _as2d(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if a.ndim == 1:
        a = a[None, :]
    return a


def fit(y, w=None, increasing=True, y_min=None, y_max=None, threads=1):
    """Fit every row of y.  Returns (z, block_start, clipped, row_nan, status).

    y, w: array-like [rows, n] or [n] (cast to float64 exactly for float32 data).
    z has the shape of the 2-D view; block_start / clipped are uint8 [rows, n];
    row_nan is uint8 [rows]; status is OK or EWEIGHT (rows with a finite weight
    <= 0 are NaN).
    """
    lib = _load()
    y2 = _as2d(y)
    rows, n = y2.shape
    w2 = None
    if w is not None:
        w2 = _as2d(w)
        if w2.shape != y2.shape:
            raise ValueError("w must have the shape of y")
    lo = -np.inf if y_min is None else float(y_min)
    hi = np.inf if y_max is None else float(y_max)
    z = np.empty((rows, n), dtype=np.float64)
    bs = np.empty((rows, n), dtype=np.uint8)
    cl = np.empty((rows, n), dtype=np.uint8)
    rn = np.zeros(rows, dtype=np.uint8)
    st = lib.iso_oracle_fit(_dptr(y2), _dptr(w2), rows, n, 1 if increasing else 0, lo, hi,
                            _dptr(z), _bptr(bs), _bptr(cl), _bptr(rn), int(threads))
    if st == EINVAL:
        raise ValueError("invalid arguments")
    return z, bs, cl, rn, st


def vjp(g, block_start, clipped=None, row_nan=None, w=None):
    """grad_y = w_j * sum_{i in B(j)} g_i [not clipped_i] / W_B over the given partition."""
    lib = _load()
    g2 = _as2d(g)
    rows, n = g2.shape
    bs = np.ascontiguousarray(np.asarray(block_start, dtype=np.uint8).reshape(rows, n))
    cl = None if clipped is None else np.ascontiguousarray(np.asarray(clipped, dtype=np.uint8).reshape(rows, n))
    rn = None if row_nan is None else np.ascontiguousarray(np.asarray(row_nan, dtype=np.uint8).reshape(rows))
    w2 = None if w is None else _as2d(w)
    out = np.empty((rows, n), dtype=np.float64)
    st = lib.iso_oracle_vjp(_dptr(g2), _bptr(bs), _bptr(cl), _bptr(rn), _dptr(w2), rows, n, _dptr(out))
    if st != OK:
        raise ValueError("invalid arguments")
    return out


def vjp_w(g, y, block_start, clipped=None, row_nan=None, w=None):
    """grad_w = (sum_{i in B(j)} g_i [not clipped_i]) * (y_j - mean_B) / W_B over the given partition
    (page "torchisotonic", "Semantics": the fit is differentiable in the weights)."""
    lib = _load()
    g2 = _as2d(g)
    rows, n = g2.shape
    y2 = _as2d(y)
    bs = np.ascontiguousarray(np.asarray(block_start, dtype=np.uint8).reshape(rows, n))
    cl = None if clipped is None else np.ascontiguousarray(np.asarray(clipped, dtype=np.uint8).reshape(rows, n))
    rn = None if row_nan is None else np.ascontiguousarray(np.asarray(row_nan, dtype=np.uint8).reshape(rows))
    w2 = None if w is None else _as2d(w)
    out = np.empty((rows, n), dtype=np.float64)
    st = lib.iso_oracle_vjp_w(_dptr(g2), _dptr(y2), _bptr(bs), _bptr(cl), _bptr(rn), _dptr(w2), rows, n,
                              _dptr(out))
    if st != OK:
        raise ValueError("invalid arguments")
    return out


def soft_rank(x, eps=1.0):
    """Soft rank with quadratic regularization (first page, Sec. 7.9): theta = x / eps is sorted in
    decreasing order into s, the non-increasing fit v of z = s - (n, n-1, ..., 1) is computed with unit
    weights, and the rank of the element at sorted position i is s_i - v_i, put back in the original order.

    The order of theta is the order of x (eps > 0), so x itself is sorted; equal values keep their index
    order (any order gives the same ranks: equal s_i pool into one block).  Returns
    (r, perm, block_start, row_nan): perm[r, i] is the index of the element at sorted position i, and
    block_start / row_nan describe the fit's partition over the sorted positions.  A row holding a NaN
    comes back NaN.
    """
    x2 = _as2d(x)
    rows, n = x2.shape
    if not (eps > 0 and np.isfinite(eps)):
        raise ValueError("eps must be positive and finite")
    perm = np.argsort(-x2, axis=1, kind="stable")
    s = np.take_along_axis(x2, perm, axis=1) / eps
    z = s - np.arange(n, 0, -1, dtype=np.float64)[None, :]
    v, bs, _cl, rn, _st = fit(z, None, increasing=False)
    r = np.empty_like(x2)
    np.put_along_axis(r, perm, s - v, axis=1)
    return r, perm, bs, rn


def soft_rank_vjp(g, eps, perm, block_start, row_nan=None):
    """Vector-Jacobian product of soft_rank in x: with g_s the upstream gradient in sorted order and A the
    block averaging of the fit (unit weights), d/dx = P^T (g_s - A g_s) / eps, P the sorting permutation."""
    g2 = _as2d(g)
    gs = np.take_along_axis(g2, perm, axis=1)
    ags = vjp(gs, block_start, None, row_nan)
    out = np.empty_like(g2)
    np.put_along_axis(out, perm, (gs - ags) / eps, axis=1)
    return out


def calibration_fit(scores, labels):
    """Calibration curve of each row (first page, Sec. 7.7; "torchisotonic" PyPI page, "What it is for":
    scikit-learn's IsotonicRegression curve), written from its definition.  The curve's points are the
    row's distinct scores in increasing order; the value at a point comes from the labels of all the
    elements holding that score, which share one fitted value: by Eq. (1) their squared errors around a
    common value v add up to c (v - mean)^2 plus a constant, so the group acts as one observation, its mean
    label, with its count c as the weight.  The curve is the non-decreasing weighted fit of those
    observations.  Returns (xs, fit, m): xs and fit [rows, n] float64 hold the m[r] points of row r and the
    curve's values there (the rest NaN).  A row holding a NaN (score or label) has no curve: m = 0.  -0 and
    +0 are one score, reported as +0."""
    s2 = _as2d(scores)
    l2 = _as2d(labels)
    if s2.shape != l2.shape:
        raise ValueError("labels must have the shape of scores")
    rows, n = s2.shape
    xs = np.full((rows, n), np.nan)
    fv = np.full((rows, n), np.nan)
    m = np.zeros(rows, dtype=np.int64)
    for r in range(rows):
        s, lab = s2[r], l2[r]
        if n == 0 or np.isnan(s).any() or np.isnan(lab).any():
            continue
        order = np.argsort(s, kind="stable")
        ss = s[order] + 0.0          # -0 becomes +0
        ll = lab[order]
        # a group of equal scores begins where the sorted score differs from the one before it
        first = np.flatnonzero(np.concatenate(([True], ss[1:] != ss[:-1])))
        last = np.append(first[1:], n)
        counts = (last - first).astype(np.float64)
        sums = np.array([math.fsum(ll[a:b]) for a, b in zip(first, last)]) if first.size < n else ll.copy()
        z, *_ = fit(sums / counts, counts, increasing=True)
        k = first.size
        xs[r, :k] = ss[first]
        fv[r, :k] = z[0]
        m[r] = k
    return xs, fv, m


def calibrate(q, xs, fv, m):
    """Calibrated values of the queries q [rows, k] on each row's curve ("torchisotonic" PyPI page, "What it
    is for"): the piecewise-linear function through the curve's points, held constant before the first point
    and after the last (numpy's interp is exactly that function); a NaN query, or a row without a curve,
    gives NaN."""
    q2 = _as2d(q)
    out = np.full(q2.shape, np.nan)
    for r in range(q2.shape[0]):
        k = int(m[r])
        if k == 0:
            continue
        out[r] = np.interp(q2[r], xs[r, :k], fv[r, :k])
        out[r, np.isnan(q2[r])] = np.nan
    return out
