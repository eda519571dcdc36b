"""Seeded synthetic inputs for batched weighted isotonic regression.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic, so both the GPU path and the CPU oracle can take their
inputs from it.  Every generator uses numpy's PCG64 with an explicit seed.

The five workloads mirror the shapes and value distributions the fit is
measured on (page "Merge Hulls Without Copying Vertices: GPU Isotonic
Regression", Sec. 7.5-7.9; page "torchisotonic" on PyPI, usage and
calibration examples).  The data families (noise, increasing, sawtooth, cliff,
constant, extreme weights, consecutive floats, cancellation) are the ones the
first page tests its accuracy and schedules on (Sec. 7.4 and 7.6, Appendix B
"Tests").  Where a page names a family without giving its formula, the formula
here is the plainest one that has the stated property.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


@dataclass
class Workload:
    name: str
    y: np.ndarray            # [rows, n]
    w: np.ndarray | None     # [rows, n] or None (unit weights)
    increasing: bool = True
    y_min: float | None = None
    y_max: float | None = None
    g: np.ndarray | None = None  # upstream gradient for the backward, if any
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.y.shape[0]

    @property
    def n(self) -> int:
        return self.y.shape[1]

    @property
    def dtype(self):
        return self.y.dtype


# --------------------------------------------------------------------------
# The five workloads.  rows / n can be shrunk for tests; the defaults are the
# full sizes.
# --------------------------------------------------------------------------

def cfg1_single_row(rows=1, n=4096, seed=1) -> Workload:
    """1 x 4096 float64, y ~ N(0,1) i.i.d., unit weights, increasing, no clip."""
    r = rng(seed)
    y = r.standard_normal((rows, n))
    return Workload("cfg1_1x4096_f64_noise", y, None, True)


def cfg2_batch_noise(rows=1000, n=5000, seed=2) -> Workload:
    """1000 x 5000 float32, y ~ N(0,1), w ~ U(0.1, 1.1) per element,
    non-increasing, clipped to [0, 1] (the PyPI page's second usage example)."""
    r = rng(seed)
    y = r.standard_normal((rows, n)).astype(np.float32)
    w = (r.random((rows, n)) + 0.1).astype(np.float32)
    return Workload("cfg2_1000x5000_f32_noise_weighted_dec_clip", y, w, False, 0.0, 1.0)


def cfg3_soft_rank(rows=4096, n=512, seed=3) -> Workload:
    """Soft-rank projection shape: 4096 x 512 float32, unit weights, increasing.

    y_i = s_i - i/512 with s the row's N(0,1) draws sorted descending: a strictly
    decreasing row, which an increasing fit pools into one block (the regime of
    the first page's Sec. 7.9 at epsilon = 1).  The upstream gradient is N(0,1).
    """
    r = rng(seed)
    s = -np.sort(-r.standard_normal((rows, n)), axis=1)
    y = (s - np.arange(n)[None, :] / 512.0).astype(np.float32)
    g = r.standard_normal((rows, n)).astype(np.float32)
    return Workload("cfg3_4096x512_f32_softrank_fwd_bwd", y, None, True, g=g)


def soft_rank_input(rows=4096, n=512, seed=3, dtype=np.float32):
    """Input of the soft-rank composition (first page, Sec. 7.9): standard normal
    scores x and a standard normal upstream gradient g, [rows, n]."""
    r = rng(seed)
    x = r.standard_normal((rows, n)).astype(dtype)
    g = r.standard_normal((rows, n)).astype(dtype)
    return x, g


def calibration_input(n=6_500_000, seed=4, dtype=np.float64):
    """Raw input of the calibration composition (first page, Sec. 7.7: one curve
    over a day of 6.5 million click-model scores; synthetic): scores N(0,1) on a
    grid of 1e-5, so that equal scores pool into runs; click labels
    Bernoulli(sigmoid(1.5 s - 3)); queries spanning and beyond the scores."""
    r = rng(seed)
    s = np.round(r.standard_normal(n), 5)
    p = 1.0 / (1.0 + np.exp(-(1.5 * s - 3.0)))
    y = (r.random(n) < p).astype(dtype)
    q = np.linspace(-6.0, 6.0, 100_001)
    return s.astype(dtype)[None, :], y[None, :], q.astype(dtype)[None, :]


def cfg4_calibration(n=6_500_000, seed=4) -> Workload:
    """Calibration-shaped single row, float64: sorted scores s ~ N(0,1),
    integer counts c ~ 1 + Poisson(2) as weights, y = Binomial(c, sigmoid(1.5 s - 3)) / c,
    increasing, clipped to [0, 1].  Stands in for the pooled click data of the
    first page's Sec. 7.7 (one curve over 6.5 million scores)."""
    r = rng(seed)
    s = np.sort(r.standard_normal(n))
    c = 1 + r.poisson(2.0, size=n)
    p = 1.0 / (1.0 + np.exp(-(1.5 * s - 3.0)))
    k = r.binomial(c, p)
    y = (k / c).astype(np.float64)[None, :]
    w = c.astype(np.float64)[None, :]
    return Workload("cfg4_1x6.5e6_f64_calibration", y, w, True, 0.0, 1.0)


def cfg5_dense(rows=32, n=1 << 22, seed=5) -> Workload:
    """32 x 2^22 float64, y_i = i/n with 1% of positions (uniform) perturbed
    downward by |N(0, 0.01)|, w ~ U(0.5, 1.5), increasing."""
    r = rng(seed)
    y = np.broadcast_to(np.arange(n, dtype=np.float64) / n, (rows, n)).copy()
    mask = r.random((rows, n)) < 0.01
    y[mask] -= np.abs(r.normal(0.0, 0.01, size=int(mask.sum())))
    w = r.random((rows, n)) + 0.5
    return Workload("cfg5_32x2^22_f64_dense", y, w, True)


CONFIGS = {
    1: cfg1_single_row,
    2: cfg2_batch_noise,
    3: cfg3_soft_rank,
    4: cfg4_calibration,
    5: cfg5_dense,
}


# --------------------------------------------------------------------------
# Data families (small sizes; used by the parity tests).
# --------------------------------------------------------------------------

def _weights(r, kind, shape, dtype):
    if kind == "unit":
        return None
    if kind == "uniform":
        return (r.random(shape) + 0.1).astype(dtype)
    if kind == "extreme":
        # weights spanning a ratio of e^8 (e^-4 .. e^4): the first page,
        # Sec. 7.6, notes that with extreme weights a sum of 32 terms can be
        # 32 e^8 times a single term
        return np.exp(r.uniform(-4.0, 4.0, size=shape)).astype(dtype)
    raise ValueError(kind)


def family(kind: str, rows: int, n: int, seed: int = 0, dtype=np.float64, weights="uniform",
           increasing=True) -> Workload:
    r = rng(seed)
    shape = (rows, n)
    i = np.arange(n, dtype=np.float64)[None, :]
    if kind == "noise":
        y = r.standard_normal(shape)
    elif kind == "trend_noise":
        y = i / max(n, 1) + 0.1 * r.standard_normal(shape)
    elif kind == "increasing":
        # every point a vertex: strictly increasing, no pooling
        y = np.broadcast_to(i / max(n, 1), shape) + 0.0 * r.random(shape)
    elif kind == "sawtooth":
        period = max(2, min(97, n // 4 + 1))
        y = np.broadcast_to((i % period) / period - i / max(n, 1), shape) + 1e-3 * r.standard_normal(shape)
    elif kind == "cliff":
        # increasing data whose last element lies far below the rest: the
        # bridge of every merge on the right spine crosses the whole row
        y = np.broadcast_to(i / max(n, 1), shape).copy()
        y[:, -1] = -10.0 * n
    elif kind == "constant":
        y = np.full(shape, 0.75)
    elif kind == "decreasing":
        y = np.broadcast_to(-i / max(n, 1), shape) + 0.0 * r.random(shape)
    elif kind == "ties":
        y = r.integers(0, 4, size=shape).astype(np.float64)
    elif kind == "consecutive":
        # consecutive floating-point numbers, each one ulp above the previous
        base = np.array(1.0, dtype=dtype)
        vals = [base]
        for _ in range(n - 1):
            vals.append(np.nextafter(vals[-1], np.array(np.inf, dtype=dtype)))
        y = np.broadcast_to(np.array(vals, dtype=dtype), shape).copy()
    elif kind == "cancellation":
        # per 64 elements: 32 x (+B), one -32B, and 31 small, nearly collinear values
        B = 10.0 ** r.integers(3, 13, size=(rows, 1))
        y = np.empty(shape)
        for k in range(n):
            p = k % 64
            if p < 32:
                y[:, k] = B[:, 0]
            elif p == 32:
                y[:, k] = -32.0 * B[:, 0]
            else:
                y[:, k] = 1e-3 * (p - 33) + 1e-9 * r.standard_normal(rows)
    else:
        raise ValueError(kind)
    y = np.ascontiguousarray(y).astype(dtype)
    w = _weights(r, weights, shape, dtype)
    return Workload(f"{kind}_{rows}x{n}_{np.dtype(dtype).name}_{weights}", y, w, increasing)


FAMILIES = ["noise", "trend_noise", "increasing", "sawtooth", "cliff", "constant", "decreasing",
            "ties", "consecutive", "cancellation"]
