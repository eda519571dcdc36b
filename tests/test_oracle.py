"""Pins for the CPU float64 oracle (no GPU).

The oracle (oracle/iso_oracle.c, pool adjacent violators) is checked against
things that do not share its algorithm:

* exact rational brute force of the min-max closed form
  fit_i = max_{j<=i} min_{k>=i} (sum_{j..k} w y) / (sum_{j..k} w)
  (classical; the page "Merge Hulls Without Copying Vertices: GPU Isotonic
  Regression" cites Barlow et al. for the equivalent hull form, Sec. 2.1 and 8);
* exact enumeration of all partitions into consecutive blocks (Eq. (1) of the
  same page minimised directly);
* invariants of Eq. (1): monotone output, preserved weighted sum, fixed points,
  idempotence, affine equivariance, weight-scale invariance, and the KKT
  multipliers of Sec. 7.6 (non-negative, zero at the end, zero where the fit
  steps up);
* scipy.optimize.isotonic_regression and sklearn.isotonic.isotonic_regression,
  which compute the same fit (PyPI page "torchisotonic", first paragraph);
* the hand-worked cases in tests/golden/hand_cases.json;
* central finite differences for the vector-Jacobian product (Appendix B,
  "Tests": gradients against finite differences in float64).
"""
from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


# ---------------------------------------------------------------- brute force

def minmax_exact(y, w):
    """Exact min-max closed form with rationals (non-decreasing fit)."""
    n = len(y)
    yq = [Fraction(v) for v in y]
    wq = [Fraction(v) for v in w]
    out = []
    for i in range(n):
        best = None
        for j in range(i + 1):
            inner = None
            for k in range(i, n):
                m = sum(wq[t] * yq[t] for t in range(j, k + 1)) / sum(wq[j:k + 1])
                inner = m if inner is None or m < inner else inner
            best = inner if best is None or inner > best else best
        out.append(best)
    return out


def partitions_exact(y, w):
    """Minimise Eq. (1) over all partitions into consecutive blocks whose means
    do not decrease (each block takes its weighted mean)."""
    n = len(y)
    yq = [Fraction(v) for v in y]
    wq = [Fraction(v) for v in w]
    best_obj, best_z = None, None
    for cuts in itertools.product([0, 1], repeat=n - 1):
        bounds = [0] + [i + 1 for i, c in enumerate(cuts) if c] + [n]
        means = []
        for a, b in zip(bounds[:-1], bounds[1:]):
            means.append(sum(wq[t] * yq[t] for t in range(a, b)) / sum(wq[a:b]))
        if any(means[k] > means[k + 1] for k in range(len(means) - 1)):
            continue
        z = []
        for (a, b), m in zip(zip(bounds[:-1], bounds[1:]), means):
            z += [m] * (b - a)
        obj = sum(wq[t] * (z[t] - yq[t]) ** 2 for t in range(n))
        if best_obj is None or obj < best_obj:
            best_obj, best_z = obj, z
    return best_z


def _rand_small(r, n):
    # small integers and halves: exact in binary, many ties and violations
    y = r.integers(-4, 5, size=n) / 2.0
    w = r.integers(1, 5, size=n) / 2.0
    return y, w


@pytest.mark.parametrize("seed", range(40))
def test_oracle_matches_minmax_exact(seed):
    r = workloads.rng(1000 + seed)
    n = int(r.integers(1, 9))
    y, w = _rand_small(r, n)
    z, *_ = oracle.fit(y, w)
    ref = [float(v) for v in minmax_exact(y, w)]
    np.testing.assert_allclose(z[0], ref, rtol=0, atol=1e-14)


@pytest.mark.parametrize("seed", range(25))
def test_oracle_matches_partition_enumeration(seed):
    r = workloads.rng(2000 + seed)
    n = int(r.integers(1, 11))
    y = r.standard_normal(n).round(3)
    w = (r.random(n) + 0.1).round(3)
    z, *_ = oracle.fit(y, w)
    ref = [float(v) for v in partitions_exact(y, w)]
    np.testing.assert_allclose(z[0], ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("seed", range(10))
def test_oracle_decreasing_minmax_exact(seed):
    r = workloads.rng(3000 + seed)
    n = int(r.integers(1, 9))
    y, w = _rand_small(r, n)
    z, *_ = oracle.fit(y, w, increasing=False)
    # non-increasing fit of y = reversed non-decreasing fit of reversed y
    ref = [float(v) for v in minmax_exact(y[::-1], w[::-1])][::-1]
    np.testing.assert_allclose(z[0], ref, rtol=0, atol=1e-14)


# ------------------------------------------------------------------ golden

def test_oracle_hand_cases():
    with open(GOLDEN) as f:
        data = json.load(f)
    for c in data["cases"]:
        z, bs, cl, rn, st = oracle.fit(c["y"], c["w"], c["increasing"], c["y_min"], c["y_max"])
        assert st == oracle.OK
        np.testing.assert_allclose(z[0], c["fit"], rtol=0, atol=1e-15, err_msg=c["why"])
        assert list(bs[0]) == c["starts"], c["why"]
        assert list(cl[0]) == c["clipped"], c["why"]
        assert rn[0] == 0
    for c in data["nan_cases"]:
        y = [float(v) for v in c["y"]]
        w = None if c["w"] is None else [float(v) for v in c["w"]]
        z, bs, cl, rn, st = oracle.fit(y, w)
        assert st == oracle.OK
        assert np.isnan(z).all() and rn[0] == 1 and bs.sum() == 0


# --------------------------------------------------------------- invariants

def kkt_residual(y, w, z):
    """Largest KKT violation of Eq. (1) (first page, Sec. 7.6): with
    lambda_i = -2 sum_{j<=i} w_j (z_j - y_j), require lambda >= 0,
    lambda_n = 0, lambda_i = 0 where z steps up; relative to 2 sum w |y|."""
    lam = -2.0 * np.cumsum(w * (z - y))
    scale = 2.0 * np.sum(w * np.abs(y))
    viol = max(0.0, -lam.min())
    viol = max(viol, abs(lam[-1]))
    up = np.nonzero(z[1:] > z[:-1])[0]
    if up.size:
        viol = max(viol, np.abs(lam[up]).max())
    return viol / scale


@pytest.mark.parametrize("kind", workloads.FAMILIES)
def test_oracle_invariants_families(kind):
    n = 300 if kind != "consecutive" else 200
    wl = workloads.family(kind, 3, n, seed=7)
    w = np.ones_like(wl.y) if wl.w is None else wl.w
    z, bs, cl, rn, st = oracle.fit(wl.y, wl.w)
    assert st == oracle.OK
    for r in range(wl.rows):
        y, wr, zr = wl.y[r], w[r], z[r]
        scale = np.abs(y).max()
        assert np.all(np.diff(zr) >= -1e-15 * scale)              # monotone
        s0, s1 = np.sum(wr * y), np.sum(wr * zr)
        assert abs(s0 - s1) <= 1e-11 * np.sum(wr * np.abs(y))    # weighted sum kept
        assert kkt_residual(y, wr, zr) < 1e-12
        # each block's value is its weighted mean
        starts = np.nonzero(bs[r])[0].tolist() + [wl.n]
        assert starts[0] == 0
        for a, b in zip(starts[:-1], starts[1:]):
            m = np.sum(wr[a:b] * y[a:b]) / np.sum(wr[a:b])
            assert np.all(np.abs(zr[a:b] - m) <= 1e-12 * max(1.0, abs(m)))
        if b - a > 0 and len(starts) > 2:
            means = [zr[a] for a in starts[:-1]]
            assert all(means[k] < means[k + 1] for k in range(len(means) - 1))


def test_oracle_fixed_point_and_idempotence():
    r = workloads.rng(11)
    y = np.sort(r.standard_normal(500))
    w = r.random(500) + 0.2
    z, *_ = oracle.fit(y, w)
    # monotone input unchanged (each element is its own block; w*y/w rounds once)
    np.testing.assert_allclose(z[0], y, rtol=4.5e-16, atol=0)
    y2 = r.standard_normal(700)
    w2 = r.random(700) + 0.2
    z2, *_ = oracle.fit(y2, w2)
    z3, *_ = oracle.fit(z2[0], w2)
    np.testing.assert_allclose(z3[0], z2[0], rtol=0, atol=1e-14)  # refitting changes nothing


def test_oracle_affine_and_weight_scale():
    r = workloads.rng(12)
    y = r.standard_normal(400)
    w = r.random(400) + 0.1
    z, *_ = oracle.fit(y, w)
    za, *_ = oracle.fit(3.0 * y - 2.0, w)
    np.testing.assert_allclose(za[0], 3.0 * z[0] - 2.0, rtol=0, atol=1e-12)
    zw, *_ = oracle.fit(y, 8.0 * w)
    np.testing.assert_allclose(zw[0], z[0], rtol=0, atol=1e-13)
    # non-increasing fit of y = minus the non-decreasing fit of -y
    zd, *_ = oracle.fit(y, w, increasing=False)
    zn, *_ = oracle.fit(-y, w, increasing=True)
    np.testing.assert_allclose(zd[0], -zn[0], rtol=0, atol=1e-13)


# ----------------------------------------------------------- library pins

@pytest.mark.parametrize("seed", range(6))
def test_oracle_matches_scipy(seed):
    from scipy.optimize import isotonic_regression
    r = workloads.rng(4000 + seed)
    n = int(r.integers(1, 3000))
    y = r.standard_normal(n) + np.linspace(0, seed, n)
    w = r.random(n) + 0.05
    inc = bool(seed % 2)
    res = isotonic_regression(y, weights=w, increasing=inc)
    z, bs, *_ = oracle.fit(y, w, increasing=inc)
    np.testing.assert_allclose(z[0], res.x, rtol=0, atol=1e-12 * np.abs(y).max())
    if inc:
        np.testing.assert_array_equal(np.nonzero(bs[0])[0], res.blocks[:-1])


@pytest.mark.parametrize("seed", range(6))
def test_oracle_matches_sklearn_clip(seed):
    from sklearn.isotonic import isotonic_regression
    r = workloads.rng(5000 + seed)
    n = int(r.integers(1, 2000))
    y = r.standard_normal(n)
    w = r.random(n) + 0.1
    inc = bool(seed % 2)
    lo, hi = -0.3, 0.4
    ref = isotonic_regression(y, sample_weight=w, y_min=lo, y_max=hi, increasing=inc)
    z, bs, cl, *_ = oracle.fit(y, w, increasing=inc, y_min=lo, y_max=hi)
    np.testing.assert_allclose(z[0], ref, rtol=0, atol=1e-12)
    zu, *_ = oracle.fit(y, w, increasing=inc)
    np.testing.assert_array_equal(cl[0].astype(bool), (zu[0] < lo) | (zu[0] > hi))


def test_oracle_configs_small_vs_scipy():
    from scipy.optimize import isotonic_regression
    for k in (1, 2, 3):
        wl = workloads.CONFIGS[k](rows=3, n=777) if k != 4 else None
        z, *_ = oracle.fit(wl.y, wl.w, wl.increasing, wl.y_min, wl.y_max)
        for r in range(wl.rows):
            wr = None if wl.w is None else wl.w[r].astype(np.float64)
            ref = isotonic_regression(wl.y[r].astype(np.float64), weights=wr, increasing=wl.increasing).x
            lo = -np.inf if wl.y_min is None else wl.y_min
            hi = np.inf if wl.y_max is None else wl.y_max
            np.testing.assert_allclose(z[r], np.clip(ref, lo, hi), rtol=0, atol=1e-12)


# ------------------------------------------------------------ error paths

def test_oracle_nan_and_weight_error_rows():
    y = np.array([[1.0, 2.0, 0.5], [1.0, np.nan, 0.0], [3.0, 1.0, 2.0], [1.0, 2.0, np.inf]])
    w = np.array([[1.0, 1.0, 1.0], [1.0, 1.0, 1.0], [1.0, 0.0, 1.0], [1.0, 1.0, 1.0]])
    z, bs, cl, rn, st = oracle.fit(y, w)
    assert st == oracle.EWEIGHT
    assert not np.isnan(z[0]).any() and rn[0] == 0
    assert np.isnan(z[1]).all() and rn[1] == 1
    assert np.isnan(z[2]).all() and rn[2] == 1
    assert np.isnan(z[3]).all() and rn[3] == 1
    z, bs, cl, rn, st = oracle.fit(y[:2], -w[:2])
    assert st == oracle.EWEIGHT


def test_oracle_empty_and_threads():
    z, *_ = oracle.fit(np.zeros((0, 5)))
    assert z.shape == (0, 5)
    z, *_ = oracle.fit(np.zeros((4, 0)))
    assert z.shape == (4, 0)
    wl = workloads.cfg2_batch_noise(rows=37, n=300)
    a = oracle.fit(wl.y, wl.w, False, 0.0, 1.0, threads=1)[0]
    b = oracle.fit(wl.y, wl.w, False, 0.0, 1.0, threads=8)[0]
    np.testing.assert_array_equal(a, b)
    with pytest.raises(ValueError):
        oracle.fit([1.0, 2.0], None, True, 2.0, 1.0)


# --------------------------------------------------------------------- VJP

@pytest.mark.parametrize("seed", range(8))
def test_oracle_vjp_finite_differences(seed):
    r = workloads.rng(6000 + seed)
    n = int(r.integers(2, 60))
    y = r.standard_normal(n)
    w = r.random(n) + 0.2
    inc = bool(seed % 2)
    lo, hi = (-0.5, 0.5) if seed % 3 == 0 else (None, None)
    g = r.standard_normal(n)
    z, bs, cl, rn, _ = oracle.fit(y, w, inc, lo, hi)
    # stay away from kinks: block means well separated, no fit at a clip bound
    starts = np.nonzero(bs[0])[0]
    means = z[0][starts]
    zu = oracle.fit(y, w, inc)[0][0]
    if (len(means) > 1 and np.min(np.abs(np.diff(oracle.fit(y, w, inc)[0][0][starts]))) < 1e-3) or \
            (lo is not None and np.min(np.minimum(np.abs(zu - lo), np.abs(zu - hi))) < 1e-3):
        pytest.skip("near a kink")
    v = oracle.vjp(g, bs, cl, rn, w)[0]
    h = 1e-6
    fd = np.empty(n)
    for j in range(n):
        yp, ym = y.copy(), y.copy()
        yp[j] += h
        ym[j] -= h
        fd[j] = (g @ oracle.fit(yp, w, inc, lo, hi)[0][0] - g @ oracle.fit(ym, w, inc, lo, hi)[0][0]) / (2 * h)
    np.testing.assert_allclose(v, fd, rtol=1e-6, atol=1e-7)


def test_oracle_vjp_unit_weight_block_mean():
    # the vector-Jacobian product averages g over each block when w = 1
    y = np.array([3.0, 1.0, 2.0, 5.0, 4.0])
    g = np.array([1.0, 2.0, 6.0, -1.0, 3.0])
    z, bs, cl, rn, _ = oracle.fit(y)
    assert list(bs[0]) == [1, 0, 0, 1, 0]
    v = oracle.vjp(g, bs, cl, rn)[0]
    np.testing.assert_allclose(v, [3.0, 3.0, 3.0, 1.0, 1.0], rtol=0, atol=1e-15)


# ------------------------------------------------------------ VJP in w
# The fit is differentiable in y and in the weights (page "torchisotonic",
# "Semantics").  Pins: central finite differences in w, a hand case derived
# from the block mean's quotient rule, and the invariance of the fit under a
# common scale of the weights (so sum_j w_j dL/dw_j = 0 on every row).

@pytest.mark.parametrize("seed", range(8))
def test_oracle_vjp_w_finite_differences(seed):
    r = workloads.rng(7000 + seed)
    n = int(r.integers(2, 60))
    y = r.standard_normal(n)
    w = r.random(n) + 0.2
    inc = bool(seed % 2)
    lo, hi = (-0.5, 0.5) if seed % 3 == 0 else (None, None)
    g = r.standard_normal(n)
    z, bs, cl, rn, _ = oracle.fit(y, w, inc, lo, hi)
    starts = np.nonzero(bs[0])[0]
    zu = oracle.fit(y, w, inc)[0][0]
    if (len(starts) > 1 and np.min(np.abs(np.diff(zu[starts]))) < 1e-3) or \
            (lo is not None and np.min(np.minimum(np.abs(zu - lo), np.abs(zu - hi))) < 1e-3):
        pytest.skip("near a kink")
    v = oracle.vjp_w(g, y, bs, cl, rn, w)[0]
    h = 1e-6
    fd = np.empty(n)
    for j in range(n):
        wp, wm = w.copy(), w.copy()
        wp[j] += h
        wm[j] -= h
        fd[j] = (g @ oracle.fit(y, wp, inc, lo, hi)[0][0] - g @ oracle.fit(y, wm, inc, lo, hi)[0][0]) / (2 * h)
    np.testing.assert_allclose(v, fd, rtol=1e-6, atol=1e-7)


def test_oracle_vjp_w_hand_cases():
    # blocks {3, 1, 2} (mean 2) and {5, 4} (mean 4.5), unit weights:
    # dL/dw_j = (sum of g over the block) * (y_j - mean) / (block weight)
    y = np.array([3.0, 1.0, 2.0, 5.0, 4.0])
    g = np.array([1.0, 2.0, 6.0, -1.0, 3.0])
    z, bs, cl, rn, _ = oracle.fit(y)
    np.testing.assert_allclose(oracle.vjp_w(g, y, bs, cl, rn)[0], [3.0, -3.0, 0.0, 0.5, -0.5], rtol=0,
                               atol=1e-15)
    # one pooled block f = (w1 y1 + w2 y2) / (w1 + w2) = 1.5 for y = (3, 1),
    # w = (1, 3): df/dw1 = (y1 - f) / W = 0.375, df/dw2 = -0.125; L = 2 f + 5 f
    y = np.array([3.0, 1.0])
    w = np.array([1.0, 3.0])
    g = np.array([2.0, 5.0])
    z, bs, cl, rn, _ = oracle.fit(y, w)
    np.testing.assert_allclose(oracle.vjp_w(g, y, bs, cl, rn, w)[0], [2.625, -0.875], rtol=0, atol=1e-15)
    # a clipped block contributes nothing
    z, bs, cl, rn, _ = oracle.fit(y, w, True, 2.0, 3.0)
    assert cl[0].all()
    np.testing.assert_array_equal(oracle.vjp_w(g, y, bs, cl, rn, w)[0], [0.0, 0.0])


@pytest.mark.parametrize("seed", range(4))
def test_oracle_vjp_w_scale_invariance(seed):
    r = workloads.rng(7100 + seed)
    y = r.standard_normal((5, 300))
    w = r.random((5, 300)) * 3 + 0.1
    g = r.standard_normal((5, 300))
    inc = bool(seed % 2)
    z, bs, cl, rn, _ = oracle.fit(y, w, inc, -0.3 if seed >= 2 else None, 0.4 if seed >= 2 else None)
    v = oracle.vjp_w(g, y, bs, cl, rn, w)
    s = np.sum(w * v, axis=1)
    assert np.max(np.abs(s)) <= 1e-12 * max(1.0, np.abs(w * v).sum(axis=1).max())


# ---------------------------------------------------------------- soft rank (first page, Sec. 7.9)

def hard_ranks(x):
    """1 for the smallest value of a row, n for the largest (distinct values)."""
    return (np.argsort(np.argsort(x, axis=-1, kind="stable"), axis=-1, kind="stable") + 1).astype(np.float64)


@pytest.mark.parametrize("n", [1, 2, 7, 64, 513])
def test_soft_rank_one_block_closed_form(n):
    """Sorted gaps below 1 make z = s - (n..1) strictly increasing, so the non-increasing fit pools the whole
    row into its mean and r = theta - mean(theta) + (n + 1) / 2."""
    r = workloads.rng(n)
    for eps in (1.0, 2.5):
        x = r.random((3, n)) * 0.99 * eps
        got, perm, bs, rn = oracle.soft_rank(x, eps)
        theta = x / eps
        want = theta - theta.mean(axis=1, keepdims=True) + (n + 1) / 2.0
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12 * n)
        assert bs[:, 0].all() and not bs[:, 1:].any() and not rn.any()


@pytest.mark.parametrize("n", [2, 5, 40, 300])
def test_soft_rank_hard_rank_regime(n):
    """Sorted gaps of at least 1 make z non-increasing already: the fit is z itself and the soft ranks are
    the hard ranks (n for the largest value)."""
    r = workloads.rng(100 + n)
    x = r.permutation(n)[None, :] * 3.0 + r.random((1, n)) * 0.5
    got, _, bs, _ = oracle.soft_rank(x, 1.0)
    np.testing.assert_allclose(got, hard_ranks(x), rtol=0, atol=1e-12 * n)
    assert bs.all()
    y = r.standard_normal((4, n))
    gap = np.min(np.diff(np.sort(y, axis=1), axis=1))
    got, *_ = oracle.soft_rank(y, gap / 2)
    np.testing.assert_allclose(got, hard_ranks(y), rtol=0, atol=1e-9 * n)


def permutahedron_projection(theta):
    """Euclidean projection of theta onto the convex hull of the permutations of (1..n), solved as a
    quadratic programme over Rado's description of that hull: the sum over any subset S is at most the
    sum of the |S| largest of (1..n), with equality for the full set."""
    from scipy.optimize import minimize
    n = len(theta)
    top = np.cumsum(np.arange(n, 0, -1, dtype=np.float64))
    cons = [{"type": "eq", "fun": lambda r: np.sum(r) - top[-1]}]
    for k in range(1, n):
        for S in itertools.combinations(range(n), k):
            idx = np.array(S)
            cons.append({"type": "ineq", "fun": lambda r, idx=idx, b=top[k - 1]: b - np.sum(r[idx])})
    x0 = np.full(n, (n + 1) / 2.0)
    res = minimize(lambda r: 0.5 * np.sum((r - theta) ** 2), x0, jac=lambda r: r - theta,
                   constraints=cons, method="SLSQP", options={"ftol": 1e-14, "maxiter": 500})
    assert res.success, res.message
    return res.x


@pytest.mark.parametrize("seed", range(12))
def test_soft_rank_is_the_permutahedron_projection(seed):
    """The soft rank of Sec. 7.9 is the projection of theta onto the permutahedron (Blondel et al.), which
    is computed here by a generic solver that shares nothing with pool adjacent violators."""
    r = workloads.rng(200 + seed)
    n = 2 + seed % 4
    eps = [0.3, 1.0, 2.0][seed % 3]
    x = r.standard_normal(n) * 1.5
    got, *_ = oracle.soft_rank(x, eps)
    want = permutahedron_projection(x / eps)
    np.testing.assert_allclose(got[0], want, rtol=0, atol=2e-6)


def test_soft_rank_invariances():
    """Shifts of theta along (1..1) do not move the projection; a permutation of x permutes the ranks;
    the ranks sum to n(n+1)/2, keep the order of x, and tied values get equal ranks."""
    r = workloads.rng(9)
    x = r.standard_normal((5, 50))
    base, *_ = oracle.soft_rank(x, 0.7)
    shifted, *_ = oracle.soft_rank(x + 3.25, 0.7)
    np.testing.assert_allclose(shifted, base, rtol=0, atol=1e-10)
    p = r.permutation(50)
    permuted, *_ = oracle.soft_rank(x[:, p], 0.7)
    np.testing.assert_allclose(permuted, base[:, p], rtol=0, atol=1e-12)
    np.testing.assert_allclose(base.sum(axis=1), 50 * 51 / 2, rtol=1e-14)
    order = np.argsort(x, axis=1)
    assert (np.diff(np.take_along_axis(base, order, axis=1), axis=1) >= -1e-12).all()
    t = x.copy()
    t[:, 7] = t[:, 3]
    t[:, 20] = t[:, 3]
    tied, *_ = oracle.soft_rank(t, 0.05)
    assert np.all(tied[:, 7] == tied[:, 3]) and np.all(tied[:, 20] == tied[:, 3])


def test_soft_rank_nan_rows():
    x = workloads.rng(4).standard_normal((3, 9))
    x[1, 4] = np.nan
    got, perm, bs, rn = oracle.soft_rank(x, 1.0)
    assert np.isnan(got[1]).all() and not np.isnan(got[[0, 2]]).any()
    assert list(rn) == [0, 1, 0]
    g = np.ones_like(x)
    d = oracle.soft_rank_vjp(g, 1.0, perm, bs, rn)
    assert np.isnan(d[1]).all() and not np.isnan(d[[0, 2]]).any()


@pytest.mark.parametrize("seed", range(8))
def test_soft_rank_vjp_finite_differences(seed):
    """The product of soft_rank_vjp against central differences of soft_rank in float64 (Appendix B,
    "Tests": gradients against finite differences on the CPU)."""
    r = workloads.rng(300 + seed)
    n = [3, 8, 17, 40][seed % 4]
    eps = [0.2, 1.0][seed % 2]
    x = r.standard_normal((2, n))
    g = r.standard_normal((2, n))
    _, perm, bs, rn = oracle.soft_rank(x, eps)
    got = oracle.soft_rank_vjp(g, eps, perm, bs, rn)
    h = 1e-6
    num = np.zeros_like(x)
    for k in range(n):
        e = np.zeros_like(x)
        e[:, k] = h
        fp, *_ = oracle.soft_rank(x + e, eps)
        fm, *_ = oracle.soft_rank(x - e, eps)
        num[:, k] = np.sum(g * (fp - fm), axis=1) / (2 * h)
    np.testing.assert_allclose(got, num, rtol=0, atol=1e-6)


# ---------------------------------------------------------------- calibration (first page, Sec. 7.7; PyPI usage)

def test_calibration_hand_cases():
    """Worked by hand: equal scores pool before the fit, and the curve interpolates linearly between its
    points and is constant beyond them."""
    xs, fv, m = oracle.calibration_fit([[1.0, 2.0, 1.0]], [[0.0, 0.0, 1.0]])
    # pooled: x = (1, 2), y = (1/2, 0), weights (2, 1); the violation pools both: (2*(1/2) + 0)/3 = 1/3
    assert m[0] == 2 and list(xs[0, :2]) == [1.0, 2.0]
    np.testing.assert_allclose(fv[0, :2], [1 / 3, 1 / 3], rtol=0, atol=1e-15)
    xs, fv, m = oracle.calibration_fit([[0.0, 1.0, 2.0, 1.0]], [[0.0, 1.0, 1.0, 0.0]])
    assert m[0] == 3
    np.testing.assert_allclose(fv[0, :3], [0.0, 0.5, 1.0], rtol=0, atol=1e-15)
    out = oracle.calibrate([[0.5, -1.0, 5.0, 1.5, 1.0, np.nan]], xs, fv, m)
    np.testing.assert_allclose(out[0, :5], [0.25, 0.0, 1.0, 0.75, 0.5], rtol=0, atol=1e-15)
    assert np.isnan(out[0, 5])
    xs, fv, m = oracle.calibration_fit([[3.0, 3.0]], [[1.0, 0.0]])
    assert m[0] == 1 and oracle.calibrate([[-7.0, 9.0]], xs, fv, m).tolist() == [[0.5, 0.5]]


@pytest.mark.parametrize("seed", range(6))
def test_calibration_matches_sklearn(seed):
    """scikit-learn's IsotonicRegression (out_of_bounds="clip") pools equal scores, fits, and interpolates
    linearly: the curve's predictions must agree, ties included."""
    from sklearn.isotonic import IsotonicRegression
    r = workloads.rng(400 + seed)
    n = [20, 200, 3000][seed % 3]
    s = np.round(r.standard_normal(n), 1 + seed % 3)  # coarse scores: many ties
    p = 1.0 / (1.0 + np.exp(-(1.5 * s - 1.0)))
    y = (r.random(n) < p).astype(np.float64) if seed % 2 == 0 else p + 0.3 * r.standard_normal(n)
    q = np.concatenate([np.linspace(s.min() - 1, s.max() + 1, 101), s[:50]])
    xs, fv, m = oracle.calibration_fit(s, y)
    got = oracle.calibrate(q, xs, fv, m)[0]
    want = IsotonicRegression(increasing=True, out_of_bounds="clip").fit(s, y).predict(q)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    assert m[0] == len(np.unique(s))


@pytest.mark.parametrize("seed", range(4))
def test_calibration_without_ties_is_the_fit_of_the_sorted_labels(seed):
    """With distinct scores there is nothing to pool: the curve at the sorted scores is the plain isotonic
    fit of the labels in score order (scipy)."""
    from scipy.optimize import isotonic_regression
    r = workloads.rng(500 + seed)
    s = r.permutation(300) + r.random(300) * 0.5
    y = r.standard_normal(300)
    xs, fv, m = oracle.calibration_fit(s, y)
    order = np.argsort(s)
    assert m[0] == 300 and np.array_equal(xs[0], s[order])
    np.testing.assert_allclose(fv[0], isotonic_regression(y[order]).x, rtol=0, atol=1e-12)


def test_calibration_equals_fit_with_tied_labels_replaced_by_their_mean():
    """A property of Eq. (1): equal neighbouring values always get equal fits, so pooling equal scores is
    the same as replacing their labels by the group mean and fitting every sample with unit weight."""
    from scipy.optimize import isotonic_regression
    r = workloads.rng(17)
    s = np.round(r.standard_normal(2000), 1)
    y = r.standard_normal(2000)
    xs, fv, m = oracle.calibration_fit(s, y)
    order = np.argsort(s, kind="stable")
    ss, yy = s[order], y[order].copy()
    u, inv = np.unique(ss, return_inverse=True)
    means = np.bincount(inv, yy) / np.bincount(inv)
    full = isotonic_regression(means[inv]).x
    np.testing.assert_allclose(full, fv[0, :m[0]][inv], rtol=0, atol=1e-12)


def test_calibration_nan_rows_and_rows():
    r = workloads.rng(23)
    s = np.round(r.standard_normal((4, 50)), 1)
    y = r.random((4, 50))
    s[1, 3] = np.nan
    y[2, 7] = np.nan
    xs, fv, m = oracle.calibration_fit(s, y)
    assert m[1] == 0 and m[2] == 0 and m[0] > 0 and m[3] > 0
    assert np.isnan(oracle.calibrate(s, xs, fv, m)[[1, 2]]).all()
    for row in (0, 3):
        xr, fr, mr = oracle.calibration_fit(s[row], y[row])
        np.testing.assert_array_equal(xr[0], xs[row])
        np.testing.assert_allclose(fr[0], fv[row], rtol=0, atol=0)
