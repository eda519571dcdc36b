"""GPU parity: the HIP path against the CPU float64 oracle on the same seeded
inputs, element by element, at the tolerances of tests/gpu_helpers.py.

Covers the five workloads at full size (the 32 x 2^22 one compared on sampled
rows, all rows checked for their invariants), ragged sizes around the wave,
group, chunk and single-workgroup limits, the data families, block partitions,
the backward pass, NaN rows and weight errors, and run-to-run determinism.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import (TOL_F32, TOL_F64, check_fit, check_partition, gpu_blocks, gpu_fit, oracle_fit, scale_of,
                         to_dev)

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def _check_vjp(wl, fit_blocks, gs, gc, grn, seed, what):
    """Both backward products on the GPU's partition (checked against the
    oracle's by check_partition first) against the oracle's products."""
    import weighted_isotonic_regression_row_amd as iso
    dtype = wl.y.dtype
    g = workloads.rng(seed).standard_normal(wl.y.shape).astype(dtype)
    gy, gw = iso.iso_vjp_yw(to_dev(g), fit_blocks, to_dev(wl.y))
    w64 = None if wl.w is None else wl.w.astype(np.float64)
    ref_y = oracle.vjp(g.astype(np.float64), gs, gc, grn, w64)
    ref_w = oracle.vjp_w(g.astype(np.float64), wl.y.astype(np.float64), gs, gc, grn, w64)
    tol = 1e-12 if dtype == np.float64 else 2e-6
    for got, ref, name in ((gy, ref_y, "grad_y"), (gw, ref_w, "grad_w")):
        got = got.cpu().numpy().astype(np.float64)
        assert np.array_equal(np.isnan(got), np.isnan(ref)), f"{what}: {name} NaN pattern"
        ok = ~np.isnan(ref)
        err = float(np.max(np.abs(got[ok] - ref[ok]), initial=0.0))
        assert err <= tol * max(1.0, float(np.abs(ref[ok]).max(initial=0.0))), f"{what}: {name} off by {err:.3e}"


@pytest.mark.parametrize("k", [1, 2, 3])
def test_config_full_size(k):
    """The workload at its full size: the fit, then its block starts and clip
    flags against the oracle's (config 2: 1000 x 5000 float32, non-increasing,
    clipped to [0, 1], on the 20-point row kernel), then both backward products."""
    wl = workloads.CONFIGS[k]()
    _print(f"config {k}: {wl.name} {wl.y.shape}")
    fit, b, *_ = gpu_fit(wl)
    z, bs, cl, rn, st = oracle_fit(wl)
    check_fit(fit.cpu().numpy(), z, wl.y, wl.y.dtype, wl.increasing, wl.name)
    gs, gc, grn = gpu_blocks(b)
    exact, rows = check_partition(gs, gc, grn, wl.y, wl.w, wl.increasing, wl.y_min, wl.y_max, wl.name)
    _print(f"config {k}: {exact} of {rows} rows without a tie position")
    _check_vjp(wl, b, gs, gc, grn, 100 + k, wl.name)


def test_config4_calibration_full():
    """1 x 6.5e6 float64 with integer counts as weights and rational labels
    (many exact ties): the fit, the partition's validity and clip flags
    against the oracle's, and both backward products at full size."""
    wl = workloads.cfg4_calibration()
    _print(f"config 4: {wl.name} {wl.y.shape}")
    fit, b, *_ = gpu_fit(wl)
    z, bs, cl, rn, st = oracle_fit(wl)
    check_fit(fit.cpu().numpy(), z, wl.y, wl.y.dtype, wl.increasing, wl.name)
    gs, gc, grn = gpu_blocks(b)
    assert grn[0] == 0
    check_partition(gs, gc, grn, wl.y, wl.w, True, 0.0, 1.0, wl.name)
    _check_vjp(wl, b, gs, gc, grn, 104, wl.name)


def test_config5_dense_full_sampled_rows():
    wl = workloads.cfg5_dense()
    _print(f"config 5: {wl.name} {wl.y.shape}")
    fit, b, *_ = gpu_fit(wl)
    f = fit.cpu().numpy()
    rows = [0, 13, 31]
    z, *_ = oracle_fit(wl, rows=rows)
    check_fit(f[rows], z, wl.y[rows], wl.y.dtype, True, wl.name)
    gs, gc, grn = gpu_blocks(b)
    check_partition(gs[rows], gc[rows], grn[rows], wl.y[rows], wl.w[rows], True, None, None, wl.name)
    # every row: monotone up to rounding and the weighted sum preserved
    s = scale_of(wl.y)
    assert np.all(np.diff(f, axis=1) >= -1e-12 * s)
    lhs = np.einsum("ij,ij->i", wl.w, f)
    rhs = np.einsum("ij,ij->i", wl.w, wl.y)
    assert np.all(np.abs(lhs - rhs) <= 1e-9 * np.abs(wl.w * wl.y).sum(axis=1))


@pytest.mark.parametrize("kind", ["increasing", "trend_noise"])
def test_rows_past_4096_chunks(kind):
    """Rows of 1.6e7 float64 elements (4465 chunks, more than the top merge keeps
    in LDS, so its descriptors stay in global memory): every point a vertex
    (increasing data, the first page's Sec. 7.5 regime) and trend plus noise.
    The fit, the partition and the clip flags against the oracle's."""
    n = 16_000_000
    wl = workloads.family(kind, 1, n, seed=17, dtype=np.float64, weights="uniform")
    wl.y_min, wl.y_max = 0.05, 0.95
    _print(f"long row: {wl.name}")
    fit, b, *_ = gpu_fit(wl)
    z, bs, cl, rn, _ = oracle_fit(wl)
    check_fit(fit.cpu().numpy(), z, wl.y, np.float64, True, wl.name)
    del z, bs, cl
    gs, gc, grn = gpu_blocks(b)
    check_partition(gs, gc, grn, wl.y, wl.w, True, wl.y_min, wl.y_max, wl.name)


# Row lengths that reach each path of the fit: one row per lane (24), two lanes
# (50), one wave with K = 2, 4, 8 points per lane (100, 200, 400), several waves
# with K = 16 (3000), K = 20 for float32 and 12 for float64 (5000), K = 12
# (6000), and the chunked path (20000).
SHAPE_SIZES = [24, 50, 100, 200, 400, 3000, 5000, 6000, 20000]


@pytest.mark.parametrize("n", SHAPE_SIZES)
@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("inc", [True, False])
def test_partition_and_clip_bits_every_row_shape(n, dtype, inc):
    """Block-start and clip bits against the oracle's on tie-free data for every
    row kernel, both dtypes, both orientations, clipped (the first page's
    Appendix B, "Tests": gradients against the CPU on data without near-ties),
    then both backward products."""
    rows = 12
    a = workloads.family("trend_noise", rows - 4, n, seed=n % 61, dtype=dtype, weights="uniform")
    b_ = workloads.family("noise", 4, n, seed=n % 67, dtype=dtype, weights="extreme")
    y = np.concatenate([a.y, b_.y])
    w = np.concatenate([a.w, b_.w])
    if not inc:
        y = y[:, ::-1].copy()
        w = w[:, ::-1].copy()
    wl = workloads.Workload(f"shapes_{rows}x{n}_{np.dtype(dtype).name}_inc{int(inc)}", y, w, inc, 0.2, 0.7)
    fit, b, *_ = gpu_fit(wl)
    z, *_ = oracle_fit(wl)
    check_fit(fit.cpu().numpy(), z, wl.y, dtype, inc, wl.name)
    gs, gc, grn = gpu_blocks(b)
    check_partition(gs, gc, grn, wl.y, wl.w, inc, 0.2, 0.7, wl.name)
    _check_vjp(wl, b, gs, gc, grn, n, wl.name)


@pytest.mark.parametrize("n", [330, 400, 450, 512])
@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("inc", [True, False])
def test_one_wave_rows_past_the_lds_list(n, dtype, inc):
    """One-wave rows (8 points per lane) whose lane hulls hold more vertices than
    the kernel's LDS list (dense data: increasing, or a sawtooth under a trend),
    so the second kernel refits them with the whole list in LDS, mixed in one
    launch with noise rows that the first kernel finishes."""
    parts = [workloads.family("increasing", 3, n, seed=n, dtype=dtype, weights="uniform"),
             workloads.family("sawtooth", 3, n, seed=n + 1, dtype=dtype, weights="extreme"),
             workloads.family("noise", 3, n, seed=n + 2, dtype=dtype, weights="uniform")]
    y = np.concatenate([p.y for p in parts])
    w = np.concatenate([p.w for p in parts])
    if not inc:
        y = y[:, ::-1].copy()
        w = w[:, ::-1].copy()
    wl = workloads.Workload(f"ovf_9x{n}_{np.dtype(dtype).name}_inc{int(inc)}", y, w, inc, -0.5, 0.9)
    fit, b, *_ = gpu_fit(wl)
    z, *_ = oracle_fit(wl)
    check_fit(fit.cpu().numpy(), z, wl.y, dtype, inc, wl.name)
    gs, gc, grn = gpu_blocks(b)
    check_partition(gs, gc, grn, wl.y, wl.w, inc, -0.5, 0.9, wl.name)
    _check_vjp(wl, b, gs, gc, grn, n + 7, wl.name)


PACK_SIZES = [33, 34, 47, 48, 63, 64, 65, 80, 81, 100, 127, 128, 129, 200, 256, 257, 300, 400, 511, 512]


@pytest.mark.parametrize("n", PACK_SIZES)
@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_packed_rows(n, dtype):
    """Rows of 33 to 512 elements: up to 128 packed several to a wave (the first page, Sec. 3.5; dense waves
    refitted by the second pass with 8 points per lane), longer ones a wave each.  1001 rows (the last wave
    ragged) of noise, trend noise, increasing data (every point a vertex), a sawtooth and integer ties,
    interleaved so that every wave mixes them, with a NaN row and a row with a weight <= 0 among them; both
    orientations, clipped.  The fit, the partition and clip bits against the oracle, and both products."""
    rows = 1001
    kinds = [("noise", "uniform"), ("trend_noise", "extreme"), ("increasing", "uniform"), ("sawtooth", "unit"),
             ("ties", "uniform")]
    parts = [workloads.family(k, rows // len(kinds) + 1, n, seed=n + 13 * j, dtype=dtype, weights=wt)
             for j, (k, wt) in enumerate(kinds)]
    ws = [p.w if p.w is not None else np.ones_like(p.y) for p in parts]
    y = np.stack([parts[q % len(kinds)].y[q // len(kinds)] for q in range(rows)])
    w = np.stack([ws[q % len(kinds)][q // len(kinds)] for q in range(rows)])
    y[7, n // 2] = np.nan
    w[500, 3] = -1.0
    for inc, clip in ((True, None), (False, (-0.4, 0.6))):
        yy = y if inc else y[:, ::-1].copy()
        ww = w if inc else w[:, ::-1].copy()
        wl = workloads.Workload(f"packed_{rows}x{n}_{np.dtype(dtype).name}_inc{int(inc)}", yy, ww, inc)
        if clip:
            wl.y_min, wl.y_max = clip
        _print(wl.name)
        fit, b, *_ = gpu_fit(wl)
        z, bs, cl, rn, st = oracle_fit(wl)
        f = fit.cpu().numpy()
        check_fit(f, z, wl.y, dtype, inc, wl.name)
        gs, gc, grn = gpu_blocks(b)
        assert grn[7] == 1 and grn[500] == 1 and grn.sum() == 2
        check_partition(gs, gc, grn, wl.y, wl.w, inc, wl.y_min, wl.y_max, wl.name)
        _check_vjp(wl, b, gs, gc, grn, n + 3, wl.name)


SIZES = [1, 2, 3, 63, 64, 65, 127, 129, 257, 513, 1000, 3583, 3584, 3585, 4096, 4097, 4500, 5120, 5121, 6143, 6144, 6145, 7168, 7169,
         8193, 12289, 20001, 65537]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_ragged_sizes(n, dtype):
    for kind, weights, inc, clip in [("noise", "uniform", True, None), ("trend_noise", "unit", False, (-0.2, 0.9))]:
        wl = workloads.family(kind, 3, n, seed=n % 97, dtype=dtype, weights=weights, increasing=inc)
        if clip:
            wl.y_min, wl.y_max = clip
        fit, b, *_ = gpu_fit(wl)
        z, *_ = oracle_fit(wl)
        check_fit(fit.cpu().numpy(), z, wl.y, dtype, inc, f"{wl.name} n={n}")
        check_partition(*gpu_blocks(b), wl.y, wl.w, inc, wl.y_min, wl.y_max, f"{wl.name} n={n}")


@pytest.mark.parametrize("kind", workloads.FAMILIES)
@pytest.mark.parametrize("n", [5000, 50000])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_families(kind, n, dtype):
    if kind == "consecutive" and n > 5000:
        n = 20000
    for weights in ("unit", "uniform", "extreme"):
        wl = workloads.family(kind, 2, n, seed=3, dtype=dtype, weights=weights)
        fit, b, *_ = gpu_fit(wl)
        z, *_ = oracle_fit(wl)
        check_fit(fit.cpu().numpy(), z, wl.y, dtype, True, f"{wl.name}")
        check_partition(*gpu_blocks(b), wl.y, wl.w, True, None, None, wl.name)


@pytest.mark.parametrize("kind", workloads.FAMILIES)
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_vjp_long_row_families(kind, dtype):
    """Rows of four 4096-element tiles and a ragged tail, of every data family,
    plus a row of two blocks that meet exactly at a tile boundary: the fit's
    partition, then both backward products against the oracle.  Decreasing
    and constant rows are one block, so whole tiles hold no block start;
    increasing rows start a block at every element."""
    n = 4 * 4096 + 77
    wl = workloads.family(kind, 3, n, seed=11, dtype=dtype, weights="uniform")
    i = np.arange(n)
    two = np.where(i < 8192, -1e-6 * i, 1.0 - 1e-6 * (i - 8192)).astype(dtype)
    wl.y = np.concatenate([wl.y, two[None, :]])
    wl.w = np.concatenate([wl.w, workloads.rng(12).uniform(0.5, 2.0, (1, n)).astype(dtype)])
    fit, b, *_ = gpu_fit(wl)
    z, *_ = oracle_fit(wl)
    check_fit(fit.cpu().numpy(), z, wl.y, dtype, True, wl.name)
    gs, gc, grn = gpu_blocks(b)
    check_partition(gs, gc, grn, wl.y, wl.w, True, None, None, wl.name)
    assert gs[3, 8192] and gs[3].sum() == 2
    _check_vjp(wl, b, gs, gc, grn, 17, wl.name)


@pytest.mark.parametrize("n", [2500, 5000, 6144])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_rows_past_the_lds_list_mixed_with_others(n, dtype):
    """One batch whose rows alternate between noise (a short vertex list, kept
    in LDS) and increasing or sawtooth data (every point or most points a
    lane-hull vertex, more than the LDS list holds: refitted with the list in
    global memory), so both kernels of the single-workgroup path write rows of
    the same launch."""
    parts = [workloads.family("noise", 2, n, seed=7, dtype=dtype, weights="uniform"),
             workloads.family("increasing", 2, n, seed=8, dtype=dtype, weights="uniform"),
             workloads.family("sawtooth", 2, n, seed=9, dtype=dtype, weights="extreme")]
    y = np.stack([parts[k % 3].y[k // 3] for k in range(6)])
    w = np.stack([parts[k % 3].w[k // 3] for k in range(6)])
    wl = workloads.Workload(f"mixed_6x{n}_{np.dtype(dtype).name}", y, w, True)
    fit, *_ = gpu_fit(wl)
    z, *_ = oracle_fit(wl)
    check_fit(fit.cpu().numpy(), z, wl.y, dtype, True, wl.name)


@pytest.mark.parametrize("n", [2500, 5000, 6144])
@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_rows_whose_wrap_gives_up(n, dtype):
    """A staircase rising by one every tenth element under small noise: the
    lanes' half hulls keep about 30% of the points (5000: about 1500, within
    the LDS list), all below the row's chord, so the output-sensitive finish
    is tried, but every wave's hull has hundreds of vertices and the wrap
    gives up at its step cap; the row is then fitted by the exact path in the
    same launch.  Mixed with noise rows (which the wrap finishes) and fitted
    in both orientations, with unit and uniform weights."""
    r = workloads.rng(4400 + n)
    i = np.arange(n)
    stairs = np.floor(i / 10.0)[None, :] + 0.1 * r.standard_normal((3, n))
    noise = r.standard_normal((3, n))
    y = np.concatenate([stairs, noise]).astype(dtype)
    for inc in (True, False):
        yy = y if inc else y[:, ::-1].copy()
        for w in (None, r.uniform(0.1, 1.1, y.shape).astype(dtype)):
            wl = workloads.Workload(f"stairs_6x{n}_{np.dtype(dtype).name}", yy, w, inc)
            fit, *_ = gpu_fit(wl)
            z, *_ = oracle_fit(wl)
            check_fit(fit.cpu().numpy(), z, wl.y, dtype, inc, f"{wl.name} inc={inc} w={w is not None}")


@pytest.mark.parametrize("n", [1, 2, 5, 15, 16, 17, 24, 31, 32, 33, 40, 48, 64, 65])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_short_rows_one_per_lane(n, dtype):
    """Rows of at most 32 elements are fitted one row per lane, rows of 33 to
    64 on two lanes whose hulls are merged across point 32 (the first page,
    Sec. 3.5: short rows packed several to a warp), 65 goes to the one-wave
    tile: many rows of several families, both orientations, clipped and not,
    with block bits and both backward products."""
    import weighted_isotonic_regression_row_amd as iso
    r = workloads.rng(900 + n)
    rows = 3000
    parts = []
    for kind, weights in (("noise", "uniform"), ("trend_noise", "extreme"), ("ties", "unit"), ("increasing", "unit"),
                          ("constant", "uniform"), ("sawtooth", "uniform")):
        parts.append(workloads.family(kind, rows // 6, n, seed=n, dtype=dtype, weights=weights))
    y = np.concatenate([p.y for p in parts])
    w = np.concatenate([p.w if p.w is not None else np.ones_like(p.y) for p in parts])
    for inc, clip in ((True, None), (False, (-0.3, 0.4))):
        wl = workloads.Workload(f"short_{rows}x{n}_{np.dtype(dtype).name}", y, w, inc)
        if clip:
            wl.y_min, wl.y_max = clip
        fit, b, yd, wd = gpu_fit(wl)
        z, bs, cl, rn, _ = oracle_fit(wl)
        check_fit(fit.cpu().numpy(), z, wl.y, dtype, inc, wl.name)
        gs, gc, grn = gpu_blocks(b)
        assert not grn.any()
        # the partition is unique away from exact ties; on tie data compare the fit only
        g = r.standard_normal(y.shape).astype(dtype)
        gy, gw = iso.iso_vjp_yw(to_dev(g), b, yd)
        ref_y = oracle.vjp(g.astype(np.float64), gs, gc, grn, w.astype(np.float64))
        ref_w = oracle.vjp_w(g.astype(np.float64), y.astype(np.float64), gs, gc, grn, w.astype(np.float64))
        tol = 1e-12 if dtype == np.float64 else 2e-6
        assert np.max(np.abs(gy.cpu().numpy().astype(np.float64) - ref_y)) <= tol * max(1.0, np.abs(ref_y).max())
        assert np.max(np.abs(gw.cpu().numpy().astype(np.float64) - ref_w)) <= tol * max(1.0, np.abs(ref_w).max())
        # block starts agree with the oracle's on the tie-free noise rows
        k = rows // 6
        np.testing.assert_array_equal(gs[:k], bs[:k])


def test_partition_is_valid_on_tie_data():
    # integer data with many exact ties: the GPU's own blocks must be blocks of
    # its fit (constant inside, the block's weighted mean)
    wl = workloads.family("ties", 3, 9000, seed=5, dtype=np.float64, weights="unit")
    fit, b, *_ = gpu_fit(wl)
    f = fit.cpu().numpy()
    gs, gc, grn = gpu_blocks(b)
    for r in range(wl.rows):
        st = np.nonzero(gs[r])[0].tolist() + [wl.n]
        assert st[0] == 0
        for a, e in zip(st[:-1], st[1:]):
            m = wl.y[r, a:e].mean()
            assert np.all(np.abs(f[r, a:e] - m) <= 1e-12 * max(1.0, abs(m)))


@pytest.mark.parametrize("n", [512, 5000, 8192, 12288, 20000, 70001])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_vjp_matches_oracle(n, dtype):
    import weighted_isotonic_regression_row_amd as iso
    wl = workloads.family("trend_noise", 3, n, seed=n % 89, dtype=dtype, weights="uniform", increasing=(n % 2 == 0))
    wl.y_min, wl.y_max = 0.1, 0.8
    r = workloads.rng(123)
    g = r.standard_normal(wl.y.shape).astype(dtype)
    fit, b, y, w = gpu_fit(wl)
    gy = iso.iso_vjp(to_dev(g), b).cpu().numpy().astype(np.float64)
    gs, gc, grn = gpu_blocks(b)
    # the oracle's VJP on the GPU's own partition (the first page's rule for
    # ties; on this data the partitions also agree, checked above)
    ref = oracle.vjp(g.astype(np.float64), gs, gc, grn, None if wl.w is None else wl.w.astype(np.float64))
    tol = (1e-12 if dtype == np.float64 else 2e-6) * max(1.0, np.abs(ref).max())
    assert np.max(np.abs(gy - ref)) <= tol


@pytest.mark.parametrize("n", [1, 63, 700, 5000, 6144, 6145, 20001])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("weighted", [True, False])
def test_vjp_w_matches_oracle(n, dtype, weighted):
    """grad_w = G_B (y_j - mean_B) / W_B (page "torchisotonic", "Semantics": the
    fit is differentiable in the weights) against the oracle on the GPU's own
    partition; single-tile and multi-tile rows, clipped, both orientations."""
    import weighted_isotonic_regression_row_amd as iso
    wl = workloads.family("trend_noise", 3, n, seed=n % 83, dtype=dtype, weights="uniform" if weighted else "unit",
                          increasing=(n % 2 == 1))
    if not weighted:
        wl.w = None
    wl.y_min, wl.y_max = 0.1, 0.8
    r = workloads.rng(321)
    g = r.standard_normal(wl.y.shape).astype(dtype)
    fit, b, y, w = gpu_fit(wl)
    gy, gw = iso.iso_vjp_yw(to_dev(g), b, y)
    gy_only = iso.iso_vjp(to_dev(g), b)
    np.testing.assert_array_equal(gy.cpu().numpy(), gy_only.cpu().numpy())
    gs, gc, grn = gpu_blocks(b)
    w64 = None if wl.w is None else wl.w.astype(np.float64)
    ref_w = oracle.vjp_w(g.astype(np.float64), wl.y.astype(np.float64), gs, gc, grn, w64)
    ref_y = oracle.vjp(g.astype(np.float64), gs, gc, grn, w64)
    tol = 1e-12 if dtype == np.float64 else 2e-6
    gwn = gw.cpu().numpy().astype(np.float64)
    gyn = gy.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(gwn - ref_w)) <= tol * max(1.0, np.abs(ref_w).max()), f"grad_w n={n}"
    assert np.max(np.abs(gyn - ref_y)) <= tol * max(1.0, np.abs(ref_y).max()), f"grad_y n={n}"
    # the fit does not change when all weights are scaled: sum_j w_j grad_w_j = 0 per row
    wv = np.ones_like(gwn) if wl.w is None else wl.w.astype(np.float64)
    assert np.max(np.abs(np.sum(wv * gwn, axis=1))) <= 50 * tol * max(1.0, np.abs(wv * gwn).sum(axis=1).max())


@pytest.mark.parametrize("n", [16, 40, 300, 5000, 20001])
def test_vjp_non_finite_gradient_stays_in_its_block(n):
    """An infinite or NaN upstream gradient reaches only its own block (the
    product is a sum over the block, Appendix C of the first page): +inf, NaN
    and -inf in one row each, on every backward kernel shape (one row per lane,
    two lanes, one workgroup, tiles with carries).  Both products match the
    oracle's on the finite elements, and the non-finite elements are exactly
    the block that holds the value (the oracle's compensated sums turn an
    infinity into NaN, so only finiteness is compared there)."""
    import weighted_isotonic_regression_row_amd as iso
    wl = workloads.family("trend_noise", 3, n, seed=n % 71, dtype=np.float64, weights="uniform")
    fit, b, y, w = gpu_fit(wl)
    gs, gc, grn = gpu_blocks(b)
    g = workloads.rng(5).standard_normal(wl.y.shape)
    pos = [n // 3, n // 2, (2 * n) // 3]
    for r, v in enumerate((np.inf, np.nan, -np.inf)):
        g[r, pos[r]] = v
    gy, gw = iso.iso_vjp_yw(to_dev(g), b, y)
    w64 = wl.w.astype(np.float64)
    ref_y = oracle.vjp(g, gs, gc, grn, w64)
    ref_w = oracle.vjp_w(g, wl.y.astype(np.float64), gs, gc, grn, w64)
    for r in range(3):
        starts = np.flatnonzero(gs[r])
        lo = starts[starts <= pos[r]].max()
        later = starts[starts > pos[r]]
        hi = later.min() if later.size else n
        block = np.zeros(n, dtype=bool)
        block[lo:hi] = True
        assert not np.isfinite(ref_y[r][block]).any()
        assert np.isfinite(ref_y[r][~block]).all()
    for got, ref, name in ((gy, ref_y, "grad_y"), (gw, ref_w, "grad_w")):
        got = got.cpu().numpy()
        assert np.array_equal(np.isfinite(got), np.isfinite(ref)), f"{name}: non-finite pattern"
        ok = np.isfinite(ref)
        err = float(np.max(np.abs(got[ok] - ref[ok]), initial=0.0))
        assert err <= 1e-12 * max(1.0, float(np.abs(ref[ok]).max(initial=0.0))), f"{name} off by {err:.3e}"


@pytest.mark.parametrize("n", [300, 20000])
def test_vjp_w_nan_rows(n):
    import weighted_isotonic_regression_row_amd as iso
    r = workloads.rng(8)
    y = r.standard_normal((3, n))
    w = r.random((3, n)) + 0.1
    y[1, n // 2] = np.nan
    wl = workloads.Workload("nan", y, w, True)
    fit, b, yd, wd = gpu_fit(wl)
    gy, gw = iso.iso_vjp_yw(to_dev(r.standard_normal((3, n))), b, yd, want_y=False)
    assert gy is None
    gwn = gw.cpu().numpy()
    assert np.isnan(gwn[1]).all() and np.isfinite(gwn[[0, 2]]).all()


def test_config3_soft_rank_forward_backward():
    import weighted_isotonic_regression_row_amd as iso
    wl = workloads.cfg3_soft_rank()
    fit, b, y, w = gpu_fit(wl)
    z, bs, cl, rn, _ = oracle_fit(wl)
    check_fit(fit.cpu().numpy(), z, wl.y, wl.y.dtype, True, wl.name)
    gy = iso.iso_vjp(to_dev(wl.g), b).cpu().numpy().astype(np.float64)
    ref = oracle.vjp(wl.g.astype(np.float64), bs, cl, rn)
    # every row is one block: the VJP is the row mean of g
    assert bs[:, 1:].sum() == 0
    np.testing.assert_allclose(gy, ref, rtol=0, atol=2e-6)
    gs, *_ = gpu_blocks(b)
    np.testing.assert_array_equal(gs, bs)


@pytest.mark.parametrize("n", [16, 300, 20000])
def test_nan_rows_and_weight_errors(n):
    import weighted_isotonic_regression_row_amd as iso
    r = workloads.rng(7)
    y = r.standard_normal((5, n))
    w = r.random((5, n)) + 0.1
    y[1, n // 3] = np.nan
    w[2, n // 2] = np.nan
    y[3, -1] = np.inf
    w[4, 0] = -1.0
    wl = workloads.Workload("nan_rows", y, w, True)
    fit, b, yd, wd = gpu_fit(wl, check=False)
    f = fit.cpu().numpy()
    z, *_ = oracle_fit(wl)
    check_fit(f, z, y, np.float64, True, "nan rows")
    assert np.isnan(f[1:]).all() and not np.isnan(f[0]).any()
    gs, gc, grn = gpu_blocks(b)
    assert list(grn) == [0, 1, 1, 1, 1]
    with pytest.raises(ValueError):
        iso.iso_fit(yd, wd, True)
    # weight error only: still reported when no row has a NaN
    wl2 = workloads.Workload("w0", y[[0, 4]].copy(), w[[0, 4]].copy(), True)
    with pytest.raises(ValueError):
        iso.iso_fit(to_dev(wl2.y), to_dev(wl2.w))
    # NaN rows alone are not an error
    iso.iso_fit(to_dev(y[[0, 1]]), to_dev(w[[0, 1]]), check=True)
    g = np.ones_like(y)
    gy = iso.iso_vjp(to_dev(g), b).cpu().numpy()
    assert np.isnan(gy[1:]).all() and np.isfinite(gy[0]).all()


@pytest.mark.parametrize("shape", [(200, 5000), (2, 300000)])
def test_deterministic(shape):
    import torch
    import weighted_isotonic_regression_row_amd as iso
    wl = workloads.family("trend_noise", shape[0], shape[1], seed=2, dtype=np.float32, weights="uniform")
    y, w = to_dev(wl.y), to_dev(wl.w)
    f0, _ = iso.iso_fit(y, w, blocks=False, check=False)
    f0 = f0.clone()
    for _ in range(5):
        f1, _ = iso.iso_fit(y, w, blocks=False, check=False)
        assert torch.equal(f0, f1)


def test_empty_inputs():
    import torch
    import weighted_isotonic_regression_row_amd as iso
    for shape in [(0, 10), (4, 0)]:
        y = torch.empty(shape, dtype=torch.float64, device="cuda:0")
        f, b = iso.iso_fit(y)
        assert f.shape == shape
        g = iso.iso_vjp(torch.empty(shape, dtype=torch.float64, device="cuda:0"), b)
        assert g.shape == shape


# ---------------------------------------------------------------- soft rank (first page, Sec. 7.9)

SR_SIZES = [1, 2, 63, 65, 100, 512, 1000, 4096, 5000, 6144, 6145, 8192, 8193, 10000, 30001]


def _soft_rank_case(x, eps, dtype, what, check_partition=None):
    import torch
    import weighted_isotonic_regression_row_amd as iso
    rows, n = x.shape
    r_gpu, st = iso.soft_rank(to_dev(x), eps)
    torch.cuda.synchronize()
    r_ref, perm, bs, rn = oracle.soft_rank(x.astype(np.float64), eps)
    # the sorting permutation is index work: bit-exact, ties in index order.  A row holding a NaN comes
    # back all NaN whatever its order, so there it only has to be a permutation.
    finite = np.isfinite(x).all(axis=1)
    gperm = st.perm().cpu().numpy()
    np.testing.assert_array_equal(gperm[finite], perm[finite], err_msg=what)
    np.testing.assert_array_equal(np.sort(gperm, axis=1), np.broadcast_to(np.arange(n), (rows, n)))
    rank = st.rank().cpu().numpy()
    np.testing.assert_array_equal(np.take_along_axis(rank, gperm, axis=1), np.broadcast_to(np.arange(n), (rows, n)))
    perm = np.where(finite[:, None], perm, gperm)
    # ranks: within the fit's tolerance of the scale of z = s - (n..1)
    scale = (float(np.abs(x[finite].astype(np.float64)).max()) / eps if finite.any() else 0.0) + n
    rg = r_gpu.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(rg), np.isnan(r_ref)), what
    ok = ~np.isnan(r_ref)
    if ok.any():
        err = float(np.max(np.abs(rg[ok] - r_ref[ok])))
        tol = (TOL_F64 if dtype == np.float64 else TOL_F32) * scale
        assert err <= tol, f"{what}: ranks off by {err:.3e} > {tol:.3e}"
        # in sorted order the ranks do not increase, up to rounding of the scale
        srt = np.take_along_axis(rg, perm, axis=1)[finite]
        up = float(np.max(np.diff(srt, axis=1), initial=0.0))
        slack = (1e-12 if dtype == np.float64 else 4 * float(np.spacing(np.float32(scale))))
        assert up <= slack, f"{what}: ranks out of order by {up:.3e}"
    gsb, gcb, grn = gpu_blocks(st.blocks)
    np.testing.assert_array_equal(grn.astype(bool), rn.astype(bool))
    if check_partition:
        np.testing.assert_array_equal(gsb[finite], bs[finite])
    return st, perm, (gsb, grn), r_ref


@pytest.mark.gpu
@pytest.mark.parametrize("n", SR_SIZES)
@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_soft_rank_matches_oracle(n, dtype):
    """Soft ranks and their product against the oracle: both strengths of the first page's Sec. 7.9
    (eps = 1, where rows pool into few blocks, and eps = 1/n, near the hard ranks); rows of one wave,
    of several waves, and beyond one workgroup's fit (6145 and more: chunked fit)."""
    import weighted_isotonic_regression_row_amd as iso
    rows = 3 if n > 1000 else 17
    x, g = workloads.soft_rank_input(rows, n, seed=n % 97, dtype=dtype)
    for eps in (1.0, 1.0 / n):
        st, perm, (gsb, grn), _ = _soft_rank_case(x, eps, dtype, f"n={n} eps={eps}",
                                                   check_partition=(dtype == np.float64))
        d = iso.soft_rank_vjp(to_dev(g), st).cpu().numpy().astype(np.float64)
        # the product on the GPU's own partition (exact ties of block means may split either way)
        ref = oracle.soft_rank_vjp(g.astype(np.float64), eps, perm, gsb, grn)
        tol = (1e-12 if dtype == np.float64 else 2e-6) * max(1.0, float(np.abs(ref).max()))
        err = float(np.max(np.abs(d - ref)))
        assert err <= tol, f"n={n} eps={eps}: product off by {err:.3e} > {tol:.3e}"


@pytest.mark.gpu
def test_soft_rank_config3_shape():
    """4096 x 512 float32 standard normal scores, eps = 1 and 1/512, forward and backward (the soft-rank
    shape of the first page's Table 6, at the size of the batch it is measured on here)."""
    import weighted_isotonic_regression_row_amd as iso
    x, g = workloads.soft_rank_input()
    for eps in (1.0, 1.0 / 512):
        st, perm, (gsb, grn), _ = _soft_rank_case(x, eps, np.float32, f"4096x512 eps={eps}")
        d = iso.soft_rank_vjp(to_dev(g), st).cpu().numpy().astype(np.float64)
        ref = oracle.soft_rank_vjp(g.astype(np.float64), eps, perm, gsb, grn)
        assert float(np.max(np.abs(d - ref))) <= 2e-6 * max(1.0, float(np.abs(ref).max()))


@pytest.mark.gpu
@pytest.mark.parametrize("rows,n,dtype", [(64, 10_000, np.float32), (1, 1_000_000, np.float32),
                                          (1, 1_000_000, np.float64)])
def test_soft_rank_long_rows(rows, n, dtype):
    """The long soft-rank shapes of the first page's Table 6 (64 x 10^4 and 1 x 10^6), sorted by tiles and
    merge passes: permutation bit for bit, ranks and the product against the oracle, at eps = 1 and 1/n."""
    import weighted_isotonic_regression_row_amd as iso
    x, g = workloads.soft_rank_input(rows, n, seed=29, dtype=dtype)
    if rows > 1:
        x[rows // 2, n // 3] = np.nan  # that row alone comes back NaN
    for eps in (1.0, 1.0 / n):
        _print(f"soft rank {rows}x{n} {np.dtype(dtype).name} eps={eps}")
        st, perm, (gsb, grn), _ = _soft_rank_case(x, eps, dtype, f"{rows}x{n} eps={eps}")
        d = iso.soft_rank_vjp(to_dev(g), st).cpu().numpy().astype(np.float64)
        ref = oracle.soft_rank_vjp(g.astype(np.float64), eps, perm, gsb, grn)
        assert np.array_equal(np.isnan(d), np.isnan(ref)), f"{rows}x{n} eps={eps}: NaN rows of the product"
        ok = ~np.isnan(ref)
        tol = (1e-12 if dtype == np.float64 else 2e-6) * max(1.0, float(np.abs(ref[ok]).max()))
        assert float(np.max(np.abs(d[ok] - ref[ok]))) <= tol, f"{rows}x{n} eps={eps}: product"


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_soft_rank_ties_signed_zeros_and_nan_rows(dtype):
    """Equal values (and -0 against +0) sort in index order and share one rank; a row holding a NaN comes
    back NaN, forward and backward, without disturbing the other rows."""
    import weighted_isotonic_regression_row_amd as iso
    r = workloads.rng(11)
    x = r.integers(-3, 4, size=(6, 300)).astype(dtype)
    x[0, ::7] = -0.0
    x[0, 3::7] = 0.0
    x[2, 150] = np.nan
    x[4, 0] = np.nan
    for eps in (1.0, 0.01):
        st, perm, (gsb, grn), r_ref = _soft_rank_case(x, eps, dtype, f"ties eps={eps}")
        rg = iso.soft_rank(to_dev(x), eps)[0].cpu().numpy()
        for row in (0, 1, 3, 5):
            for v in np.unique(x[row]):
                vals = rg[row][x[row] == v]
                assert np.all(vals == vals[0])
        g = np.ones_like(x)
        d = iso.soft_rank_vjp(to_dev(g), st).cpu().numpy()
        assert np.isnan(d[[2, 4]]).all() and not np.isnan(d[[0, 1, 3, 5]]).any()


# ---------------------------------------------------------------- calibration (first page, Sec. 7.7; PyPI usage)

def _calibration_case(s, y, q, what):
    import torch
    import weighted_isotonic_regression_row_amd as iso
    dtype = s.dtype
    xs, fit, m = iso.calibration_fit(to_dev(s), to_dev(y))
    p = iso.calibrate(to_dev(q), xs, fit, m)
    torch.cuda.synchronize()
    rx, rf, rm = oracle.calibration_fit(s.astype(np.float64), y.astype(np.float64))
    gm = m.cpu().numpy()
    np.testing.assert_array_equal(gm, rm, err_msg=what)           # the number of distinct scores: exact
    gx = xs.cpu().numpy().astype(np.float64)
    gf = fit.cpu().numpy().astype(np.float64)
    finite = np.isfinite(y)
    scale = float(np.abs(y[finite]).max()) if finite.any() else 1.0
    tol = (TOL_F64 if dtype == np.float64 else TOL_F32) * max(scale, 1e-300)
    for r in range(s.shape[0]):
        k = int(rm[r])
        if k == 0:
            continue
        assert np.array_equal(gx[r, :k], rx[r, :k]), f"{what}: distinct scores of row {r}"
        assert np.isnan(gx[r, k:]).all(), f"{what}: xs past m in row {r}"
        err = float(np.max(np.abs(gf[r, :k] - rf[r, :k])))
        assert err <= tol, f"{what}: curve of row {r} off by {err:.3e} > {tol:.3e}"
        assert (np.diff(gf[r, :k]) >= -MONO_SLACK[np.dtype(dtype)] * scale).all(), f"{what}: curve of row {r} decreases"
    ref = oracle.calibrate(q.astype(np.float64), rx, rf, rm)
    gp = p.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(gp), np.isnan(ref)), f"{what}: NaN pattern of the predictions"
    ok = ~np.isnan(ref)
    if ok.any():
        err = float(np.max(np.abs(gp[ok] - ref[ok])))
        assert err <= 2 * tol, f"{what}: predictions off by {err:.3e}"


MONO_SLACK = {np.dtype(np.float64): 1e-12, np.dtype(np.float32): 4 * 2.0 ** -23}
CAL_SIZES = [1, 2, 100, 2048, 2049, 8192, 8193, 20000, 70001]


@pytest.mark.gpu
@pytest.mark.parametrize("n", CAL_SIZES)
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_calibration_matches_oracle(n, dtype):
    """Curves and predictions against the oracle: one pool tile and ragged ones, one sort tile and several
    merged (8193 and more), coarse scores (many ties), Bernoulli and continuous labels, several rows."""
    r = workloads.rng(600 + n % 101)
    rows = 3 if n <= 20000 else 1
    s = np.round(r.standard_normal((rows, n)), 2).astype(dtype)
    p = 1.0 / (1.0 + np.exp(-(1.5 * s.astype(np.float64) - 1.0)))
    y = (r.random((rows, n)) < p).astype(dtype)
    if rows > 1:
        y[1] = (p[1] + 0.2 * r.standard_normal(n)).astype(dtype)
    q = np.concatenate([np.linspace(-5, 5, 257)[None, :].repeat(rows, 0), s[:, :64]], axis=1).astype(dtype)
    _calibration_case(s, y, q, f"n={n}")


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_calibration_edge_rows(dtype):
    """All scores equal (one point: a constant curve), -0 against +0 (one score), distinct scores (nothing to
    pool), and rows holding a NaN score or label (no curve: m = 0, NaN predictions)."""
    r = workloads.rng(31)
    n = 3000
    s = r.standard_normal((6, n))
    s[0] = 0.25
    s[1, ::2] = -0.0
    s[1, 1::2] = 0.0
    s[2] = r.permutation(n)
    s[3, 17] = np.nan
    y = r.random((6, n))
    y[4, 5] = np.nan
    s, y = s.astype(dtype), y.astype(dtype)
    q = np.concatenate([np.linspace(-3, 3, 101)[None, :].repeat(6, 0), s[:, :20]], axis=1).astype(dtype)
    q[5, 3] = np.nan
    _calibration_case(s, y, q, "edge rows")


@pytest.mark.gpu
def test_calibration_day_of_scores():
    """6.5 million float64 scores of one curve (the first page's Sec. 7.7 day, synthetic): scores on a grid
    of 1e-5 (pooled runs of equal scores), click labels from a logistic curve."""
    s, y, q = workloads.calibration_input()
    _calibration_case(s, y, q, "6.5e6 scores")


@pytest.mark.gpu
@pytest.mark.parametrize("n", [5000, 300, 24, 20000])
def test_fit_replayed_from_a_hip_graph(n):
    """The fit call captured in a HIP graph (it records kernel launches only, no memset) gives the eager
    result bit for bit on every replay, with eager work and synchronisations between the replays;
    one-workgroup rows, one-wave rows, one-row-per-lane rows and chunked rows (several launches)."""
    import torch
    import weighted_isotonic_regression_row_amd as iso
    rows = 64 if n <= 5000 else 4
    wl = workloads.family("noise", rows, n, seed=n, dtype=np.float32, weights="uniform", increasing=False)
    wl.y_min, wl.y_max = 0.0, 1.0
    y, w = to_dev(wl.y), to_dev(wl.w)
    ws = iso.workspace(rows, n, y.dtype, y.device)
    eager = iso.iso_fit(y, w, False, 0.0, 1.0, ws=ws, blocks=False, check=True)[0].clone()
    out = torch.empty_like(y)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # a first call on the capture stream sets any launch attributes
        iso.iso_fit(y, w, False, 0.0, 1.0, out=out, ws=ws, blocks=False, check=False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        iso.iso_fit(y, w, False, 0.0, 1.0, out=out, ws=ws, blocks=False, check=False)
    for k in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {k}"
        other = iso.iso_fit(y * 0.5, w, True, ws=iso.workspace(rows, n, y.dtype, y.device), blocks=False,
                            check=False)[0]
        torch.cuda.synchronize()
        del other


@pytest.mark.parametrize("n", [24, 50, 300, 5000, 20000])
def test_status_belongs_to_the_latest_call(n):
    """A weight error is reported by iso_status for the call that made it and
    not for a later clean call on the same workspace (the status words live in
    the workspace: the call's epoch and its last error), on every first kernel
    of the fit (one row per lane, two lanes, one workgroup, chunks)."""
    import torch
    import weighted_isotonic_regression_row_amd as iso
    r = workloads.rng(n)
    y = to_dev(r.standard_normal((4, n)))
    w_ok = r.random((4, n)) + 0.1
    w_bad = w_ok.copy()
    w_bad[2, n // 2] = 0.0
    ws = iso.workspace(4, n, torch.float64, y.device)
    for w, want in ((w_bad, iso.ISO_EWEIGHT), (w_ok, iso.ISO_OK), (w_ok, iso.ISO_OK), (w_bad, iso.ISO_EWEIGHT),
                    (w_ok, iso.ISO_OK)):
        iso.iso_fit(y, to_dev(w), ws=ws, blocks=False, check=False)
        assert iso.iso_status(ws) == want
