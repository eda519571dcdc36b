"""GPU tests of the view entry points (include/iso.h, iso_fit_view and
iso_vjp_view) and of `isotonic`, the operator with the PyPI page's semantics
("Semantics": weights of y's shape or broadcast to it, `dim` picks the axis,
float16 and bfloat16 computed in float32, integer input made float,
differentiable in y and in the weights).

The views only gather inputs into contiguous rows of the compute type and
scatter the result, so on the same values they must give the contiguous
entry point's result bit for bit; the tests compare them that way (the
contiguous path's own parity with the oracle is tests/test_gpu_parity.py),
and the float16 / bfloat16 / integer results also against the oracle on the
inputs' exact float64 values.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import TOL_F32, check_partition, gpu_blocks, row_scales

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def _torch():
    import torch
    return torch


def _iso():
    import weighted_isotonic_regression_row_amd as iso
    return iso


def _rand(shape, seed, dtype, lo=None, hi=None):
    torch = _torch()
    r = workloads.rng(seed)
    a = r.standard_normal(shape) if lo is None else r.uniform(lo, hi, shape)
    return torch.from_numpy(a.astype(np.float64)).to("cuda:0", dtype)


def _same(a, b, what):
    torch = _torch()
    torch.cuda.synchronize()
    a, b = a.cpu(), b.cpu()
    assert a.dtype == b.dtype and a.shape == b.shape, f"{what}: {a.dtype}{tuple(a.shape)} vs {b.dtype}{tuple(b.shape)}"
    eq = (a == b) | (torch.isnan(a) & torch.isnan(b))
    assert bool(eq.all()), f"{what}: {int((~eq).sum())} elements differ"


def _bits_same(b1, b2, what):
    for x, y, name in zip(b1.bits(), b2.bits(), ("start", "clip", "row_nan")):
        _same(x, y, f"{what} {name} bits")


@pytest.mark.parametrize("dtype", ["float32", "float64"])
@pytest.mark.parametrize("n", [1, 16, 40, 500, 5000, 9000])
def test_contiguous_view_is_iso_fit(dtype, n):
    """Contiguous rows of the compute type pass straight through: same result and partition as iso_fit."""
    torch, iso = _torch(), _iso()
    dt = getattr(torch, dtype)
    y = _rand((7, n), 1, dt)
    w = _rand((7, n), 2, dt, 0.5, 1.5)
    f1, b1 = iso.iso_fit(y, w, False, -0.5, 0.5)
    f2, b2 = iso.iso_fit_view(y, w, False, -0.5, 0.5)
    _same(f2, f1, f"contiguous {dtype} n={n}")
    _bits_same(b2, b1, f"contiguous {dtype} n={n}")


@pytest.mark.parametrize("dtype", ["float32", "float64"])
@pytest.mark.parametrize("n,b", [(5000, 37), (70, 1000), (3, 130), (9000, 5), (64, 64), (1, 9)])
def test_fit_along_dim0(dtype, n, b):
    """A fit down the columns of a row-major [n, b] matrix (dim=0): the tiled transposes in and out."""
    torch, iso = _torch(), _iso()
    dt = getattr(torch, dtype)
    y = _rand((n, b), 3, dt)
    w = _rand((n, b), 4, dt, 0.1, 1.1)
    f, blk = iso.iso_fit_view(y, w, True, None, None, dim=0)
    ref, rb = iso.iso_fit(y.t().contiguous(), w.t().contiguous(), True)
    _same(f.t().contiguous(), ref, f"dim0 {dtype} {n}x{b}")
    _bits_same(blk, rb, f"dim0 {dtype} {n}x{b}")


@pytest.mark.parametrize("shape,dim", [((3, 700, 5), 1), ((4, 6, 300), 0), ((2, 3, 4, 50), 3), ((5, 1, 800), 2)])
def test_fit_along_any_axis(shape, dim):
    """N-d tensors: the batch axes fold into at most two strides."""
    torch, iso = _torch(), _iso()
    y = _rand(shape, 5, torch.float32)
    f, _ = iso.iso_fit_view(y, None, True, dim=dim)
    yt = y.movedim(dim, -1).contiguous()
    ref, _ = iso.iso_fit(yt.reshape(-1, yt.shape[-1]))
    _same(f.movedim(dim, -1).contiguous().reshape(-1, yt.shape[-1]), ref, f"shape {shape} dim {dim}")


def test_layout_beyond_two_batch_strides_is_refused():
    torch, iso = _torch(), _iso()
    y = _rand((3, 4, 5, 60), 6, torch.float32).permute(1, 0, 2, 3)  # [4, 3, 5, 60]: no two batch axes fold
    with pytest.raises(ValueError):
        iso.iso_fit_view(y, None, True, dim=2)


@pytest.mark.parametrize("wshape", ["row", "col", "scalar", "one_row", "full"])
def test_broadcast_weights(wshape):
    """Weights that broadcast to y's shape give the fit of the expanded weights."""
    torch, iso = _torch(), _iso()
    rows, n = 300, 2000
    y = _rand((rows, n), 7, torch.float64)
    w = {"row": _rand((n,), 8, torch.float64, 0.5, 2.0),
         "col": _rand((rows, 1), 9, torch.float64, 0.5, 2.0),
         "scalar": torch.tensor(1.7, dtype=torch.float64, device="cuda:0"),
         "one_row": _rand((1, n), 10, torch.float64, 0.5, 2.0),
         "full": _rand((rows, n), 11, torch.float64, 0.5, 2.0)}[wshape]
    f, blk = iso.iso_fit_view(y, w, True, 0.0, None)
    ref, rb = iso.iso_fit(y, w.expand(rows, n).contiguous(), True, 0.0, None)
    _same(f, ref, f"weights {wshape}")
    _bits_same(blk, rb, f"weights {wshape}")


def test_expanded_y_with_one_weight_row_each():
    """The PyPI page's bootstrap band: one y expanded over many rows, a weight row each."""
    torch, iso = _torch(), _iso()
    n = 3000
    y = _rand((n,), 12, torch.float32)
    w = torch.empty(64, n, device="cuda:0").exponential_(generator=torch.Generator("cuda:0").manual_seed(13))
    f, _ = iso.iso_fit_view(y.expand(64, n), w)
    ref, _ = iso.iso_fit(y.expand(64, n).contiguous(), w)
    _same(f, ref, "expanded y")


def _oracle_rows(y, w, increasing=True, y_min=None, y_max=None):
    y64 = y.double().cpu().numpy()
    w64 = None if w is None else w.double().expand(y.shape).cpu().numpy()
    return oracle.fit(y64, w64, increasing, y_min, y_max, threads=8)


@pytest.mark.parametrize("dtype,ulp", [("float16", 2.0 ** -10), ("bfloat16", 2.0 ** -7)])
@pytest.mark.parametrize("n", [24, 300, 5000, 20000])
def test_half_inputs(dtype, ulp, n):
    """float16 / bfloat16 y and w are computed in float32 and stored in their own dtype: bit for bit the
    float32 path's result rounded to nearest even, and within the float32 bound plus one ulp of the format of
    the oracle's fit of the same (exactly representable) values."""
    torch, iso = _torch(), _iso()
    dt = getattr(torch, dtype)
    rows = 64
    y = _rand((rows, n), 14, dt)
    w = _rand((rows, n), 15, dt, 0.25, 2.0)
    f, blk = iso.iso_fit_view(y, w, False, -1.0, 1.0)
    assert f.dtype == dt
    ref32, b32 = iso.iso_fit(y.float(), w.float(), False, -1.0, 1.0)
    _same(f, ref32.to(dt), f"{dtype} n={n} against float32 rounded")
    _bits_same(blk, b32, f"{dtype} n={n}")
    z, *_ = _oracle_rows(y, w, False, -1.0, 1.0)
    got = f.double().cpu().numpy()
    s = row_scales(y.double().cpu().numpy())
    err = np.abs(got - z).max(axis=1)
    assert (err <= (TOL_F32 + ulp) * s).all(), f"{dtype} n={n}: max error {err.max():.3e}"
    gs, gc, grn = gpu_blocks(blk)
    check_partition(gs, gc, grn, y.float().cpu().numpy(), w.float().cpu().numpy(), False, -1.0, 1.0,
                    f"{dtype} n={n}")


def test_half_nan_rows_and_weight_errors():
    torch, iso = _torch(), _iso()
    y = _rand((4, 100), 16, torch.float16)
    y[1, 50] = float("nan")
    f, blk = iso.iso_fit_view(y, None)
    assert bool(torch.isnan(f[1]).all()) and not bool(torch.isnan(f[[0, 2, 3]]).any())
    w = _rand((100,), 17, torch.bfloat16, 0.5, 1.5)
    w[3] = 0.0
    with pytest.raises(ValueError):
        iso.iso_fit_view(y, w)


@pytest.mark.parametrize("ydt,wdt", [("int64", None), ("int32", "int64"), ("float32", "int32")])
def test_integer_inputs(ydt, wdt):
    """Integer y becomes the default float dtype; integer weights (counts) are converted exactly."""
    torch, iso = _torch(), _iso()
    r = workloads.rng(18)
    y = torch.from_numpy(r.integers(-50, 50, (40, 3000))).to("cuda:0", getattr(torch, ydt))
    w = None if wdt is None else torch.from_numpy(r.integers(1, 9, (40, 3000))).to("cuda:0", getattr(torch, wdt))
    f, _ = iso.iso_fit_view(y, w)
    assert f.dtype == torch.get_default_dtype()
    ref, _ = iso.iso_fit(y.to(torch.float32), None if w is None else w.to(torch.float32))
    _same(f, ref, f"integer {ydt}/{wdt}")
    z, *_ = _oracle_rows(y, w)
    s = row_scales(y.double().cpu().numpy())
    assert (np.abs(f.double().cpu().numpy() - z).max(axis=1) <= TOL_F32 * s).all()


@pytest.mark.parametrize("dtype", ["float32", "float64", "float16"])
def test_vjp_views_dim0_broadcast_weights(dtype):
    """Both backward products through views (dim=0, weights broadcast along the batch axis, a transposed
    upstream gradient) equal iso_vjp_yw on the contiguous transposed problem bit for bit (float16: on its float32
    values, rounded)."""
    torch, iso = _torch(), _iso()
    dt = getattr(torch, dtype)
    cdt = torch.float64 if dtype == "float64" else torch.float32
    n, b = 2500, 48
    y = _rand((n, b), 19, dt)
    w = _rand((n, 1), 20, dt, 0.5, 1.5)
    g = _rand((b, n), 21, dt).t()  # a non-contiguous gradient of y's shape
    f, blk = iso.iso_fit_view(y, w, True, None, 0.5, dim=0)
    gy, gw = iso.iso_vjp_view(g, blk, y)
    assert gy.dtype == dt and gw.dtype == dt and gy.shape == y.shape
    yt = y.t().contiguous().to(cdt)
    wt = w.expand(n, b).t().contiguous().to(cdt)
    ref, rb = iso.iso_fit(yt, wt, True, None, 0.5)
    _same(f.t().contiguous(), ref.to(dt), f"vjp {dtype} fit")
    ry, rw = iso.iso_vjp_yw(g.t().contiguous().to(cdt), rb, yt)
    _same(gy.t().contiguous(), ry.to(dt), f"vjp {dtype} grad_y")
    _same(gw.t().contiguous(), rw.to(dt), f"vjp {dtype} grad_w")
    gy2, gw2 = iso.iso_vjp_view(g, blk, None)
    assert gw2 is None
    _same(gy2, gy, f"vjp {dtype} grad_y alone")


def test_isotonic_autograd_with_broadcast_weights():
    """isotonic() is differentiable in y and w; for weights broadcast along the rows the product in w is the
    per-element product summed over the rows (autograd's reduction of the expand)."""
    torch, iso = _torch(), _iso()
    rows, n = 50, 800
    y = _rand((rows, n), 22, torch.float64).requires_grad_(True)
    w = _rand((n,), 23, torch.float64, 0.5, 1.5).requires_grad_(True)
    g = _rand((rows, n), 24, torch.float64)
    f = iso.isotonic(y, w, increasing=False, y_min=-1.0)
    gy, gw = torch.autograd.grad(f, (y, w), g)
    assert gw.shape == w.shape
    ref, rb = iso.iso_fit(y.detach(), w.detach().expand(rows, n).contiguous(), False, -1.0, None)
    _same(f.detach(), ref, "isotonic fit")
    ry, rw = iso.iso_vjp_yw(g, rb, y.detach())
    _same(gy, ry, "isotonic grad_y")
    torch.testing.assert_close(gw, rw.sum(0), rtol=1e-12, atol=1e-12)
    # no gradient wanted: plain fit, no handle
    with torch.no_grad():
        _same(iso.isotonic(y, w, increasing=False, y_min=-1.0), ref, "isotonic without grad")


def test_isotonic_autograd_half_along_dim0():
    torch, iso = _torch(), _iso()
    y = _rand((600, 12), 25, torch.bfloat16).requires_grad_(True)
    f = iso.isotonic(y, dim=0)
    assert f.dtype == torch.bfloat16
    (gy,) = torch.autograd.grad(f.float().sum(), (y,))
    assert gy.dtype == torch.bfloat16 and gy.shape == y.shape
    # unit weights: the product in y of an all-ones gradient is 1 everywhere
    assert bool((gy == 1).all())


@pytest.mark.parametrize("shape", [(0, 5), (5, 0), (0, 0)])
def test_empty_views(shape):
    torch, iso = _torch(), _iso()
    y = torch.empty(shape, dtype=torch.float16, device="cuda:0")
    f, blk = iso.iso_fit_view(y, None)
    assert f.shape == y.shape and f.dtype == torch.float16
    f2, _ = iso.iso_fit_view(y, None, dim=0)
    assert f2.shape == y.shape
