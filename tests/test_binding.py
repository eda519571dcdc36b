"""Argument checks of the Python binding, on the CPU: a caller's out=, ws= or
input tensor of the wrong shape, dtype, device or layout is refused with a
ValueError before anything reaches the library, so it can never become an
out-of-bounds write or a device fault.  Host tensors are refused outright
(every operation runs on the GPU; there is no CPU fallback)."""
from __future__ import annotations

import pytest
import torch

import weighted_isotonic_regression_row_amd as iso


def _y(dtype=torch.float64, shape=(3, 100)):
    return torch.zeros(shape, dtype=dtype)


def test_host_tensors_are_refused():
    with pytest.raises(ValueError, match="GPU"):
        iso.iso_fit(_y())
    with pytest.raises(ValueError, match="GPU"):
        iso.soft_rank(_y())
    with pytest.raises(ValueError, match="GPU"):
        iso.calibration_fit(_y(), _y())


@pytest.mark.parametrize("out", [
    torch.zeros((3, 100), dtype=torch.float32),          # wrong dtype
    torch.zeros((3, 99), dtype=torch.float64),           # wrong shape
    torch.zeros((100, 3), dtype=torch.float64).t(),      # not contiguous
    torch.zeros((3, 100), dtype=torch.float64, device="meta"),  # wrong device
])
def test_fit_out_is_checked(out):
    with pytest.raises(ValueError, match="out"):
        iso.iso_fit(_y(), out=out)


@pytest.mark.parametrize("ws", [
    torch.zeros(4096, dtype=torch.int32),
    torch.zeros(4096, dtype=torch.uint8, device="meta"),
    torch.zeros((2, 4096), dtype=torch.uint8).t(),
])
def test_fit_ws_is_checked(ws):
    with pytest.raises(ValueError, match="ws"):
        iso.iso_fit(_y(), ws=ws)


def test_fit_w_is_checked():
    with pytest.raises(ValueError, match="w must"):
        iso.iso_fit(_y(), _y(torch.float32))
    with pytest.raises(ValueError, match="w must"):
        iso.iso_fit(_y(), _y(shape=(3, 101)))


def _blocks(rows=3, n=100, dtype=iso.ISO_F64, device="cpu"):
    c = iso.IsoBlocksC()
    c.rows, c.n, c.words, c.dtype, c.valid = rows, n, (n + 63) // 64, dtype, 1
    return iso.Blocks(c, torch.zeros(4096, dtype=torch.uint8, device=device), None, (rows, n))


def test_vjp_arguments_are_checked():
    b = _blocks()
    with pytest.raises(ValueError, match="grad"):
        iso.iso_vjp(_y(shape=(3, 99)), b)
    with pytest.raises(ValueError, match="grad"):
        iso.iso_vjp(_y(torch.float32), b)
    with pytest.raises(ValueError, match="grad must be on"):
        iso.iso_vjp(_y().to("meta"), b)
    with pytest.raises(ValueError, match="out"):
        iso.iso_vjp(_y(), b, out=_y(torch.float32))
    with pytest.raises(ValueError, match="ws"):
        iso.iso_vjp(_y(), b, ws=torch.zeros(10, dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        iso.iso_vjp(_y(), b)


def test_vjp_yw_arguments_are_checked():
    b = _blocks()
    with pytest.raises(ValueError, match="y must be on"):
        iso.iso_vjp_yw(_y(), b, _y().to("meta"))
    with pytest.raises(ValueError, match="y must"):
        iso.iso_vjp_yw(_y(), b, _y(torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        iso.iso_vjp_yw(_y(), b, _y())


def test_soft_rank_arguments_are_checked():
    with pytest.raises(ValueError, match="out"):
        iso.soft_rank(_y(), out=_y(shape=(3, 5)))
    with pytest.raises(ValueError, match="ws"):
        iso.soft_rank(_y(), ws=torch.zeros(10))
    st = iso.SoftRankState(iso.IsoSoftRankStateC(), torch.zeros(4096, dtype=torch.uint8), (3, 100))
    st.c.blocks = _blocks().c
    with pytest.raises(ValueError, match="grad must be on"):
        iso.soft_rank_vjp(_y().to("meta"), st)
    with pytest.raises(ValueError, match="out"):
        iso.soft_rank_vjp(_y(), st, out=_y(torch.float32))


def test_calibration_arguments_are_checked():
    with pytest.raises(ValueError, match="labels"):
        iso.calibration_fit(_y(), _y(torch.float32))
    with pytest.raises(ValueError, match="ws"):
        iso.calibration_fit(_y(), _y(), ws=torch.zeros(10))
    xs, fit, m = _y(), _y(), torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError, match="fit"):
        iso.calibrate(_y(shape=(3, 7)), xs, _y(torch.float32), m)
    with pytest.raises(ValueError, match="m must"):
        iso.calibrate(_y(shape=(3, 7)), xs, fit, torch.zeros(3, dtype=torch.int64))
    with pytest.raises(ValueError, match="q must be on"):
        iso.calibrate(_y(shape=(3, 7)).to("meta"), xs, fit, m)
    with pytest.raises(ValueError, match="out"):
        iso.calibrate(_y(shape=(3, 7)), xs, fit, m, out=_y(shape=(3, 8)))
    with pytest.raises(ValueError, match="GPU"):
        iso.calibrate(_y(shape=(3, 7)), xs, fit, m)


def test_view_entry_points_need_device_tensors():
    with pytest.raises(ValueError, match="GPU"):
        iso.iso_fit_view(_y())
    with pytest.raises(ValueError, match="GPU"):
        iso.isotonic(_y(), dim=0)


def test_fold_gives_the_logical_rows():
    """_fold reads only shapes and strides: the [outer, inner, n] geometry of a fit along an axis."""
    y = torch.zeros(6, 50)
    assert iso._fold(y.shape, 1, [y]) == (1, 6, 50, [(0, 50, 1)])
    assert iso._fold(y.shape, 0, [y]) == (1, 50, 6, [(0, 1, 50)])          # down the columns
    z = torch.zeros(3, 70, 5)
    assert iso._fold(z.shape, 1, [z]) == (3, 5, 70, [(350, 1, 5)])         # two batch strides
    q = torch.zeros(2, 3, 4, 9)
    assert iso._fold(q.shape, 3, [q]) == (1, 24, 9, [(0, 9, 1)])           # batch axes folded into one
    w = torch.zeros(9).expand(2, 3, 4, 9)
    assert iso._fold(q.shape, 3, [q, w]) == (1, 24, 9, [(0, 9, 1), (0, 0, 1)])  # a shared weight vector
    c = torch.zeros(6, 1).expand(6, 50)
    assert iso._fold(y.shape, 1, [y, c]) == (1, 6, 50, [(0, 50, 1), (0, 1, 0)])  # one weight per row
    one = torch.zeros(1, 7)
    assert iso._fold(one.shape, 1, [one]) == (1, 1, 7, [(0, 0, 1)])
    assert iso._fold((5, 1), 1, [torch.zeros(5, 1)])[2:] == (1, [(0, 1, 1)])  # n = 1: elements adjacent
    p = torch.zeros(3, 4, 5, 60).permute(1, 0, 2, 3)
    with pytest.raises(ValueError, match="two batch strides"):
        iso._fold(p.shape, 3, [p])


def test_result_dtype_follows_the_semantics():
    assert iso._result_dtype(torch.zeros(2, dtype=torch.float16)) == torch.float16
    assert iso._result_dtype(torch.zeros(2, dtype=torch.bfloat16)) == torch.bfloat16
    assert iso._result_dtype(torch.zeros(2, dtype=torch.int64)) == torch.get_default_dtype()
    with pytest.raises(TypeError):
        iso._result_dtype(torch.zeros(2, dtype=torch.complex64))
