"""The GPU tests' comparison helpers, exercised on the CPU: the oracle's own
results pass them, and planted mistakes (a moved or dropped block start, a
wrong clip flag, an error just above a row's own tolerance in a batch whose
other row has a far larger scale) fail them.  This shows that the checks
bite before they are trusted with the GPU's results."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import check_fit, check_partition, row_scales


def _case(dtype=np.float64, inc=True, clip=(0.2, 0.7)):
    wl = workloads.family("trend_noise", 4, 700, seed=5, dtype=dtype, weights="uniform", increasing=inc)
    z, bs, cl, rn, _ = oracle.fit(wl.y.astype(np.float64), wl.w.astype(np.float64), inc, *clip)
    return wl, z, bs, cl, rn


@pytest.mark.parametrize("inc", [True, False])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_oracle_results_pass(inc, dtype):
    wl, z, bs, cl, rn = _case(dtype, inc)
    check_fit(z.astype(dtype), z, wl.y, dtype, inc, "self")
    exact, rows = check_partition(bs, cl, rn, wl.y, wl.w, inc, 0.2, 0.7, "self")
    assert rows == 4 and exact >= 3  # trend plus noise: most rows hold no tie position


def test_a_moved_block_start_fails():
    wl, z, bs, cl, rn = _case()
    gs = bs.copy()
    i = int(np.flatnonzero(bs[1])[5])
    gs[1, i] = 0
    gs[1, i + 1] = 1
    with pytest.raises(AssertionError, match="row 1"):
        check_partition(gs, cl, rn, wl.y, wl.w, True, 0.2, 0.7, "moved")


def test_a_dropped_block_start_fails():
    wl, z, bs, cl, rn = _case()
    gs = bs.copy()
    gs[2, int(np.flatnonzero(bs[2])[3])] = 0
    with pytest.raises(AssertionError, match="row 2"):
        check_partition(gs, cl, rn, wl.y, wl.w, True, 0.2, 0.7, "dropped")


def test_a_split_at_a_collinear_point_passes():
    # (2, 0, 2, 0) pools into one block of mean 1 (the oracle pools ties); a
    # split after the first pair leaves two blocks of that same mean, which is
    # a valid partition of the fit
    y = np.array([[2.0, 0.0, 2.0, 0.0, 5.0]])
    z, bs, cl, rn, _ = oracle.fit(y)
    gs = bs.copy()
    gs[0, 2] = 1
    check_partition(gs, cl, rn, y, None, True, None, None, "collinear")


def test_a_wrong_clip_bit_fails():
    wl, z, bs, cl, rn = _case()
    gc = cl.copy()
    i = int(np.flatnonzero(cl[0])[0])
    gc[0, i] = 0
    with pytest.raises(AssertionError, match="clip bit"):
        check_partition(bs, gc, rn, wl.y, wl.w, True, 0.2, 0.7, "clip")


def test_tolerance_is_taken_per_row():
    # two rows whose scales differ by 1e8: an error of 1e-9 in the small row
    # passes a whole-batch scale but fails the row's own (1e-10 * 1)
    y = np.stack([np.linspace(0, 1e8, 64), np.linspace(0, 1, 64)])
    z = y.copy()
    zg = z.copy()
    zg[1, 10] += 1e-9
    with pytest.raises(AssertionError, match="row 1"):
        check_fit(zg, z, y, np.float64, True, "per row")
    zg[1, 10] = z[1, 10] + 5e-11
    check_fit(zg, z, y, np.float64, True, "per row")
    assert row_scales(y)[1] == 1.0


def test_float32_monotonicity_is_taken_per_row():
    y = np.stack([np.linspace(0, 1e6, 64), np.linspace(0, 1, 64)]).astype(np.float32)
    z = y.astype(np.float64)
    zg = z.copy()
    zg[1, 11] = zg[1, 10] - 1e-5  # a wrong-way step far above 4 ulp of 1, far below 4 ulp of 1e6
    zg[1, 12:] = np.maximum(zg[1, 12:], zg[1, 10])
    with pytest.raises(AssertionError, match="row 1"):
        check_fit(zg, z, y, np.float32, True, "mono")


def test_a_difference_away_from_ties_fails_in_a_row_with_ties():
    # a row holding an exact tie somewhere still has every other position compared
    y = np.concatenate([[2.0, 0.0, 2.0, 0.0], np.linspace(1.5, 3.0, 40) + 0.01 * np.sin(np.arange(40))])[None, :]
    z, bs, cl, rn, _ = oracle.fit(y)
    gs = bs.copy()
    gs[0, 2] = 1  # the tie: allowed
    check_partition(gs, cl, rn, y, None, True, None, None, "tie")
    j = int(np.flatnonzero(bs[0])[-1])
    gs[0, j] = 0  # a clear start dropped (its pooled block's mean is then off the fit as well)
    with pytest.raises(AssertionError, match="row 0"):
        check_partition(gs, cl, rn, y, None, True, None, None, "tie")
