"""iso_fit_noalloc (include/iso.h) against iso_fit, through the C ABI: the
same kernels on the library's static scratch instead of a caller's workspace,
so the fit, the block-start and clip bits and the row-NaN flags must equal
iso_fit's bit for bit, and the fit must match the oracle at the usual
tolerance.  Each case makes two calls in a row on the shared scratch, the
second on a smaller input, so a leftover of the first call cannot pass
unnoticed."""
from __future__ import annotations

import ctypes
import math

import numpy as np
import pytest

import workloads
from gpu_helpers import check_fit, oracle_fit, to_dev

pytestmark = pytest.mark.gpu


def _noalloc(lib, iso, wl):
    """One call of iso_fit_noalloc through ctypes; returns (fit, start bits, clip bits, row NaN)."""
    import torch
    y = to_dev(wl.y)
    w = to_dev(wl.w)
    out = torch.full_like(y, float("nan"))
    mem = torch.zeros(max(iso.iso_blocks_bytes(wl.rows, wl.n), 256), dtype=torch.uint8, device=y.device)
    bc = iso.IsoBlocksC()
    lo = -math.inf if wl.y_min is None else wl.y_min
    hi = math.inf if wl.y_max is None else wl.y_max
    code = lib.iso_fit_noalloc(y.data_ptr(), None if w is None else w.data_ptr(), wl.rows, wl.n,
                               1 if wl.increasing else 0, lo, hi, iso.ISO_F32 if wl.y.dtype == np.float32 else iso.ISO_F64,
                               out.data_ptr(), ctypes.byref(bc), mem.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    assert code == iso.ISO_OK, iso.strerror(code)
    torch.cuda.synchronize()
    b = iso.Blocks(bc, mem, w, tuple(y.shape))
    sb, cb, rn = b.bits()
    return out, sb.clone(), cb.clone(), rn.clone()


def _reference(iso, wl):
    import torch
    fit, b = iso.iso_fit(to_dev(wl.y), to_dev(wl.w), wl.increasing, wl.y_min, wl.y_max, check=False)
    torch.cuda.synchronize()
    sb, cb, rn = b.bits()
    return fit, sb, cb, rn


def _batch(rows, n, dtype, seed, inc=True, clip=None):
    wl = workloads.family("trend_noise" if seed % 2 else "noise", rows, n, seed=seed, dtype=dtype,
                          weights="uniform", increasing=inc)
    if clip:
        wl.y_min, wl.y_max = clip
    return wl


# pairs of calls: a larger problem, then a smaller one of another shape, on each path of the fit
CASES = [
    ("batch rows", _batch(1000, 5000, np.float32, 2, False, (0.0, 1.0)), _batch(37, 777, np.float64, 3)),
    ("long rows", _batch(2, 30000, np.float64, 5), _batch(1, 9000, np.float32, 7, False, (-0.5, 0.5))),
    ("short rows", _batch(5000, 50, np.float32, 9), _batch(300, 24, np.float64, 11, True, (-1.0, 1.0))),
    ("one long row", _batch(1, 6_500_000, np.float64, 13), _batch(3, 20001, np.float64, 15)),
    ("packed rows", _batch(300_000, 65, np.float32, 17), _batch(1001, 128, np.float64, 19, False, (-0.5, 0.5))),
    ("one-wave rows", _batch(20_000, 300, np.float32, 21, True, (-1.0, 1.0)), _batch(77, 512, np.float64, 23)),
]


@pytest.mark.parametrize("name,first,second", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_iso_fit(name, first, second):
    import torch
    import weighted_isotonic_regression_row_amd as iso
    lib = iso.load_library()
    for wl in (first, second):
        print(f"noalloc {name}: {wl.name}", flush=True)
        got = _noalloc(lib, iso, wl)
        ref = _reference(iso, wl)
        for g, r, what in zip(got, ref, ("fit", "start bits", "clip bits", "row NaN")):
            assert torch.equal(g, r), f"{name} {wl.name}: {what} differ from iso_fit's"
        z, *_ = oracle_fit(wl)
        check_fit(got[0].cpu().numpy(), z, wl.y, wl.y.dtype, wl.increasing, f"noalloc {wl.name}")


def test_noalloc_refuses_a_problem_past_its_scratch():
    import torch
    import weighted_isotonic_regression_row_amd as iso
    y = torch.zeros((2000, 5000), dtype=torch.float32, device="cuda:0")
    out = torch.full_like(y, 7.0)
    with pytest.raises(iso.IsoError) as e:
        iso.iso_fit_noalloc(y, out=out)
    assert e.value.code == iso.ISO_ETOOBIG
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())  # nothing was queued
