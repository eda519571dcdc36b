"""The C ABI library builds, loads, exports every declared symbol, and rejects
bad arguments on the host before anything is queued (no GPU needed).

Arguments are those of include/iso.h; every call below fails validation, so
no HIP call is made and no device memory is touched (the pointers are never
dereferenced on this path).
"""
from __future__ import annotations

import ctypes
import math
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "iso.h")
LIB = os.path.join(ROOT, "weighted_isotonic_regression_row_amd", "libiso.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(iso_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libiso.so not built (run __graft_entry__.build())")
    import weighted_isotonic_regression_row_amd as iso
    return iso.load_library()


def test_header_declares_the_boundary():
    fns = declared_functions()
    assert fns == sorted(["iso_blocks_bytes", "iso_fit", "iso_fit_noalloc", "iso_status", "iso_strerror", "iso_vjp", "iso_vjp_yw",
                          "iso_workspace_bytes", "iso_soft_rank", "iso_soft_rank_vjp", "iso_soft_rank_state_bytes",
                          "iso_soft_rank_workspace_bytes", "iso_calibration_workspace_bytes", "iso_calibration_fit",
                          "iso_calibrate", "iso_view_workspace_bytes", "iso_view_blocks_bytes", "iso_fit_view",
                          "iso_vjp_view"])


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (iso_\w+)$", out, flags=re.M))
    for fn in declared_functions():
        assert fn in exported, fn
        assert hasattr(lib, fn)


def test_binding_lists_the_same_symbols():
    import weighted_isotonic_regression_row_amd as iso
    assert sorted(iso.SYMBOLS) == declared_functions()


def test_sizes(lib):
    assert lib.iso_workspace_bytes(-1, 5, 0) == 0
    assert lib.iso_workspace_bytes(5, 5, 7) == 0
    assert lib.iso_workspace_bytes(1000, 5000, 0) >= 256
    small = lib.iso_workspace_bytes(1000, 5000, 0)
    big = lib.iso_workspace_bytes(32, 1 << 22, 1)
    # chunk hulls of long rows live in the workspace: a vertex bit set, group
    # starts and up to 1024 explicit vertices per chunk of 3584 elements
    assert 32 * (1 << 22) * 0.25 < big < 32 * (1 << 22) * 12
    # single-workgroup rows: room for each row's vertex list in case its lane
    # hulls do not fit in LDS (18 bytes per point)
    assert 1000 * 5001 * 18 <= small < 1000 * 5001 * 19
    assert lib.iso_blocks_bytes(4, 130) >= 2 * 4 * 3 * 8 + 4 * 4
    assert lib.iso_blocks_bytes(-1, 3) == 0


def test_strerror(lib):
    assert lib.iso_strerror(0) == b"success"
    assert b"positive" in lib.iso_strerror(-3)
    assert b"scratch" in lib.iso_strerror(-4)
    assert lib.iso_strerror(-99) == b"unknown error"


def _fit(lib, y=256, w=None, rows=2, n=3, inc=1, lo=-math.inf, hi=math.inf, dt=0, fit=512, bo=None, bm=None,
         ws=4096, wsb=1 << 20, stream=None):
    import weighted_isotonic_regression_row_amd as iso
    return lib.iso_fit(y, w, rows, n, inc, lo, hi, dt, fit, bo, bm, ws, wsb, stream)


def test_fit_rejects_bad_arguments_on_host(lib):
    import weighted_isotonic_regression_row_amd as iso
    E = iso.ISO_EINVAL
    assert _fit(lib, rows=-1) == E
    assert _fit(lib, n=-1) == E
    assert _fit(lib, dt=2) == E
    assert _fit(lib, inc=2) == E
    assert _fit(lib, lo=1.0, hi=0.0) == E
    assert _fit(lib, y=None) == E
    assert _fit(lib, fit=None) == E
    assert _fit(lib, ws=None) == E
    assert _fit(lib, ws=4096 + 8) == E           # misaligned workspace
    assert _fit(lib, wsb=8) == E                 # workspace too small
    big = lib.iso_workspace_bytes(2, 20000, 0)
    assert _fit(lib, n=20000, wsb=big - 1) == E
    assert _fit(lib, fit=256) == E               # output aliases y
    bc = iso.IsoBlocksC()
    assert _fit(lib, bo=ctypes.byref(bc)) == E   # handle without memory
    assert _fit(lib, bm=8192) == E               # memory without handle


def test_fit_empty_is_a_noop(lib):
    import weighted_isotonic_regression_row_amd as iso
    bc = iso.IsoBlocksC()
    assert _fit(lib, rows=0, y=None, fit=None, ws=None, bo=ctypes.byref(bc), bm=8192) == iso.ISO_OK
    assert bc.valid == 1 and bc.rows == 0
    assert _fit(lib, n=0, y=None, fit=None, ws=None) == iso.ISO_OK
    # NaN bounds mean "no bound"
    assert _fit(lib, rows=0, lo=math.nan, hi=math.nan) == iso.ISO_OK


def test_vjp_rejects_bad_arguments_on_host(lib):
    import weighted_isotonic_regression_row_amd as iso
    bc = iso.IsoBlocksC()
    assert lib.iso_vjp(256, ctypes.byref(bc), 512, 4096, 1 << 20, None) == iso.ISO_EINVAL  # invalid handle
    assert lib.iso_vjp(256, None, 512, 4096, 1 << 20, None) == iso.ISO_EINVAL
    bc.valid = 1
    bc.rows, bc.n, bc.words, bc.dtype = 2, 3, 1, 0
    bc.start_bits_dev, bc.clip_bits_dev, bc.row_nan_dev = 8192, 8192 + 256, 8192 + 512
    assert lib.iso_vjp(None, ctypes.byref(bc), 512, 4096, 1 << 20, None) == iso.ISO_EINVAL
    assert lib.iso_vjp(256, ctypes.byref(bc), 512, 4096, 1, None) == iso.ISO_EINVAL
    assert lib.iso_vjp(256, ctypes.byref(bc), None, 4096, 1 << 20, None) == iso.ISO_EINVAL  # no output
    bc.dtype = 5
    assert lib.iso_vjp(256, ctypes.byref(bc), 512, 4096, 1 << 20, None) == iso.ISO_EINVAL


def test_vjp_yw_rejects_bad_arguments_on_host(lib):
    import weighted_isotonic_regression_row_amd as iso
    E = iso.ISO_EINVAL
    bc = iso.IsoBlocksC()
    assert lib.iso_vjp_yw(256, ctypes.byref(bc), 128, 512, 640, 4096, 1 << 20, None) == E  # invalid handle
    bc.valid = 1
    bc.rows, bc.n, bc.words, bc.dtype = 2, 3, 1, 0
    bc.start_bits_dev, bc.clip_bits_dev, bc.row_nan_dev = 8192, 8192 + 256, 8192 + 512
    assert lib.iso_vjp_yw(256, ctypes.byref(bc), 128, None, None, 4096, 1 << 20, None) == E  # no output
    assert lib.iso_vjp_yw(256, ctypes.byref(bc), None, 512, 640, 4096, 1 << 20, None) == E   # grad_w without y
    assert lib.iso_vjp_yw(None, ctypes.byref(bc), 128, 512, 640, 4096, 1 << 20, None) == E
    assert lib.iso_vjp_yw(256, ctypes.byref(bc), 128, 512, 640, 4096 + 8, 1 << 20, None) == E  # misaligned
    assert lib.iso_vjp_yw(256, ctypes.byref(bc), 128, 512, 640, 4096, 1, None) == E  # workspace too small
    bc.rows = 0
    assert lib.iso_vjp_yw(None, ctypes.byref(bc), None, None, None, None, 0, None) == iso.ISO_OK  # empty


def test_soft_rank_sizes(lib):
    assert lib.iso_soft_rank_workspace_bytes(4096, 512, 0) >= 2 * 4096 * 512 * 4
    # longer than one workgroup sorts: the tiled sort's keys and indices too
    assert lib.iso_soft_rank_workspace_bytes(4, 8193, 0) >= lib.iso_soft_rank_workspace_bytes(4, 8192, 0) + 4 * 8193 * 24
    assert lib.iso_soft_rank_workspace_bytes(1, 1 << 31, 0) == 0
    assert lib.iso_soft_rank_workspace_bytes(4, 8192, 1) >= 2 * 4 * 8192 * 8
    assert lib.iso_soft_rank_workspace_bytes(-1, 5, 0) == 0
    assert lib.iso_soft_rank_workspace_bytes(2, 5, 3) == 0
    # the permutation, its inverse and the block bits
    assert lib.iso_soft_rank_state_bytes(4096, 512) >= 2 * 4 * 4096 * 512 + lib.iso_blocks_bytes(4096, 512)
    assert lib.iso_soft_rank_state_bytes(-1, 5) == 0


def _sr(lib, x=256, rows=2, n=3, eps=1.0, dt=0, r=512, st=True, mem=8192, ws=1 << 16, wsb=1 << 20):
    import weighted_isotonic_regression_row_amd as iso
    sc = iso.IsoSoftRankStateC()
    code = lib.iso_soft_rank(x, rows, n, eps, dt, r, ctypes.byref(sc) if st else None, mem, ws, wsb, None)
    return code, sc


def test_soft_rank_rejects_bad_arguments_on_host(lib):
    import weighted_isotonic_regression_row_amd as iso
    E = iso.ISO_EINVAL
    for kw in ({"rows": -1}, {"n": -1}, {"n": 1 << 31}, {"rows": 1 << 31}, {"dt": 2}, {"eps": 0.0}, {"eps": -1.0}, {"eps": math.inf},
               {"eps": math.nan}, {"st": False}, {"mem": None}, {"mem": 8192 + 8}, {"x": None}, {"r": None},
               {"ws": None}, {"ws": (1 << 16) + 8}, {"wsb": 8}, {"r": 256 + 4}):
        assert _sr(lib, **kw)[0] == E, kw


def test_soft_rank_empty_is_a_noop(lib):
    import weighted_isotonic_regression_row_amd as iso
    code, sc = _sr(lib, rows=0, x=None, r=None, ws=None)
    assert code == iso.ISO_OK and sc.valid == 1 and sc.blocks.valid == 1
    assert lib.iso_soft_rank_vjp(None, ctypes.byref(sc), None, None, 0, None) == iso.ISO_OK


def test_soft_rank_vjp_rejects_bad_arguments_on_host(lib):
    import weighted_isotonic_regression_row_amd as iso
    E = iso.ISO_EINVAL
    sc = iso.IsoSoftRankStateC()
    assert lib.iso_soft_rank_vjp(256, ctypes.byref(sc), 512, 1 << 16, 1 << 20, None) == E  # invalid state
    assert lib.iso_soft_rank_vjp(256, None, 512, 1 << 16, 1 << 20, None) == E
    code, sc = _sr(lib, x=None)   # fails, leaves the state invalid
    assert code == E and sc.valid == 0
    assert lib.iso_soft_rank_vjp(256, ctypes.byref(sc), 512, 1 << 16, 1 << 20, None) == E
    sc.valid = 1
    sc.blocks.valid = 1
    sc.blocks.rows, sc.blocks.n, sc.blocks.words, sc.blocks.dtype = 2, 3, 1, 0
    sc.blocks.start_bits_dev, sc.blocks.clip_bits_dev, sc.blocks.row_nan_dev = 8192, 8192 + 256, 8192 + 512
    sc.perm_dev, sc.rank_dev, sc.eps = 8192 + 1024, 8192 + 2048, 1.0
    assert lib.iso_soft_rank_vjp(None, ctypes.byref(sc), 512, 1 << 16, 1 << 20, None) == E
    assert lib.iso_soft_rank_vjp(256, ctypes.byref(sc), None, 1 << 16, 1 << 20, None) == E
    assert lib.iso_soft_rank_vjp(256, ctypes.byref(sc), 512, (1 << 16) + 8, 1 << 20, None) == E
    assert lib.iso_soft_rank_vjp(256, ctypes.byref(sc), 512, 1 << 16, 8, None) == E
    sc.eps = 0.0
    assert lib.iso_soft_rank_vjp(256, ctypes.byref(sc), 512, 1 << 16, 1 << 20, None) == E
    sc.eps, sc.perm_dev = 1.0, None
    assert lib.iso_soft_rank_vjp(256, ctypes.byref(sc), 512, 1 << 16, 1 << 20, None) == E


def test_calibration_sizes(lib):
    # sorted (key, index) entries twice, run starts and label prefixes, pooled means and weights
    assert lib.iso_calibration_workspace_bytes(1, 6_500_000, 1) >= 6_500_000 * (2 * 12 + 4 + 16 + 16)
    assert lib.iso_calibration_workspace_bytes(-1, 5, 0) == 0
    assert lib.iso_calibration_workspace_bytes(2, 5, 4) == 0
    assert lib.iso_calibration_workspace_bytes(1, 1 << 31, 0) == 0


def _cal(lib, s=256, y=512, rows=2, n=3, dt=0, xs=1024, fit=2048, m=4096, ws=1 << 16, wsb=1 << 24):
    return lib.iso_calibration_fit(s, y, rows, n, dt, xs, fit, m, ws, wsb, None)


def test_calibration_rejects_bad_arguments_on_host(lib):
    import weighted_isotonic_regression_row_amd as iso
    E = iso.ISO_EINVAL
    for kw in ({"rows": -1}, {"n": -1}, {"dt": 2}, {"s": None}, {"y": None}, {"xs": None}, {"fit": None},
               {"m": None}, {"ws": None}, {"ws": (1 << 16) + 8}, {"wsb": 8}, {"xs": 2048}, {"xs": 256 + 4},
               {"fit": 512}):
        assert _cal(lib, **kw) == E, kw
    assert _cal(lib, rows=0, s=None, y=None, xs=None, fit=None, m=None, ws=None) == iso.ISO_OK
    assert _cal(lib, n=0, s=None, y=None, xs=None, fit=None, m=None, ws=None) == iso.ISO_OK
    # evaluation
    assert lib.iso_calibrate(256, 512, 1024, 2, 3, 2048, 5, 2, 4096, None) == E       # dtype
    assert lib.iso_calibrate(None, 512, 1024, 2, 3, 2048, 5, 0, 4096, None) == E
    assert lib.iso_calibrate(256, 512, None, 2, 3, 2048, 5, 0, 4096, None) == E
    assert lib.iso_calibrate(256, 512, 1024, 2, 3, 2048, 5, 0, None, None) == E
    assert lib.iso_calibrate(256, 512, 1024, 2, 3, 2048, -1, 0, 4096, None) == E
    assert lib.iso_calibrate(None, None, None, 2, 3, None, 0, 0, None, None) == iso.ISO_OK  # no queries


def test_status_without_calls(lib):
    import weighted_isotonic_regression_row_amd as iso
    assert lib.iso_status(None, None) == iso.ISO_EINVAL
    # a workspace's status lives in its own first 16 bytes (no host map per
    # workspace), so any other call reads device memory and is for the GPU tests


def test_binding_refuses_host_tensors():
    import torch
    import weighted_isotonic_regression_row_amd as iso
    with pytest.raises(ValueError):
        iso.iso_fit(torch.zeros(3, 4))


def test_noalloc_refuses_problems_past_its_scratch_on_host(lib):
    """iso_fit_noalloc checks the problem's workspace against its static scratch
    before any HIP call: too large gives ISO_ETOOBIG, bad sizes ISO_EINVAL, an
    empty problem fills the handle and returns ISO_OK."""
    import weighted_isotonic_regression_row_amd as iso
    f = lib.iso_fit_noalloc
    assert f(256, None, 32, 1 << 22, 1, -math.inf, math.inf, 1, 512, None, None, None) == iso.ISO_ETOOBIG
    assert f(256, None, 2000, 5000, 1, -math.inf, math.inf, 0, 512, None, None, None) == iso.ISO_ETOOBIG
    assert f(256, None, -1, 5, 1, -math.inf, math.inf, 0, 512, None, None, None) == iso.ISO_EINVAL
    assert f(256, None, 2, 5, 1, -math.inf, math.inf, 9, 512, None, None, None) == iso.ISO_EINVAL
    bc = iso.IsoBlocksC()
    assert f(None, None, 0, 5, 1, -math.inf, math.inf, 0, None, ctypes.byref(bc), 8192, None) == iso.ISO_OK
    assert bc.valid == 1 and bc.rows == 0
    assert lib.iso_workspace_bytes(1000, 6144, 0) <= iso.NOALLOC_SCRATCH_BYTES
    assert lib.iso_workspace_bytes(1, 12_000_000, 1) <= iso.NOALLOC_SCRATCH_BYTES


def test_view_sizes(lib):
    import weighted_isotonic_regression_row_amd as iso
    base = lib.iso_workspace_bytes(100, 5000, 0)
    # the solver's workspace and four converted [rows, n] arrays of the compute type
    assert lib.iso_view_workspace_bytes(100, 5000, iso.ISO_F32) >= base + 4 * 100 * 5000 * 4
    assert lib.iso_view_workspace_bytes(100, 5000, iso.ISO_F64) >= lib.iso_workspace_bytes(100, 5000, 1) + 4 * 100 * 5000 * 8
    assert lib.iso_view_workspace_bytes(100, 5000, iso.ISO_F16) == 0   # not a compute type
    assert lib.iso_view_workspace_bytes(-1, 5, iso.ISO_F32) == 0
    b = lib.iso_view_blocks_bytes(100, 5000, iso.ISO_F32, 0)
    assert b >= lib.iso_blocks_bytes(100, 5000)
    assert lib.iso_view_blocks_bytes(100, 5000, iso.ISO_F32, 1) >= b + 100 * 5000 * 4
    assert lib.iso_view_blocks_bytes(100, 5000, iso.ISO_I32, 1) == 0


def _v(data=256, dt=0, so=3, si=0, se=1):
    import weighted_isotonic_regression_row_amd as iso
    return ctypes.byref(iso.IsoViewC(data, dt, so, si, se))


def _fitv(lib, y=None, w=None, outer=2, inner=1, n=3, inc=1, lo=-math.inf, hi=math.inf, fit=None, bo=None,
          bm=None, ws=1 << 16, wsb=1 << 26):
    y = _v() if y is None else y
    fit = _v(data=1 << 20) if fit is None else fit
    return lib.iso_fit_view(y, w, outer, inner, n, inc, lo, hi, fit, bo, bm, ws, wsb, None)


def test_fit_view_rejects_bad_arguments_on_host(lib):
    import weighted_isotonic_regression_row_amd as iso
    E = iso.ISO_EINVAL
    assert lib.iso_fit_view(None, None, 2, 1, 3, 1, -math.inf, math.inf, _v(), None, None, 1 << 16, 1 << 26,
                            None) == E
    assert _fitv(lib, outer=-1) == E
    assert _fitv(lib, n=-1) == E
    assert _fitv(lib, y=_v(dt=9)) == E                    # unknown dtype
    assert _fitv(lib, fit=_v(data=1 << 20, dt=iso.ISO_I32)) == E   # integer output
    assert _fitv(lib, y=_v(dt=iso.ISO_F64), fit=_v(data=1 << 20, dt=iso.ISO_F16)) == E  # float16 from float64
    assert _fitv(lib, y=_v(data=None)) == E
    assert _fitv(lib, y=_v(data=258)) == E               # not aligned to its element
    assert _fitv(lib, y=_v(se=-1)) == E                  # negative stride
    assert _fitv(lib, w=_v(dt=iso.ISO_F16, so=-3)) == E
    assert _fitv(lib, fit=_v(data=1 << 20, se=0)) == E    # an output that repeats itself
    assert _fitv(lib, ws=None) == E
    assert _fitv(lib, wsb=8) == E                        # workspace too small
    assert _fitv(lib, ws=(1 << 16) + 8) == E             # misaligned workspace
    assert _fitv(lib, inc=2) == E
    assert _fitv(lib, lo=1.0, hi=0.0) == E
    assert _fitv(lib, outer=1 << 62, inner=1 << 10) == E  # the row count overflows
    bc = iso.IsoBlocksC()
    assert _fitv(lib, bo=ctypes.byref(bc)) == E           # handle without memory


def test_fit_view_empty_is_a_noop(lib):
    import weighted_isotonic_regression_row_amd as iso
    bc = iso.IsoBlocksC()
    assert _fitv(lib, outer=0, ws=None, bo=ctypes.byref(bc), bm=8192) == iso.ISO_OK
    assert bc.valid == 1 and bc.rows == 0
    assert _fitv(lib, n=0, ws=None, y=_v(dt=iso.ISO_BF16), fit=_v(data=1 << 20, dt=iso.ISO_BF16)) == iso.ISO_OK


def test_vjp_view_rejects_bad_arguments_on_host(lib):
    import weighted_isotonic_regression_row_amd as iso
    E = iso.ISO_EINVAL
    bc = iso.IsoBlocksC()
    g, out = _v(), _v(data=1 << 20)
    assert lib.iso_vjp_view(g, ctypes.byref(bc), None, out, None, 2, 1, 1 << 16, 1 << 26, None) == E  # invalid
    bc.valid = 1
    bc.rows, bc.n, bc.words, bc.dtype = 2, 3, 1, 0
    bc.start_bits_dev, bc.clip_bits_dev, bc.row_nan_dev = 8192, 8192 + 256, 8192 + 512
    call = lambda g=g, y=None, gy=out, gw=None, outer=2, inner=1, ws=1 << 16, wsb=1 << 26: lib.iso_vjp_view(  # noqa
        g, ctypes.byref(bc), y, gy, gw, outer, inner, ws, wsb, None)
    assert call(g=None) == E
    assert call(gy=None) == E                              # no output
    assert call(gw=_v(data=1 << 21)) == E                  # grad_w without y
    assert call(outer=3) == E                              # rows differ from the handle's
    assert call(gy=_v(data=1 << 20, dt=iso.ISO_F64)) == E  # float64 output of a float32 fit
    assert call(gy=_v(data=1 << 20, se=0)) == E
    assert call(ws=None) == E
    assert call(wsb=8) == E
    bc.rows = 0
    assert call(outer=0) == iso.ISO_OK
