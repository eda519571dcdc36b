"""Batched weighted isotonic regression on AMD Instinct MI355X (gfx950).

Thin ctypes binding over libiso.so, whose C ABI is declared in include/iso.h.
The binding only marshals arguments: torch supplies device memory and the
current HIP stream; every step of the fit and of its backward pass runs in
the library's HIP kernels.  There is no CPU fallback: without the built
library (or without a GPU) the calls raise.

    fit, blocks = iso_fit(y, w, increasing=True, y_min=None, y_max=None)
    grad_y = iso_vjp(grad, blocks)
    grad_y, grad_w = iso_vjp_yw(grad, blocks, y)
    ranks, state = soft_rank(x, eps)
    grad_x = soft_rank_vjp(grad, state)
    xs, curve, m = calibration_fit(scores, labels)
    p = calibrate(new_scores, xs, curve, m)

The fit of each row is the weighted least-squares monotone sequence (page
"Merge Hulls Without Copying Vertices: GPU Isotonic Regression", Eq. (1)),
with the semantics of the "torchisotonic" PyPI page ("Semantics").  The soft rank is the composition of the first page's
Sec. 7.9: a per-row sort, the non-increasing fit of s - (n..1), and s minus
that fit in the original order.  The calibration curve is that of Sec. 7.7
and of the PyPI page's usage: scores sorted, equal scores pooled, the
weighted non-decreasing fit of the pooled means, evaluated by linear
interpolation.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch  # loaded first: libiso.so then binds to torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libiso.so")

ISO_F32 = 0
ISO_F64 = 1
ISO_F16 = 2
ISO_BF16 = 3
ISO_I32 = 4
ISO_I64 = 5
ISO_OK = 0
ISO_EINVAL = -1
ISO_EHIP = -2
ISO_EWEIGHT = -3
ISO_ETOOBIG = -4
NOALLOC_SCRATCH_BYTES = 128 << 20

SYMBOLS = ("iso_workspace_bytes", "iso_blocks_bytes", "iso_fit", "iso_fit_noalloc", "iso_vjp", "iso_vjp_yw", "iso_soft_rank_state_bytes",
           "iso_soft_rank_workspace_bytes", "iso_soft_rank", "iso_soft_rank_vjp", "iso_calibration_workspace_bytes",
           "iso_calibration_fit", "iso_calibrate", "iso_status", "iso_strerror", "iso_view_workspace_bytes",
           "iso_view_blocks_bytes", "iso_fit_view", "iso_vjp_view")


class IsoBlocksC(ctypes.Structure):
    """Mirror of struct iso_blocks (include/iso.h)."""

    _fields_ = [
        ("start_bits_dev", ctypes.c_void_p),
        ("clip_bits_dev", ctypes.c_void_p),
        ("row_nan_dev", ctypes.c_void_p),
        ("w_dev", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("n", ctypes.c_int64),
        ("words", ctypes.c_int64),
        ("dtype", ctypes.c_int),
        ("valid", ctypes.c_int),
    ]


class IsoSoftRankStateC(ctypes.Structure):
    """Mirror of struct iso_soft_rank_state (include/iso.h)."""

    _fields_ = [
        ("blocks", IsoBlocksC),
        ("perm_dev", ctypes.c_void_p),
        ("rank_dev", ctypes.c_void_p),
        ("eps", ctypes.c_double),
        ("valid", ctypes.c_int),
    ]


class IsoViewC(ctypes.Structure):
    """Mirror of struct iso_view (include/iso.h)."""

    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int),
        ("stride_outer", ctypes.c_int64),
        ("stride_inner", ctypes.c_int64),
        ("stride_elem", ctypes.c_int64),
    ]


class IsoError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


_lib = None


def load_library(path: str | None = None):
    """Load libiso.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with weighted_isotonic_regression_row_amd.build.build()")
    lib = ctypes.CDLL(p)
    vp, i64, c_int, c_size, c_double = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_double
    lib.iso_workspace_bytes.restype = c_size
    lib.iso_workspace_bytes.argtypes = [i64, i64, c_int]
    lib.iso_blocks_bytes.restype = c_size
    lib.iso_blocks_bytes.argtypes = [i64, i64]
    lib.iso_fit.restype = c_int
    lib.iso_fit.argtypes = [vp, vp, i64, i64, c_int, c_double, c_double, c_int, vp,
                            ctypes.POINTER(IsoBlocksC), vp, vp, c_size, vp]
    lib.iso_fit_noalloc.restype = c_int
    lib.iso_fit_noalloc.argtypes = [vp, vp, i64, i64, c_int, c_double, c_double, c_int, vp,
                                    ctypes.POINTER(IsoBlocksC), vp, vp]
    lib.iso_vjp.restype = c_int
    lib.iso_vjp.argtypes = [vp, ctypes.POINTER(IsoBlocksC), vp, vp, c_size, vp]
    lib.iso_vjp_yw.restype = c_int
    lib.iso_vjp_yw.argtypes = [vp, ctypes.POINTER(IsoBlocksC), vp, vp, vp, vp, c_size, vp]
    lib.iso_soft_rank_state_bytes.restype = c_size
    lib.iso_soft_rank_state_bytes.argtypes = [i64, i64]
    lib.iso_soft_rank_workspace_bytes.restype = c_size
    lib.iso_soft_rank_workspace_bytes.argtypes = [i64, i64, c_int]
    lib.iso_soft_rank.restype = c_int
    lib.iso_soft_rank.argtypes = [vp, i64, i64, c_double, c_int, vp, ctypes.POINTER(IsoSoftRankStateC), vp, vp,
                                  c_size, vp]
    lib.iso_soft_rank_vjp.restype = c_int
    lib.iso_soft_rank_vjp.argtypes = [vp, ctypes.POINTER(IsoSoftRankStateC), vp, vp, c_size, vp]
    lib.iso_calibration_workspace_bytes.restype = c_size
    lib.iso_calibration_workspace_bytes.argtypes = [i64, i64, c_int]
    lib.iso_calibration_fit.restype = c_int
    lib.iso_calibration_fit.argtypes = [vp, vp, i64, i64, c_int, vp, vp, vp, vp, c_size, vp]
    lib.iso_calibrate.restype = c_int
    lib.iso_calibrate.argtypes = [vp, vp, vp, i64, i64, vp, i64, c_int, vp, vp]
    lib.iso_view_workspace_bytes.restype = c_size
    lib.iso_view_workspace_bytes.argtypes = [i64, i64, c_int]
    lib.iso_view_blocks_bytes.restype = c_size
    lib.iso_view_blocks_bytes.argtypes = [i64, i64, c_int, c_int]
    pv = ctypes.POINTER(IsoViewC)
    lib.iso_fit_view.restype = c_int
    lib.iso_fit_view.argtypes = [pv, pv, i64, i64, i64, c_int, c_double, c_double, pv, ctypes.POINTER(IsoBlocksC),
                                 vp, vp, c_size, vp]
    lib.iso_vjp_view.restype = c_int
    lib.iso_vjp_view.argtypes = [pv, ctypes.POINTER(IsoBlocksC), pv, pv, pv, i64, i64, vp, c_size, vp]
    lib.iso_status.restype = c_int
    lib.iso_status.argtypes = [vp, vp]
    lib.iso_strerror.restype = ctypes.c_char_p
    lib.iso_strerror.argtypes = [c_int]
    if path is None:
        _lib = lib
    return lib


def strerror(code: int) -> str:
    try:
        return load_library().iso_strerror(int(code)).decode()
    except ImportError:
        return f"error {code}"


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return ISO_F32
    if t.dtype == torch.float64:
        return ISO_F64
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or float64)")


def _stream_ptr(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def iso_workspace_bytes(rows: int, n: int, dtype: torch.dtype) -> int:
    code = ISO_F32 if dtype == torch.float32 else ISO_F64
    return int(load_library().iso_workspace_bytes(rows, n, code))


def iso_blocks_bytes(rows: int, n: int) -> int:
    return int(load_library().iso_blocks_bytes(rows, n))


def workspace(rows: int, n: int, dtype: torch.dtype, device) -> torch.Tensor:
    """Allocate a workspace tensor (uint8, 256-byte aligned by torch's allocator)."""
    return torch.empty(max(iso_workspace_bytes(rows, n, dtype), 256), dtype=torch.uint8, device=device)


class Blocks:
    """Partition handle of a fit (struct iso_blocks plus the memory behind it)."""

    def __init__(self, c: IsoBlocksC, mem: torch.Tensor, w: torch.Tensor | None, shape):
        self.c = c
        self.mem = mem
        self.w = w  # keeps the borrowed weights alive
        self.shape = shape

    def bits(self):
        """(start_bits, clip_bits, row_nan) as device tensors (views of the memory)."""
        rows, words = self.c.rows, self.c.words
        m = self.mem
        nb = rows * words * 8
        stride = (nb + 255) // 256 * 256
        sb = m[:nb].view(torch.int64).view(rows, words)
        cb = m[stride:stride + nb].view(torch.int64).view(rows, words)
        rn = m[2 * stride:2 * stride + 4 * rows].view(torch.int32)
        return sb, cb, rn


def _check_like(t: torch.Tensor | None, like: torch.Tensor, name: str) -> None:
    """t must be a contiguous tensor of like's shape (as rows), dtype and device."""
    if t is None:
        return
    t2 = t.unsqueeze(0) if t.dim() == 1 else t
    if tuple(t2.shape) != tuple(like.shape) or t.dtype != like.dtype or t.device != like.device:
        raise ValueError(f"{name} must be a tensor of shape {tuple(like.shape)}, dtype {like.dtype} on {like.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_ws(ws: torch.Tensor | None, device, name: str = "ws") -> None:
    """A caller's workspace: a contiguous uint8 tensor on the device of the data (its size is checked by the
    library, which returns ISO_EINVAL when it is too small)."""
    if ws is None:
        return
    if ws.dtype != torch.uint8 or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"{name} must be a contiguous uint8 tensor on {device}")


def _check_device(t: torch.Tensor, device, name: str) -> None:
    if t.device != device:
        raise ValueError(f"{name} must be on {device} (it is on {t.device})")


def _require_cuda(t: torch.Tensor, what: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{what} runs on the GPU: its tensors must be device tensors")


def _as_rows(t: torch.Tensor) -> torch.Tensor:
    if t.dim() == 1:
        return t.unsqueeze(0)
    if t.dim() != 2:
        raise ValueError("expected a [rows, n] or [n] tensor")
    return t


def iso_fit(y: torch.Tensor, w: torch.Tensor | None = None, increasing: bool = True,
            y_min: float | None = None, y_max: float | None = None, *, out: torch.Tensor | None = None,
            blocks: bool = True, ws: torch.Tensor | None = None, check: bool = True):
    """Fit every row of y on the GPU.  Returns (fit, blocks or None).

    y, w: [rows, n] (or [n]) contiguous float32/float64 device tensors of one
    dtype; w None means unit weights.  check=True synchronises once to raise
    ValueError if a weight was not strictly positive (those rows are NaN).
    """
    shape = y.shape
    y2 = _as_rows(y)
    if not y2.is_contiguous():
        raise ValueError("y must be contiguous")
    rows, n = y2.shape
    dt = _dtype_code(y2)
    w2 = None
    if w is not None:
        w2 = _as_rows(w)
        _check_like(w2, y2, "w")
    _check_like(out, y2, "out")
    _check_ws(ws, y2.device)
    _require_cuda(y2, "iso_fit")
    lib = load_library()
    if out is None:
        out = torch.empty_like(y2)
    if ws is None:
        ws = workspace(rows, n, y2.dtype, y2.device)
    bc = IsoBlocksC()
    mem = None
    if blocks:
        mem = torch.empty(max(iso_blocks_bytes(rows, n), 256), dtype=torch.uint8, device=y2.device)
    lo = -math.inf if y_min is None else float(y_min)
    hi = math.inf if y_max is None else float(y_max)
    code = lib.iso_fit(y2.data_ptr(), None if w2 is None else w2.data_ptr(), rows, n, 1 if increasing else 0,
                       lo, hi, dt, out.data_ptr(), ctypes.byref(bc) if blocks else None,
                       None if mem is None else mem.data_ptr(), ws.data_ptr(), ws.numel(),
                       _stream_ptr(y2.device))
    if code != ISO_OK:
        raise IsoError(code, "iso_fit")
    if check:
        st = lib.iso_status(ws.data_ptr(), _stream_ptr(y2.device))
        if st == ISO_EWEIGHT:
            raise ValueError("weights must be strictly positive")
        if st != ISO_OK:
            raise IsoError(st, "iso_status")
    return out.view(shape), (Blocks(bc, mem, w2, shape) if blocks else None)


def iso_fit_noalloc(y: torch.Tensor, w: torch.Tensor | None = None, increasing: bool = True,
                    y_min: float | None = None, y_max: float | None = None, *, out: torch.Tensor,
                    blocks_mem: torch.Tensor | None = None):
    """iso_fit with the library's static scratch as its workspace (include/iso.h, iso_fit_noalloc): the caller
    passes the output (and, for the partition, blocks_mem of iso_blocks_bytes(rows, n) bytes) and nothing is
    allocated.  Returns (out, Blocks or None).  Raises IsoError(ISO_ETOOBIG) for problems whose workspace
    exceeds NOALLOC_SCRATCH_BYTES.  Calls on one GPU share the scratch: overlapping calls race."""
    shape = y.shape
    y2 = _as_rows(y)
    if not y2.is_contiguous():
        raise ValueError("y must be contiguous")
    rows, n = y2.shape
    dt = _dtype_code(y2)
    w2 = None
    if w is not None:
        w2 = _as_rows(w)
        _check_like(w2, y2, "w")
    _check_like(out, y2, "out")
    if blocks_mem is not None:
        _check_ws(blocks_mem, y2.device, "blocks_mem")
    _require_cuda(y2, "iso_fit_noalloc")
    lib = load_library()
    bc = IsoBlocksC()
    if blocks_mem is not None and blocks_mem.numel() < iso_blocks_bytes(rows, n):
        raise ValueError("blocks_mem holds fewer than iso_blocks_bytes(rows, n) bytes")
    lo = -math.inf if y_min is None else float(y_min)
    hi = math.inf if y_max is None else float(y_max)
    code = lib.iso_fit_noalloc(y2.data_ptr(), None if w2 is None else w2.data_ptr(), rows, n,
                               1 if increasing else 0, lo, hi, dt, out.data_ptr(),
                               ctypes.byref(bc) if blocks_mem is not None else None,
                               None if blocks_mem is None else blocks_mem.data_ptr(), _stream_ptr(y2.device))
    if code != ISO_OK:
        raise IsoError(code, "iso_fit_noalloc")
    return out.view(shape), (Blocks(bc, blocks_mem, w2, shape) if blocks_mem is not None else None)


def iso_vjp(grad: torch.Tensor, blocks: Blocks, *, out: torch.Tensor | None = None,
            ws: torch.Tensor | None = None) -> torch.Tensor:
    """grad_y = w_j * sum_{i in B(j), clip inactive} grad_i / sum_{i in B(j)} w_i."""
    g2 = _as_rows(grad)
    rows, n = blocks.c.rows, blocks.c.n
    if tuple(g2.shape) != (rows, n) or not g2.is_contiguous():
        raise ValueError("grad must be a contiguous tensor of the fit's shape")
    if _dtype_code(g2) != blocks.c.dtype:
        raise ValueError("grad must have the fit's dtype")
    _check_device(g2, blocks.mem.device, "grad")
    _check_like(out, g2, "out")
    _check_ws(ws, g2.device)
    _require_cuda(g2, "iso_vjp")
    lib = load_library()
    if out is None:
        out = torch.empty_like(g2)
    if ws is None:
        ws = workspace(rows, n, g2.dtype, g2.device)
    code = lib.iso_vjp(g2.data_ptr(), ctypes.byref(blocks.c), out.data_ptr(), ws.data_ptr(), ws.numel(),
                       _stream_ptr(g2.device))
    if code != ISO_OK:
        raise IsoError(code, "iso_vjp")
    return out.view(blocks.shape)


def iso_vjp_yw(grad: torch.Tensor, blocks: Blocks, y: torch.Tensor, *, want_y: bool = True,
               ws: torch.Tensor | None = None):
    """(grad_y or None, grad_w): grad_w = G_B (y_j - mean_B) / W_B over the fit's blocks, where y is the
    tensor the fit was computed from (page "torchisotonic", "Semantics": differentiable in y and in w)."""
    g2 = _as_rows(grad)
    y2 = _as_rows(y)
    rows, n = blocks.c.rows, blocks.c.n
    for t, name in ((g2, "grad"), (y2, "y")):
        if tuple(t.shape) != (rows, n) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor of the fit's shape")
        if _dtype_code(t) != blocks.c.dtype:
            raise ValueError(f"{name} must have the fit's dtype")
        _check_device(t, blocks.mem.device, name)
    _check_ws(ws, g2.device)
    _require_cuda(g2, "iso_vjp_yw")
    lib = load_library()
    gy = torch.empty_like(g2) if want_y else None
    gw = torch.empty_like(g2)
    if ws is None:
        ws = workspace(rows, n, g2.dtype, g2.device)
    code = lib.iso_vjp_yw(g2.data_ptr(), ctypes.byref(blocks.c), y2.data_ptr(),
                          None if gy is None else gy.data_ptr(), gw.data_ptr(), ws.data_ptr(), ws.numel(),
                          _stream_ptr(g2.device))
    if code != ISO_OK:
        raise IsoError(code, "iso_vjp_yw")
    return (None if gy is None else gy.view(blocks.shape)), gw.view(blocks.shape)


# ---------------------------------------------------------------------------
# views: any axis, broadcast weights, float16 / bfloat16 / integer inputs
# (page "torchisotonic", "Semantics")
# ---------------------------------------------------------------------------

_VIEW_CODES = {torch.float32: ISO_F32, torch.float64: ISO_F64, torch.float16: ISO_F16, torch.bfloat16: ISO_BF16,
               torch.int32: ISO_I32, torch.int64: ISO_I64}


def _view_code(t: torch.Tensor, output: bool = False) -> int:
    c = _VIEW_CODES.get(t.dtype)
    if c is None or (output and c > ISO_BF16):
        raise TypeError(f"unsupported dtype {t.dtype}")
    return c


def _result_dtype(y: torch.Tensor) -> torch.dtype:
    """Float input keeps its dtype; integer input becomes the default float dtype (PyPI page, "Semantics")."""
    if y.dtype in (torch.float16, torch.bfloat16, torch.float32, torch.float64):
        return y.dtype
    if y.dtype in (torch.int32, torch.int64, torch.int16, torch.int8, torch.uint8, torch.bool):
        return torch.get_default_dtype()
    raise TypeError(f"unsupported dtype {y.dtype}")


def _fold(shape, axis: int, tensors):
    """The logical [outer, inner, n] geometry of a fit along `axis`: the other axes, in order, with size-1 axes
    dropped and neighbours merged where every tensor's strides allow it.  Returns (outer, inner, n, strides),
    strides[k] = (outer, inner, elem) element strides of tensors[k]; ValueError if more than two batch strides
    remain."""
    n = shape[axis]
    groups = []  # [size, [stride of each tensor at the group's innermost axis]]
    for k, size in enumerate(shape):
        if k == axis or size == 1:
            continue
        st = [t.stride(k) for t in tensors]
        if groups and all(g == s_ * size for g, s_ in zip(groups[-1][1], st)):
            groups[-1][0] *= size
            groups[-1][1] = st
        else:
            groups.append([size, st])
    if len(groups) > 2:
        raise ValueError("this layout needs more than two batch strides; pass a contiguous tensor")
    while len(groups) < 2:
        groups.insert(0, [1, [0] * len(tensors)])
    (outer, so), (inner, si) = groups
    strides = [(so[k], si[k], t.stride(axis) if n > 1 else 1) for k, t in enumerate(tensors)]
    return outer, inner, n, strides


def _view(t: torch.Tensor | None, strides, output: bool = False):
    if t is None:
        return None
    return IsoViewC(t.data_ptr(), _view_code(t, output), *strides)


def _view_ws(rows: int, n: int, cdt: int, device) -> torch.Tensor:
    return torch.empty(max(int(load_library().iso_view_workspace_bytes(rows, n, cdt)), 256), dtype=torch.uint8,
                       device=device)


class ViewBlocks(Blocks):
    """Partition handle of iso_fit_view: the logical rows r = o * inner + j of the fit, plus the geometry."""

    def __init__(self, c, mem, w, shape, axis, outer, inner, out_dtype):
        super().__init__(c, mem, w, shape)
        self.axis, self.outer, self.inner, self.out_dtype = axis, outer, inner, out_dtype


def iso_fit_view(y: torch.Tensor, w: torch.Tensor | None = None, increasing: bool = True,
                 y_min: float | None = None, y_max: float | None = None, *, dim: int = -1, blocks: bool = True,
                 ws: torch.Tensor | None = None, check: bool = True):
    """Fit y along axis `dim` (include/iso.h, iso_fit_view).  y: any strided device tensor of float16, bfloat16,
    float32, float64, int32 or int64; w: None or a tensor that broadcasts to y's shape.  The result has y's shape
    and y's dtype (integer y: the default float dtype).  Returns (fit, ViewBlocks or None)."""
    _require_cuda(y, "iso_fit_view")
    if y.dim() == 0:
        raise ValueError("y needs at least one axis")
    axis = dim % y.dim()
    shape = tuple(y.shape)
    if w is not None:
        _check_device(w, y.device, "w")
        try:
            w = w.expand(shape)
        except RuntimeError as e:
            raise ValueError(f"w of shape {tuple(w.shape)} does not broadcast to {shape}") from e
    _check_ws(ws, y.device)
    # the output keeps y's layout when y is dense (so it folds as y does), else it is contiguous
    out = torch.empty_like(y, dtype=_result_dtype(y), memory_format=torch.preserve_format)
    tensors = [y, out] + ([w] if w is not None else [])
    outer, inner, n, strides = _fold(shape, axis, tensors)
    rows = outer * inner
    cdt = ISO_F64 if (y.dtype == torch.float64 or out.dtype == torch.float64) else ISO_F32
    lib = load_library()
    if ws is None:
        ws = _view_ws(rows, n, cdt, y.device)
    bc = IsoBlocksC()
    mem = None
    if blocks:
        nb = int(lib.iso_view_blocks_bytes(rows, n, cdt, 1 if w is not None else 0))
        mem = torch.empty(max(nb, 256), dtype=torch.uint8, device=y.device)
    lo = -math.inf if y_min is None else float(y_min)
    hi = math.inf if y_max is None else float(y_max)
    yv, ov = _view(y, strides[0]), _view(out, strides[1], output=True)
    wv = _view(w, strides[2]) if w is not None else None
    code = lib.iso_fit_view(ctypes.byref(yv), None if wv is None else ctypes.byref(wv), outer, inner, n,
                            1 if increasing else 0, lo, hi, ctypes.byref(ov), ctypes.byref(bc) if blocks else None,
                            None if mem is None else mem.data_ptr(), ws.data_ptr(), ws.numel(),
                            _stream_ptr(y.device))
    if code != ISO_OK:
        raise IsoError(code, "iso_fit_view")
    if check and rows * n > 0:
        st = lib.iso_status(ws.data_ptr(), _stream_ptr(y.device))
        if st == ISO_EWEIGHT:
            raise ValueError("weights must be strictly positive")
        if st != ISO_OK:
            raise IsoError(st, "iso_status")
    vb = ViewBlocks(bc, mem, w, shape, axis, outer, inner, out.dtype) if blocks else None
    return out, vb


def iso_vjp_view(grad: torch.Tensor, blocks: ViewBlocks, y: torch.Tensor | None = None, *, want_y: bool = True,
                 ws: torch.Tensor | None = None):
    """(grad_y or None, grad_w or None) of a fit made by iso_fit_view (include/iso.h, iso_vjp_view).  grad has
    the fit's shape; grad_w (when y, the tensor the fit was given, is passed) is per element of y's shape: for
    broadcast weights its sum over the broadcast axes is the product in the caller's weights."""
    _require_cuda(grad, "iso_vjp_view")
    shape = blocks.shape
    if tuple(grad.shape) != shape:
        raise ValueError(f"grad must have the fit's shape {shape}")
    _check_device(grad, blocks.mem.device, "grad")
    if y is not None:
        if tuple(y.shape) != shape:
            raise ValueError(f"y must have the fit's shape {shape}")
        _check_device(y, grad.device, "y")
    if not want_y and y is None:
        raise ValueError("nothing to compute: want_y=False and no y for the product in w")
    _check_ws(ws, grad.device)
    like = y if y is not None else grad
    gy = torch.empty_like(like, dtype=blocks.out_dtype, memory_format=torch.preserve_format) if want_y else None
    gw = torch.empty_like(like, dtype=blocks.out_dtype, memory_format=torch.preserve_format) if y is not None else None
    tensors = [grad] + [t for t in (y, gy, gw) if t is not None]
    outer, inner, n, strides = _fold(shape, blocks.axis, tensors)
    if outer * inner != blocks.c.rows:
        raise ValueError("grad's layout does not match the fit's rows")
    k = iter(strides[1:])
    yv = _view(y, next(k)) if y is not None else None
    gyv = _view(gy, next(k), output=True) if gy is not None else None
    gwv = _view(gw, next(k), output=True) if gw is not None else None
    gv = _view(grad, strides[0])
    lib = load_library()
    if ws is None:
        ws = _view_ws(outer * inner, n, blocks.c.dtype, grad.device)
    ref = lambda v: None if v is None else ctypes.byref(v)  # noqa: E731
    code = lib.iso_vjp_view(ctypes.byref(gv), ctypes.byref(blocks.c), ref(yv), ref(gyv), ref(gwv), outer, inner,
                            ws.data_ptr(), ws.numel(), _stream_ptr(grad.device))
    if code != ISO_OK:
        raise IsoError(code, "iso_vjp_view")
    return gy, gw


class _Isotonic(torch.autograd.Function):
    """The fit as a differentiable function of y and of (broadcast-expanded) w."""

    @staticmethod
    def forward(ctx, y, w, increasing, y_min, y_max, dim):
        fit, blocks = iso_fit_view(y, w, increasing, y_min, y_max, dim=dim)
        ctx.blocks = blocks
        ctx.save_for_backward(y)
        return fit

    @staticmethod
    def backward(ctx, grad):
        (y,) = ctx.saved_tensors
        need_y, need_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        gy, gw = iso_vjp_view(grad, ctx.blocks, y if need_w else None, want_y=True)
        return (gy if need_y else None), gw, None, None, None, None


def isotonic(y: torch.Tensor, w: torch.Tensor | None = None, *, increasing: bool = True,
             y_min: float | None = None, y_max: float | None = None, dim: int = -1) -> torch.Tensor:
    """The isotonic fit with the PyPI page's semantics ("Semantics"): strictly positive weights of y's shape or
    broadcast to it, clipping to [y_min, y_max] after the fit, `dim` picks the axis, a row holding a NaN comes
    back NaN, float input keeps its dtype (float16 and bfloat16 computed in float32), integer input becomes the
    default float dtype; differentiable in y and in w (for a broadcast w, autograd sums the per-element product
    over the broadcast axes)."""
    if w is not None and w.requires_grad:
        w = w.expand(y.shape)  # the expand's backward reduces grad_w to w's shape
    if torch.is_grad_enabled() and (y.requires_grad or (w is not None and w.requires_grad)):
        return _Isotonic.apply(y, w, increasing, y_min, y_max, dim)
    fit, _ = iso_fit_view(y, w, increasing, y_min, y_max, dim=dim, blocks=False)
    return fit


class SoftRankState:
    """Backward state of soft_rank (struct iso_soft_rank_state plus the memory behind it)."""

    def __init__(self, c: IsoSoftRankStateC, mem: torch.Tensor, shape):
        self.c = c
        self.mem = mem
        self.shape = shape
        self.blocks = Blocks(c.blocks, mem, None, shape)

    def perm(self) -> torch.Tensor:
        """[rows, n] int32 view: index of the element at each sorted position."""
        rows, n = self.c.blocks.rows, self.c.blocks.n
        off = self.c.perm_dev - self.mem.data_ptr()
        return self.mem[off:off + 4 * rows * n].view(torch.int32).view(rows, n)

    def rank(self) -> torch.Tensor:
        """[rows, n] int32 view: sorted position of each element (the inverse of perm)."""
        rows, n = self.c.blocks.rows, self.c.blocks.n
        off = self.c.rank_dev - self.mem.data_ptr()
        return self.mem[off:off + 4 * rows * n].view(torch.int32).view(rows, n)


def soft_rank_workspace(rows: int, n: int, dtype: torch.dtype, device) -> torch.Tensor:
    code = ISO_F32 if dtype == torch.float32 else ISO_F64
    nb = int(load_library().iso_soft_rank_workspace_bytes(rows, n, code))
    if nb == 0:
        raise ValueError(f"bad soft-rank sizes {rows} x {n} or dtype {dtype}")
    return torch.empty(nb, dtype=torch.uint8, device=device)


def soft_rank(x: torch.Tensor, eps: float = 1.0, *, out: torch.Tensor | None = None,
              ws: torch.Tensor | None = None):
    """Soft ranks of every row of x (first page, Sec. 7.9): the projection of x / eps onto the
    permutahedron of (1..n).  Returns (ranks, state); rows of any length (longer than 8192: sorted by tiles
    and merge passes)."""
    shape = x.shape
    x2 = _as_rows(x)
    if not x2.is_contiguous():
        raise ValueError("x must be contiguous")
    rows, n = x2.shape
    dt = _dtype_code(x2)
    _check_like(out, x2, "out")
    _check_ws(ws, x2.device)
    _require_cuda(x2, "soft_rank")
    lib = load_library()
    if out is None:
        out = torch.empty_like(x2)
    if ws is None:
        ws = soft_rank_workspace(rows, n, x2.dtype, x2.device)
    mem = torch.empty(max(int(lib.iso_soft_rank_state_bytes(rows, n)), 256), dtype=torch.uint8, device=x2.device)
    st = IsoSoftRankStateC()
    code = lib.iso_soft_rank(x2.data_ptr(), rows, n, float(eps), dt, out.data_ptr(), ctypes.byref(st), mem.data_ptr(),
                             ws.data_ptr(), ws.numel(), _stream_ptr(x2.device))
    if code != ISO_OK:
        raise IsoError(code, "iso_soft_rank")
    return out.view(shape), SoftRankState(st, mem, shape)


def soft_rank_vjp(grad: torch.Tensor, state: SoftRankState, *, out: torch.Tensor | None = None,
                  ws: torch.Tensor | None = None) -> torch.Tensor:
    """Gradient in x of <grad, soft_rank(x, eps)>: P^T (g_s - A g_s) / eps over the fit's blocks."""
    g2 = _as_rows(grad)
    rows, n = state.c.blocks.rows, state.c.blocks.n
    if tuple(g2.shape) != (rows, n) or not g2.is_contiguous():
        raise ValueError("grad must be a contiguous tensor of the ranks' shape")
    if _dtype_code(g2) != state.c.blocks.dtype:
        raise ValueError("grad must have the ranks' dtype")
    _check_device(g2, state.mem.device, "grad")
    _check_like(out, g2, "out")
    _check_ws(ws, g2.device)
    _require_cuda(g2, "soft_rank_vjp")
    lib = load_library()
    if out is None:
        out = torch.empty_like(g2)
    if ws is None:
        ws = soft_rank_workspace(rows, n, g2.dtype, g2.device)
    code = lib.iso_soft_rank_vjp(g2.data_ptr(), ctypes.byref(state.c), out.data_ptr(), ws.data_ptr(), ws.numel(),
                                 _stream_ptr(g2.device))
    if code != ISO_OK:
        raise IsoError(code, "iso_soft_rank_vjp")
    return out.view(state.shape)


def calibration_workspace(rows: int, n: int, dtype: torch.dtype, device) -> torch.Tensor:
    code = ISO_F32 if dtype == torch.float32 else ISO_F64
    return torch.empty(max(int(load_library().iso_calibration_workspace_bytes(rows, n, code)), 256), dtype=torch.uint8,
                       device=device)


def calibration_fit(scores: torch.Tensor, labels: torch.Tensor, *, ws: torch.Tensor | None = None):
    """Calibration curve of every row (first page, Sec. 7.7; PyPI page, "What it is for"): returns (xs, fit, m),
    the m[r] distinct scores of row r in increasing order and the curve there (entries past m[r] unspecified)."""
    s2 = _as_rows(scores)
    l2 = _as_rows(labels)
    if s2.shape != l2.shape or s2.dtype != l2.dtype or s2.device != l2.device:
        raise ValueError("labels must have the shape, dtype and device of scores")
    if not s2.is_contiguous() or not l2.is_contiguous():
        raise ValueError("scores and labels must be contiguous")
    rows, n = s2.shape
    dt = _dtype_code(s2)
    _check_ws(ws, s2.device)
    _require_cuda(s2, "calibration_fit")
    lib = load_library()
    xs = torch.empty_like(s2)
    fit = torch.empty_like(s2)
    m = torch.empty(rows, dtype=torch.int32, device=s2.device)
    if ws is None:
        ws = calibration_workspace(rows, n, s2.dtype, s2.device)
    code = lib.iso_calibration_fit(s2.data_ptr(), l2.data_ptr(), rows, n, dt, xs.data_ptr(), fit.data_ptr(),
                                   m.data_ptr(), ws.data_ptr(), ws.numel(), _stream_ptr(s2.device))
    if code != ISO_OK:
        raise IsoError(code, "iso_calibration_fit")
    return xs, fit, m


def calibrate(q: torch.Tensor, xs: torch.Tensor, fit: torch.Tensor, m: torch.Tensor, *,
              out: torch.Tensor | None = None) -> torch.Tensor:
    """Calibrated values of the queries q [rows, k] on the curves (linear between points, constant beyond)."""
    shape = q.shape
    q2 = _as_rows(q)
    if xs.dim() != 2 or not xs.is_contiguous():
        raise ValueError("xs must be the contiguous [rows, n] points of calibration_fit")
    _check_like(fit, xs, "fit")
    if not q2.is_contiguous() or q2.dtype != xs.dtype or q2.shape[0] != xs.shape[0]:
        raise ValueError("q must be contiguous, of the curve's dtype, one row per curve")
    if m.dtype != torch.int32 or m.numel() != xs.shape[0] or not m.is_contiguous():
        raise ValueError("m must be the int32 counts of calibration_fit")
    for t, name in ((q2, "q"), (m, "m")):
        _check_device(t, xs.device, name)
    _check_like(out, q2, "out")
    _require_cuda(q2, "calibrate")
    lib = load_library()
    rows, k = q2.shape
    if out is None:
        out = torch.empty_like(q2)
    code = lib.iso_calibrate(xs.data_ptr(), fit.data_ptr(), m.data_ptr(), rows, xs.shape[1], q2.data_ptr(), k,
                             _dtype_code(q2), out.data_ptr(), _stream_ptr(q2.device))
    if code != ISO_OK:
        raise IsoError(code, "iso_calibrate")
    return out.view(shape)


def iso_status(ws: torch.Tensor) -> int:
    return int(load_library().iso_status(ws.data_ptr(), _stream_ptr(ws.device)))


__all__ = ["isotonic", "iso_fit_view", "iso_vjp_view", "ViewBlocks", "iso_fit", "iso_fit_noalloc", "iso_vjp", "iso_vjp_yw", "soft_rank", "soft_rank_vjp", "SoftRankState", "soft_rank_workspace",
           "calibration_fit", "calibrate", "calibration_workspace",
           "iso_status", "iso_workspace_bytes", "iso_blocks_bytes", "workspace",
           "Blocks", "IsoError", "load_library", "SYMBOLS"]
