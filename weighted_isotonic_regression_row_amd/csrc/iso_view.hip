// Strided, typed views of the fit's inputs and outputs (include/iso.h,
// iso_fit_view and iso_vjp_view): the operator's input semantics of the
// "torchisotonic" PyPI page ("Semantics": weights of y's shape or broadcast
// to it, `dim` picks the axis, float16 and bfloat16 computed in float32,
// integer input made float).
//
// The fit itself always runs on contiguous rows of the compute type.  A view
// that is already such rows is passed through; any other is converted by a
// gather kernel into the workspace first, and an output view that is not is
// written by a scatter kernel from the workspace afterwards.  Both move each
// element once: straight through when a view's rows are contiguous, else
// through an LDS tile of 64 rows x 64 elements, so that reads and writes are
// both along the axis that is contiguous in memory (a fit along dim 0 of a
// row-major matrix reads down its columns).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/iso.h"
#include "iso_internal.hpp"
#include "iso_prepare.hpp"

namespace iso {
namespace {

struct VArg {
    char* p;
    int dt;
    int64_t so, si, se;
};

constexpr int kTile = 64;
constexpr int kViewThreads = 256;

// element offset of (row r, element i) of a view over rows of `inner`
__device__ __forceinline__ int64_t view_off(const VArg& v, int64_t r, int64_t inner, int64_t i) {
    int64_t o = r, j = 0;
    if (inner > 1) {
        o = r / inner;
        j = r - o * inner;
    }
    return o * v.so + j * v.si + i * v.se;
}

template <typename D>
__device__ __forceinline__ D load_as(const char* p, int dt, int64_t off) {
    switch (dt) {
        case ISO_F32:
            return (D)((const float*)p)[off];
        case ISO_F64:
            return (D)((const double*)p)[off];
        case ISO_F16:
            return (D)(float)((const _Float16*)p)[off];
        case ISO_BF16:
            // bfloat16 is the high half of a binary32
            return (D)__uint_as_float((uint32_t)((const uint16_t*)p)[off] << 16);
        case ISO_I32:
            return (D)((const int32_t*)p)[off];
        default:
            return (D)((const int64_t*)p)[off];
    }
}

// binary32 to bfloat16, rounding to nearest with ties to even on the 16 bits
// dropped; a NaN stays a (quiet) NaN of the same sign
__device__ __forceinline__ uint16_t bf16_of(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <typename D>
__device__ __forceinline__ void store_as(char* p, int dt, int64_t off, D x) {
    switch (dt) {
        case ISO_F32:
            ((float*)p)[off] = (float)x;
            break;
        case ISO_F64:
            ((double*)p)[off] = (double)x;
            break;
        case ISO_F16:
            ((_Float16*)p)[off] = (_Float16)(float)x;
            break;
        default:
            ((uint16_t*)p)[off] = bf16_of((float)x);
            break;
    }
}

// view -> contiguous [rows, n] of D, one element per thread and step
template <typename D>
__global__ __launch_bounds__(kViewThreads) void k_gather_rows(VArg v, int64_t rows, int64_t n, int64_t inner,
                                                              D* __restrict__ out) {
    const int64_t total = rows * n;
    for (int64_t e = (int64_t)blockIdx.x * kViewThreads + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * kViewThreads) {
        const int64_t r = e / n, i = e - r * n;
        out[e] = load_as<D>(v.p, v.dt, view_off(v, r, inner, i));
    }
}

// contiguous [rows, n] of D -> view
template <typename D>
__global__ __launch_bounds__(kViewThreads) void k_scatter_rows(const D* __restrict__ in, int64_t rows, int64_t n,
                                                               int64_t inner, VArg v) {
    const int64_t total = rows * n;
    for (int64_t e = (int64_t)blockIdx.x * kViewThreads + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * kViewThreads) {
        const int64_t r = e / n, i = e - r * n;
        store_as<D>(v.p, v.dt, view_off(v, r, inner, i), in[e]);
    }
}

// One 64 x 64 tile (rows r0.., elements i0..) per workgroup for views whose
// consecutive rows, not elements, are adjacent in memory: the view side walks
// along rows, the contiguous side along elements, and LDS transposes.
template <typename D>
__global__ __launch_bounds__(kViewThreads) void k_gather_tiles(VArg v, int64_t rows, int64_t n, int64_t inner,
                                                               int64_t tiles_n, D* __restrict__ out) {
    __shared__ D tile[kTile][kTile + 1];
    const int64_t r0 = (int64_t)(blockIdx.x / tiles_n) * kTile, i0 = (int64_t)(blockIdx.x % tiles_n) * kTile;
    const int t = threadIdx.x, a = t / kTile, b = t % kTile;
#pragma unroll 4
    for (int k = 0; k < kTile; k += kViewThreads / kTile) {
        const int64_t r = r0 + b, i = i0 + k + a;  // consecutive threads: consecutive rows
        if (r < rows && i < n) tile[b][k + a] = load_as<D>(v.p, v.dt, view_off(v, r, inner, i));
    }
    __syncthreads();
#pragma unroll 4
    for (int k = 0; k < kTile; k += kViewThreads / kTile) {
        const int64_t r = r0 + k + a, i = i0 + b;  // consecutive threads: consecutive elements
        if (r < rows && i < n) out[r * n + i] = tile[k + a][b];
    }
}

template <typename D>
__global__ __launch_bounds__(kViewThreads) void k_scatter_tiles(const D* __restrict__ in, int64_t rows, int64_t n,
                                                                int64_t inner, int64_t tiles_n, VArg v) {
    __shared__ D tile[kTile][kTile + 1];
    const int64_t r0 = (int64_t)(blockIdx.x / tiles_n) * kTile, i0 = (int64_t)(blockIdx.x % tiles_n) * kTile;
    const int t = threadIdx.x, a = t / kTile, b = t % kTile;
#pragma unroll 4
    for (int k = 0; k < kTile; k += kViewThreads / kTile) {
        const int64_t r = r0 + k + a, i = i0 + b;
        if (r < rows && i < n) tile[k + a][b] = in[r * n + i];
    }
    __syncthreads();
#pragma unroll 4
    for (int k = 0; k < kTile; k += kViewThreads / kTile) {
        const int64_t r = r0 + b, i = i0 + k + a;
        if (r < rows && i < n) store_as<D>(v.p, v.dt, view_off(v, r, inner, i), tile[b][k + a]);
    }
}

size_t esize(int dt) {
    switch (dt) {
        case ISO_F16:
        case ISO_BF16:
            return 2;
        case ISO_F32:
        case ISO_I32:
            return 4;
        default:
            return 8;
    }
}

bool input_dtype(int d) { return d >= ISO_F32 && d <= ISO_I64; }
bool output_dtype(int d) { return d >= ISO_F32 && d <= ISO_BF16; }

// a view's own checks: data present and aligned to its element, strides >= 0
bool view_ok(const iso_view* v, bool output) {
    if (!v || !v->data) return false;
    if (output ? !output_dtype(v->dtype) : !input_dtype(v->dtype)) return false;
    if (v->stride_outer < 0 || v->stride_inner < 0 || v->stride_elem < 0) return false;
    return ((uintptr_t)v->data % esize(v->dtype)) == 0;
}

// the view is contiguous rows of dtype dt: row r at r * n
bool plain(const iso_view* v, int dt, int64_t outer, int64_t inner, int64_t n) {
    return v->dtype == dt && (n == 1 || v->stride_elem == 1) && (inner == 1 || v->stride_inner == n) &&
           (outer == 1 || v->stride_outer == inner * n);
}

// whether consecutive rows are adjacent in memory while elements are not
bool rows_adjacent(const iso_view* v, int64_t inner, int64_t n) {
    if (n == 1 || v->stride_elem == 1) return false;
    return inner > 1 ? v->stride_inner == 1 : v->stride_outer == 1;
}

VArg varg(const iso_view* v) { return VArg{(char*)v->data, v->dtype, v->stride_outer, v->stride_inner, v->stride_elem}; }

unsigned grid_rows(int64_t total) {
    const int64_t b = (total + kViewThreads - 1) / kViewThreads;
    return (unsigned)(b < 8192 ? b : 8192);
}

template <typename D>
hipError_t gather(const iso_view* v, int64_t rows, int64_t n, int64_t inner, void* out, hipStream_t st) {
    if (rows_adjacent(v, inner, n)) {
        const int64_t tn = (n + kTile - 1) / kTile, tr = (rows + kTile - 1) / kTile;
        k_gather_tiles<D><<<dim3((unsigned)(tn * tr)), dim3(kViewThreads), 0, st>>>(varg(v), rows, n, inner, tn,
                                                                                     (D*)out);
    } else {
        k_gather_rows<D><<<dim3(grid_rows(rows * n)), dim3(kViewThreads), 0, st>>>(varg(v), rows, n, inner, (D*)out);
    }
    return hipGetLastError();
}

template <typename D>
hipError_t scatter(const void* in, const iso_view* v, int64_t rows, int64_t n, int64_t inner, hipStream_t st) {
    if (rows_adjacent(v, inner, n)) {
        const int64_t tn = (n + kTile - 1) / kTile, tr = (rows + kTile - 1) / kTile;
        k_scatter_tiles<D><<<dim3((unsigned)(tn * tr)), dim3(kViewThreads), 0, st>>>((const D*)in, rows, n, inner,
                                                                                      tn, varg(v));
    } else {
        k_scatter_rows<D><<<dim3(grid_rows(rows * n)), dim3(kViewThreads), 0, st>>>((const D*)in, rows, n, inner,
                                                                                     varg(v));
    }
    return hipGetLastError();
}

hipError_t gather_c(int cdt, const iso_view* v, int64_t rows, int64_t n, int64_t inner, void* out, hipStream_t st) {
    return cdt == ISO_F32 ? gather<float>(v, rows, n, inner, out, st) : gather<double>(v, rows, n, inner, out, st);
}

hipError_t scatter_c(int cdt, const void* in, const iso_view* v, int64_t rows, int64_t n, int64_t inner,
                     hipStream_t st) {
    return cdt == ISO_F32 ? scatter<float>(in, v, rows, n, inner, st) : scatter<double>(in, v, rows, n, inner, st);
}

// the logical row count, or -1 when outer * inner overflows or a size is negative
int64_t row_count(int64_t outer, int64_t inner, int64_t n) {
    if (outer < 0 || inner < 0 || n < 0) return -1;
    if (inner > 0 && outer > INT64_MAX / inner) return -1;
    const int64_t rows = outer * inner;
    if (rows > 0 && n > INT64_MAX / rows / 8) return -1;
    return rows;
}

// Workspace of the view entry points: the solver's layout, then four arrays
// of [rows, n] in the compute type (converted inputs and outputs).
size_t staging_bytes(int64_t rows, int64_t n, int cdt) {
    return align256((size_t)rows * (size_t)n * (cdt == ISO_F32 ? 4 : 8));
}

size_t view_ws_bytes(int64_t rows, int64_t n, int cdt) {
    return align256(make_layout(rows, n).total) + 4 * staging_bytes(rows, n, cdt);
}

// The compute type: float64 when y or the output is float64, else float32.
// Outputs of float16 / bfloat16 come from float32 only.
int compute_type(int y_dt, int out_dt) {
    const int c = (y_dt == ISO_F64 || out_dt == ISO_F64) ? ISO_F64 : ISO_F32;
    if ((out_dt == ISO_F16 || out_dt == ISO_BF16) && c != ISO_F32) return -1;
    return c;
}

}  // namespace
}  // namespace iso

extern "C" {

size_t iso_view_workspace_bytes(int64_t rows, int64_t n, int compute_dtype) {
    if (rows < 0 || n < 0 || (compute_dtype != ISO_F32 && compute_dtype != ISO_F64)) return 0;
    return iso::view_ws_bytes(rows, n, compute_dtype);
}

size_t iso_view_blocks_bytes(int64_t rows, int64_t n, int compute_dtype, int weighted) {
    if (rows < 0 || n < 0 || (compute_dtype != ISO_F32 && compute_dtype != ISO_F64)) return 0;
    const size_t b = iso::align256(iso_blocks_bytes(rows, n));
    return weighted ? b + iso::staging_bytes(rows, n, compute_dtype) : b;
}

int iso_fit_view(const iso_view* y, const iso_view* w, int64_t outer, int64_t inner, int64_t n, int increasing,
                 double y_min, double y_max, const iso_view* fit, iso_blocks* blocks_out, void* blocks_mem,
                 void* workspace, size_t workspace_bytes, void* stream) {
    using namespace iso;
    const int64_t rows = row_count(outer, inner, n);
    if (rows < 0 || !y || !fit) return ISO_EINVAL;
    if (!input_dtype(y->dtype) || !output_dtype(fit->dtype) || (w && !input_dtype(w->dtype))) return ISO_EINVAL;
    const int cdt = compute_type(y->dtype, fit->dtype);
    if (cdt < 0) return ISO_EINVAL;
    if (rows > 0 && n > 0) {
        if (!view_ok(y, false) || !view_ok(fit, true) || (w && !view_ok(w, false))) return ISO_EINVAL;
        if (!workspace || workspace_bytes < view_ws_bytes(rows, n, cdt)) return ISO_EINVAL;
        if (fit->stride_elem == 0 && n > 1) return ISO_EINVAL;  // the output may not repeat itself
    }
    char* ws = (char*)workspace;
    const size_t base = rows > 0 && n > 0 ? align256(make_layout(rows, n).total) : 0;
    const size_t area = staging_bytes(rows, n, cdt);
    const bool yp = rows == 0 || n == 0 || plain(y, cdt, outer, inner, n);
    const bool wp = !w || rows == 0 || n == 0 || plain(w, cdt, outer, inner, n);
    const bool fp = rows == 0 || n == 0 || plain(fit, cdt, outer, inner, n);
    const void* yc = yp ? y->data : (const void*)(ws + base);
    const void* wc = !w ? nullptr
                        : wp ? w->data
                             : (const void*)(blocks_mem ? (char*)blocks_mem + align256(iso_blocks_bytes(rows, n))
                                                        : ws + base + area);
    void* fc = fp ? fit->data : (void*)(ws + base + 2 * area);
    FitLaunch a{};
    const int rc = fit_prepare(yc, wc, rows, n, increasing, y_min, y_max, cdt, fc, blocks_out, blocks_mem, workspace,
                               workspace_bytes, stream, a);
    if (rc != 1) return rc;
    const hipStream_t st = (hipStream_t)stream;
    if (!yp && gather_c(cdt, y, rows, n, inner, (void*)yc, st) != hipSuccess) return ISO_EHIP;
    if (!wp && gather_c(cdt, w, rows, n, inner, (void*)wc, st) != hipSuccess) return ISO_EHIP;
    if (launch_fit(a) != hipSuccess) return ISO_EHIP;
    if (!fp && scatter_c(cdt, fc, fit, rows, n, inner, st) != hipSuccess) return ISO_EHIP;
    if (blocks_out) blocks_out->valid = 1;
    return ISO_OK;
}

int iso_vjp_view(const iso_view* grad, const iso_blocks* blocks, const iso_view* y, const iso_view* grad_y,
                 const iso_view* grad_w, int64_t outer, int64_t inner, void* workspace, size_t workspace_bytes,
                 void* stream) {
    using namespace iso;
    if (!blocks || !blocks->valid || !grad) return ISO_EINVAL;
    const int cdt = blocks->dtype;
    if (cdt != ISO_F32 && cdt != ISO_F64) return ISO_EINVAL;
    const int64_t n = blocks->n;
    const int64_t rows = row_count(outer, inner, n);
    if (rows < 0 || rows != blocks->rows) return ISO_EINVAL;
    if (!grad_y && !grad_w) return ISO_EINVAL;
    if (grad_w && !y) return ISO_EINVAL;
    for (const iso_view* o : {grad_y, grad_w})
        if (o && (!output_dtype(o->dtype) || compute_type(cdt, o->dtype) != cdt)) return ISO_EINVAL;
    if (!input_dtype(grad->dtype) || (y && !input_dtype(y->dtype))) return ISO_EINVAL;
    if (rows == 0 || n == 0) return ISO_OK;
    if (!view_ok(grad, false) || (y && !view_ok(y, false))) return ISO_EINVAL;
    for (const iso_view* o : {grad_y, grad_w})
        if (o && (!view_ok(o, true) || (o->stride_elem == 0 && n > 1))) return ISO_EINVAL;
    if (!workspace || workspace_bytes < view_ws_bytes(rows, n, cdt)) return ISO_EINVAL;
    char* ws = (char*)workspace;
    const size_t base = align256(make_layout(rows, n).total);
    const size_t area = staging_bytes(rows, n, cdt);
    const bool gp = plain(grad, cdt, outer, inner, n);
    const bool yp = !y || plain(y, cdt, outer, inner, n);
    const bool gyp = !grad_y || plain(grad_y, cdt, outer, inner, n);
    const bool gwp = !grad_w || plain(grad_w, cdt, outer, inner, n);
    const void* gc = gp ? grad->data : (const void*)(ws + base);
    const void* yc = !y ? nullptr : yp ? y->data : (const void*)(ws + base + area);
    void* gyc = !grad_y ? nullptr : gyp ? grad_y->data : (void*)(ws + base + 2 * area);
    void* gwc = !grad_w ? nullptr : gwp ? grad_w->data : (void*)(ws + base + 3 * area);
    VjpLaunch v{};
    const int rc = vjp_prepare(gc, blocks, grad_w ? yc : nullptr, gyc, gwc, workspace, workspace_bytes, stream, v);
    if (rc != 1) return rc;
    const hipStream_t st = (hipStream_t)stream;
    if (!gp && gather_c(cdt, grad, rows, n, inner, (void*)gc, st) != hipSuccess) return ISO_EHIP;
    if (grad_w && !yp && gather_c(cdt, y, rows, n, inner, (void*)yc, st) != hipSuccess) return ISO_EHIP;
    if (launch_vjp(v) != hipSuccess) return ISO_EHIP;
    if (grad_y && !gyp && scatter_c(cdt, gyc, grad_y, rows, n, inner, st) != hipSuccess) return ISO_EHIP;
    if (grad_w && !gwp && scatter_c(cdt, gwc, grad_w, rows, n, inner, st) != hipSuccess) return ISO_EHIP;
    return ISO_OK;
}

}  // extern "C"
