// C ABI of libiso.so: argument checks, workspace layout, launches, status.
// The operations are specified in include/iso.h.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "../../include/iso.h"
#include "iso_compose.hpp"
#include "iso_internal.hpp"
#include "iso_prepare.hpp"

namespace {

// Every iso_fit call gets a fresh epoch (never 0).  Its first kernel stores
// the epoch in the workspace's second status word, and a data error is
// recorded in the first as epoch << 8 | code, so the status words never need
// clearing and iso_status reports an error only when it belongs to the
// latest call that used the workspace.  No host state is kept per workspace.
std::atomic<unsigned long long> g_epoch{0};

bool valid_dtype(int d) { return d == ISO_F32 || d == ISO_F64; }

}  // namespace

namespace iso {

// iso_fit's argument checks, the partition handle and the launch record:
// returns 1 when kernels are to be launched (a is filled), else the code the
// call returns (ISO_OK for an empty problem, ISO_EINVAL).  Nothing is queued.
int fit_prepare(const void* y, const void* w, int64_t rows, int64_t n, int increasing, double y_min, double y_max,
                int dtype, void* fit, iso_blocks* blocks_out, void* blocks_mem, void* workspace,
                size_t workspace_bytes, void* stream, FitLaunch& a) {
    if (rows < 0 || n < 0 || !valid_dtype(dtype)) return ISO_EINVAL;
    if (increasing != 0 && increasing != 1) return ISO_EINVAL;
    if ((blocks_out == nullptr) != (blocks_mem == nullptr)) return ISO_EINVAL;
    if (isnan(y_min)) y_min = -INFINITY;
    if (isnan(y_max)) y_max = INFINITY;
    if (y_min > y_max) return ISO_EINVAL;
    if (n > (int64_t)INT32_MAX) return ISO_EINVAL;
    const int64_t words = (n + 63) / 64;
    if (blocks_out) {
        memset(blocks_out, 0, sizeof(*blocks_out));
        char* bm = (char*)blocks_mem;
        const size_t bits = iso::align256(8 * (size_t)words * (size_t)rows);
        blocks_out->start_bits_dev = (uint64_t*)bm;
        blocks_out->clip_bits_dev = (uint64_t*)(bm + bits);
        blocks_out->row_nan_dev = (uint32_t*)(bm + 2 * bits);
        blocks_out->w_dev = w;
        blocks_out->rows = rows;
        blocks_out->n = n;
        blocks_out->words = words;
        blocks_out->dtype = dtype;
        blocks_out->valid = 0;
    }
    if (rows == 0 || n == 0) {
        if (blocks_out) blocks_out->valid = 1;
        return ISO_OK;
    }
    if (!y || !fit || !workspace) return ISO_EINVAL;
    if (((uintptr_t)workspace & 255u) != 0) return ISO_EINVAL;
    if (blocks_mem && ((uintptr_t)blocks_mem & 255u) != 0) return ISO_EINVAL;
    const iso::Layout L = iso::make_layout(rows, n);
    if (workspace_bytes < L.total) return ISO_EINVAL;
    if (L.m > 0 && rows * L.m > (int64_t)UINT32_MAX) return ISO_EINVAL;
    if (L.m == 0 && rows > (int64_t)UINT32_MAX) return ISO_EINVAL;
    const size_t esz = dtype == ISO_F32 ? 4 : 8;
    const size_t bytes = (size_t)rows * (size_t)n * esz;
    const char* fb = (const char*)fit;
    auto overlaps = [&](const void* p) {
        const char* b = (const char*)p;
        return p && b < fb + bytes && fb < b + bytes;
    };
    if (overlaps(y) || overlaps(w)) return ISO_EINVAL;

    const unsigned long long epoch = ++g_epoch;
    a = iso::FitLaunch{};
    a.y = y;
    a.w = w;
    a.fit = fit;
    a.rows = rows;
    a.n = n;
    a.increasing = increasing;
    a.dtype = dtype;
    a.lo = y_min;
    a.hi = y_max;
    a.start_bits = blocks_out ? blocks_out->start_bits_dev : nullptr;
    a.clip_bits = blocks_out ? blocks_out->clip_bits_dev : nullptr;
    a.row_nan = blocks_out ? blocks_out->row_nan_dev : nullptr;
    a.words = words;
    a.ws = (char*)workspace;
    a.L = L;
    a.epoch = epoch;
    a.stream = (hipStream_t)stream;
    return 1;
}

// iso_vjp_yw's argument checks and launch record (returns as fit_prepare).
int vjp_prepare(const void* grad, const iso_blocks* blocks, const void* y, void* grad_y, void* grad_w,
                void* workspace, size_t workspace_bytes, void* stream, VjpLaunch& v) {
    if (!blocks || !blocks->valid) return ISO_EINVAL;
    if (blocks->rows < 0 || blocks->n < 0 || !valid_dtype(blocks->dtype)) return ISO_EINVAL;
    if (blocks->rows == 0 || blocks->n == 0) return ISO_OK;
    if (!grad || !workspace) return ISO_EINVAL;
    if (!grad_y && !grad_w) return ISO_EINVAL;
    if (grad_w && !y) return ISO_EINVAL;
    if (!blocks->start_bits_dev || !blocks->clip_bits_dev || !blocks->row_nan_dev) return ISO_EINVAL;
    if (((uintptr_t)workspace & 255u) != 0) return ISO_EINVAL;
    const iso::Layout L = iso::make_layout(blocks->rows, blocks->n);
    if (workspace_bytes < L.total) return ISO_EINVAL;
    v = iso::VjpLaunch{};
    v.g = grad;
    v.w = blocks->w_dev;
    v.y = y;
    v.out = grad_y;
    v.out_w = grad_w;
    v.rows = blocks->rows;
    v.n = blocks->n;
    v.words = blocks->words;
    v.dtype = blocks->dtype;
    v.start_bits = blocks->start_bits_dev;
    v.clip_bits = blocks->clip_bits_dev;
    v.row_nan = blocks->row_nan_dev;
    v.ws = (char*)workspace;
    v.L = L;
    v.stream = (hipStream_t)stream;
    return 1;
}

}  // namespace iso

extern "C" {

size_t iso_workspace_bytes(int64_t rows, int64_t n, int dtype) {
    if (rows < 0 || n < 0 || !valid_dtype(dtype)) return 0;
    return iso::make_layout(rows, n).total;
}

size_t iso_blocks_bytes(int64_t rows, int64_t n) {
    if (rows < 0 || n < 0) return 0;
    const size_t words = (size_t)((n + 63) / 64);
    const size_t bits = iso::align256(8 * words * (size_t)rows);
    return 2 * bits + iso::align256(4 * (size_t)rows) + 256;
}

int iso_fit(const void* y, const void* w, int64_t rows, int64_t n, int increasing, double y_min, double y_max,
            int dtype, void* fit, iso_blocks* blocks_out, void* blocks_mem, void* workspace,
            size_t workspace_bytes, void* stream) {
    iso::FitLaunch a{};
    const int rc = iso::fit_prepare(y, w, rows, n, increasing, y_min, y_max, dtype, fit, blocks_out, blocks_mem,
                                    workspace, workspace_bytes, stream, a);
    if (rc != 1) return rc;
    if (iso::launch_fit(a) != hipSuccess) return ISO_EHIP;
    if (blocks_out) blocks_out->valid = 1;
    return ISO_OK;
}

int iso_vjp_yw(const void* grad, const iso_blocks* blocks, const void* y, void* grad_y, void* grad_w,
               void* workspace, size_t workspace_bytes, void* stream) {
    iso::VjpLaunch v{};
    const int rc = iso::vjp_prepare(grad, blocks, y, grad_y, grad_w, workspace, workspace_bytes, stream, v);
    if (rc != 1) return rc;
    if (iso::launch_vjp(v) != hipSuccess) return ISO_EHIP;
    return ISO_OK;
}

int iso_vjp(const void* grad, const iso_blocks* blocks, void* grad_y, void* workspace, size_t workspace_bytes,
            void* stream) {
    return iso_vjp_yw(grad, blocks, nullptr, grad_y, nullptr, workspace, workspace_bytes, stream);
}

size_t iso_soft_rank_state_bytes(int64_t rows, int64_t n) {
    if (rows < 0 || n < 0) return 0;
    const size_t idx = iso::align256(4 * (size_t)rows * (size_t)n);
    return iso::align256(iso_blocks_bytes(rows, n)) + 2 * idx;
}

size_t iso_soft_rank_workspace_bytes(int64_t rows, int64_t n, int dtype) {
    if (rows < 0 || n < 0 || n > (int64_t)INT32_MAX || !valid_dtype(dtype)) return 0;
    const size_t esz = dtype == ISO_F32 ? 4 : 8;
    const size_t zoff = iso::align256(iso::make_layout(rows, n).total);
    const size_t voff = zoff + iso::align256(esz * (size_t)rows * (size_t)n);
    const size_t end = voff + iso::align256(esz * (size_t)rows * (size_t)n);
    // rows sorted by tiles and merge passes also hold the sort's keys and indices
    return n > iso::kRankMaxN ? iso::rank_sort_areas(rows, n, voff, esz).end : end;
}

namespace {

iso::RankLaunch rank_launch(const iso_soft_rank_state* st, void* workspace) {
    iso::RankLaunch l{};
    const int64_t rows = st->blocks.rows, n = st->blocks.n;
    const size_t esz = st->blocks.dtype == ISO_F32 ? 4 : 8;
    l.rows = rows;
    l.n = n;
    l.words = st->blocks.words;
    l.dtype = st->blocks.dtype;
    l.eps = st->eps;
    l.perm = st->perm_dev;
    l.rank = st->rank_dev;
    l.start_bits = st->blocks.start_bits_dev;
    l.clip_bits = st->blocks.clip_bits_dev;
    l.row_nan = st->blocks.row_nan_dev;
    l.ws = (char*)workspace;
    l.L = iso::make_layout(rows, n);
    l.zoff = iso::align256(l.L.total);
    l.voff = l.zoff + iso::align256(esz * (size_t)rows * (size_t)n);
    return l;
}

}  // namespace

int iso_soft_rank(const void* x, int64_t rows, int64_t n, double eps, int dtype, void* r,
                  iso_soft_rank_state* state_out, void* state_mem, void* workspace, size_t workspace_bytes,
                  void* stream) {
    if (rows < 0 || n < 0 || !valid_dtype(dtype)) return ISO_EINVAL;
    if (n > (int64_t)INT32_MAX || rows > (int64_t)INT32_MAX) return ISO_EINVAL;
    // the merge passes' grids: one workgroup per 2048 outputs of every row
    if (n > iso::kRankMaxN && rows * ((n + 2047) / 2048) > (int64_t)UINT32_MAX) return ISO_EINVAL;
    if (!(eps > 0.0) || !isfinite(eps)) return ISO_EINVAL;
    if (!state_out || !state_mem) return ISO_EINVAL;
    if (((uintptr_t)state_mem & 255u) != 0) return ISO_EINVAL;
    memset(state_out, 0, sizeof(*state_out));
    const int64_t words = (n + 63) / 64;
    char* sm = (char*)state_mem;
    const size_t bits = iso::align256(8 * (size_t)words * (size_t)rows);
    const size_t bb = iso::align256(iso_blocks_bytes(rows, n));
    const size_t idx = iso::align256(4 * (size_t)rows * (size_t)n);
    iso_blocks* b = &state_out->blocks;
    b->start_bits_dev = (uint64_t*)sm;
    b->clip_bits_dev = (uint64_t*)(sm + bits);
    b->row_nan_dev = (uint32_t*)(sm + 2 * bits);
    b->w_dev = nullptr;
    b->rows = rows;
    b->n = n;
    b->words = words;
    b->dtype = dtype;
    b->valid = 1;
    state_out->perm_dev = (int32_t*)(sm + bb);
    state_out->rank_dev = (int32_t*)(sm + bb + idx);
    state_out->eps = eps;
    if (rows == 0 || n == 0) {
        state_out->valid = 1;
        return ISO_OK;
    }
    if (!x || !r || !workspace) return ISO_EINVAL;
    if (((uintptr_t)workspace & 255u) != 0) return ISO_EINVAL;
    if (workspace_bytes < iso_soft_rank_workspace_bytes(rows, n, dtype)) return ISO_EINVAL;
    const iso::Layout L = iso::make_layout(rows, n);
    if (L.m > 0 && rows * L.m > (int64_t)UINT32_MAX) return ISO_EINVAL;  // the chunk grids of the fit
    const size_t bytes = (size_t)rows * (size_t)n * (dtype == ISO_F32 ? 4 : 8);
    const char* rb = (const char*)r;
    const char* xb = (const char*)x;
    if (xb < rb + bytes && rb < xb + bytes) return ISO_EINVAL;
    iso::RankLaunch l = rank_launch(state_out, workspace);
    l.in = x;
    l.out = r;
    l.stream = (hipStream_t)stream;
    if (iso::launch_soft_rank(l) != hipSuccess) return ISO_EHIP;
    state_out->valid = 1;
    return ISO_OK;
}

int iso_soft_rank_vjp(const void* grad, const iso_soft_rank_state* state, void* grad_x, void* workspace,
                      size_t workspace_bytes, void* stream) {
    if (!state || !state->valid || !state->blocks.valid) return ISO_EINVAL;
    const int64_t rows = state->blocks.rows, n = state->blocks.n;
    if (rows < 0 || n < 0 || n > (int64_t)INT32_MAX || !valid_dtype(state->blocks.dtype)) return ISO_EINVAL;
    if (rows == 0 || n == 0) return ISO_OK;
    if (!grad || !grad_x || !workspace || !state->perm_dev || !state->rank_dev) return ISO_EINVAL;
    if (!state->blocks.start_bits_dev || !state->blocks.clip_bits_dev || !state->blocks.row_nan_dev)
        return ISO_EINVAL;
    if (!(state->eps > 0.0) || !isfinite(state->eps)) return ISO_EINVAL;
    if (((uintptr_t)workspace & 255u) != 0) return ISO_EINVAL;
    if (workspace_bytes < iso_soft_rank_workspace_bytes(rows, n, state->blocks.dtype)) return ISO_EINVAL;
    iso::RankLaunch l = rank_launch(state, workspace);
    l.in = grad;
    l.out = grad_x;
    l.stream = (hipStream_t)stream;
    if (iso::launch_soft_rank_vjp(l) != hipSuccess) return ISO_EHIP;
    return ISO_OK;
}

size_t iso_calibration_workspace_bytes(int64_t rows, int64_t n, int dtype) {
    if (rows < 0 || n < 0 || n > (int64_t)INT32_MAX || !valid_dtype(dtype)) return 0;
    return iso::make_cal_layout(rows, n, dtype == ISO_F32 ? 4 : 8).total;
}

int iso_calibration_fit(const void* scores, const void* labels, int64_t rows, int64_t n, int dtype, void* xs,
                        void* fit, int32_t* m, void* workspace, size_t workspace_bytes, void* stream) {
    if (rows < 0 || n < 0 || !valid_dtype(dtype) || n > (int64_t)INT32_MAX) return ISO_EINVAL;
    if (rows == 0 || n == 0) return ISO_OK;
    if (!scores || !labels || !xs || !fit || !m || !workspace) return ISO_EINVAL;
    if (((uintptr_t)workspace & 255u) != 0) return ISO_EINVAL;
    const size_t esz = dtype == ISO_F32 ? 4 : 8;
    const iso::CalLayout C = iso::make_cal_layout(rows, n, esz);
    if (workspace_bytes < C.total) return ISO_EINVAL;
    if (rows * ((n + 2047) / 2048) > (int64_t)UINT32_MAX) return ISO_EINVAL;  // merge and pooling grids
    const size_t bytes = (size_t)rows * (size_t)n * esz;
    auto overlap = [&](const void* p, const void* q) {
        const char* a = (const char*)p;
        const char* b = (const char*)q;
        return a < b + bytes && b < a + bytes;
    };
    if (overlap(xs, fit) || overlap(xs, scores) || overlap(xs, labels) || overlap(fit, scores) ||
        overlap(fit, labels))
        return ISO_EINVAL;
    iso::CalLaunch l{};
    l.scores = scores;
    l.labels = labels;
    l.rows = rows;
    l.n = n;
    l.dtype = dtype;
    l.xs = xs;
    l.fit = fit;
    l.m = m;
    l.ws = (char*)workspace;
    l.C = C;
    l.stream = (hipStream_t)stream;
    if (iso::launch_calibration_fit(l) != hipSuccess) return ISO_EHIP;
    return ISO_OK;
}

int iso_calibrate(const void* xs, const void* fit, const int32_t* m, int64_t rows, int64_t n, const void* q,
                  int64_t k, int dtype, void* out, void* stream) {
    if (rows < 0 || n < 0 || k < 0 || !valid_dtype(dtype)) return ISO_EINVAL;
    if (rows == 0 || k == 0) return ISO_OK;
    if (n == 0 || !xs || !fit || !m || !q || !out) return ISO_EINVAL;
    iso::CalPredictLaunch l{};
    l.xs = xs;
    l.fit = fit;
    l.m = m;
    l.q = q;
    l.out = out;
    l.rows = rows;
    l.n = n;
    l.k = k;
    l.dtype = dtype;
    l.stream = (hipStream_t)stream;
    if (iso::launch_calibrate(l) != hipSuccess) return ISO_EHIP;
    return ISO_OK;
}

int iso_status(const void* workspace, void* stream) {
    if (!workspace) return ISO_EINVAL;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return ISO_EHIP;
    unsigned long long word[2] = {0, 0};
    if (hipMemcpy(word, workspace, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess) return ISO_EHIP;
    if (word[1] != 0 && (word[0] >> 8) == word[1]) return -(int)(word[0] & 0xff);
    return ISO_OK;
}

const char* iso_strerror(int code) {
    switch (code) {
        case ISO_OK:
            return "success";
        case ISO_EINVAL:
            return "invalid argument";
        case ISO_EHIP:
            return "HIP runtime error";
        case ISO_EWEIGHT:
            return "a weight is not strictly positive";
        case ISO_ETOOBIG:
            return "the problem needs more workspace than iso_fit_noalloc's static scratch holds";
        default:
            return "unknown error";
    }
}

}  // extern "C"
