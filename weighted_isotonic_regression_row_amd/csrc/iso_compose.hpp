// Host-side plan of the calibration composition (iso_calib.hip), shared with
// the C ABI.
#pragma once

#include "iso_internal.hpp"

namespace iso {

// Calibration (first page, Sec. 7.7): workspace regions after the solver's
// own layout L (offset 0): two ping-pong copies of the sorted (key, index)
// entries, per-tile and per-row pooling records, the start and label prefix of
// every run of equal scores, and the padded pooled means and weights.
struct CalLayout {
    Layout L;
    size_t k0, k1, i0, i1;        // u64 / u32 [rows * n]
    size_t trec, tmax, tnan;      // [rows * ceil(n / 2048)]: double4, double, int
    size_t rtot, rnan;            // [rows]: double4, int
    size_t start, pst;            // [rows * n]: int32, double2
    size_t ys;                    // [rows * n] of the data type: labels in score order
    size_t yp, wp;                // [rows * n] of the data type
    size_t total;
};

inline CalLayout make_cal_layout(int64_t rows, int64_t n, size_t esz) {
    CalLayout C{};
    C.L = make_layout(rows, n);
    size_t off = align256(C.L.total);
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    const size_t rn = (size_t)rows * (size_t)n;
    const size_t pt = (size_t)rows * (size_t)((n + 2047) / 2048);
    C.k0 = take(8 * rn);
    C.k1 = take(8 * rn);
    C.i0 = take(4 * rn);
    C.i1 = take(4 * rn);
    C.trec = take(32 * pt);
    C.tmax = take(8 * pt);
    C.tnan = take(4 * pt);
    C.rtot = take(32 * (size_t)rows);
    C.rnan = take(4 * (size_t)rows);
    C.start = take(4 * rn);
    C.pst = take(16 * rn);
    C.ys = take(esz * rn);
    C.yp = take(esz * rn);
    C.wp = take(esz * rn);
    C.total = off;
    return C;
}

struct CalLaunch {
    const void* scores;
    const void* labels;
    int64_t rows, n;
    int dtype;
    void* xs;
    void* fit;
    int32_t* m;
    char* ws;
    CalLayout C;
    hipStream_t stream;
};

struct CalPredictLaunch {
    const void* xs;
    const void* fit;
    const int32_t* m;
    const void* q;
    void* out;
    int64_t rows, n, k;
    int dtype;
    hipStream_t stream;
};

// Soft-rank rows longer than one workgroup sorts: the sort's key and index
// buffers follow the z and v arrays of the soft-rank workspace (v at voff).
struct RankSortAreas {
    size_t k0, k1, i0, i1, end;
};

inline RankSortAreas rank_sort_areas(int64_t rows, int64_t n, size_t voff, size_t esz) {
    const size_t rn = (size_t)rows * (size_t)n;
    RankSortAreas A{};
    A.k0 = voff + align256(esz * rn);
    A.k1 = A.k0 + align256(8 * rn);
    A.i0 = A.k1 + align256(8 * rn);
    A.i1 = A.i0 + align256(4 * rn);
    A.end = A.i1 + align256(4 * rn);
    return A;
}

hipError_t launch_calibration_fit(const CalLaunch& l);
// Every row of x ([rows, n] of dtype) sorted by tiles of 2048 and merge passes
// (iso_calib.hip) in decreasing order of x, or of -x when neg: K[cur] holds
// the sorted keys and I[cur] the elements' indices within the row (float64;
// float32 keeps the complemented index in the key's low word).  K[0..1] are
// [rows * n] u64 and I[0..1] [rows * n] u32 buffers (I unused for float32).
hipError_t launch_sort_rows(int dtype, const void* x, int64_t rows, int64_t n, int neg, uint64_t* const K[2],
                           uint32_t* const I[2], hipStream_t stream, int& cur);
hipError_t launch_calibrate(const CalPredictLaunch& l);

}  // namespace iso
