// Host-side plan and workspace layout shared by the C ABI and the launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace iso {

// Rows of at most this many elements are fitted one per lane (the whole row's
// hull in registers: 16 points per lane up to 16 elements, else 32); the
// backward pass handles them the same way.
constexpr int kLaneRow = 32;
// LDS of one CU (bytes).
constexpr int kLdsBytes = 163840;
// Rows of at most this many elements are fitted by one workgroup each, the
// lane hulls' vertices listed in LDS (18 bytes per vertex plus about 60 per
// lane; 512 lanes of 12 elements at most).
constexpr int64_t kSingleMax = 6144;
// Rows of kPackedMin to kPackedMax elements are packed several to a wave
// (shorter rows take the lane kernels).  Rows of 33 to 64 on three or four
// lanes of 16 points measured about twice as fast on noise as two lanes of 32
// (1e6x48 float32: 0.40 against 0.97 ms), a third slower on rows whose every
// point is a vertex.  Longer rows take a wave each (k_row_fit with 4 or 8
// points per lane), whose output-sensitive finish measured as fast as the
// packed kernels on noise rows of 160 to 256 and faster on rows whose every
// point is a vertex (1e5 rows, float32: increasing rows of 160, 0.29 against
// 0.41 ms packed).
constexpr int kPackedMin = kLaneRow + 1;
constexpr int kPackedMax = 128;
// Rows of up to this many elements take one wave (k_row_fit with 2, 4 or 8
// points per lane); longer ones several.
constexpr int64_t kOneWaveMax = 512;
// Longer rows are cut into chunks of this many elements (first page, Sec. 3:
// chunks of 1024 to 4096 points), one workgroup of 256 threads, 224 of them
// holding 16 elements each (76 KiB of LDS, so that two chunks share a CU),
// whose hulls are merged as segment lists.
constexpr int kChunk = 3584;
constexpr int kLaneK = 16;
constexpr int kChunkLanes = 256;
// Stored form of a chunk hull (written once by the chunk kernel):
//   vertex bit set, bit p-1 <-> chunk point p (point 0 is always a vertex);
constexpr int kMaskWords = kChunk / 64;
//   starts of the 256-element groups relative to the chunk start
//   (double-double), from which the merge tree recomputes a vertex's
//   coordinates with at most 128 element reads;
constexpr int kGroup = 256;
constexpr int kGroups = kChunk / kGroup;
//   the coordinates of the first and last kVMax/2 vertices (of all of them
//   when the hull has at most kVMax), which cover the walks of the merges,
//   as those start at the shared points.
constexpr int kVMax = 1024;
// The lower levels of the merge tree run on subtrees of this many chunks.
constexpr int kSub = 64;
// Segment descriptors of a row are kept in LDS up to this many chunks (the
// top merge's LDS also holds the waves' merge windows).
constexpr int64_t kMergeLdsChunks = 3584;
// Elements per tile of the backward pass on long rows.
constexpr int kVjpTile = 4096;

// A segment of a node's hull: vertex ranks l..h of chunk c's hull (first
// page, Sec. 3.3: a node's list lives in the descriptor slots of its chunks).
struct Desc {
    int c;
    unsigned short l, h;
};

// How one merge of a level rewrites its node's list: the left node keeps its
// first newA descriptors (the last one ending at rank alk), the right node's
// descriptors bs .. bs+nBk-1 follow (the first one starting at rank bek).
struct MRec {
    int newA, bs, nBk, alk, bek;
};

struct Rec {
    int lo;    // chunk-local point where the chunk's surviving segment starts
    int hi;    // chunk-local point where it ends
    int mode;  // 0: has a segment; 1: lies under one edge; 2: NaN row
    int pad;
    double sin;   // slope of the edge entering the segment
    double sout;  // slope of the edge leaving it (or spanning the chunk)
};

// Offsets (bytes) of the workspace regions for one problem.
struct Layout {
    int64_t rows, n, m;  // m = chunks per row (0 on the single-workgroup path)
    size_t status;       // u64 status word
    size_t tot;          // double4 [rows*m] chunk totals (double-double x, y)
    size_t nv;           // int [rows*m] vertices of each chunk hull
    size_t cflag;        // int [rows*m]
    size_t starts;       // double4 [rows*m]
    size_t rec;          // Rec [rows*m]
    size_t desc0, desc1; // Desc [rows*m] (upper merge levels ping-pong between them)
    size_t gsd;          // Desc [rows*m] the subtrees' lists
    size_t gsn;          // int [rows*ceil(m/kSub)]
    size_t nc;           // int [rows*m]
    size_t cover;        // int [rows*m] 1 where the chunk kernel's first pass left the chunk to its second
    size_t clist;        // int [rows*m] those chunks, listed
    size_t cctr;         // u64 [2] the list's count (tagged with the call's epoch), the epoch of a full scan
    size_t mrec;         // MRec [rows*m]
    size_t so;           // double [rows*m]
    size_t cmask;        // u64 [rows*m*kMaskWords]
    size_t cpre;         // int [rows*m*kMaskWords] rank of the first vertex >= each word
    size_t cgs;          // double4 [rows*m*kGroups]
    size_t cvx;          // double4 [rows*m*kVMax]
    size_t cvi;          // int [rows*m*kVMax]
    size_t ovf;          // single-workgroup rows: per-row vertex lists for rows whose lane hulls overflow LDS
    size_t ovf_stride;   // bytes per row of ovf
    size_t ovfrow;       // int [rows] single-workgroup rows: 1 where the row's list went to ovf
    size_t vjp;          // backward tile records (alias the fit regions)
    size_t total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline Layout make_layout(int64_t rows, int64_t n) {
    Layout L{};
    L.rows = rows;
    L.n = n;
    L.m = (n > kSingleMax) ? (n + kChunk - 1) / kChunk : 0;
    const size_t rm = (size_t)rows * (size_t)L.m;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    L.status = take(16);  // [0] last data error (epoch << 8 | code), [1] epoch of the last call
    L.vjp = off;  // the backward reuses everything after the status word
    L.tot = take(32 * rm);
    L.nv = take(4 * rm);
    L.cflag = take(4 * rm);
    L.starts = take(32 * rm);
    L.rec = take(sizeof(Rec) * rm);
    L.desc0 = take(sizeof(Desc) * rm);
    L.desc1 = take(sizeof(Desc) * rm);
    L.gsd = take(sizeof(Desc) * rm);
    L.gsn = take(4 * (size_t)rows * (size_t)((L.m + kSub - 1) / kSub));
    L.nc = take(4 * rm);
    L.cover = take(4 * rm);
    L.clist = take(4 * rm);
    L.cctr = take(16);
    L.mrec = take(sizeof(MRec) * rm);
    L.so = take(8 * rm);
    L.cmask = take(8 * rm * kMaskWords);
    L.cpre = take(4 * rm * kMaskWords);
    L.cgs = take(32 * rm * kGroups);
    L.cvx = take(32 * rm * kVMax);
    L.cvi = take(4 * rm * kVMax);
    if (L.m == 0 && n > kOneWaveMax) {
        // rows of several waves (k_row_fit): a vertex list per row for lane
        // hulls that overflow the LDS list, and a flag per row
        L.ovf_stride = align256(16 * ((size_t)n + 1) + 2 * ((size_t)n + 1));
        L.ovf = take(L.ovf_stride * (size_t)rows);
        L.ovfrow = take(4 * (size_t)rows);
    } else if (L.m == 0 && n > kPackedMax) {
        // rows of one wave: a flag per row for k_row_ovf, which refits a
        // flagged row with its whole list in LDS
        L.ovfrow = take(4 * (size_t)rows);
    } else if (L.m == 0 && n >= kPackedMin) {
        // packed rows (iso_pack.hip): 16 counters 256 bytes apart, then lists
        // of at most one entry per wave (fewer than rows + 16 in all)
        L.ovf = take(16 * 256 + 4 * ((size_t)rows + 16));
    }
    // backward: per tile head, tail, carry, total (up to three doubles each) + flag
    const size_t tiles = (n > kSingleMax) ? (size_t)rows * (size_t)((n + kVjpTile - 1) / kVjpTile) : 0;
    const size_t vjp_end = L.vjp + align256(tiles * (4 * 24 + 8));
    L.total = (off > vjp_end ? off : vjp_end);
    if (L.total < 256) L.total = 256;
    return L;
}

struct FitLaunch {
    const void* y;
    const void* w;
    void* fit;
    int64_t rows, n;
    int increasing;
    int dtype;
    double lo, hi;
    uint64_t* start_bits;
    uint64_t* clip_bits;
    uint32_t* row_nan;
    int64_t words;
    char* ws;
    Layout L;
    unsigned long long epoch;
    hipStream_t stream;
};

struct VjpLaunch {
    const void* g;
    const void* w;
    const void* y;  // needed for out_w
    void* out;      // grad_y or nullptr
    void* out_w;    // grad_w or nullptr
    int64_t rows, n, words;
    int dtype;
    const uint64_t* start_bits;
    const uint64_t* clip_bits;
    const uint32_t* row_nan;
    char* ws;
    Layout L;
    hipStream_t stream;
};

// Raises a kernel's dynamic-LDS limit to at least `bytes` on the current
// device.  The attribute belongs to the device, so `seen` (the call site's
// static table, one entry per device id) records what each device was given;
// concurrent first calls may both set it, which is harmless.
constexpr int kMaxDevices = 64;
inline hipError_t ensure_lds(const void* fn, size_t bytes, size_t (&seen)[kMaxDevices]) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (seen[dev] >= bytes) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) seen[dev] = bytes;
    return e;
}

// Compute units of the current device (256 on MI355X), cached per device id.
inline int num_cus() {
    static int cus[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// Soft rank (first page, Sec. 7.9): rows of at most this many elements are
// sorted by one workgroup in LDS (12 bytes per entry for float64).
constexpr int64_t kRankMaxN = 8192;

// Soft rank and its backward: `in` is x (forward) or the upstream gradient
// (backward), `out` the ranks or the gradient in x.  The workspace holds the
// solver's layout L from offset 0, then two [rows, n] arrays of the data type
// at zoff and voff (z and its fit; the sorted gradient and its block averages).
struct RankLaunch {
    const void* in;
    void* out;
    int64_t rows, n, words;
    int dtype;
    double eps;
    int32_t* perm;
    int32_t* rank;
    uint64_t* start_bits;
    uint64_t* clip_bits;
    uint32_t* row_nan;
    char* ws;
    Layout L;
    size_t zoff, voff;
    hipStream_t stream;
};

// Launchers (iso_fit.hip, iso_vjp.hip, iso_rank.hip).  Return hipSuccess or
// the launch error.
hipError_t launch_fit(const FitLaunch& a);
hipError_t launch_vjp(const VjpLaunch& l);
hipError_t launch_soft_rank(const RankLaunch& l);
hipError_t launch_soft_rank_vjp(const RankLaunch& l);

}  // namespace iso
