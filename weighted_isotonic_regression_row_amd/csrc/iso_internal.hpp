// Host-side plan and workspace layout shared by the C ABI and the launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace iso {

// Rows of at most this many elements are fitted by one workgroup each, the
// whole row held in LDS (16 bytes per point: 8192 points = 128 KiB of the
// 160 KiB of a gfx950 CU).
constexpr int64_t kSingleMax = 8192;
// Longer rows are cut into chunks of this many elements (first page, Sec. 3:
// chunks of 1024 to 4096 points), whose hulls are merged as segment lists.
constexpr int kChunk = 4096;
// Vertex slot per chunk: C + 1 points (neighbouring chunks share one).
constexpr int64_t kVSlot = kChunk + 1;
// Segment descriptors of a row are kept in LDS up to this many chunks.
constexpr int64_t kMergeLdsChunks = 4096;
// Elements per tile of the backward pass on long rows.
constexpr int kVjpTile = 4096;

struct Desc {
    int c;  // chunk
    int l;  // first vertex (rank in the chunk hull)
    int h;  // last vertex
    int pad;
};

struct Rec {
    int lo;    // chunk-local element where the chunk's surviving segment starts
    int hi;    // chunk-local element where it ends
    int mode;  // 0: has a segment; 1: lies under one edge; 2: NaN row
    int pad;
    double sin;   // slope of the edge entering the segment
    double sout;  // slope of the edge leaving it (or spanning the chunk)
};

// Offsets (bytes) of the workspace regions for one problem.
struct Layout {
    int64_t rows, n, m;  // m = chunks per row (0 on the single-workgroup path)
    size_t status;       // u64 status word
    size_t totals;       // double4 [rows*m] (double-double x, y)
    size_t nv;           // int [rows*m]
    size_t cflag;        // int [rows*m]
    size_t starts;       // double4 [rows*m]
    size_t rec;          // Rec [rows*m]
    size_t desc;         // Desc [rows*m]
    size_t nc;           // int [rows*m]
    size_t seg;          // int [rows*m]
    size_t so;           // double [rows*m]
    size_t vxy;          // double4 [rows*m*kVSlot] (double-double x, y)
    size_t vidx;         // int [rows*m*kVSlot]
    size_t vjp;          // backward tile records (aliases the fit regions)
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
    L.status = off;
    off = align256(off + 8);
    L.vjp = off;  // the backward reuses everything after the status word
    L.totals = off;
    off = align256(off + 32 * rm);
    L.nv = off;
    off = align256(off + 4 * rm);
    L.cflag = off;
    off = align256(off + 4 * rm);
    L.starts = off;
    off = align256(off + 32 * rm);
    L.rec = off;
    off = align256(off + sizeof(Rec) * rm);
    L.desc = off;
    off = align256(off + sizeof(Desc) * rm);
    L.nc = off;
    off = align256(off + 4 * rm);
    L.seg = off;
    off = align256(off + 4 * rm);
    L.so = off;
    off = align256(off + 8 * rm);
    L.vxy = off;
    off = align256(off + 32 * rm * (size_t)kVSlot);
    L.vidx = off;
    off = align256(off + 4 * rm * (size_t)kVSlot);
    // backward: per tile head, tail, carry, total (double2 each) + flag
    const size_t tiles = (n > kSingleMax) ? (size_t)rows * (size_t)((n + kVjpTile - 1) / kVjpTile) : 0;
    const size_t vjp_end = L.vjp + align256(tiles * (4 * 16 + 8));
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
    void* out;
    int64_t rows, n, words;
    int dtype;
    const uint64_t* start_bits;
    const uint64_t* clip_bits;
    const uint32_t* row_nan;
    char* ws;
    Layout L;
    hipStream_t stream;
};

// Launchers (iso_fit.hip, iso_vjp.hip).  Return hipSuccess or the launch error.
hipError_t launch_fit(const FitLaunch& a);
hipError_t launch_vjp(const VjpLaunch& a);

}  // namespace iso
