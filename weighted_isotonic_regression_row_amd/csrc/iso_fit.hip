// Forward kernels of the isotonic fit for gfx950.
//
// Page "Merge Hulls Without Copying Vertices: GPU Isotonic Regression":
//   k_row_fit      rows of at most 6144 elements: one workgroup per row builds
//                  the row's hull in LDS and writes the fit (Sec. 3: a row that
//                  fits in one chunk is finished by the chunk level).  Noisy
//                  float32 rows are finished by gift wrapping a few candidate
//                  vertices; the others merge their lane hulls in rounds.
//   k_chunk_hull   longer rows: one workgroup per chunk of 3584 elements builds
//                  the chunk's hull once and stores it compactly (vertex bit
//                  set, group starts, the coordinates of its end vertices),
//                  the chunk totals, and a tentative fit from the chunk's own
//                  hull.
//   k_merge_sub    the lower levels of the merge tree on segment lists, at
//                  most one segment per chunk (Sec. 3.3, Theorem 4.4): one
//                  workgroup per subtree of 64 chunks;
//   k_merge_top    one workgroup per long row: double-double chunk starts
//                  (exclusive scan of the chunk totals, Sec. 3.3 and App. B),
//                  the upper levels, then per-chunk records of the root list
//                  (Sec. 3.4).
//   k_fixup        per chunk, rewrites only the elements that lie outside the
//                  chunk's surviving segment (the edge rule after Theorem 4.4:
//                  they lie under the edge entering or leaving the segment, or
//                  a chunk without a segment lies under one edge).
#include <math.h>

#include <algorithm>

#include "iso_internal.hpp"
#include "iso_pack.hpp"
#include "iso_tile.hpp"

namespace iso {

struct RowArgs {
    const void* y;
    const void* w;
    void* fit;
    int64_t n;
    int increasing;
    double lo, hi;
    uint64_t* start_bits;
    uint64_t* clip_bits;
    uint32_t* row_nan;
    int64_t words;
    unsigned long long* status;
    unsigned long long epoch;
    int cap;             // vertices the LDS list holds (row kernel)
    char* ovf;           // per-row vertex lists in global memory for rows whose lane hulls exceed cap
    int64_t ovf_stride;  // bytes per row of ovf
    int* ovf_row;        // [rows] 1 where the row kernel left the row to k_row_ovf
    int stage;           // row kernel: read the inputs through LDS (lane_load_staged)
};

template <typename T>
__device__ inline void wg_write_nan(int64_t N, T* out, uint64_t* sbits, uint64_t* cbits) {
    for (int64_t i = threadIdx.x; i < N; i += blockDim.x) out[i] = (T)NAN;
    if (sbits) {
        const int64_t words = (N + 63) / 64;
        for (int64_t q = threadIdx.x; q < words; q += blockDim.x) {
            sbits[q] = 0ull;
            cbits[q] = 0ull;
        }
    }
}

// Steps 1-2 of the tile pipeline (lane hulls, lane starts) on the elements at
// y, w.  Returns the tile's flag (non-zero: a non-finite input or a bad
// weight); nvert = the number of lane-hull vertices.  The lane's points stay
// in xs, ys.
// With stage set, the inputs pass through the still unused vertex list (each
// wave K * 64 elements of it).  With nxp, the masks are those of the hulls of
// the lanes' parts (a superset of the lane hulls' vertices, gw_parts); without
// HULL the masks are 0 (the caller chooses candidates, lane_chords).
// Float32 rows of K = 12 or 20 (lanes of 48 or 80 bytes) are always staged:
// the launcher reserves the room in the list.
template <typename T, int K>
constexpr bool always_staged() {
    return sizeof(T) == 4 && (K * 4) % 64 != 0 && (K * 4) % 16 == 0;
}

template <typename T, int K, bool HULL = true>
__device__ inline int tile_build(const Tile& t, const T* y, const T* w, int increasing, uint64_t& mask,
                                 double (&xs)[K], double (&ys)[K], int& nvert, bool stage = false,
                                 uint64_t (*nxp)[3] = nullptr) {
    constexpr bool ABS = sizeof(T) == 4;
    const int l = threadIdx.x;
    const int cnt = min(max(t.N - l * K, 0), K);
    int f = 0;
    constexpr bool SO = always_staged<T, K>();
    if (SO || stage) {
        const int e0 = (l & ~(kWave - 1)) * K;  // the wave's first element
        T* st = (T*)t.VXY + e0;
        mask = lane_hull<T, K, HULL, SO>(y + e0, w ? w + e0 : nullptr, cnt, !increasing, xs, ys, f, st,
                                         min(max(t.N - e0, 0), K * kWave), nxp);
    } else {
        mask = lane_hull<T, K, HULL>(y + (int64_t)l * K, w ? w + (int64_t)l * K : nullptr, cnt, !increasing, xs, ys, f,
                               nullptr, 0, nxp);
    }
    nvert = tile_lane_starts<!ABS>(t, make_double2(xs[K - 1], ys[K - 1]), f, __popcll(mask));
    return t.flag[0];
}

// The stores of step 4, the list holding the edges' values (tile_edge_slopes
// or tile_hull_to_front): fit (and bits) of the tile's elements.
template <typename T, int K>
__device__ inline void tile_store(const Tile& t, uint64_t mask, T* out, uint64_t* sb, uint64_t* cb) {
    double vals[K];
    uint64_t clipm;
    tile_expand<K>(t, mask, vals, clipm);
    const int l = threadIdx.x;
    const int cnt = min(max(t.N - l * K, 0), K);
    store_lane<T, K>(out + (int64_t)l * K, cnt, vals);
    if (sb) {
        t.CM[l] = clipm;
        __syncthreads();
        tile_bits<K>(t, sb, cb);
    }
}

// Step 4 and the stores: fit (and bits) of the tile's elements.  Overwrites
// the list's coordinates with edge slopes.  QR > 0: the list is the QuickHull
// list (list_compact) of at most QR entries per thread.
template <typename T, int K, int QR = 0>
__device__ inline void tile_finish(const Tile& t, uint64_t mask, int increasing, double lo, double hi, T* out,
                                   uint64_t* sb, uint64_t* cb) {
    constexpr bool ABS = sizeof(T) == 4;
    if constexpr (QR > 0)
        list_edge_slopes<QR>(t, increasing, lo, hi);
    else
        tile_edge_slopes<K, ABS>(t, increasing, lo, hi);
    double vals[K];
    uint64_t clipm;
    tile_expand<K>(t, mask, vals, clipm);
    const int l = threadIdx.x;
    const int cnt = min(max(t.N - l * K, 0), K);
    store_lane<T, K>(out + (int64_t)l * K, cnt, vals);
    if (sb) {
        t.CM[l] = clipm;
        __syncthreads();
        tile_bits<K>(t, sb, cb);
    }
}

// The row kernel's exact path, to the end of the row: the lane hulls built
// again from the inputs, merged in rounds, the fit and bits stored.  Its own
// function (not inlined), so that its registers are allocated apart from the
// wrap's.  A row whose lane hulls' vertices overflow the LDS list keeps its
// list in the row's area of the workspace.
template <typename T, int K>
__device__ __attribute__((noinline)) void row_exact(const T* y, const T* w, T* out, uint64_t* sb, uint64_t* cb,
                                                    uint32_t* row_nan, char* ovf, int n, int increasing, double lo,
                                                    double hi, int cap, int stage) {
    // the arguments are plain values, passed in registers (a structure passed
    // by value would be staged through scratch memory by every thread)
    extern __shared__ __align__(32) char smem[];
    Tile t = tile_carve(smem, blockDim.x, cap, K, n, sizeof(T) == 4);
    uint64_t mask;
    double xs[K], ys[K];
    int nvert;
    (void)tile_build<T, K>(t, y, w, increasing, mask, xs, ys, nvert, stage != 0);  // inputs already checked
    if (nvert > cap + 1) {  // uniform
        t.VXY = (double2*)ovf;
        t.V = (unsigned short*)(ovf + 16 * ((int64_t)n + 1));
    }
    tile_merges<K, sizeof(T) == 4>(t, mask, xs, ys);
    tile_finish<T, K>(t, mask, increasing, lo, hi, out, sb, cb);
    if (row_nan && threadIdx.x == 0) *row_nan = 0u;
}

// ---------------------------------------------------------------------------
// one workgroup per row.  The row's phases are latency-bound, so the register
// budget is capped at 128 VGPRs (four waves per SIMD).  The vertex list lives
// in LDS; a row whose lane hulls hold more vertices than it has room for is
// flagged and left to k_row_ovf, which keeps the list in global memory (one
// code path per kernel keeps this one free of register spills).
// ---------------------------------------------------------------------------
template <typename T, int K>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void k_row_fit(RowArgs a) {
    extern __shared__ __align__(32) char smem[];
    mark_epoch(a.status, a.epoch);
    const int64_t row = blockIdx.x;
    const int N = (int)a.n;
    const Tile t = tile_carve(smem, blockDim.x, a.cap, K, N, sizeof(T) == 4);
    const T* y = (const T*)a.y + row * a.n;
    const T* w = a.w ? (const T*)a.w + row * a.n : nullptr;
    T* out = (T*)a.fit + row * a.n;
    uint64_t* sb = a.start_bits ? a.start_bits + row * a.words : nullptr;
    uint64_t* cb = a.clip_bits ? a.clip_bits + row * a.words : nullptr;
    uint64_t mask;
    double xs[K], ys[K];
    int nvert;
    uint64_t nxp[3];
    constexpr bool HALVES = K >= 12;                  // rows of several waves
    constexpr bool CHORDS = HALVES && sizeof(T) == 4;  // float32 ones take chord candidates (lane_chords)
    const int flag = tile_build<T, K, !CHORDS>(t, y, w, a.increasing, mask, xs, ys, nvert, a.stage != 0,
                                               (HALVES && !CHORDS) ? &nxp : nullptr);
    if (flag) {
        wg_write_nan<T>(N, out, sb, cb);
        if (threadIdx.x == 0) {
            if (a.ovf_row) a.ovf_row[row] = 0;
            if (a.row_nan) a.row_nan[row] = 1u;
            if (flag == 2) report_weight_error(a.status, a.epoch);
        }
        return;
    }
    constexpr bool ABS = sizeof(T) == 4;
    bool over = false;
    if constexpr (HALVES) {
        // Noisy rows have few hull vertices among few candidates, found
        // output-sensitively: float32 rows by QuickHull over the points under
        // the hull of the lane ends, float64 rows by wrapping the vertices of
        // the lanes' half hulls.  The rest take the exact path (row_exact, its
        // own function, which also handles lists beyond the LDS), so this
        // kernel holds one path's registers.  The list holds point 0 and cap
        // vertices; every condition here is uniform.
        if constexpr (ABS) {
            // candidates: the points not above the hull of the lane ends
            // (found by QuickHull, one lane end per thread), then the exact
            // hull of the candidates by QuickHull again, one per thread.  A
            // row with more candidates than threads, or without the LDS room,
            // takes the exact path.
            const int cnt = min(max(N - (int)threadIdx.x * K, 0), K);
            const int used = (N + K - 1) / K;
            if (8 * qh_slot_words(used) <= 16 * (a.cap + 1)) {
                int ea, eb;  // the hull edge of the lane ends over this lane
                (void)tile_quickhull((const double2*)t.LS, used, (unsigned long long*)t.VXY, 0.0, ea, eb);
                mask = lane_coarse_filter<K>(t, xs, ys, cnt, ea, eb);
                // at most one candidate per thread, with room for the slots after them
                const int mmax = min((int)blockDim.x, (16 * (a.cap + 1) - 8 * qh_slot_words(0) - 16) / 40);
                nvert = tile_compact_upto<K, ABS>(t, mask, xs, ys, mmax + 1);
                const int m = nvert - 1;
                if (m <= mmax) {
                    int qa, qb;
                    const bool vert =
                        tile_quickhull(t.VXY, m, (unsigned long long*)(t.VXY + m + 1), 0x1p-48, qa, qb);
                    tile_hull_to_front(t, m, vert, qa, a.increasing, a.lo, a.hi);
                    tile_masks_short<K>(t, mask);
                    tile_store<T, K>(t, mask, out, sb, cb);
                    if (a.row_nan && threadIdx.x == 0) a.row_nan[row] = 0u;
                    return;
                }
            }
            row_exact<T, K>(y, w, out, sb, cb, a.row_nan ? a.row_nan + row : nullptr, a.ovf + row * a.ovf_stride, N,
                            a.increasing, a.lo, a.hi, a.cap, a.stage);
            return;
        } else {
            bool done = false;
            if (5 * nvert <= 3 * N + 5 && nvert <= a.cap + 1) {
                tile_compact<K, ABS>(t, mask, xs, ys);
                if (tile_wrap<K, ABS>(t)) {
                    tile_masks_short<K>(t, mask);
                    done = true;
                }
            }
            if (!done) {
                row_exact<T, K>(y, w, out, sb, cb, a.row_nan ? a.row_nan + row : nullptr, a.ovf + row * a.ovf_stride,
                                N, a.increasing, a.lo, a.hi, a.cap, a.stage);
                return;
            }
        }
    } else {
        over = nvert > a.cap + 1;
        if (!over) tile_merges<K, ABS>(t, mask, xs, ys, true);
    }
    if (a.ovf_row && threadIdx.x == 0) a.ovf_row[row] = over ? 1 : 0;
    if (over) return;
    tile_finish<T, K>(t, mask, a.increasing, a.lo, a.hi, out, sb, cb);
    if (a.row_nan && threadIdx.x == 0) a.row_nan[row] = 0u;
}

// The rows k_row_fit flagged: the same pipeline with room for every point in
// the vertex list, in LDS when a.cap == N (one-wave rows: 13 KiB at most) or
// else in the row's area of the workspace.  Other rows return at once.
template <typename T, int K>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void k_row_ovf(RowArgs a) {
    extern __shared__ __align__(32) char smem[];
    const int64_t row = blockIdx.x;
    if (a.ovf_row[row] == 0) return;
    const int N = (int)a.n;
    const bool in_lds = a.cap >= N;
    Tile t = tile_carve(smem, blockDim.x, in_lds ? N : 0, K, N);
    if (!in_lds) {
        char* o = a.ovf + row * a.ovf_stride;
        t.VXY = (double2*)o;
        t.V = (unsigned short*)(o + 16 * (a.n + 1));
    }
    const T* y = (const T*)a.y + row * a.n;
    const T* w = a.w ? (const T*)a.w + row * a.n : nullptr;
    T* out = (T*)a.fit + row * a.n;
    uint64_t* sb = a.start_bits ? a.start_bits + row * a.words : nullptr;
    uint64_t* cb = a.clip_bits ? a.clip_bits + row * a.words : nullptr;
    uint64_t mask;
    double xs[K], ys[K];
    int nvert;
    (void)tile_build<T, K>(t, y, w, a.increasing, mask, xs, ys, nvert);  // inputs already checked
    constexpr bool ABS = sizeof(T) == 4;
    tile_merges<K, ABS>(t, mask, xs, ys);
    tile_finish<T, K>(t, mask, a.increasing, a.lo, a.hi, out, sb, cb);
    if (a.row_nan && threadIdx.x == 0) a.row_nan[row] = 0u;
}

// ---------------------------------------------------------------------------
// rows of at most kLaneRow elements, one row per lane (first page, Sec. 3.5:
// short rows are packed several to a warp; here each lane holds a whole row).
// The lane's hull is the row's hull, so there is nothing to merge: a forward
// pass over the points gives the slope of each hull edge at its end vertex,
// and a backward pass hands every element the slope of the first vertex at or
// after its right point.  No LDS, no barriers.
// ---------------------------------------------------------------------------
template <typename T, int K>
// At most 256 registers a lane (two waves per SIMD): beyond that the
// accumulation registers count too and only one wave fits.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_rows_lane(RowArgs a, int64_t rows) {
    mark_epoch(a.status, a.epoch);
    const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= rows) return;
    const int N = (int)a.n;
    const T* y = (const T*)a.y + row * a.n;
    const T* w = a.w ? (const T*)a.w + row * a.n : nullptr;
    T* out = (T*)a.fit + row * a.n;
    uint64_t* sb = a.start_bits ? a.start_bits + row * a.words : nullptr;  // one word: n <= 64
    uint64_t* cb = a.clip_bits ? a.clip_bits + row * a.words : nullptr;
    double xs[K], ys[K];
    int f = 0;
    const uint64_t mask = lane_hull<T, K>(y, w, N, !a.increasing, xs, ys, f);
    if (f) {
        for (int j = 0; j < N; ++j) out[j] = (T)NAN;
        if (sb) {
            *sb = 0ull;
            *cb = 0ull;
        }
        if (a.row_nan) a.row_nan[row] = 1u;
        if (f == 2) report_weight_error(a.status, a.epoch);
        return;
    }
    // E[b] = slope of the hull edge ending at point b + 1 (where that point is
    // a vertex); the edge starts at the previous vertex (px, py)
    double E[K];
    double px = 0.0, py = 0.0;
#pragma unroll
    for (int b = 0; b < K; ++b) {
        E[b] = 0.0;
        if (b < N && ((mask >> b) & 1ull)) {
            E[b] = (ys[b] - py) / (xs[b] - px);
            px = xs[b];
            py = ys[b];
        }
    }
    double vals[K];
    uint64_t clipm = 0ull;
    double cur = 0.0;
#pragma unroll
    for (int b = K - 1; b >= 0; --b) {
        if (b < N && ((mask >> b) & 1ull)) cur = E[b];  // point N is always a vertex
        bool c = false;
        vals[b] = finish(cur, a.increasing, a.lo, a.hi, c);
        if (b < N && c) clipm |= 1ull << b;
    }
    store_lane<T, K>(out, N, vals);
    if (sb) {
        *sb = ((mask << 1) | 1ull) & bits_upto(N - 1);  // element j starts a block iff point j is a vertex
        *cb = clipm;
    }
    if (a.row_nan) a.row_nan[row] = 0u;
}

// ---------------------------------------------------------------------------
// chunk hulls of long rows
// ---------------------------------------------------------------------------
struct ChunkArgs {
    RowArgs r;
    int64_t m;         // chunks per row
    double4* tot;      // [rows*m] chunk totals (double-double x, y)
    int* nv;           // [rows*m] vertices of the chunk hull
    int* cflag;        // [rows*m]
    uint64_t* cmask;   // [rows*m*kMaskWords]
    int* cpre;         // [rows*m*kMaskWords]
    double4* cgs;      // [rows*m*kGroups]
    double4* cvx;      // [rows*m*kVMax]
    int* cvi;          // [rows*m*kVMax]
    int* cover;        // [rows*m] 1 where the first pass left the chunk to the second, else 0
    int* clist;        // [rows*m] the chunks the first pass left, in the order they were listed
    unsigned long long* cctr;  // [2] clist's count word (cover_append), the epoch of a full scan
    int64_t nchunks;   // rows * m
    int cap;           // list entries of this pass (kChunk in the second)
    int early;         // the call has chunks enough to keep the second pass busy
};

// The first pass gives each chunk a list of kChunkCap entries, small enough
// for four chunks to share a CU's LDS; a chunk that merges lane hulls with
// more survivors than that (rare on dense rows, whose merging chunks keep
// about 650 to 1300 of 3585 points; every chunk of a row whose every point is
// a vertex) is flagged, listed, and fitted by the second pass, whose list
// holds every point.  Every chunk writes its flag.
constexpr int kChunkCap = (kLdsBytes / 4 - 512 - (int)tile_smem_bytes(kChunkLanes, 0, kLaneK)) / 18;
// Candidates the first pass finishes by QuickHull: its list (32 bytes an
// entry) takes the list's room, its three slot arrays (24 bytes an entry) the
// lane starts, masks, bridges and lane indices, which are contiguous in the
// tile's LDS and free while it runs.
constexpr int kChunkQh = std::min((16 * (kChunkCap + 1)) / 32 - 1,
                                  (int)((32 * (kChunkLanes + 1) + 16 * kChunkLanes + 8 * (kChunkLanes / 2 + 1) +
                                         4 * kChunkLanes - 48) / 24));
static_assert(kChunkQh <= 3 * kChunkLanes && kChunkQh <= 1023, "three QuickHull entries per thread, 10-bit keys");

// The first pass lists the chunks it leaves to the second.  The count word
// holds the call's epoch (its low 40 bits, above) and the count (24 bits:
// more chunks than that would not fit in memory), so that a word left by an
// earlier call reads as an empty list and nothing needs clearing.  Should an
// entry fall outside the list (a word of another process's call with the same
// tag), the second pass is told to scan every chunk's flag instead; stale
// entries are harmless, as the second pass fits only chunks whose flag (written
// by every chunk of this call) is set.
constexpr unsigned long long kCoverTagShift = 24;
__device__ inline unsigned long long cover_tag(unsigned long long epoch) {
    return (epoch & ((1ull << 40) - 1ull)) << kCoverTagShift;
}
__device__ inline void cover_append(const ChunkArgs& a, int64_t bid) {
    const unsigned long long tag = cover_tag(a.r.epoch), cnt_mask = (1ull << kCoverTagShift) - 1ull;
    // one atomic add per entry; only the call's first appenders, which find
    // an earlier call's word, replace it by this call's tag (one of them wins
    // and takes entry 0, the others then add to the new word)
    unsigned long long old = atomicAdd(a.cctr, 1ull);
    while ((old & ~cnt_mask) != tag) {
        const unsigned long long cur = atomicCAS(a.cctr, old + 1ull, tag + 1ull);
        if (cur == old + 1ull) {
            old = tag;
            break;
        }
        old = ((cur & ~cnt_mask) == tag) ? atomicAdd(a.cctr, 1ull) : cur - 1ull;
    }
    const int64_t slot = (int64_t)(old & cnt_mask);
    if (slot < a.nchunks)
        a.clist[slot] = (int)bid;
    else
        atomicExch(a.cctr + 1, a.r.epoch);
}

// One chunk by the workgroup: its hull stored, its tentative fit written.
// PASS 0: the first pass (every chunk, a list of kChunkCap entries); 1: the
// second (the chunks the first left, a list of every point).
template <typename T, int PASS>
__device__ inline void chunk_fit(const ChunkArgs& a, int64_t bid) {
    constexpr int K = kLaneK;
    constexpr bool ABS = sizeof(T) == 4;
    extern __shared__ __align__(32) char smem[];
    const int64_t row = bid / a.m, c = bid % a.m;
    const int64_t e0 = c * kChunk;
    const int N = (int)((a.r.n - e0) < kChunk ? (a.r.n - e0) : kChunk);
    const Tile t = tile_carve(smem, blockDim.x, a.cap, K, N);
    const T* y = (const T*)a.r.y + row * a.r.n + e0;
    const T* w = a.r.w ? (const T*)a.r.w + row * a.r.n + e0 : nullptr;
    T* out = (T*)a.r.fit + row * a.r.n + e0;
    uint64_t* sb = a.r.start_bits ? a.r.start_bits + row * a.r.words + e0 / 64 : nullptr;
    uint64_t* cb = a.r.clip_bits ? a.r.clip_bits + row * a.r.words + e0 / 64 : nullptr;
    uint64_t mask;
    double xs[K], ys[K];
    int nvert;
    // the points and lane starts only: the lane hulls are built below, by the
    // chunks that merge them
    const int flag = tile_build<T, K, false>(t, y, w, a.r.increasing, mask, xs, ys, nvert);
    if (flag) {
        // the whole row comes back NaN; k_fixup writes it
        if (threadIdx.x == 0) {
            a.cflag[bid] = flag;
            a.nv[bid] = 0;
            if (PASS == 0) a.cover[bid] = 0;
        }
        return;
    }
    const int l = threadIdx.x;
    // starts of the 256-element groups and the chunk's total (QuickHull
    // overwrites the lane starts)
    constexpr int LPG = kGroup / K;
    if ((l % LPG) == 0 && l * K < N) a.cgs[bid * kGroups + l / LPG] = t.LS[l];
    if (l == 0) a.tot[bid] = t.LS[t.nl];
    // Only points under the hull of the lane ends can be vertices of the
    // chunk's hull (its edges are chords between points of the chunk), so
    // the candidates are the points not above the edge of that coarse hull
    // over their lane (dense data: about 400 of 3584, noise: about 80), and
    // the chunk's last point.  The coarse hull is found by QuickHull (one
    // lane end per thread) on a plain copy of the lane starts.
    const int cnt = min(max(N - (int)threadIdx.x * K, 0), K);
    // The second pass first tests whether the lanes' hulls already form one
    // convex chain (every point of the chunk a vertex, the first page's Sec.
    // 7.5 regime): that chain is then the chunk's hull, and neither the coarse
    // filter nor the merges run.  (A convex chain lies under the chord of any
    // two of its points, so the filter would keep every point of it.)
    bool chain = false;
    if constexpr (PASS == 1 && !ABS) {
        mask = lane_gift_wrap<K>(xs, ys, cnt);
        tile_compact<K, ABS>(t, mask, xs, ys);
        chain = tile_junctions_left<K, ABS>(t, mask);  // uniform
    }
    uint64_t cand = ~0ull;
    if (!chain) {
        const int used = (N + K - 1) / K;
        double2* E = (double2*)t.VXY;  // free until the candidates are listed
        unsigned long long* slots = (unsigned long long*)(E + kChunkLanes + 1);
        for (int l = threadIdx.x; l <= used; l += blockDim.x) E[l] = lane_start2(t, l);
        __syncthreads();
        int ea, eb;
        (void)tile_quickhull(E, used, slots, 0.0, ea, eb);
        cand = lane_coarse_filter<K>(t, xs, ys, cnt, ea, eb, E);
        if ((int)threadIdx.x == used - 1) cand |= 1ull << (cnt - 1);
        __syncthreads();  // E and the slots are read before the list reuses them
    }
    // few candidates: their hull by QuickHull on the list, with the merges'
    // vertex test; no lane hulls are needed (m is uniform: read as a scalar,
    // so that the branches below hold registers apart)
    int m = kChunk;
    if constexpr (PASS == 0) m = __builtin_amdgcn_readfirstlane(list_compact<K>(t, cand, xs, ys, kChunkQh + 1) - 1);
    if (PASS == 0 && a.early && m > a.cap && m >= N) {
        // every point a candidate, more than the first pass's list holds
        // (every point of an increasing row is a vertex): the second pass
        // fits the chunk, with room for every point.  Chunks whose lane hulls
        // may still shrink their candidates below the list's size stay here,
        // and so do all chunks of a call with few of them, where the second
        // pass would take one chunk's latency per workgroup.
        if (threadIdx.x == 0) {
            a.cover[bid] = 1;
            cover_append(a, bid);
        }
        return;
    }
    const bool merged = m > kChunkQh;
    if (!merged) {
        bool vert[3];
        list_quickhull<3>(t, m, (unsigned long long*)t.LS, vert);
        list_to_front<3>(t, m, vert);
        tile_masks<K>(t, mask);
    } else if (!chain) {
        // the lane hulls' vertices among the candidates, and every lane's
        // last point, so that each lane's node is still a convex chain from
        // its start to its end (the merges need both ends: a node starts at
        // the previous lane's end and shares it).  The first pass forms the
        // lane's points again from the inputs (the same loads and sums), so
        // that they are not held in registers through QuickHull.
        const uint64_t end = (cnt > 0) ? (1ull << (cnt - 1)) : 0ull;
        if constexpr (PASS == 0) {
            int f2 = 0;
            mask = lane_hull<T, K>(y + (int64_t)l * K, w ? w + (int64_t)l * K : nullptr, cnt, !a.r.increasing, xs,
                                   ys, f2);
        } else if constexpr (ABS) {
            mask = lane_gift_wrap<K>(xs, ys, cnt);
        }  // (the second pass's float64 lane hulls are in mask already)
        mask &= cand | end;
        if constexpr (PASS == 0) {
            const bool over = tile_count(t, mask) > a.cap + 1;  // uniform
            if (over) {
                if (threadIdx.x == 0) {
                    a.cover[bid] = 1;
                    cover_append(a, bid);
                }
                return;  // nothing else written: the second pass fits the chunk
            }
        }
        tile_merges<K, ABS>(t, mask, xs, ys, false, 1 << 30, PASS == 1);
    }
    if (PASS == 0 && threadIdx.x == 0) a.cover[bid] = 0;
    __syncthreads();  // every lane's final mask in M
    const int nv = t.flag[1];  // vertices of the chunk hull; rank r is list entry r
    // explicit coordinates (relative to the chunk start) of the end windows,
    // or of every vertex of a hull of at most kVMax vertices
    for (int q = l; q < kVMax; q += blockDim.x) {
        const int r = (nv <= kVMax || q < kVMax / 2) ? q : nv - kVMax + q;
        if (r < nv) {
            const int p = t.V[r];
            double4 c4;
            if (merged) {
                const double2 c = t.VXY[r];
                c4 = ABS ? make_double4(c.x, 0.0, c.y, 0.0) : dd4_add_d(t.LS[lane_of<K>(p)], c);
            } else {
                c4 = list_dd(t)[r];
                if (ABS) c4 = make_double4(c4.x, 0.0, c4.z, 0.0);
            }
            a.cvi[bid * kVMax + q] = p;
            a.cvx[bid * kVMax + q] = c4;
        }
    }
    // vertex bit set and the rank of each word's first vertex
    constexpr int LPW = 64 / K;
    if ((l % LPW) == 0 && l * K < N) {
        uint64_t word = 0ull;
#pragma unroll
        for (int k = 0; k < LPW; ++k) word |= t.M[l + k] << (k * K);
        a.cmask[bid * kMaskWords + l / LPW] = word;
        a.cpre[bid * kMaskWords + l / LPW] = t.I[l];
    }
    if (l == 0) {
        a.nv[bid] = nv;
        a.cflag[bid] = 0;
    }
    // tentative fit from the chunk's own hull; k_fixup corrects the elements
    // outside the chunk's surviving segment
    if (merged)
        tile_finish<T, K>(t, mask, a.r.increasing, a.r.lo, a.r.hi, out, sb, cb);
    else
        tile_finish<T, K, 3>(t, mask, a.r.increasing, a.r.lo, a.r.hi, out, sb, cb);
}

// The first pass: one workgroup per chunk.
template <typename T>
__global__ __launch_bounds__(kChunkLanes) void k_chunk_hull(ChunkArgs a) {
    mark_epoch(a.r.status, a.r.epoch);
    chunk_fit<T, 0>(a, blockIdx.x);
}

// The second pass: workgroup b of the grid takes the listed chunks b, b + G,
// b + 2G, ... (G workgroups, each chunk to one workgroup while there are at
// most G).  The first pass has completed in stream order.  When the list
// overflowed, every workgroup instead reads the flags of the chunks b, b + G,
// ..., 256 at a time (flagged chunks come in runs, which this spreads over
// the grid), and fits the flagged ones.  Registers are held to 256 a lane, so
// that two workgroups (the LDS's limit) fit on a CU.
template <typename T>
__global__ __launch_bounds__(kChunkLanes) __attribute__((amdgpu_waves_per_eu(2))) void k_chunk_cover(ChunkArgs a) {
    const int64_t G = gridDim.x;
    const unsigned long long word = a.cctr[0], tag = cover_tag(a.r.epoch);
    if (a.cctr[1] != a.r.epoch) {
        int64_t cnt = ((word >> kCoverTagShift) == (tag >> kCoverTagShift))
                          ? (int64_t)(word & ((1ull << kCoverTagShift) - 1ull))
                          : 0;
        if (cnt > a.nchunks) cnt = a.nchunks;
        for (int64_t i = blockIdx.x; i < cnt; i += G) {
            const int64_t c = a.clist[i];
            if (c >= 0 && c < a.nchunks && a.cover[c] != 0) {  // uniform
                chunk_fit<T, 1>(a, c);
                __syncthreads();  // the next chunk reuses the LDS
            }
        }
        return;
    }
    __shared__ uint64_t sel[kChunkLanes / kWave];
    for (int64_t i0 = 0; (int64_t)blockIdx.x + i0 * G < a.nchunks; i0 += kChunkLanes) {
        const int64_t c = (int64_t)blockIdx.x + (i0 + threadIdx.x) * G;
        const uint64_t b = __ballot(c < a.nchunks && a.cover[c] != 0);
        if (lane_id() == 0) sel[threadIdx.x / kWave] = b;
        __syncthreads();
        for (int q = 0; q < kChunkLanes / kWave; ++q) {
            uint64_t pend = sel[q];  // the same in every thread
            while (pend) {
                const int bit = lo_bit(pend);
                pend &= pend - 1ull;
                chunk_fit<T, 1>(a, (int64_t)blockIdx.x + (i0 + q * kWave + bit) * G);
                __syncthreads();  // the next chunk reuses the LDS
            }
        }
        __syncthreads();  // every thread has read sel before it is rewritten
    }
}

// ---------------------------------------------------------------------------
// merge tree of one long row
// ---------------------------------------------------------------------------

// Read access to the stored chunk hulls of one row.
struct HullView {
    const int* nv;
    const double4* tot;
    const uint64_t* mask;
    const int* pre;
    const double4* gs;
    const double4* vx;
    const int* vi;
    const void* y;  // the row's elements
    const void* w;
    int negate;
    int64_t n;
};

struct Vtx {
    int p;      // chunk-local point
    double4 v;  // coordinates relative to the chunk start (double-double x, y)
};

template <typename T>
__device__ inline double2 elem_wt(const HullView& H, int64_t e) {
    const double yv = (double)((const T*)H.y)[e];
    const double wv = H.w ? (double)((const T*)H.w)[e] : 1.0;
    double t = wv * yv;
    if (H.negate) t = -t;
    return make_double2(wv, t);
}

// Vertex of rank r of chunk c's hull.  The end windows are read directly;
// any other vertex is found in the bit set (rank of each word's first vertex,
// then the bit) and its coordinates are summed from the nearer end of its
// 256-element group.
template <typename T>
__device__ inline Vtx vtx_n(const HullView& H, int c, int r, int nv) {
    int s = -1;
    if (nv <= kVMax || r < kVMax / 2)
        s = r;
    else if (r >= nv - kVMax / 2)
        s = r - nv + kVMax;
    if (s >= 0) return Vtx{H.vi[c * kVMax + s], H.vx[c * kVMax + s]};
    const int64_t e0 = (int64_t)c * kChunk;
    const int Nc = (int)((H.n - e0) < kChunk ? (H.n - e0) : kChunk);
    const int words = (Nc + 63) / 64;
    const int* pre = H.pre + (int64_t)c * kMaskWords;
    const uint64_t* mk = H.mask + (int64_t)c * kMaskWords;
    int lo = 0, hi = words - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= r)
            lo = mid;
        else
            hi = mid - 1;
    }
    uint64_t m = mk[lo];
    for (int k = r - pre[lo]; k > 0 && m; --k) m &= m - 1ull;
    const int p = m ? lo * 64 + lo_bit(m) + 1 : lo * 64 + 1;
    const int G = (Nc + kGroup - 1) / kGroup;
    int g = p / kGroup;
    if (g > G - 1) g = G - 1;
    const int gs0 = g * kGroup, ge = (gs0 + kGroup < Nc) ? gs0 + kGroup : Nc;
    // compensated sums (two-sum), so that the partial sum adds no more than
    // a unit of rounding of its own magnitude
    double X = 0.0, Xe = 0.0, Y = 0.0, Ye = 0.0;
    double4 v;
    if (p - gs0 <= ge - p) {
        for (int e = gs0; e < p; ++e) {
            const double2 q = elem_wt<T>(H, e0 + e);
            double se;
            two_sum(X, q.x, X, se);
            Xe += se;
            two_sum(Y, q.y, Y, se);
            Ye += se;
        }
        const double4 G0 = H.gs[(int64_t)c * kGroups + g];
        v = dd4_add(G0, make_double4(X, Xe, Y, Ye));
    } else {
        for (int e = p; e < ge; ++e) {
            const double2 q = elem_wt<T>(H, e0 + e);
            double se;
            two_sum(X, q.x, X, se);
            Xe += se;
            two_sum(Y, q.y, Y, se);
            Ye += se;
        }
        const double4 B = (g + 1 < G) ? H.gs[(int64_t)c * kGroups + g + 1] : H.tot[c];
        v = dd4_add(B, make_double4(-X, -Xe, -Y, -Ye));
    }
    return Vtx{p, v};
}

template <typename T>
__device__ inline Vtx vtx(const HullView& H, int c, int r) {
    return vtx_n<T>(H, c, r, H.nv[c]);
}

struct MergeArgs {
    const void* y;
    const void* w;
    int64_t n, m;
    int nsub;     // subtrees of kSub chunks per row
    int negate;
    HullView H0;  // row 0's pointers; offset per row in the kernels
    const int* cflag;
    double4* starts;
    Desc* gsd;    // [rows*m] each subtree's hull as a list, in the slots of its chunks
    int* gsn;     // [rows*nsub] their lengths
    Desc* gd0;    // [rows*m] top levels' lists when they do not fit in LDS
    Desc* gd1;
    int* gnc;
    MRec* gmr;
    int* gnv;     // unused slot kept for layout symmetry
    double* gso;
    Rec* rec;
    uint32_t* row_nan;
    unsigned long long* status;
    unsigned long long epoch;
    int use_lds;
};

// a point of the row as one double-double pair (chunk start + chunk-relative
// vertex, summed exactly), so that the difference of two points loses nothing
// to the size of the chunk starts (first page, App. B, "Merge levels")
struct PtD {
    double4 a;
};

// What a merge reads: the descriptors of the current level, the chunk starts
// in the merge's frame (st[c - st_off]; a subtree uses starts relative to its
// first chunk, as the hull of a node does not change under translation), and
// the vertex counts (nvc[c - nv_off]).
struct MCtx {
    const Desc* D;
    const double4* st;
    int st_off;
    const int* nvc;
    int nv_off;
    HullView H;
};

struct VR {
    int s;  // descriptor slot
    int k;  // vertex rank in the chunk hull
};

// a + b of two double-double numbers with one exact sum of the high parts and
// the low parts added once (Dekker's shorter addition): its error is of the
// order of the low parts' rounding, far below what a difference of two points
// keeps (pdx, pdy round to a double)
__device__ __forceinline__ void dd_add_short(double ah, double al, double bh, double bl, double& rh, double& rl) {
    double s, e;
    two_sum(ah, bh, s, e);
    e += al + bl;
    fast_two_sum(s, e, rh, rl);
}

template <typename T>
__device__ __forceinline__ PtD ptd(const MCtx& X, int c, int k) {
    const double4 a = X.st[c - X.st_off], b = vtx_n<T>(X.H, c, k, X.nvc[c - X.nv_off]).v;
    PtD p;
    dd_add_short(a.x, a.y, b.x, b.y, p.a.x, p.a.y);
    dd_add_short(a.z, a.w, b.z, b.w, p.a.z, p.a.w);
    return p;
}
template <typename T>
__device__ __forceinline__ PtD ptv(const MCtx& X, VR v) {
    return ptd<T>(X, X.D[v.s].c, v.k);
}

// b - a, rounded to a double, part by part (high parts, then low parts): the
// high parts of two nearby points cancel exactly, and the rounding of a
// distant pair's difference is that of the result itself
__device__ __forceinline__ double pdx(const PtD& a, const PtD& b) { return (b.a.x - a.a.x) + (b.a.y - a.a.y); }
__device__ __forceinline__ double pdy(const PtD& a, const PtD& b) { return (b.a.z - a.a.z) + (b.a.w - a.a.w); }
__device__ __forceinline__ double turnD(const PtD& a, const PtD& b, const PtD& d) {
    return pdx(a, b) * pdy(a, d) - pdy(a, b) * pdx(a, d);
}
__device__ __forceinline__ double slopeD(const PtD& a, const PtD& b) { return pdy(a, b) / pdx(a, b); }

// successor of v in the list whose last slot is s1
__device__ __forceinline__ bool vsucc(const MCtx& X, VR v, int s1, VR& n) {
    if (v.k < (int)X.D[v.s].h) {
        n.s = v.s;
        n.k = v.k + 1;
        return true;
    }
    if (v.s < s1) {
        n.s = v.s + 1;
        n.k = X.D[v.s + 1].l;
        return true;
    }
    return false;
}
// predecessor of v in the list whose first slot is s0
__device__ __forceinline__ bool vpred(const MCtx& X, VR v, int s0, VR& p) {
    if (v.k > (int)X.D[v.s].l) {
        p.s = v.s;
        p.k = v.k - 1;
        return true;
    }
    if (v.s > s0) {
        p.s = v.s - 1;
        p.k = X.D[v.s - 1].h;
        return true;
    }
    return false;
}
// the vertex g places before v in the list whose first slot is s0
__device__ inline bool step_back(const MCtx& X, VR v, int s0, int g, VR& out) {
    int s = v.s, k = v.k;
    while (g > 0) {
        const int avail = k - (int)X.D[s].l;
        if (g <= avail) {
            k -= g;
            g = 0;
        } else {
            if (s == s0) return false;
            g -= avail + 1;
            --s;
            k = X.D[s].h;
        }
    }
    out = VR{s, k};
    return true;
}
// the vertex g places after v in the list whose last slot is s1
__device__ inline bool step_fwd(const MCtx& X, VR v, int s1, int g, VR& out) {
    int s = v.s, k = v.k;
    while (g > 0) {
        const int avail = (int)X.D[s].h - k;
        if (g <= avail) {
            k += g;
            g = 0;
        } else {
            if (s == s1) return false;
            g -= avail + 1;
            ++s;
            k = X.D[s].l;
        }
    }
    out = VR{s, k};
    return true;
}

// First vertex of the view (slots s0..s1, last slot ending at lastH) for which
// a monotone predicate (false ... false true ... true) holds; the view's last
// vertex must satisfy it.  Bisection first over segments, then within one
// (first page, Sec. 3.3).
template <class Pred>
__device__ inline VR first_true(const MCtx& X, int s0, int s1, int lastH, Pred pred) {
    int lo = s0, hi = s1 + 1;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (pred(VR{mid, (int)X.D[mid].l}))
            hi = mid;
        else
            lo = mid + 1;
    }
    if (lo == s0) return VR{s0, (int)X.D[s0].l};
    const int sg = lo - 1;
    const int hv = (sg == s1) ? lastH : (int)X.D[sg].h;
    int rlo = (int)X.D[sg].l + 1, rhi = hv + 1;
    while (rlo < rhi) {
        const int mid = (rlo + rhi) >> 1;
        if (pred(VR{sg, mid}))
            rhi = mid;
        else
            rlo = mid + 1;
    }
    if (rlo <= hv) return VR{sg, rlo};
    // only reached if rounding broke the predicate's guarantee at the view's
    // last vertex: stay inside the view
    if (lo > s1) return VR{s1, lastH};
    return VR{lo, (int)X.D[lo].l};
}

// Lower tangent from p (left of every vertex of B) to B = slots jB..sB1: the
// vertex minimising the slope from p, the farthest one on ties.
template <typename T>
__device__ inline VR tangent_b(const MCtx& X, const PtD& p, int jB, int sB1) {
    return first_true(X, jB, sB1, X.D[sB1].h, [&](VR v) -> bool {
        VR nx;
        if (!vsucc(X, v, sB1, nx)) return true;
        return turnD(p, ptv<T>(X, v), ptv<T>(X, nx)) > 0.0;
    });
}

// The bridge by nested bisection (Sec. 3.3, Thm. 5.2): a candidate a of A is
// tested against its tangent to B; a is left of the bridge while A's next
// vertex lies strictly below the line from a to its tangent point.
// Candidates end at the predecessor of the shared point.
template <typename T>
__device__ inline void bisect_bridge(const MCtx& X, int j0, int la, int jB, int sB1, VR& al, VR& be) {
    const Desc dA = X.D[la];
    int aS1 = la, aLastH = (int)dA.h - 1;
    if (aLastH < (int)dA.l) {
        aS1 = la - 1;
        aLastH = X.D[la - 1].h;
    }
    al = first_true(X, j0, aS1, aLastH, [&](VR a) -> bool {
        VR an;
        vsucc(X, a, la, an);
        const PtD Pa = ptv<T>(X, a);
        const VR b = tangent_b<T>(X, Pa, jB, sB1);
        return !(turnD(Pa, ptv<T>(X, an), ptv<T>(X, b)) > 0.0);
    });
    be = tangent_b<T>(X, ptv<T>(X, al), jB, sB1);
}

// Window steps a merge may take before it switches to bisection.
constexpr int kWindowSteps = 64;

// LDS of one wave's window search (window_bridge): kBW vertices of each list
// nearest the shared point.
constexpr int kBW = 128;
struct BWin {
    double2 A[kBW], B[kBW];    // coordinates relative to the shared point
    int2 IA[kBW], IB[kBW];     // (slot, rank) of each entry
    int cA[kWave], cB[kWave];  // vertices in the first 1..64 descriptors read from the shared point
};

// The bridge of a merge from windows of the two lists, with the calling wave
// (first page, Sec. 4, Lemma 4.2 and the walk after it, at LDS latency).  The
// kBW vertices of A before the shared point s (A[0] = s, A[i] = the i-th
// predecessor) and of B after it are read once, as double-double differences
// from s rounded to float64 (a difference loses nothing to the size of the
// coordinates, first page, App. B), together with their (slot, rank); then the
// walk of find_merge runs on them, 64 candidates per step.  Returns false when
// the walk reaches the end of a window that does not hold its whole list (the
// bridge may lie beyond it); the caller then walks the lists themselves.
template <typename T>
__device__ __forceinline__ bool window_bridge(const MCtx& X, int j0, int la, int jB, int sB1, int g, BWin* W, VR& al,
                                     VR& be) {
    const Desc* D = X.D;
    int lenA = 0, lenB = 0;
    if (la - g >= j0) {
        const Desc d = D[la - g];
        lenA = (int)d.h - (int)d.l + 1;
    }
    if (jB + g <= sB1) {
        const Desc d = D[jB + g];
        lenB = (int)d.h - (int)d.l + 1;
    }
    const int cumA = wave_incl_scan_int(lenA), cumB = wave_incl_scan_int(lenB);
    W->cA[g] = cumA;
    W->cB[g] = cumB;
    const int totA = __builtin_amdgcn_readlane(cumA, kWave - 1), totB = __builtin_amdgcn_readlane(cumB, kWave - 1);
    const bool allA = la - (kWave - 1) <= j0 && totA <= kBW;  // the window holds all of A
    const bool allB = jB + (kWave - 1) >= sB1 && totB <= kBW;
    const int nA = min(totA, kBW), nB = min(totB, kBW);
    const PtD Ps = ptv<T>(X, VR{la, (int)D[la].h});
    wave_sync();
    // entries g, g + 64 of each window: one vertex read per pass (a loop, not
    // unrolled, keeps one vertex access inlined)
#pragma unroll 1
    for (int q = 0; q < 2 * (kBW / kWave); ++q) {
        const bool onA = q < kBW / kWave;
        const int i = g + kWave * (onA ? q : q - kBW / kWave);
        const int* cnt = onA ? W->cA : W->cB;
        if (i < (onA ? nA : nB)) {
            int lo = 0, hi = kWave - 1;  // the first descriptor whose count passes i
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (cnt[mid] > i)
                    hi = mid;
                else
                    lo = mid + 1;
            }
            const int off = i - (lo ? cnt[lo - 1] : 0);
            const int sl = onA ? la - lo : jB + lo;
            const int k = onA ? (int)D[sl].h - off : (int)D[sl].l + off;
            const PtD P = ptd<T>(X, D[sl].c, k);
            const double2 rel = make_double2(pdx(Ps, P), pdy(Ps, P));
            if (onA) {
                W->A[i] = rel;
                W->IA[i] = make_int2(sl, k);
            } else {
                W->B[i] = rel;
                W->IB[i] = make_int2(sl, k);
            }
        }
    }
    wave_sync();
    auto turn = [](double2 a, double2 b, double2 d) { return (b.x - a.x) * (d.y - a.y) - (b.y - a.y) * (d.x - a.x); };
    int ia = 1, ib = 1;  // the neighbours of s
    for (int it = 0; it < kWindowSteps; ++it) {
        // left side against B[ib]: pass over a while it is not a strict
        // vertex of {pred(a), a, B[ib]}
        const double2 pb = W->B[ib];
        for (;;) {
            const int i = ia + g;
            bool cont = false;
            if (i + 1 < nA) cont = !(turn(W->A[i + 1], W->A[i], pb) > 0.0);
            const int run = trailing_ones(__ballot(cont));
            ia += run;
            if (run < kWave) break;
        }
        if (ia == nA - 1 && !allA) return false;
        // right side against the new A[ia]
        const double2 pa = W->A[ia];
        bool moved = false;
        for (;;) {
            const int j = ib + g;
            bool cont = false;
            if (j + 1 < nB) cont = !(turn(pa, W->B[j], W->B[j + 1]) > 0.0);
            const int run = trailing_ones(__ballot(cont));
            ib += run;
            moved = moved || run > 0;
            if (run < kWave) break;
        }
        if (ib == nB - 1 && !allB) return false;
        if (!moved) {
            const int2 a2 = W->IA[ia], b2 = W->IB[ib];
            al = VR{a2.x, a2.y};
            be = VR{b2.x, b2.y};
            return true;
        }
    }
    return false;
}

// Merge of the node at slots j0.. (cntA descriptors) with its right neighbour
// at jB.. (cntB) by a group of G lanes (g = 0..G-1, G a power of two <= 64)
// (Sec. 3.3, Lemma 4.2, Theorem 4.4).  From the neighbours of the shared
// point the walk of Sec. 4 advances each side to its tangent point against
// the other side's current end, G candidates per step; a walk longer than
// kWindowSteps steps is finished by nested bisection.  Returns the rewrite of
// the merged list; reads the descriptors only.
template <typename T>
__device__ __forceinline__ MRec find_merge(const MCtx& X, int j0, int jB, int cntA, int cntB, int g, int G,
                                  BWin* win = nullptr) {
    const Desc* D = X.D;
    const int la = j0 + cntA - 1;
    const int sB1 = jB + cntB - 1;
    const Desc dA = D[la];
    const Desc dB = D[jB];
    // s: the last vertex of A and the first of B (chunk jB's point 0)
    const VR sA{la, dA.h};
    const VR sB{jB, dB.l};
    VR pA, nB;
    vpred(X, sA, j0, pA);   // A has at least two vertices
    vsucc(X, sB, sB1, nB);  // and so has B
    MRec r;
    PtD Pbe = ptv<T>(X, nB);
    if (turnD(ptv<T>(X, pA), ptv<T>(X, sB), Pbe) > 0.0) {
        // convex at s: keep s once, in B's first segment
        if ((int)dA.h - 1 < (int)dA.l) {
            r.newA = cntA - 1;
            r.alk = D[la - 1].h;
        } else {
            r.newA = cntA;
            r.alk = (int)dA.h - 1;
        }
        r.bs = jB;
        r.nBk = cntB;
        r.bek = dB.l;
        return r;
    }
    const int gb = lane_id() & ~(G - 1);
    VR al = pA, be = nB;
    int steps = 0;
    // the walk, until it converges (true), or has taken cap steps of G
    // candidates in all, or (iters) that many steps of any length (false)
    auto walk = [&](int cap, int iters) -> bool {
        Pbe = ptv<T>(X, be);  // a walk that stopped inside the right side left it behind be
        for (;;) {
            // left side against be: pass over a while it is not a strict vertex
            // of {pred(a), a, be}
            for (;;) {
                VR c0 = al, c1 = al;
                const bool v0 = step_back(X, al, j0, g, c0);
                const bool v1 = v0 && step_back(X, c0, j0, 1, c1);
                bool cont = false;
                if (v1) cont = !(turnD(ptv<T>(X, c1), ptv<T>(X, c0), Pbe) > 0.0);
                const int run = trailing_ones(group_bits(__ballot(cont), G));
                const int step = run < G ? run : G;
                const int src = gb + (step < G ? step : G - 1);
                const int ts = __shfl(step < G ? c0.s : c1.s, src, kWave);
                const int tk = __shfl(step < G ? c0.k : c1.k, src, kWave);
                if (step > 0) al = VR{ts, tk};
                if (--iters < 0) return false;
                if (step < G) break;
                if (++steps > cap) return false;
            }
            // right side against the new al
            const PtD Pal = ptv<T>(X, al);
            bool movedB = false;
            for (;;) {
                VR c0 = be, c1 = be;
                const bool v0 = step_fwd(X, be, sB1, g, c0);
                const bool v1 = v0 && step_fwd(X, c0, sB1, 1, c1);
                bool cont = false;
                if (v1) cont = !(turnD(Pal, ptv<T>(X, c0), ptv<T>(X, c1)) > 0.0);
                const int run = trailing_ones(group_bits(__ballot(cont), G));
                const int step = run < G ? run : G;
                const int src = gb + (step < G ? step : G - 1);
                const int ts = __shfl(step < G ? c0.s : c1.s, src, kWave);
                const int tk = __shfl(step < G ? c0.k : c1.k, src, kWave);
                if (step > 0) {
                    be = VR{ts, tk};
                    movedB = true;
                }
                if (--iters < 0) return false;
                if (step < G) break;
                if (++steps > cap) return false;
            }
            if (!movedB) return true;
            Pbe = ptv<T>(X, be);
        }
    };
    // with windows, the walk first runs on them at LDS latency; else (or when
    // the bridge lies beyond them) on the lists, to its cap; then bisection.
    // Windows pay where the segments at the shared point are short (noisy
    // rows: chunk hulls of a few vertices, bridges many segments away); long
    // ones (dense rows: hundreds of vertices a chunk) have their bridge close
    // to the shared point, which the walk reaches in a step or two.
    const bool shortseg = ((int)dA.h - (int)dA.l) + ((int)dB.h - (int)dB.l) + 2 <= kBW;
    if (win && G == kWave && shortseg && window_bridge<T>(X, j0, la, jB, sB1, g, win, al, be)) {
        r.newA = al.s - j0 + 1;
        r.alk = al.k;
        r.bs = be.s;
        r.nBk = sB1 - be.s + 1;
        r.bek = be.k;
        return r;
    }
    const bool ok = walk(kWindowSteps, 1 << 30);
    if (!ok) {
        int as = 0, ak = 0, bs = 0, bk = 0;
        if (g == 0) {
            VR a2, b2;
            bisect_bridge<T>(X, j0, la, jB, sB1, a2, b2);
            as = a2.s;
            ak = a2.k;
            bs = b2.s;
            bk = b2.k;
        }
        al = VR{__shfl(as, gb, kWave), __shfl(ak, gb, kWave)};
        be = VR{__shfl(bs, gb, kWave), __shfl(bk, gb, kWave)};
    }
    r.newA = al.s - j0 + 1;
    r.alk = al.k;
    r.bs = be.s;
    r.nBk = sB1 - be.s + 1;
    r.bek = be.k;
    return r;
}

// Rewrites every slot of the merged lists of one level into Dn (one thread per
// slot), and the node lengths in NC.
__device__ inline void rewrite_level(const Desc* Dc, Desc* Dn, int* NC, const MRec* MR, int m, int h, int nm) {
    for (int j = threadIdx.x; j < m; j += blockDim.x) {
        const int k = j / (2 * h);
        if (k < nm) {
            const int j0 = k * 2 * h;
            const MRec r = MR[k];
            const int pos = j - j0;
            if (pos < r.newA) {
                Desc d = Dc[j0 + pos];
                if (pos == r.newA - 1) d.h = (unsigned short)r.alk;
                Dn[j] = d;
            } else if (pos < r.newA + r.nBk) {
                Desc d = Dc[r.bs + pos - r.newA];
                if (pos == r.newA) d.l = (unsigned short)r.bek;
                Dn[j] = d;
            }
            if (pos == 0) NC[j0] = r.newA + r.nBk;
        } else {
            Dn[j] = Dc[j];
        }
    }
}

__device__ inline HullView row_view(const MergeArgs& a, int64_t row) {
    const int64_t base = row * a.m;
    HullView H = a.H0;
    H.nv += base;
    H.tot += base;
    H.mask += base * kMaskWords;
    H.pre += base * kMaskWords;
    H.gs += base * kGroups;
    H.vx += base * kVMax;
    H.vi += base * kVMax;
    return H;
}

constexpr int kMergeThreads = 512;

// Lower levels of the merge tree: one workgroup per subtree of kSub chunks,
// in coordinates relative to the subtree's first chunk.  Writes the
// subtree's hull as a list of at most kSub segments.
template <typename T>
__global__ __launch_bounds__(kMergeThreads) void k_merge_sub(MergeArgs a) {
    extern __shared__ __align__(32) char smem[];
    BWin* wins = (BWin*)smem;  // one window per wave
    __shared__ Desc D0[kSub], D1[kSub];
    __shared__ int NC[kSub], nvl[kSub];
    __shared__ MRec MR[kSub / 2];
    __shared__ double4 stl[kSub];
    __shared__ int sflag;
    const int64_t row = blockIdx.x / a.nsub;
    const int sub = (int)(blockIdx.x % a.nsub);
    const int m = (int)a.m;
    const int c0 = sub * kSub, ms = min(kSub, m - c0);
    const int64_t base = row * a.m;
    const int tid = threadIdx.x;
    if (tid == 0) sflag = 0;
    __syncthreads();
    if (tid < ms && a.cflag[base + c0 + tid]) atomicOr(&sflag, 1);
    __syncthreads();
    if (sflag) return;  // a NaN or a bad weight: k_merge_top writes the row's records
    HullView H = row_view(a, row);
    H.y = (const char*)a.y + row * a.n * (int64_t)sizeof(T);
    H.w = a.w ? (const void*)((const char*)a.w + row * a.n * (int64_t)sizeof(T)) : nullptr;
    if (tid < kWave) {
        double4 v = (tid < ms) ? H.tot[c0 + tid] : make_double4(0.0, 0.0, 0.0, 0.0);
        v = wave_scan_incl(v, [](double4 p, double4 q) { return dd4_add(p, q); });
        const double4 ex = wave_shift_up1(v);
        if (tid < ms) {
            const int nv = H.nv[c0 + tid];
            stl[tid] = ex;
            nvl[tid] = nv;
            Desc dsc;
            dsc.c = c0 + tid;
            dsc.l = 0;
            dsc.h = (unsigned short)(nv - 1);
            D0[tid] = dsc;
            NC[tid] = 1;
        }
    }
    __syncthreads();
    MCtx X;
    X.st = stl;
    X.st_off = c0;
    X.nvc = nvl;
    X.nv_off = c0;
    X.H = H;
    Desc* Dc = D0;
    Desc* Dn = D1;
    const int nwv = blockDim.x / kWave, wid = tid / kWave, g = lane_id();
    for (int h = 1; h < ms; h <<= 1) {
        const int nm = (ms - h + 2 * h - 1) / (2 * h);
        X.D = Dc;
        // one wave per merge, or groups of 16 or 32 lanes when the level has
        // more merges than waves (the lower levels: several merges of a wave
        // then run side by side; their bridges lie within a few group steps
        // of the shared point, and a wave's merges would otherwise run in
        // turn); the LDS windows need a whole wave
        int G = kWave;
        while (G > 16 && (kWave / G) * nwv < nm) G >>= 1;
        const int per = kWave / G, grp = g / G, gl = g % G;
        for (int k0 = wid * per; k0 < nm; k0 += nwv * per) {
            const int k = k0 + grp;
            if (k < nm) {
                const int j0 = k * 2 * h;
                const MRec r =
                    find_merge<T>(X, j0, j0 + h, NC[j0], NC[j0 + h], gl, G, G == kWave ? wins + wid : nullptr);
                if (gl == 0) MR[k] = r;
            }
        }
        __syncthreads();
        rewrite_level(Dc, Dn, NC, MR, ms, h, nm);
        __syncthreads();
        Desc* t = Dc;
        Dc = Dn;
        Dn = t;
    }
    const int cnt = NC[0];
    for (int i = tid; i < cnt; i += blockDim.x) a.gsd[base + c0 + i] = Dc[i];
    if (tid == 0) a.gsn[row * a.nsub + sub] = cnt;
}

// LDS of the merge windows (one per wave).
constexpr size_t kMergeWinBytes = sizeof(BWin) * (kMergeThreads / kWave);

__host__ __device__ inline size_t merge_top_smem_bytes(int64_t m, int use_lds) {
    const size_t scan = sizeof(double4) * kMergeThreads;
    const size_t mr = sizeof(MRec) * (size_t)(m / (2 * kSub) + 1);
    size_t b = (scan > mr ? scan : mr) + 16;
    if (use_lds) b += (2 * sizeof(Desc) + 2 * sizeof(int)) * (size_t)m;
    return ((b + 15) & ~(size_t)15) + kMergeWinBytes;
}

// Upper levels of the merge tree of one long row: double-double chunk starts
// (exclusive scan of the chunk totals, Sec. 3.3 and App. B), the levels above
// the subtrees, then per-chunk records of the root list (Sec. 3.4).
template <typename T>
__global__ __launch_bounds__(kMergeThreads) void k_merge_top(MergeArgs a) {
    extern __shared__ __align__(32) char smem[];
    const int64_t row = blockIdx.x;
    const int m = (int)a.m;
    const int tid = threadIdx.x;
    const int NT = blockDim.x;
    const int64_t base = row * a.m;
    char* p = smem;
    double4* sbuf = (double4*)p;  // the scan's partial sums, then the merge records
    MRec* MR = (MRec*)p;
    {
        const size_t scan = sizeof(double4) * kMergeThreads;
        const size_t mr = sizeof(MRec) * (size_t)(m / (2 * kSub) + 1);
        p += (scan > mr ? scan : mr);
    }
    int* sflag = (int*)p;
    p += 16;
    HullView H = row_view(a, row);
    H.y = (const char*)a.y + row * a.n * (int64_t)sizeof(T);
    H.w = a.w ? (const void*)((const char*)a.w + row * a.n * (int64_t)sizeof(T)) : nullptr;
    Desc *Dc, *Dn;
    int *NC, *nvl;
    if (a.use_lds) {
        Dc = (Desc*)p;
        p += sizeof(Desc) * (size_t)m;
        Dn = (Desc*)p;
        p += sizeof(Desc) * (size_t)m;
        NC = (int*)p;
        p += sizeof(int) * (size_t)m;
        nvl = (int*)p;
    } else {
        Dc = a.gd0 + base;
        Dn = a.gd1 + base;
        NC = a.gnc + base;
        MR = a.gmr + base;
        nvl = nullptr;
    }
    Rec* rec = a.rec + base;
    BWin* wins = (BWin*)(smem + merge_top_smem_bytes(m, a.use_lds) - kMergeWinBytes);

    // 1. row flag: any chunk with a NaN / infinite input or a bad weight
    if (tid == 0) sflag[0] = 0;
    __syncthreads();
    int f = 0;
    for (int c = tid; c < m; c += NT) f |= a.cflag[base + c];
    if (f) atomicOr(sflag, f);
    __syncthreads();
    f = sflag[0];
    if (f) {
        for (int c = tid; c < m; c += NT) {
            Rec r{};
            r.mode = 2;
            rec[c] = r;
        }
        if (tid == 0) {
            if (a.row_nan) a.row_nan[row] = 1u;
            if ((f & 1) == 0) report_weight_error(a.status, a.epoch);
        }
        return;
    }

    // 2. chunk starts: exclusive double-double scan of the chunk totals
    const int per = (m + NT - 1) / NT;
    const int c0 = min(m, tid * per), c1 = min(m, c0 + per);
    double4 loc = make_double4(0.0, 0.0, 0.0, 0.0);
    for (int c = c0; c < c1; ++c) loc = dd4_add(loc, H.tot[c]);
    // the threads' sums scanned in each wave (DPP), then the waves' totals
    // added in order: one barrier
    const int wv = tid >> 6;
    const double4 inc = wave_scan_incl(loc, [](double4 p, double4 q) { return dd4_add(p, q); });
    if (lane_id() == kWave - 1) sbuf[wv] = inc;
    __syncthreads();
    double4 ex = make_double4(0.0, 0.0, 0.0, 0.0);
    for (int k = 0; k < wv; ++k) ex = dd4_add(ex, sbuf[k]);
    ex = dd4_add(ex, wave_shift_up1(inc));
    for (int c = c0; c < c1; ++c) {
        a.starts[base + c] = ex;
        ex = dd4_add(ex, H.tot[c]);
    }
    // 3. the subtrees' lists, one node per subtree at its first chunk's slot
    for (int c = tid; c < m; c += NT) {
        const int sub = c / kSub;
        const int cnt = a.gsn[row * a.nsub + sub];
        if (c - sub * kSub < cnt) Dc[c] = a.gsd[base + c];
        if (c == sub * kSub) NC[c] = cnt;
        if (nvl) nvl[c] = H.nv[c];
    }
    __threadfence();
    __syncthreads();

    MCtx X;
    X.st = a.starts + base;
    X.st_off = 0;
    X.nvc = nvl ? nvl : H.nv;
    X.nv_off = 0;
    X.H = H;

    // 4. the upper levels, one wave per merge
    const int nw = NT / kWave, wid = tid / kWave, g = lane_id();
    for (int h = kSub; h < m; h <<= 1) {
        const int nm = (m - h + 2 * h - 1) / (2 * h);
        X.D = Dc;
        for (int k = wid; k < nm; k += nw) {
            const int j0 = k * 2 * h;
            const MRec r = find_merge<T>(X, j0, j0 + h, NC[j0], NC[j0 + h], g, kWave, wins + wid);
            if (g == 0) MR[k] = r;
        }
        __threadfence_block();
        __syncthreads();
        rewrite_level(Dc, Dn, NC, MR, m, h, nm);
        __threadfence_block();
        __syncthreads();
        Desc* t = Dc;
        Dc = Dn;
        Dn = t;
    }
    X.D = Dc;

    // 5. per-chunk records of the root list
    const int K = NC[0];
    double* so = a.gso + base;
    for (int k = tid; k < K - 1; k += NT) {
        const Desc d0 = Dc[k], d1 = Dc[k + 1];
        so[k] = slopeD(ptd<T>(X, d0.c, d0.h), ptd<T>(X, d1.c, d1.l));
    }
    __threadfence();
    __syncthreads();
    for (int c = tid; c < m; c += NT) {
        // last root segment whose chunk is <= c
        int lo = 0, hi = K;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (Dc[mid].c <= c)
                lo = mid;
            else
                hi = mid;
        }
        const Desc d = Dc[lo];
        Rec r{};
        if (d.c == c) {
            const int nv = X.nvc[c];
            r.mode = 0;
            r.lo = vtx_n<T>(H, c, d.l, nv).p;
            r.hi = vtx_n<T>(H, c, d.h, nv).p;
            r.sin = (lo > 0) ? so[lo - 1] : 0.0;
            r.sout = (lo < K - 1) ? so[lo] : 0.0;
        } else {
            r.mode = 1;
            r.lo = 0;
            r.hi = 0;
            r.sin = 0.0;
            r.sout = so[lo];
        }
        rec[c] = r;
    }
    if (tid == 0 && a.row_nan) a.row_nan[row] = 0u;
}

// ---------------------------------------------------------------------------
// fix-up of the elements outside each chunk's surviving segment
// ---------------------------------------------------------------------------
struct FixArgs {
    void* fit;
    int64_t n, m, words;
    int increasing;
    double lo, hi;
    const Rec* rec;
    uint64_t* start_bits;
    uint64_t* clip_bits;
};

template <typename T>
__global__ __launch_bounds__(256) void k_fixup(FixArgs a) {
    const int64_t bid = blockIdx.x;
    const int64_t row = bid / a.m, c = bid % a.m;
    const int64_t e0 = c * kChunk;
    const int N = (int)((a.n - e0) < kChunk ? (a.n - e0) : kChunk);
    T* out = (T*)a.fit + row * a.n + e0;
    uint64_t* sb = a.start_bits ? a.start_bits + row * a.words + e0 / 64 : nullptr;
    uint64_t* cb = a.clip_bits ? a.clip_bits + row * a.words + e0 / 64 : nullptr;
    const Rec r = a.rec[bid];
    const int nwords = (N + 63) / 64;
    if (r.mode == 2) {
        for (int i = threadIdx.x; i < N; i += blockDim.x) out[i] = (T)NAN;
        if (sb)
            for (int q = threadIdx.x; q < nwords; q += blockDim.x) {
                sb[q] = 0ull;
                cb[q] = 0ull;
            }
        return;
    }
    bool cin = false, cout = false;
    const double vin = finish(r.sin, a.increasing, a.lo, a.hi, cin);
    const double vout = finish(r.sout, a.increasing, a.lo, a.hi, cout);
    const int lo = (r.mode == 0) ? r.lo : 0;
    const int hi = (r.mode == 0) ? r.hi : 0;
    for (int i = threadIdx.x; i < lo; i += blockDim.x) out[i] = (T)vin;
    for (int i = hi + threadIdx.x; i < N; i += blockDim.x) out[i] = (T)vout;
    if (sb) {
        for (int q = threadIdx.x; q < nwords; q += blockDim.x) {
            const int b0 = q * 64;
            const int cnt = min(64, N - b0);
            const uint64_t valid = (cnt >= 64) ? ~0ull : ((1ull << cnt) - 1ull);
            // elements e < lo of this word, and e >= hi
            const uint64_t mIn = (lo <= b0) ? 0ull : ((lo - b0 >= 64) ? ~0ull : ((1ull << (lo - b0)) - 1ull));
            const uint64_t mOut = (hi <= b0) ? ~0ull : ((hi - b0 >= 64) ? 0ull : ~((1ull << (hi - b0)) - 1ull));
            uint64_t s = sb[q], cl = cb[q];
            if (r.mode == 0) {
                // keep block starts only at the segment's vertices lo..hi
                const uint64_t keep = ~(mIn | mOut) | ((hi >= b0 && hi < b0 + 64) ? (1ull << (hi - b0)) : 0ull);
                s &= keep;
            } else {
                s = 0ull;
            }
            const uint64_t ins = mIn & valid, outs = mOut & valid;
            cl = (cl & ~(ins | outs)) | (cin ? ins : 0ull) | (cout ? outs : 0ull);
            sb[q] = s & valid;
            cb[q] = cl & valid;
        }
    }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------

// Lanes and elements per lane for a row of N <= kSingleMax elements: a single
// wave for short rows, else 16 elements per lane and ceil(N/16) lanes rounded
// up to whole waves (at most 384).
static void row_shape(int N, bool f32, int& K, int& nl) {
    if (N <= 128) {
        K = 2;
        nl = 64;
    } else if (N <= 256) {
        K = 4;
        nl = 64;
    } else if (N <= kOneWaveMax) {
        K = 8;
        nl = 64;
    } else if (N <= 4096) {
        K = 16;
        nl = ((N + 15) / 16 + 63) / 64 * 64;  // at most four waves
    } else if (f32 && N <= 5120) {
        K = 20;  // four waves (float64 rows would spill at this K)
        nl = 256;
    } else {
        K = 12;
        nl = ((N + 11) / 12 + 63) / 64 * 64;  // five to eight waves
    }
}

// Vertices the LDS list of a row holds.  A CU runs at most four waves per
// SIMD at these kernels' register budget.  A workgroup of W <= 4 waves puts
// one wave on each of W SIMDs, so 16 / W of them share a CU; one of W > 4
// waves puts ceil(W/4) of them on its busiest SIMD, so 4 / ceil(W/4) share
// it.  The list takes what their share of the 160 KiB leaves (at least a
// quarter of the points).  Rows that need more go to k_row_ovf.
static int row_list_cap(int N, int nl, int K, bool ls2, int stage_bytes = 0) {
    const int W = nl / 64;
    const int per_simd = (W + 3) / 4;
    const long wgs = (W <= 4) ? 16 / W : (per_simd >= 4 ? 1 : 4 / per_simd);
    const long target = kLdsBytes / wgs - 512;
    const long fixed = (long)tile_smem_bytes(nl, 0, K, ls2);
    const long room = (target - fixed) / 18;
    long cap = room > N / 4 ? room : N / 4;
    cap = cap < N ? cap : N;
    // a list of 16-byte entries that holds the staged inputs of every wave
    const long stage = (stage_bytes + 15) / 16 - 1;
    return (int)(cap > stage ? cap : stage);
}

template <typename T, int K>
static hipError_t launch_row(const FitLaunch& a, RowArgs r, int nl) {
    constexpr bool ls2 = sizeof(T) == 4;  // float32 tiles: plain lane starts
    constexpr bool SO = always_staged<T, K>();
    r.cap = row_list_cap((int)a.n, nl, K, ls2, SO ? nl * K * (int)sizeof(T) : 0);
    const size_t smem = tile_smem_bytes(nl, r.cap, K, ls2);
    static size_t seen[kMaxDevices] = {};
    (void)ensure_lds((const void*)k_row_fit<T, K>, smem, seen);
    r.ovf = a.ws + a.L.ovf;
    r.ovf_stride = (int64_t)a.L.ovf_stride;
    // stage the inputs through LDS when a lane's K elements are not whole
    // 64-byte segments and the list has room for every wave's span
    r.stage = SO || (((K * (int)sizeof(T)) % 64 != 0) && ((K * (int)sizeof(T)) % 16 == 0) &&
                     ((size_t)nl * K * sizeof(T) <= tile_list_len(nl, r.cap, K) * 16));
    // rows of several waves keep an overflowing list in the workspace within
    // k_row_fit (row_exact); one-wave rows leave it to k_row_ovf
    const bool may_overflow = r.cap < a.n && K < 12;
    r.ovf_row = may_overflow ? (int*)(a.ws + a.L.ovfrow) : nullptr;
    hipLaunchKernelGGL((k_row_fit<T, K>), dim3((unsigned)a.rows), dim3(nl), smem, a.stream, r);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !may_overflow) return e;
    // the flagged rows again: one-wave rows keep the whole list in LDS (a
    // dozen rows still share a CU), wider rows keep it in the workspace
    RowArgs o = r;
    o.cap = nl == 64 ? (int)a.n : 0;
    const size_t osmem = tile_smem_bytes(nl, o.cap, K);
    static size_t oseen[kMaxDevices] = {};
    (void)ensure_lds((const void*)k_row_ovf<T, K>, osmem, oseen);
    hipLaunchKernelGGL((k_row_ovf<T, K>), dim3((unsigned)a.rows), dim3(nl), osmem, a.stream, o);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_fit_t(const FitLaunch& a) {
    unsigned long long* status = (unsigned long long*)(a.ws + a.L.status);
    const RowArgs r{a.y, a.w, a.fit, a.n, a.increasing, a.lo, a.hi, a.start_bits, a.clip_bits, a.row_nan,
                    a.words, status, a.epoch, 0, nullptr, 0, nullptr, 0};
    if (a.n <= kLaneRow) {
        const unsigned grid = (unsigned)((a.rows + 255) / 256);
        if (a.n <= 16)
            hipLaunchKernelGGL((k_rows_lane<T, 16>), dim3(grid), dim3(256), 0, a.stream, r, (int64_t)a.rows);
        else
            hipLaunchKernelGGL((k_rows_lane<T, 32>), dim3(grid), dim3(256), 0, a.stream, r, (int64_t)a.rows);
        return hipGetLastError();
    }
    if (a.n <= kPackedMax) {
        const PackedLaunch p{a.y,         a.w,       a.fit,   a.rows,  a.n,
                             a.increasing, sizeof(T) == 4 ? 0 : 1, a.lo, a.hi,
                             a.start_bits, a.clip_bits, a.row_nan, a.words, status,
                             a.epoch,     (int*)(a.ws + a.L.ovf), a.stream};
        return launch_rows_packed(p);
    }
    if (a.n <= kSingleMax) {
        int K, nl;
        row_shape((int)a.n, sizeof(T) == 4, K, nl);
        switch (K) {
            case 2:
                return launch_row<T, 2>(a, r, nl);
            case 4:
                return launch_row<T, 4>(a, r, nl);
            case 8:
                return launch_row<T, 8>(a, r, nl);
            case 12:
                return launch_row<T, 12>(a, r, nl);
            case 20:
                if constexpr (sizeof(T) == 4) return launch_row<T, 20>(a, r, nl);
                return hipErrorInvalidValue;  // row_shape gives float64 rows no K = 20
            default:
                return launch_row<T, 16>(a, r, nl);
        }
    }
    const int64_t m = a.L.m;
    ChunkArgs ca;
    ca.r = r;
    ca.m = m;
    ca.tot = (double4*)(a.ws + a.L.tot);
    ca.nv = (int*)(a.ws + a.L.nv);
    ca.cflag = (int*)(a.ws + a.L.cflag);
    ca.cmask = (uint64_t*)(a.ws + a.L.cmask);
    ca.cpre = (int*)(a.ws + a.L.cpre);
    ca.cgs = (double4*)(a.ws + a.L.cgs);
    ca.cvx = (double4*)(a.ws + a.L.cvx);
    ca.cvi = (int*)(a.ws + a.L.cvi);
    ca.cover = (int*)(a.ws + a.L.cover);
    ca.clist = (int*)(a.ws + a.L.clist);
    ca.cctr = (unsigned long long*)(a.ws + a.L.cctr);
    ca.nchunks = a.rows * m;
    {
        const size_t smem1 = tile_smem_bytes(kChunkLanes, kChunk, kLaneK);
        const size_t smem0 = tile_smem_bytes(kChunkLanes, kChunkCap, kLaneK);
        static size_t seen0[kMaxDevices] = {}, seen1[kMaxDevices] = {};
        (void)ensure_lds((const void*)k_chunk_hull<T>, smem0, seen0);
        (void)ensure_lds((const void*)k_chunk_cover<T>, smem1, seen1);
        const int64_t chunks = a.rows * m;
        ca.cap = kChunkCap;
        ca.early = (chunks >= 16 * (int64_t)num_cus()) ? 1 : 0;
        hipLaunchKernelGGL(k_chunk_hull<T>, dim3((unsigned)chunks), dim3(kChunkLanes), smem0, a.stream, ca);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        // two workgroups per CU (the full list) run at a time: one such
        // generation of workgroups, each taking at most one listed chunk
        // while there are at most that many
        ca.cap = kChunk;
        const int64_t cover_grid = std::min<int64_t>(chunks, 2 * (int64_t)num_cus());
        hipLaunchKernelGGL(k_chunk_cover<T>, dim3((unsigned)cover_grid), dim3(kChunkLanes), smem1, a.stream, ca);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    MergeArgs ma;
    ma.y = a.y;
    ma.w = a.w;
    ma.n = a.n;
    ma.m = m;
    ma.nsub = (int)((m + kSub - 1) / kSub);
    ma.negate = !a.increasing;
    ma.H0 = HullView{ca.nv, ca.tot, ca.cmask, ca.cpre, ca.cgs, ca.cvx, ca.cvi, nullptr, nullptr, !a.increasing, a.n};
    ma.cflag = ca.cflag;
    ma.starts = (double4*)(a.ws + a.L.starts);
    ma.gsd = (Desc*)(a.ws + a.L.gsd);
    ma.gsn = (int*)(a.ws + a.L.gsn);
    ma.gd0 = (Desc*)(a.ws + a.L.desc0);
    ma.gd1 = (Desc*)(a.ws + a.L.desc1);
    ma.gnc = (int*)(a.ws + a.L.nc);
    ma.gmr = (MRec*)(a.ws + a.L.mrec);
    ma.gnv = nullptr;
    ma.gso = (double*)(a.ws + a.L.so);
    ma.rec = (Rec*)(a.ws + a.L.rec);
    ma.row_nan = a.row_nan;
    ma.status = status;
    ma.epoch = a.epoch;
    ma.use_lds = (m <= kMergeLdsChunks) ? 1 : 0;
    {
        static size_t seen[kMaxDevices] = {};
        (void)ensure_lds((const void*)k_merge_sub<T>, kMergeWinBytes, seen);
    }
    // Eight waves per subtree finish its levels in fewer steps, but only one
    // such workgroup fits on a CU (registers); with more subtrees than CUs,
    // workgroups of four waves (three to a CU) run them in one generation.
    const int64_t subtrees = a.rows * ma.nsub;
    const int sub_threads = subtrees > 256 ? kMergeThreads / 2 : kMergeThreads;
    hipLaunchKernelGGL(k_merge_sub<T>, dim3((unsigned)subtrees), dim3(sub_threads),
                       sizeof(BWin) * (sub_threads / kWave), a.stream, ma);
    {
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    {
        static size_t seen[kMaxDevices] = {};
        (void)ensure_lds((const void*)k_merge_top<T>, merge_top_smem_bytes(kMergeLdsChunks, 1), seen);
        hipLaunchKernelGGL(k_merge_top<T>, dim3((unsigned)a.rows), dim3(kMergeThreads),
                           merge_top_smem_bytes(m, ma.use_lds), a.stream, ma);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    FixArgs fa{a.fit, a.n, m, a.words, a.increasing, a.lo, a.hi, ma.rec, a.start_bits, a.clip_bits};
    hipLaunchKernelGGL(k_fixup<T>, dim3((unsigned)(a.rows * m)), dim3(256), 0, a.stream, fa);
    return hipGetLastError();
}

hipError_t launch_fit(const FitLaunch& a) {
    if (a.dtype == 0) return launch_fit_t<float>(a);
    return launch_fit_t<double>(a);
}

}  // namespace iso
