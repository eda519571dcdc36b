// One workgroup builds the lower convex hull of the cumulative sum diagram of
// N consecutive elements (a "tile") and the slope of the hull edge above every
// element (page "Merge Hulls Without Copying Vertices: GPU Isotonic
// Regression", Sec. 2.1 Eq. (2)-(3), Sec. 3.1-3.2 and 3.4).
//
// Work split (gfx950, wave64):
//   1. lane hull each lane (thread) owns K consecutive elements, i.e. the
//                points lK+1 .. lK+K, reads them from global memory (through
//                LDS when K elements are not whole 64-byte segments), forms
//                their float64 prefix sums of (w, w*y) relative to the lane's
//                start, and builds its hull by gift wrapping with compile-time
//                register indices (the first page's lane hull, Sec. 3.1);
//   2. starts    an exclusive DPP scan of the lane totals gives each lane's
//                start relative to the tile's first point (double-double for
//                float64 data);
//   3. merges    the lane-hull vertices are compacted once into a sorted list
//                in LDS; a lane's node is an index range of it.  Rounds inside
//                each wave merge neighbouring nodes, a group of G lanes per
//                merge finding the bridge (Sec. 4, Lemma 4.2 and the walk
//                after it) and moving the right node's surviving suffix
//                behind the left node's surviving prefix; then a tree over
//                the waves' nodes.  Tiles whose candidates are few first try
//                an output-sensitive finish instead (tile_wrap): every wave
//                gift-wraps its candidates, one step per hull edge, and the
//                waves' vertices are reduced to the tile's hull by a parallel
//                vertex test; the rounds run only if a wrap exceeds its cap.
//                Candidates may be any superset of the hull's vertices: the
//                lane hulls' vertices, or for float32 rows of several waves
//                those of the lanes' half hulls below the tile's chord.
//                Float32 rows of several waves, and the chunks of long rows
//                with few candidates, skip the lane hulls and the rounds: the
//                points under the hull of the lane ends are listed and their
//                hull is found by a workgroup QuickHull (tile_quickhull on
//                absolute float64 points, list_quickhull on double-double
//                coordinates);
//   4. expand    every lane computes the slope of the hull edge above each of
//                its elements (Sec. 3.4: the edge from the last vertex at or
//                before the element's left point to the first vertex at or
//                after its right point) and stores the fit.
//
// Coordinates.  For float64 data a point is its lane's start (double-double)
// plus a local float64 sum of at most K terms, and differences are formed part
// by part (the first page's Appendix B, "Merge levels").  For float32 data the
// products w*y are exact in float64 and a float64 coordinate relative to the
// tile's first point is accurate far beyond float32 output, so points carry
// one float64 pair and differences are direct.  A turn of zero counts as
// non-convex, so collinear middle points are dropped (Sec. 2.1 and Sec. 4).
//
// Point p of the tile (p = 0..N) is P_p; element i lies between P_i and
// P_{i+1}.  Point 0 is always a vertex and belongs to no lane; point p >= 1
// belongs to lane (p-1)/K as its local point p - lK, and is bit p-1-lK of that
// lane's mask.
#pragma once

#include "iso_device.hpp"

namespace iso {

// LDS of a tile.  The workgroup has nl threads, a whole number of waves; lane
// l holds the elements lK .. lK+K-1 that are < N <= cap (lanes past the end
// hold none).
struct Tile {
    unsigned short* V;  // the current vertices, sorted (point indices): the tile's list, or one per wave
    double2* VXY;       // their coordinates (local to the point's lane, or absolute)
    double4* LS;        // [nl + 1] lane starts (double-double pairs), LS[nl] = tile total; plain
                        // (x, y) double pairs instead when ls2 (tiles whose starts are not double-double)
    uint64_t* M;        // [nl] final lane vertex masks
    uint64_t* CM;       // [nl] lane clip masks
    int* I;             // [nl] index in V of each lane's first vertex
    int2* MR;           // [nl / 2 + 1] bridge (alpha, beta) points of the merges of a round
    int* R;             // wrap results: [nw * kWrapWave] per wave, then (nw > 1) the tile's candidates and hull
    int* W;             // [32] per-wave scratch
    int* flag;          // [4]
    int nl;             // lanes (= threads of the workgroup)
    int N;              // elements
    bool ls2;           // LS holds double2 entries
};

// Step caps of the output-sensitive finish (tile_wrap): hull vertices a wave
// may find among its lane hulls' vertices, and the tile among the waves'.
constexpr int kWrapWave = 32;
constexpr int kWrapTile = 128;
__host__ __device__ constexpr size_t tile_wrap_ints(int nl) {
    const int nw = nl / 64;
    return (size_t)nw * kWrapWave + (nw > 1 ? (size_t)(4 + nw * kWrapWave + kWrapTile) : 0);
}

// List capacity: the tile's vertices plus point 0.
__host__ __device__ constexpr size_t tile_list_len(int nl, int cap, int K) {
    (void)nl;
    (void)K;
    return (size_t)cap + 1;
}

// The wrap's results share the clip-mask array when they fit in it (the two
// are never in use at once).
__host__ __device__ constexpr size_t tile_wrap_own_bytes(int nl) {
    const size_t b = 4 * tile_wrap_ints(nl);
    return b <= 8 * (size_t)nl ? 0 : ((b + 15) & ~(size_t)15);
}

// ls2: lane starts as plain double pairs (16 bytes a lane instead of 32).
__host__ __device__ constexpr size_t tile_smem_bytes(int nl, int cap, int K, bool ls2 = false) {
    const size_t n = tile_list_len(nl, cap, K);
    const size_t v = (2 * n + 15) & ~(size_t)15;
    return v + 16 * n + (ls2 ? 16 : 32) * (size_t)(nl + 1) + 16 * (size_t)nl + 4 * (size_t)nl +
           8 * (size_t)(nl / 2 + 1) + 128 + 16 + 128 + tile_wrap_own_bytes(nl);
}

__device__ inline Tile tile_carve(char* base, int nl, int cap, int K, int N, bool ls2 = false) {
    Tile t;
    char* p = base;
    const size_t n = tile_list_len(nl, cap, K);
    t.VXY = (double2*)p;
    p += 16 * n;
    t.LS = (double4*)p;
    t.ls2 = ls2;
    p += (ls2 ? 16 : 32) * (size_t)(nl + 1);
    t.M = (uint64_t*)p;
    p += 8 * (size_t)nl;
    t.CM = (uint64_t*)p;
    p += 8 * (size_t)nl;
    t.MR = (int2*)p;
    p += 8 * (size_t)(nl / 2 + 1);
    t.I = (int*)p;
    p += 4 * (size_t)nl;
    t.W = (int*)p;
    p += 128;
    t.flag = (int*)p;
    p += 16;
    if (tile_wrap_own_bytes(nl)) {
        t.R = (int*)p;
        p += tile_wrap_own_bytes(nl);
    } else {
        t.R = (int*)t.CM;
    }
    t.V = (unsigned short*)p;
    t.nl = nl;
    t.N = N;
    return t;
}

template <int K>
__device__ __forceinline__ int lane_of(int p) {
    return p <= 0 ? 0 : (p - 1) / K;
}

// Coordinates of list entries i, j: P_j - P_i.
template <int K, bool ABS>
__device__ __forceinline__ double2 vdiff(const Tile& t, int i, int j) {
    const double2 A = t.VXY[i], B = t.VXY[j];
    if (ABS) return sub2(B, A);
    const int li = lane_of<K>(t.V[i]), lj = lane_of<K>(t.V[j]);
    if (li == lj) return sub2(B, A);
    const double2 d = dd4_diff(t.LS[li], t.LS[lj]);
    return make_double2(d.x + (B.x - A.x), d.y + (B.y - A.y));
}

template <int K, bool ABS>
__device__ __forceinline__ double vturn(const Tile& t, int i, int j, int k) {
    return cross2(vdiff<K, ABS>(t, i, j), vdiff<K, ABS>(t, i, k));
}

// ---------------------------------------------------------------------------
// 1. lane hull, in registers
// Gift wrapping over the lane's points (xs, ys)[0..cnt) (point j+1 of the
// lane at index j; the lane's start is the origin).  From point j the next
// vertex is the point k of least slope (the farthest one on ties); the
// pointers are kept as offsets nx - j - 1, PB bits each, PE per word.
template <int K>
struct GiftWrap {
    static constexpr int PB = (K <= 16) ? 4 : 5, PE = 64 / PB, PW = (K + PE - 1) / PE;
    static_assert(PW <= 3, "next-vertex offsets are packed in at most three words");
};

// Pointers of the points j in [J0, J1) over the candidates k <= KMAX.
template <int K, int J0, int J1, int KMAX>
__device__ __forceinline__ void gw_ptrs(const double (&xs)[K], const double (&ys)[K], int cnt, uint64_t (&nxp)[3]) {
    constexpr int PB = GiftWrap<K>::PB, PE = GiftWrap<K>::PE;
#pragma unroll
    for (int j = J0; j < J1; ++j) {
        const double xj = j ? xs[j - 1] : 0.0, yj = j ? ys[j - 1] : 0.0;
        double bdx = xs[j] - xj, bdy = ys[j] - yj;
        int bk = 0;
#pragma unroll
        for (int k = j + 2; k <= KMAX; ++k) {
            const double dx = xs[k - 1] - xj, dy = ys[k - 1] - yj;
            const bool take = (k <= cnt) && (dy * bdx <= bdy * dx);
            bdx = take ? dx : bdx;
            bdy = take ? dy : bdy;
            bk = take ? (k - j - 1) : bk;
        }
        const uint64_t field = ((1ull << PB) - 1ull) << (PB * (j % PE));
        nxp[j / PE] = (nxp[j / PE] & ~field) | ((uint64_t)bk << (PB * (j % PE)));
    }
}

// The chain of pointers from point v0 until it reaches min(vend, cnt): the
// mask of the points it visits (bit j for point j+1).
template <int K>
__device__ __forceinline__ uint64_t gw_walk(const uint64_t (&nxp)[3], int v0, int vend, int cnt) {
    constexpr int PB = GiftWrap<K>::PB, PE = GiftWrap<K>::PE, PW = GiftWrap<K>::PW;
    const int end = min(vend, cnt);
    uint64_t mask = 0ull;
    int v = v0;
    for (int s = 0; s < K && v < end; ++s) {
        uint64_t word = nxp[0];
#pragma unroll
        for (int q = 1; q < PW; ++q) word = v >= q * PE ? nxp[q] : word;
        v += 1 + (int)((word >> (PB * (v % PE))) & ((1ull << PB) - 1ull));
        mask |= 1ull << (v - 1);
    }
    return mask;
}

// The lane's hull: the mask of its vertices (bit j for point j+1).  All
// K(K+1)/2 pairs are compared with compile-time indices: no divergence and no
// indexed access to the lane's registers.
template <int K>
__device__ __forceinline__ uint64_t lane_gift_wrap(const double (&xs)[K], const double (&ys)[K], int cnt) {
    uint64_t nxp[3] = {0ull, 0ull, 0ull};
    gw_ptrs<K, 0, K, K>(xs, ys, cnt, nxp);
    return gw_walk<K>(nxp, 0, K, cnt);
}

// The hulls of P consecutive parts of the lane (points 0..K/P, K/P..2K/P, ...),
// a P-th of the comparisons or less: their vertices include every vertex of
// the lane's hull (subset lemma), so they serve as candidates where a superset
// will do.  nxp keeps the pointers.
template <int K, int P>
__device__ __forceinline__ uint64_t gw_parts(const double (&xs)[K], const double (&ys)[K], int cnt,
                                             uint64_t (&nxp)[3]) {
    static_assert(K % P == 0, "equal parts");
    constexpr int S = K / P;
    nxp[0] = nxp[1] = nxp[2] = 0ull;
    uint64_t m = 0ull;
    gw_ptrs<K, 0, S, S>(xs, ys, cnt, nxp);
    m |= gw_walk<K>(nxp, 0, S, cnt);
    if constexpr (P > 1) {
        gw_ptrs<K, S, 2 * S, 2 * S>(xs, ys, cnt, nxp);
        m |= gw_walk<K>(nxp, S, 2 * S, cnt);
    }
    if constexpr (P > 2) {
        gw_ptrs<K, 2 * S, 3 * S, 3 * S>(xs, ys, cnt, nxp);
        m |= gw_walk<K>(nxp, 2 * S, 3 * S, cnt);
    }
    if constexpr (P > 3) {
        gw_ptrs<K, 3 * S, 4 * S, 4 * S>(xs, ys, cnt, nxp);
        m |= gw_walk<K>(nxp, 3 * S, 4 * S, cnt);
    }
    static_assert(P <= 4, "at most four parts");
    return m;
}

// ---------------------------------------------------------------------------

// The wave's K * 64 elements of one input through LDS, for lanes whose K
// elements are not a whole number of 64-byte segments (per-lane 16-byte loads
// then touch each segment from several lanes and instructions, and HBM serves
// some segments more than once): consecutive lanes read consecutive 16-byte
// pieces (one contiguous KiB per load instruction) into the wave's stage, and
// each lane then reads its own K values.  avail = elements of the span that
// exist; the rest read as 0.
//
// stage_fetch is the global half (a 16-byte aligned span): the lane's pieces
// into registers, every load issued before any is used, so that a caller
// fetching two inputs waits for memory once; stage_put writes them to the
// stage.
template <typename T, int K>
struct StagePieces {
    static constexpr int VW = 16 / (int)sizeof(T);
    static constexpr int NQ = K / VW;  // 16-byte pieces per lane
    static_assert(K % VW == 0, "a lane's span is a whole number of 16-byte pieces");
    uint4 v[NQ];
};

template <typename T, int K>
__device__ __forceinline__ void stage_fetch(const T* __restrict__ base, int avail, StagePieces<T, K>& P) {
    constexpr int VW = StagePieces<T, K>::VW, NQ = StagePieces<T, K>::NQ;
    const int lane = lane_id();
    if (avail >= K * kWave) {  // uniform: the whole span exists
#pragma unroll
        for (int q = 0; q < NQ; ++q) P.v[q] = *(const uint4*)(base + (q * kWave + lane) * VW);
    } else {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int e = (q * kWave + lane) * VW;
            if (e + VW <= avail) {
                P.v[q] = *(const uint4*)(base + e);
            } else {
                T tv[VW];
#pragma unroll
                for (int r = 0; r < VW; ++r) tv[r] = (e + r < avail) ? base[e + r] : (T)0;
                P.v[q] = *(const uint4*)tv;
            }
        }
    }
}

template <typename T, int K>
__device__ __forceinline__ void stage_put(const StagePieces<T, K>& P, T* stage) {
    constexpr int VW = StagePieces<T, K>::VW, NQ = StagePieces<T, K>::NQ;
    const int lane = lane_id();
#pragma unroll
    for (int q = 0; q < NQ; ++q) *(uint4*)(stage + (q * kWave + lane) * VW) = P.v[q];
}

template <typename T, int K>
__device__ __forceinline__ void stage_wave(const T* __restrict__ base, int avail, T* stage) {
    if ((((uintptr_t)base) & 15) == 0) {
        StagePieces<T, K> P;
        stage_fetch<T, K>(base, avail, P);
        stage_put<T, K>(P, stage);
    } else {
        for (int e = lane_id(); e < K * kWave; e += kWave) stage[e] = (e < avail) ? base[e] : (T)0;
    }
    wave_sync();
}

// The lane's K values from the stage (after stage_put and a wave_sync).
template <typename T, int K>
__device__ __forceinline__ void stage_read(const T* stage, T (&v)[K]) {
    constexpr int VW = 16 / (int)sizeof(T);
    const int lane = lane_id();
#pragma unroll
    for (int q = 0; q < K / VW; ++q) {
        const uint4 u = *(const uint4*)(stage + lane * K + q * VW);
        const T* pu = (const T*)&u;
#pragma unroll
        for (int r = 0; r < VW; ++r) v[q * VW + r] = pu[r];
    }
}

template <typename T, int K>
__device__ __forceinline__ void lane_load_staged(const T* __restrict__ base, int avail, T* stage, T (&v)[K]) {
    static_assert((K * (int)sizeof(T)) % 16 == 0, "a lane's values are read back as 16-byte pieces");
    stage_wave<T, K>(base, avail, stage);
    stage_read<T, K>(stage, v);
    wave_sync();  // every lane has its values before the stage is reused
}

// Loads the lane's elements, forms the local points (xs, ys)[j] = point j+1
// relative to the lane's start, and returns the lane's hull as a mask (bit b
// <-> local point b+1; point 0 is implicit).  f |= 1 for a non-finite input,
// 2 for a weight <= 0.  With a stage (LDS, K * 64 elements for the calling
// wave), the inputs come through lane_load_staged from the wave's span
// starting at y, w with avail elements; otherwise each lane reads its own
// elements at y, w.
//
// The hull is found by gift wrapping: from every local point j the next hull
// vertex is the point k > j of least slope (the farthest one on ties, so
// collinear middle points are dropped), compared by cross-multiplication;
// the hull is the chain of these pointers from point 0.  All K(K+1)/2 pairs
// are compared with compile-time indices: no divergence and no indexed access
// to the lane's registers.
// With nxp, the hulls of the lane's two halves instead: a superset of the
// lane hull's vertices (gw_parts).  Without HULL only the points are formed
// (mask 0): the caller picks its candidates itself (lane_chords).
// STAGED: the caller always passes a stage (the other load paths are left
// out of the code, which keeps the kernel's registers for the points).
template <typename T, int K, bool HULL = true, bool STAGED = false>
__device__ inline uint64_t lane_hull(const T* __restrict__ y, const T* __restrict__ w, int cnt, int negate,
                                     double (&xs)[K], double (&ys)[K], int& f, T* stage = nullptr,
                                     int avail = 0, uint64_t (*nxp)[3] = nullptr) {
    static_assert(K <= 32, "next-vertex offsets are packed in at most three words");
    double X = 0.0, Y = 0.0;
    // float32 inputs take no branches: a product of two floats is exact in
    // float64, so the fused multiply-add rounds as the sum of the product
    // does; a non-finite input leaves a lane total non-finite (infinities and
    // NaN absorb finite terms, opposite infinities give NaN) while finite
    // inputs cannot overflow, so the totals are checked once at the end; the
    // least weight finds a weight <= 0.
    constexpr bool F32 = sizeof(T) == 4;
    const double sg = negate ? -1.0 : 1.0;
    float wmin = INFINITY;
    // The staged path gives zeros past cnt (zero = true), which leave the sums
    // as they are; only the least weight skips them.
    auto take = [&](int j, double yi, double wi, bool zero = false) {
        if constexpr (F32) {
            const bool in = j < cnt;
            if (!zero) {
                wi = in ? wi : 0.0;
                yi = in ? yi : 0.0;
            }
            X += wi;
            Y = fma(wi * sg, yi, Y);
            wmin = fminf(wmin, in ? (float)wi : 1.f);
        } else {
            // no branches either: the flags and sums take selects
            const bool in = j < cnt, fin = isfinite(yi) && isfinite(wi);
            f |= (in && !fin) ? 1 : 0;
            f |= (in && fin && !(wi > 0.0)) ? 2 : 0;
            X += in ? wi : 0.0;
            Y += in ? (wi * sg) * yi : 0.0;
        }
        xs[j] = X;
        ys[j] = Y;
    };
    auto checks = [&]() {
        if constexpr (F32) {
            if (!isfinite(X) || !isfinite(Y)) f |= 1;
            if (!(wmin > 0.f)) f |= 2;
        }
    };
    constexpr int VW = 16 / (int)sizeof(T);
    bool done = false;
    if constexpr ((K * (int)sizeof(T)) % 16 == 0) {
        if (stage) {
            // the weights first, into registers; then y through the stage,
            // read back 16 bytes at a time as the sums consume it (the values
            // of y never all sit in registers beside the points)
            T wv[K];
            if ((((uintptr_t)y) & 15) == 0 && (w == nullptr || (((uintptr_t)w) & 15) == 0)) {
                // both inputs' loads in flight together
                StagePieces<T, K> PW, PY;
                if (w) stage_fetch<T, K>(w, avail, PW);
                stage_fetch<T, K>(y, avail, PY);
                if (w) {
                    stage_put<T, K>(PW, stage);
                    wave_sync();
                    stage_read<T, K>(stage, wv);
                    wave_sync();  // every lane has its weights before the values replace them
                }
                stage_put<T, K>(PY, stage);
                wave_sync();
            } else {
                if (w) lane_load_staged<T, K>(w, avail, stage, wv);
                stage_wave<T, K>(y, avail, stage);
            }
            if (!w) {
#pragma unroll
                for (int j = 0; j < K; ++j) wv[j] = (j < cnt) ? (T)1 : (T)0;
            }
            const int lane = lane_id();
#pragma unroll
            for (int q = 0; q < K / VW; ++q) {
                const uint4 u = *(const uint4*)(stage + lane * K + q * VW);
                const T* pu = (const T*)&u;
#pragma unroll
                for (int r = 0; r < VW; ++r) take(q * VW + r, (double)pu[r], (double)wv[q * VW + r], true);
            }
            wave_sync();  // every lane has its values before the stage is reused
            done = true;
        }
    }
    if constexpr (K % VW == 0 && !STAGED) {
        // whole, aligned lanes: 16-byte loads, all issued before the sums
        // consume them (one memory latency for the lane, not one per load)
        if (!done && cnt == K && (((uintptr_t)y) & 15) == 0 && (w == nullptr || (((uintptr_t)w) & 15) == 0)) {
            if constexpr (sizeof(T) == 4) {
                float4 a[K / 4], b[K / 4];
#pragma unroll
                for (int q = 0; q < K / 4; ++q) a[q] = ((const float4*)y)[q];
                if (w) {
#pragma unroll
                    for (int q = 0; q < K / 4; ++q) b[q] = ((const float4*)w)[q];
                } else {
#pragma unroll
                    for (int q = 0; q < K / 4; ++q) b[q] = make_float4(1.f, 1.f, 1.f, 1.f);
                }
#pragma unroll
                for (int q = 0; q < K / 4; ++q) {
                    take(4 * q, a[q].x, b[q].x);
                    take(4 * q + 1, a[q].y, b[q].y);
                    take(4 * q + 2, a[q].z, b[q].z);
                    take(4 * q + 3, a[q].w, b[q].w);
                }
            } else {
                double2 a[K / 2], b[K / 2];
#pragma unroll
                for (int q = 0; q < K / 2; ++q) a[q] = ((const double2*)y)[q];
                if (w) {
#pragma unroll
                    for (int q = 0; q < K / 2; ++q) b[q] = ((const double2*)w)[q];
                } else {
#pragma unroll
                    for (int q = 0; q < K / 2; ++q) b[q] = make_double2(1.0, 1.0);
                }
#pragma unroll
                for (int q = 0; q < K / 2; ++q) {
                    take(2 * q, a[q].x, b[q].x);
                    take(2 * q + 1, a[q].y, b[q].y);
                }
            }
            done = true;
        }
    }
    if (!STAGED && !done) {
        // element loads, all issued before the sums use them
        T yv[K], wv[K];
#pragma unroll
        for (int j = 0; j < K; ++j) yv[j] = (j < cnt) ? y[j] : (T)0;
        if (w) {
#pragma unroll
            for (int j = 0; j < K; ++j) wv[j] = (j < cnt) ? w[j] : (T)0;
        } else {
#pragma unroll
            for (int j = 0; j < K; ++j) wv[j] = (j < cnt) ? (T)1 : (T)0;
        }
#pragma unroll
        for (int j = 0; j < K; ++j) take(j, (double)yv[j], (double)wv[j]);
    }
    checks();
    if constexpr (!HULL) return 0ull;
    if (nxp) return gw_parts<K, 2>(xs, ys, cnt, *nxp);
    return lane_gift_wrap<K>(xs, ys, cnt);
}

// The same on values already in registers, with unit weights: yv[j] for
// j < cnt (f as in lane_hull; a non-finite value sets bit 1).
template <int K>
__device__ inline uint64_t lane_hull_vals(const double (&yv)[K], int cnt, int negate, double (&xs)[K],
                                          double (&ys)[K], int& f) {
    double X = 0.0, Y = 0.0;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        if (j < cnt) {
            if (!isfinite(yv[j])) f |= 1;
            X += 1.0;
            Y += negate ? -yv[j] : yv[j];
        }
        xs[j] = X;
        ys[j] = Y;
    }
    return lane_gift_wrap<K>(xs, ys, cnt);
}

// ---------------------------------------------------------------------------
// 2. lane starts: exclusive scan of the lane totals into LS[0..nl-1], LS[nl]
// = the tile's total (double-double when DD, else plain float64 in .x/.z).
// Also combines the lane flags into flag[0], and returns the number of lane
// hull vertices of the tile (point 0 included).  Ends with a barrier.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double4 add4(bool dd, double4 a, double4 b) {
    return dd ? dd4_add(a, b) : make_double4(a.x + b.x, 0.0, a.z + b.z, 0.0);
}

template <bool DD>
__device__ inline int tile_lane_starts(const Tile& t, double2 total, int f, int pc) {
    const int lane = lane_id(), wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    double4* wsum = (double4*)t.CM;  // nw <= 16 entries
    const uint64_t b1 = __ballot(f & 1), b2 = __ballot(f & 2);
    const int pcs = wave_incl_scan_int(pc);
    if (threadIdx.x == 0) t.flag[0] = 0;
    double4 v = make_double4(total.x, 0.0, total.y, 0.0);
    if constexpr (DD) {
        v = wave_scan_incl(v, [](double4 a, double4 b) { return dd4_add(a, b); });
    } else {
        v.x = wave_scan_incl(v.x, [](double a, double b) { return a + b; });
        v.z = wave_scan_incl(v.z, [](double a, double b) { return a + b; });
    }
    if (lane == kWave - 1) {
        wsum[wid] = v;
        t.W[wid] = pcs;
    }
    __syncthreads();
    if (lane == 0 && (b1 | b2)) atomicOr(t.flag, (b1 ? 1 : 0) | (b2 ? 2 : 0));
    double4 acc = make_double4(0.0, 0.0, 0.0, 0.0), all = acc;
    int nvert = 1;
    for (int k = 0; k < nw; ++k) {
        const double4 s = wsum[k];
        if (k < wid) acc = add4(DD, acc, s);
        all = add4(DD, all, s);
        nvert += t.W[k];
    }
    const double4 ex = wave_shift_up1(v);
    const double4 st = add4(DD, acc, ex);
    if (!DD && t.ls2) {
        ((double2*)t.LS)[threadIdx.x] = make_double2(st.x, st.z);
        if (threadIdx.x == 0) ((double2*)t.LS)[t.nl] = make_double2(all.x, all.z);
    } else {
        t.LS[threadIdx.x] = st;
        if (threadIdx.x == 0) t.LS[t.nl] = all;
    }
    __syncthreads();
    return nvert;
}

// Drops from the lane's mask the points that lie above the chord from the
// tile's first point to its last by more than rounding: the lower hull lies
// on or below that chord (its ends are hull vertices and the hull is convex),
// so no such point is a vertex.  Absolute coordinates (float32 tiles, lane
// starts as plain pairs); needs the lane starts written.
template <int K>
__device__ inline uint64_t chord_filter(const Tile& t, uint64_t mask, const double (&xs)[K], const double (&ys)[K]) {
    const double2 tot = ((const double2*)t.LS)[t.nl], st = ((const double2*)t.LS)[threadIdx.x];
    // the cross product of point (st + (xs, ys)[b]) with the chord splits into
    // a part of the lane's start and one of the local point; its rounding is
    // bounded by the magnitudes of the four products (scaled once per lane)
    constexpr double e = 1e-13;
    const double c0 = st.y * tot.x - tot.y * st.x;
    const double a0 = (fabs(st.y * tot.x) + fabs(tot.y * st.x)) * e, ax = fabs(tot.x) * e, ay = fabs(tot.y) * e;
    uint64_t keep = 0ull;
#pragma unroll
    for (int b = 0; b < K; ++b) {
        const double d = c0 + fma(ys[b], tot.x, -(tot.y * xs[b]));
        const double tol = fma(fabs(ys[b]), ax, fma(ay, xs[b], a0));
        keep |= (d <= tol ? 1ull : 0ull) << b;
    }
    return mask & keep;
}

// Candidates of a noisy float32 tile without lane hulls: the lane's points
// that no chord between two points of the tile lies clearly below.  The lower
// hull lies on or below every chord between two of its points, so a point
// strictly above the chord of two points on either side of it is not a
// vertex; the chords used, all between points of the tile, are
//   - the lane's: from its start (local origin) to its last point E, and,
//     split at the interior point v lowest under it, from the start to v and
//     from v to E (any point v would do; the lowest removes the most: one
//     level of QuickHull inside the lane);
//   - the wave's: from the start of its first lane to the end of its last;
//   - the tile's: from point 0 to point N.
// A point is dropped only when its cross product with a chord exceeds a
// bound on the rounding of that product and of the float64 coordinates the
// later steps use (absolute, the lane start plus the local point), so every
// vertex of the tile's hull in those coordinates is kept.  About 10% of the
// points of N(0,1) noise remain (half hulls below the tile's chord keep 14%),
// at about a twentieth of the comparisons.  Needs the lane starts written
// (plain pairs, ls2).  Returns the lane's mask (bit b <-> local point b+1).
template <int K>
__device__ inline uint64_t lane_chords(const Tile& t, const double (&xs)[K], const double (&ys)[K], int cnt) {
    if (cnt <= 0) return 0ull;
    const int l = threadIdx.x, wid = l >> 6;
    const double2* LS = (const double2*)t.LS;
    const double2 st = LS[l];
    // the tile's and the wave's chords are the same in every lane of a wave
    const int wend = min((wid + 1) * kWave, t.nl);
    const double2 wa = LS[wid * kWave], wb = LS[wend], tt = LS[t.nl];
    const double2 tot = make_double2(uniform_d(tt.x), uniform_d(tt.y));
    // local points past cnt repeat the lane's last one (their weights are 0)
    const double ex = xs[K - 1], ey = ys[K - 1];
    double ymax = 0.0;
#pragma unroll
    for (int j = 0; j < K; ++j) ymax = fmax(ymax, fabs(ys[j]));
    // rounding bound of every cross product below, in local units: the
    // coordinates the wrap compares carry errors of an ulp of their absolute
    // size (st + local), times the lane's extents; the local products' own
    // rounding is smaller than the slack factor covers
    const double xa = st.x + ex, ya = fabs(st.y) + ymax;
    const double tol = 0x1p-44 * (xa * ymax + ya * ex + ex * ymax);
    // the wave's and the tile's chords on absolute points st + (xs, ys): the
    // cross product splits into a part of the lane's start and a local one
    uint32_t keep = 0u;
    {
        const double wax = uniform_d(wa.x), way = uniform_d(wa.y);
        const double wdx = uniform_d(wb.x - wa.x), wdy = uniform_d(wb.y - wa.y);
        const double wc = fma(st.y - way, wdx, -(wdy * (st.x - wax)));
        const double wtol = 0x1p-44 * ((fabs(st.y) + fabs(way) + ymax) * wdx + fabs(wdy) * xa);
        const double tc = fma(st.y, tot.x, -(tot.y * st.x));
        const double ttol = 0x1p-44 * ((fabs(st.y) + ymax) * tot.x + fabs(tot.y) * xa);
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const double dw = wc + fma(ys[j], wdx, -(wdy * xs[j]));
            const double dt = tc + fma(ys[j], tot.x, -(tot.y * xs[j]));
            keep |= (dw <= wtol && dt <= ttol && j < cnt) ? (1u << j) : 0u;
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // the lane's chord and its lowest interior point
    double dmin = INFINITY;
    int v = -1;
#pragma unroll
    for (int j = 0; j + 1 < K; ++j) {
        const double d = fma(ys[j], ex, -(ey * xs[j]));
        const bool take = j + 1 < cnt && d < dmin;
        dmin = take ? d : dmin;
        v = take ? j : v;
    }
    double xv = 0.0, yv = 0.0;
#pragma unroll
    for (int j = 0; j + 1 < K; ++j) {
        xv = (j == v) ? xs[j] : xv;
        yv = (j == v) ? ys[j] : yv;
    }
    const bool split = v >= 0 && dmin <= tol;  // some interior point lies under (or on) the lane's chord
    static_assert(K <= 32, "a lane's candidates fit one 32-bit word");
    __builtin_amdgcn_sched_barrier(0);
    {
        const double rdx = ex - xv, rdy = ey - yv;
        const double rc = fma(-yv, rdx, rdy * xv);
        uint32_t lq = 1u << (K - 1);  // the lane's last point (E): no lane chord spans it
#pragma unroll
        for (int j = 0; j + 1 < K; ++j) {
            // left of v: chord start-v; right of v: chord v-E; v itself is kept
            const double cl = fma(ys[j], xv, -(yv * xs[j]));
            const double cr = fma(ys[j], rdx, rc) - rdy * xs[j];
            const double c = (j < v) ? cl : cr;
            bool k = split && (j == v || c <= tol);
            k = (j + 1 == cnt) ? true : k;  // a partial lane's last point is its E
            lq |= k ? (1u << j) : 0u;
        }
        keep &= lq;
    }
    return (uint64_t)keep;
}

// ---------------------------------------------------------------------------
// QuickHull by the workgroup (the lower hull of a few hundred points, one per
// thread).  Entries 0..m of E hold points in increasing x; thread t holds
// entry e = t + 1, entries 0 and m are the ends and always vertices.  Each
// level, every interior point still strictly below the chord of its segment
// (a, b) offers its cross product with the chord (its depth below the chord,
// scaled by the chord's length) to the segment's slot; the deepest point of
// each segment is a vertex and splits it, and every thread follows the part
// that holds it.  A point on or above its segment's chord is not a vertex and
// stays above the chords of the parts, so it drops out.  Strictly below
// means a cross product under -tolrel times the magnitude of its two terms
// (collinear points are not vertices).
// A slot's key orders by the cross product (its sign, exponent and first 42
// bits of mantissa) and then by the entry (10 bits), one 64-bit LDS atomic
// minimum per point and level; the slots of a level are keyed by the
// segment's first entry, in three arrays used in turn (an array is cleared
// one level after its last read and one level before its next use), each
// with a word that says whether any point made an offer (plain stores of 1).
// Returns whether the calling thread's entry is a vertex, with (a, b) the
// entries of the hull edge over the interval [e - 1, e] (for a vertex: the
// previous vertex and e).  slots: 3 (m + 2) words of LDS.  Block scope; every
// thread calls it; m <= min(1023, blockDim.x).
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned long long qh_key(double d, int e) {
    // d < 0: the complement of its bits orders by depth (deeper = smaller)
    const unsigned long long b = ~(unsigned long long)__double_as_longlong(d);
    return (b & ~1023ull) | (unsigned long long)e;
}

__host__ __device__ inline int qh_slot_words(int m) { return 3 * (m + 2); }

__device__ inline bool tile_quickhull(const double2* E, int m, unsigned long long* slots, double tolrel, int& a,
                                      int& b) {
    const int tid = threadIdx.x, e = tid + 1, ns = m + 1;
    unsigned long long* F = slots + 3 * ns;  // the offer words of the three arrays
    for (int i = tid; i < 3 * ns + 3; i += blockDim.x) slots[i] = (i < 3 * ns) ? ~0ull : 0ull;
    a = 0;
    b = m;
    const bool held = e <= m;
    double2 A = E[0], B = E[m];
    const double2 P = held ? E[e] : make_double2(0.0, 0.0);
    bool vert = e == m, cand = e < m;
    __syncthreads();
    for (int k = 0;; ++k) {
        const int r = k % 3;
        unsigned long long* cur = slots + r * ns;
        if (cand) {
            const double dx = B.x - A.x, dy = B.y - A.y, px = P.x - A.x, py = P.y - A.y;
            const double t1 = py * dx, t2 = dy * px;
            const double d = t1 - t2;
            if (d < -tolrel * (fabs(t1) + fabs(t2)) && d < 0.0) {
                atomicMin(cur + a, qh_key(d, e));
                F[r] = 1ull;
            } else {
                cand = false;
            }
        }
        __syncthreads();
        const unsigned long long f = F[r];                // both reads in flight at once
        const unsigned long long w = held ? cur[a] : ~0ull;
        if (f == 0ull) break;  // uniform: no segment split
        if (held) {
            if (w != ~0ull) {
                const int v = (int)(w & 1023ull);
                if (v == e) {
                    vert = true;
                    cand = false;
                    b = e;
                    B = P;
                } else if (e < v) {
                    b = v;
                    B = E[v];
                } else {
                    a = v;
                    A = E[v];
                }
            }
        }
        const int o = (k + 2) % 3;
        unsigned long long* old = slots + o * ns;
        for (int i = tid; i < ns; i += blockDim.x) old[i] = ~0ull;
        if (tid == 0) F[o] = 0ull;
    }
    return vert;
}

// Candidates of a noisy float32 tile: the lane's points that do not lie
// clearly above the hull of the lanes' end points.  Every edge of that coarse
// hull joins two points of the tile, and the tile's lower hull lies on or
// below every such chord over its span, so a point strictly above the coarse
// edge that spans its lane is not a vertex.  (a, b): the coarse edge over the
// lane, as lane-end indices into the lane starts (tile_quickhull on LS).  A
// point is dropped only when its cross product with the edge exceeds a bound
// on the rounding of that product and of the coordinates the later steps use
// (absolute: the lane start plus the local point).  On N(0,1) noise rows of
// 5000 elements about 80 points remain (1.6%).  Needs the lane starts (plain
// pairs, ls2).  Returns the lane's mask (bit b <-> local point b+1).
// A lane start as one float64 pair, from either layout of LS.
__device__ __forceinline__ double2 lane_start2(const Tile& t, int l) {
    if (t.ls2) return ((const double2*)t.LS)[l];
    const double4 s = t.LS[l];
    return make_double2(s.x + s.y, s.z + s.w);
}

// E: the lane ends as pairs (entry l = the start of lane l); nullptr reads
// them from LS (plain pairs, ls2).
template <int K>
__device__ inline uint64_t lane_coarse_filter(const Tile& t, const double (&xs)[K], const double (&ys)[K], int cnt,
                                              int a, int b, const double2* E = nullptr) {
    if (cnt <= 0) return 0ull;
    const double2* LS = E ? E : (const double2*)t.LS;
    const double2 st = LS[threadIdx.x], A = LS[a], B = LS[b];
    const double ex = xs[K - 1];
    double ymax = 0.0;
#pragma unroll
    for (int j = 0; j < K; ++j) ymax = fmax(ymax, fabs(ys[j]));
    const double xa = st.x + ex;
    const double dx = B.x - A.x, dy = B.y - A.y;
    const double c0 = fma(st.y - A.y, dx, -(dy * (st.x - A.x)));
    const double tol = 0x1p-44 * ((fabs(st.y) + fabs(A.y) + ymax) * dx + fabs(dy) * xa);
    static_assert(K <= 32, "a lane's candidates fit one 32-bit word");
    uint32_t keep = 0u;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const double d = c0 + fma(ys[j], dx, -(dy * xs[j]));
        keep |= (d <= tol && j < cnt) ? (1u << j) : 0u;
    }
    return (uint64_t)keep;
}

// The QuickHull list: entry r is point V[r] with its coordinates relative to
// the tile's first point as a double-double pair, L[r] = (x, x_lo, y, y_lo)
// (the lane's start plus the local point, exact), 32 bytes an entry in the
// list's room at VXY.  Differences of two entries are formed part by part, as
// the merges form them across lanes.
__device__ __forceinline__ double4* list_dd(const Tile& t) { return (double4*)t.VXY; }

// tile_compact_upto for the QuickHull list: the candidates of mask (point 0
// first) are listed only when their number, point 0 included, is at most
// maxv; returns that number.  Ends with a barrier.
template <int K>
__device__ inline int list_compact(const Tile& t, uint64_t mask, const double (&xs)[K], const double (&ys)[K],
                                   int maxv) {
    const int l = threadIdx.x, lane = lane_id(), wid = l >> 6, nw = blockDim.x >> 6;
    double4* L = list_dd(t);
    const int pc = __popcll(mask);
    const int incl = wave_incl_scan_int(pc);
    if (lane == kWave - 1) t.W[wid] = incl;
    __syncthreads();
    int r = 1, tot = 1;
    for (int k = 0; k < nw; ++k) {
        const int c = t.W[k];
        r += (k < wid) ? c : 0;
        tot += c;
    }
    if (tot <= maxv) {  // uniform
        r += incl - pc;
        if (l == 0) {
            t.flag[1] = tot;
            t.V[0] = 0;
            L[0] = make_double4(0.0, 0.0, 0.0, 0.0);
        }
        if (mask) {
            double4 st;
            if (t.ls2) {
                const double2 s2 = ((const double2*)t.LS)[l];
                st = make_double4(s2.x, 0.0, s2.y, 0.0);
            } else {
                st = t.LS[l];
            }
#pragma unroll
            for (int b = 0; b < K; ++b) {
                if ((mask >> b) & 1ull) {
                    t.V[r] = (unsigned short)(l * K + b + 1);
                    L[r] = dd4_add_d(st, make_double2(xs[b], ys[b]));
                    ++r;
                }
            }
        }
    }
    __syncthreads();
    return tot;
}

// QuickHull over the QuickHull list: the lower hull of entries 0..m (points
// in increasing order; entries 0 and m are its ends and always vertices).  R
// entries per thread, e = 1 + tid + r * blockDim.x.  Each level, every entry
// still strictly below the chord of its segment (a, b) (the turn (a, e, b)
// positive, the merges' vertex test) offers minus that turn to the segment's
// slot as tile_quickhull does; the deepest entry of each segment is a vertex
// and splits it, and the other entries follow the part that holds them.  An
// entry on or above its chord drops out.  vert[r]: entry e is an interior
// vertex.  slots: 3 (m + 2) words of LDS apart from the list.  Block scope;
// the list is complete (a barrier after its last write);
// m <= min(1023, R * blockDim.x).  Ends with a barrier.
template <int R>
__device__ inline void list_quickhull(const Tile& t, int m, unsigned long long* slots, bool (&vert)[R]) {
    const double4* L = list_dd(t);
    const int tid = threadIdx.x, nt = blockDim.x, ns = m + 1;
    unsigned long long* F = slots + 3 * ns;  // the offer words of the three arrays
    for (int i = tid; i < 3 * ns + 3; i += nt) slots[i] = (i < 3 * ns) ? ~0ull : 0ull;
    int a[R], b[R];
    double2 dP[R], dB[R];  // P_e - P_a and P_b - P_a
    bool cand[R];
    const double4 L0 = L[0], Lm = L[m];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int e = 1 + tid + r * nt;
        vert[r] = false;
        cand[r] = e < m;
        a[r] = 0;
        b[r] = m;
        dP[r] = dd4_diff(L0, cand[r] ? L[e] : L0);
        dB[r] = dd4_diff(L0, Lm);
    }
    __syncthreads();  // the slots are clear
    for (int k = 0;; ++k) {
        const int q = k % 3;
        unsigned long long* cur = slots + q * ns;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (cand[r]) {
                const double turn = cross2(dP[r], dB[r]);
                if (turn > 0.0) {
                    atomicMin(cur + a[r], qh_key(-turn, 1 + tid + r * nt));
                    F[q] = 1ull;
                } else {
                    cand[r] = false;
                }
            }
        }
        __syncthreads();
        const unsigned long long f = F[q];
        unsigned long long wv[R];
#pragma unroll
        for (int r = 0; r < R; ++r) wv[r] = cand[r] ? cur[a[r]] : ~0ull;
        if (f == 0ull) break;  // uniform: no segment split
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (cand[r]) {
                const int e = 1 + tid + r * nt, v = (int)(wv[r] & 1023ull);
                if (v == e) {
                    vert[r] = true;
                    cand[r] = false;
                } else {
                    const bool left = e < v;
                    a[r] = left ? a[r] : v;
                    b[r] = left ? v : b[r];
                    const double4 A = L[a[r]], B = L[b[r]], P = L[e];
                    dP[r] = dd4_diff(A, P);
                    dB[r] = dd4_diff(A, B);
                }
            }
            __builtin_amdgcn_sched_barrier(0);  // one entry's loads in flight at a time (registers)
        }
        const int o = (k + 2) % 3;
        unsigned long long* old = slots + o * ns;
        for (int i = tid; i < ns; i += nt) old[i] = ~0ull;
        if (tid == 0) F[o] = 0ull;
    }
}

// After list_quickhull: its vertices (entry 0, the entries with vert, entry
// m) move to the front of the list in order (V and L), flag[1] = their
// number.  Every read precedes the first barrier.  Ends with a barrier.
template <int R>
__device__ inline void list_to_front(const Tile& t, int m, const bool (&vert)[R]) {
    double4* L = list_dd(t);
    const int tid = threadIdx.x, nt = blockDim.x, lane = lane_id(), wid = tid >> 6, nw = nt >> 6;
    static_assert(R * 8 <= 32, "per-wave counts in W");
    unsigned short pv[R];
    double4 xy[R];
    uint64_t bal[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int e = 1 + tid + r * nt;
        bal[r] = __ballot(vert[r]);
        if (lane == 0) t.W[r * nw + wid] = __popcll(bal[r]);
        pv[r] = 0;
        xy[r] = make_double4(0.0, 0.0, 0.0, 0.0);
        if (vert[r]) {
            pv[r] = t.V[e];
            xy[r] = L[e];
        }
    }
    const unsigned short pm = t.V[m];
    const double4 xym = L[m];
    __syncthreads();
    int base = 1;  // entry 0 stays
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int before = base;
        for (int q = 0; q < nw; ++q) {
            const int c = t.W[r * nw + q];
            before += (q < wid) ? c : 0;
            base += c;
        }
        if (vert[r]) {
            const int i = before + __popcll(bal[r] & bits_upto(lane - 1));
            t.V[i] = pv[r];
            L[i] = xy[r];
        }
    }
    if (tid == 0) {
        t.V[base] = pm;
        L[base] = xym;
        t.flag[1] = base + 1;
    }
    __syncthreads();
}

// tile_edge_slopes on the QuickHull list (after list_to_front): VXY[i] =
// (slope of the edge from entry i to i + 1, oriented and clipped; clip
// flag), at most R edges per thread.  Reads precede the barrier that the
// writes follow (VXY[i] overlaps the list).  Ends with a barrier.
template <int R>
__device__ inline void list_edge_slopes(const Tile& t, int increasing, double clo, double chi) {
    const double4* L = list_dd(t);
    const int nv = t.flag[1];
    double sv[R];
    bool cv[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int i = threadIdx.x + k * t.nl;
        sv[k] = 0.0;
        cv[k] = false;
        if (i < nv - 1) {
            const double2 d = dd4_diff(L[i], L[i + 1]);
            sv[k] = finish(d.y / d.x, increasing, clo, chi, cv[k]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int i = threadIdx.x + k * t.nl;
        if (i < nv - 1) t.VXY[i] = make_double2(sv[k], cv[k] ? 1.0 : 0.0);
    }
    __syncthreads();
}

// After tile_compact and tile_quickhull over the list (absolute coordinates):
// the hull's vertices (vert in the thread holding entry tid + 1, whose
// previous vertex is entry a; entry 0 always) move to the front of the list
// in order, flag[1] = their number, and each vertex's thread writes the value
// of the edge that ends at it over the coordinates of the entry before it:
// VXY[i] = (the slope of the edge from vertex i to vertex i + 1, oriented and
// clipped; 1 where clipping changed it, else 0), as tile_edge_slopes does.
// Entries only move down, and every read precedes the first barrier.  Ends
// with a barrier.
__device__ inline void tile_hull_to_front(const Tile& t, int m, bool vert, int a, int increasing, double lo,
                                          double hi) {
    const int tid = threadIdx.x, e = tid + 1, lane = lane_id(), wid = tid >> 6, nw = blockDim.x >> 6;
    const bool mine = vert && e <= m;
    unsigned short pv = 0;
    double sl = 0.0;
    bool cl = false;
    if (mine) {
        pv = t.V[e];
        const double2 d = sub2(t.VXY[e], t.VXY[a]);
        sl = finish(d.y / d.x, increasing, lo, hi, cl);
    }
    const uint64_t bal = __ballot(mine);
    if (lane == 0) t.W[wid] = __popcll(bal);
    __syncthreads();
    int before = 1, total = 1;
    for (int q = 0; q < nw; ++q) {
        const int c = t.W[q];
        before += (q < wid) ? c : 0;
        total += c;
    }
    if (mine) {
        const int r = before + __popcll(bal & bits_upto(lane - 1));
        t.V[r] = pv;
        t.VXY[r - 1] = make_double2(sl, cl ? 1.0 : 0.0);
    }
    if (tid == 0) t.flag[1] = total;
    __syncthreads();
}

// Vertices of the tile's lane masks, point 0 included (block scope; ends
// with a barrier).
__device__ inline int tile_count(const Tile& t, uint64_t mask) {
    const int lane = lane_id(), wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int incl = wave_incl_scan_int(__popcll(mask));
    if (lane == kWave - 1) t.W[24 + wid] = incl;
    __syncthreads();
    int tot = 1;
    for (int k = 0; k < nw; ++k) tot += t.W[24 + k];
    return tot;
}

// ---------------------------------------------------------------------------
// 3. compaction of the vertex set and the merge rounds
// ---------------------------------------------------------------------------

// the calling lane's group's bits of a wave ballot (G consecutive lanes)
__device__ __forceinline__ uint64_t group_bits(uint64_t ballot, int G) {
    if (G >= 64) return ballot;
    return (ballot >> (lane_id() & ~(G - 1))) & ((1ull << G) - 1ull);
}
// number of consecutive set bits from bit 0
__device__ __forceinline__ int trailing_ones(uint64_t m) { return (m == ~0ull) ? 64 : lo_bit(~m); }


// Block scope.  Writes the sorted vertex list of the whole tile: V[0] = point
// 0, then every lane's vertices; I[l] = index of lane l's first vertex;
// flag[1] = number of vertices.  The coordinates are local to the point's lane
// (or absolute when ABS).  Ends with a barrier.
template <int K, bool ABS>
__device__ inline void tile_compact(const Tile& t, uint64_t mask, const double (&xs)[K], const double (&ys)[K]) {
    const int l = threadIdx.x, lane = lane_id(), wid = l >> 6, nw = blockDim.x >> 6;
    const int pc = __popcll(mask);
    const int incl = wave_incl_scan_int(pc);
    if (lane == kWave - 1) t.W[wid] = incl;
    __syncthreads();
    int r = 1;
    for (int k = 0; k < wid; ++k) r += t.W[k];
    r += incl - pc;
    if (l == 0) {
        int tot = 1;
        for (int k = 0; k < nw; ++k) tot += t.W[k];
        t.flag[1] = tot;
        t.V[0] = 0;
        t.VXY[0] = make_double2(0.0, 0.0);
    }
    t.I[l] = r;
    double sx = 0.0, sy = 0.0;
    if (ABS) {
        if (t.ls2) {
            const double2 s = ((const double2*)t.LS)[l];
            sx = s.x;
            sy = s.y;
        } else {
            const double4 s = t.LS[l];
            sx = s.x;
            sy = s.z;
        }
    }
#pragma unroll
    for (int b = 0; b < K; ++b) {
        if ((mask >> b) & 1ull) {
            t.V[r] = (unsigned short)(l * K + b + 1);
            t.VXY[r] = ABS ? make_double2(sx + xs[b], sy + ys[b]) : make_double2(xs[b], ys[b]);
            ++r;
        }
    }
    __syncthreads();
}

// tile_count and tile_compact in one: the number of candidates (point 0
// included) is returned, and the list is written (as tile_compact does) only
// when that number is at most maxv.  One scan and two barriers; ends with a
// barrier.
template <int K, bool ABS>
__device__ inline int tile_compact_upto(const Tile& t, uint64_t mask, const double (&xs)[K], const double (&ys)[K],
                                        int maxv) {
    const int l = threadIdx.x, lane = lane_id(), wid = l >> 6, nw = blockDim.x >> 6;
    const int pc = __popcll(mask);
    const int incl = wave_incl_scan_int(pc);
    if (lane == kWave - 1) t.W[wid] = incl;
    __syncthreads();
    int r = 1, tot = 1;
    for (int k = 0; k < nw; ++k) {
        const int c = t.W[k];
        r += (k < wid) ? c : 0;
        tot += c;
    }
    if (tot <= maxv) {  // uniform
        r += incl - pc;
        if (l == 0) {
            t.flag[1] = tot;
            t.V[0] = 0;
            t.VXY[0] = make_double2(0.0, 0.0);
        }
        t.I[l] = r;
        double sx = 0.0, sy = 0.0;
        if (ABS) {
            const double2 s = lane_start2(t, l);
            sx = s.x;
            sy = s.y;
        }
        if (mask) {
#pragma unroll
            for (int b = 0; b < K; ++b) {
                if ((mask >> b) & 1ull) {
                    t.V[r] = (unsigned short)(l * K + b + 1);
                    t.VXY[r] = ABS ? make_double2(sx + xs[b], sy + ys[b]) : make_double2(xs[b], ys[b]);
                    ++r;
                }
            }
        }
    }
    __syncthreads();
    return tot;
}

// One test of the pairs nearest the shared point (points with absolute
// coordinates).  The cells (i, j) of a D x D grid stand for a = iS - i in A
// and b = jS + j in B; the group's lanes take PASSES cells each and evaluate
//   t1(i, j): a is a strict vertex of {pred(a), a, b} (true at A's first entry),
//   t3(i, j): b is a strict vertex of {a, b, succ(b)} (true at B's last entry).
// Along each convex side these flip once, so the walk described below stops
// exactly at the cell where t1 holds and fails one step nearer the shared
// point on A, and t3 holds and fails one step nearer on B: the bridge (first
// page, Sec. 4, Lemma 4.2), here checked at every cell at once.  All loads are
// issued before any test (indices clamped into the nodes), so the whole grid
// costs one LDS round trip.  Returns false when no cell qualifies (the bridge
// lies farther out, or rounding broke the monotonicity); the caller walks.
template <int PASSES>
__device__ inline bool grid_bridge(const Tile& t, int iA0, int iS, int jS, int jB1, int g, int G, int2& ab) {
    constexpr int D = 8;
    double2 pa1[PASSES], pa[PASSES], pb[PASSES], pb1[PASSES];
#pragma unroll
    for (int m = 0; m < PASSES; ++m) {
        const int c = m * G + g, i = c / D, j = c % D;
        const int a = max(iS - i, iA0), b = min(jS + j, jB1);
        pa1[m] = t.VXY[max(a - 1, 0)];
        pa[m] = t.VXY[a];
        pb[m] = t.VXY[b];
        pb1[m] = t.VXY[min(b + 1, jB1)];
    }
    uint64_t T1 = 0ull, T3 = 0ull;
#pragma unroll
    for (int m = 0; m < PASSES; ++m) {
        const int c = m * G + g, i = c / D, j = c % D;
        const int a = iS - i, b = jS + j;
        const bool in = (a >= iA0) && (b <= jB1);
        const double u1 = cross2(sub2(pa[m], pa1[m]), sub2(pb[m], pa1[m]));
        const double u3 = cross2(sub2(pb[m], pa[m]), sub2(pb1[m], pa[m]));
        const bool t1 = in && j >= 1 && (a == iA0 || u1 > 0.0);
        const bool t3 = in && i >= 1 && (b == jB1 || u3 > 0.0);
        T1 |= group_bits(__ballot(t1), G) << (m * G);
        T3 |= group_bits(__ballot(t3), G) << (m * G);
    }
    if ((T1 >> 1) & 1ull) {  // convex at the shared point
        ab = make_int2(iS, jS);
        return true;
    }
    const int imax = min(D - 1, iS - iA0), jmax = min(D - 1, jB1 - jS);
    const uint64_t rows = (imax >= D - 1) ? ~0xFFull : (((1ull << (D * (imax + 1))) - 1ull) & ~0xFFull);
    const uint64_t cols = ((1ull << (jmax + 1)) - 2ull) * 0x0101010101010101ull;  // j = 1 .. jmax in every row
    const uint64_t cand = T1 & ~(T1 << D) & T3 & ~(T3 << 1) & rows & cols;
    if (!cand) return false;
    const int c = lo_bit(cand);
    ab = make_int2(iS - c / D, jS + c % D);
    return true;
}

// The bridge of two nodes that share one point, found by the calling group of
// G lanes (g = 0..G-1): A = list entries [iA0, iS] and B = [jS, jB1], where
// entries iS and jS hold the shared point (iS == jS when the two lists are
// adjacent).  Returns the list indices (alpha in A, beta in B); (iS, jS) when
// the chain is convex at the shared point.  With absolute coordinates, groups
// of 16 or more lanes first test the 8 x 8 pairs nearest the shared point at
// once.  Otherwise, and when
// that test finds nothing, from the neighbours of the shared point the walk of
// the first page (Sec. 4, after Lemma 4.2) advances each side to its tangent
// point against the other side's current end, G candidates per step: a is
// passed over while it is not a strict vertex of {pred(a), a, b}, and b while
// it is not one of {a, b, succ(b)}.
template <int K, bool ABS>
__device__ inline int2 group_bridge(const Tile& t, int iA0, int iS, int jS, int jB1, int g, int G) {
    if constexpr (ABS) {
        int2 ab;
        if (G == 64) {
            if (grid_bridge<1>(t, iA0, iS, jS, jB1, g, G, ab)) return ab;
        } else if (G == 32) {
            if (grid_bridge<2>(t, iA0, iS, jS, jB1, g, G, ab)) return ab;
        } else if (G == 16) {
            if (grid_bridge<4>(t, iA0, iS, jS, jB1, g, G, ab)) return ab;
        }
    }
    if (vturn<K, ABS>(t, iS - 1, iS, jS + 1) > 0.0) return make_int2(iS, jS);
    int al = iS - 1, be = jS + 1;
    for (;;) {
        for (;;) {
            const int i = al - g;
            bool cont = false;
            if (i > iA0) cont = !(vturn<K, ABS>(t, i - 1, i, be) > 0.0);
            const int run = trailing_ones(group_bits(__ballot(cont), G));
            const int step = run < G ? run : G;
            al -= step;
            if (step < G) break;
        }
        bool movedB = false;
        for (;;) {
            const int j = be + g;
            bool cont = false;
            if (j < jB1) cont = !(vturn<K, ABS>(t, al, j, j + 1) > 0.0);
            const int run = trailing_ones(group_bits(__ballot(cont), G));
            const int step = run < G ? run : G;
            be += step;
            if (step > 0) movedB = true;
            if (step < G) break;
        }
        if (!movedB) break;
    }
    return make_int2(al, be);
}

// Copies list entries [s0, s1] to d0.. (d0 <= s0) with the calling group of G
// lanes, four blocks of G entries per step.  A step's blocks are read by all
// lanes before any of them is written; a step's destinations end where the
// next step's sources start (d0 <= s0), so no later source is overwritten.
// The caller orders the writes before its next reads of the list (wave_sync
// or barrier).
__device__ inline void group_move(const Tile& t, int s0, int s1, int d0, int g, int G) {
    constexpr int kB = 4;
    const int cnt = s1 - s0 + 1;
    if (d0 == s0 || cnt <= 0) return;  // uniform in the group
    for (int off = 0; off < cnt; off += kB * G) {
        unsigned short pv[kB];
        double2 xy[kB];
#pragma unroll
        for (int b = 0; b < kB; ++b) {
            const int q = off + b * G + g;
            pv[b] = 0;
            xy[b] = make_double2(0.0, 0.0);
            if (q < cnt) {
                pv[b] = t.V[s0 + q];
                xy[b] = t.VXY[s0 + q];
            }
        }
        wave_sync();
#pragma unroll
        for (int b = 0; b < kB; ++b) {
            const int q = off + b * G + g;
            if (q < cnt) {
                t.V[d0 + q] = pv[b];
                t.VXY[d0 + q] = xy[b];
            }
        }
    }
}

// Merges the nodes A = entries [a0, a1] and B = [b0, b1] (a1 and b0 hold the
// same point) with the calling group: the bridge, then B's surviving suffix is
// copied behind A's surviving prefix.  Returns the merged node's last index
// (it starts at a0).
template <int K, bool ABS>
__device__ inline int group_merge(const Tile& t, int a0, int a1, int b0, int b1, int g, int G) {
    const int2 ab = group_bridge<K, ABS>(t, a0, a1, b0, b1, g, G);
    int al = ab.x, be = ab.y;
    if (be == b0) {
        // convex at the shared point: keep A's copy of it
        al = a1;
        be = b0 + 1;
    }
    group_move(t, be, b1, al + 1, g, G);
    return al + 1 + (b1 - be);
}

template <int K>
__device__ inline void tile_masks(const Tile& t, uint64_t& mask);
template <int K>
__device__ inline void tile_masks_short(const Tile& t, uint64_t& mask);

// ---------------------------------------------------------------------------
// Output-sensitive finish.  Every vertex of the tile's hull is a vertex of
// its lane's hull (the subset lemma of the first page, Sec. 3.1), so the hull
// of the compacted list is the tile's hull, and from a hull vertex v the next
// one is the entry after v of least slope from v (the farthest of equal
// slopes, so collinear middle points are dropped): a gift wrap whose steps
// are the hull's edges.  Noisy tiles end with a few dozen vertices out of
// thousands of points, so a few steps replace the merge rounds; a wrap that
// takes more than its cap of steps gives up and the rounds run instead on
// the untouched list.
// ---------------------------------------------------------------------------

// One wrap by the calling wave over the candidates c0 .. c1 (list entries
// cand(c)), from c0 (a hull vertex) to c1 (the last point, always a vertex).
// Writes the candidates it steps to, c1 last, to out[0..) and returns their
// number, or -1 after cap steps short of c1.  Each lane keeps the best of its
// strided candidates by exact cross-multiplied comparison; the wave's least
// slope then picks the winner, and the few lanes whose slopes lie within
// rounding of it are compared exactly (ties to the farthest).
template <int K, bool ABS, class Cand>
__device__ inline int wave_wrap(const Tile& t, int c0, int c1, Cand cand, int* out, int cap) {
    const int lane = lane_id();
    int v = c0, n = 0;
    while (v < c1) {
        if (n == cap) return -1;
        const int ev = cand(v);
        double bx = 1.0, by = 0.0;
        int bc = -1;
        for (int c = v + 1 + lane; c <= c1; c += kWave) {
            const double2 d = vdiff<K, ABS>(t, ev, cand(c));
            // candidates come in increasing order: on equal slopes the later one
            if (bc < 0 || d.y * bx <= by * d.x) {
                bx = d.x;
                by = d.y;
                bc = c;
            }
        }
        const double sl = (bc < 0) ? INFINITY : by / bx;
        const double m = wave_min(sl);
        const uint64_t con = __ballot(bc >= 0 && sl <= m + fabs(m) * 2e-15);
        int wl = lo_bit(con);
        if (con & (con - 1)) {
            double wx = readlane_d(bx, wl), wy = readlane_d(by, wl);
            int wc = __builtin_amdgcn_readlane(bc, wl);
            for (uint64_t rest = con & (con - 1); rest; rest &= rest - 1) {
                const int q = lo_bit(rest);
                const double qx = readlane_d(bx, q), qy = readlane_d(by, q);
                const int qc = __builtin_amdgcn_readlane(bc, q);
                const double lhs = qy * wx, rhs = wy * qx;
                if (lhs < rhs || (lhs == rhs && qc > wc)) {
                    wx = qx;
                    wy = qy;
                    wc = qc;
                }
            }
            v = wc;
        } else {
            v = __builtin_amdgcn_readlane(bc, wl);
        }
        if (lane == 0) out[n] = v;
        ++n;
    }
    return n;
}

// The same wrap with the candidates held in registers, Q per lane (lane l
// holds c0 + 1 + l + 64q), for tiles with absolute coordinates and at most
// 64 Q candidates: a step then reads no LDS.  Each lane's best is found by
// exact comparisons; across lanes a float32 image of the slopes picks the
// winner, and the lanes whose images lie within its rounding are compared
// exactly.  The next origin is the old one plus the winner's difference
// (within a few ulp of the vertex: enough to pick the next one, whose
// coordinates the list keeps exactly).
template <int K, int Q, class Cand>
__device__ inline int wave_wrap_regs(const Tile& t, int c0, int c1, Cand cand, int* out, int cap) {
    const int lane = lane_id();
    double X[Q], Y[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int c = c0 + 1 + lane + kWave * q;
        const double2 p = (c <= c1) ? t.VXY[cand(c)] : make_double2(0.0, 0.0);
        X[q] = p.x;
        Y[q] = p.y;
    }
    const double2 p0 = t.VXY[cand(c0)];
    double xv = p0.x, yv = p0.y;
    int v = c0, n = 0;
    while (v < c1) {
        if (n == cap) return -1;
        double bx = 1.0, by = 0.0;
        int bq = -1;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            if (c0 + kWave * (q + 1) > v) {  // uniform: the slot holds candidates after v
                const int c = c0 + 1 + lane + kWave * q;
                const double dx = X[q] - xv, dy = Y[q] - yv;
                // later slots hold later candidates: on equal slopes the later one
                const bool take = c > v && c <= c1 && (bq < 0 || dy * bx <= by * dx);
                bx = take ? dx : bx;
                by = take ? dy : by;
                bq = take ? q : bq;
            }
        }
        const int bc = (bq < 0) ? -1 : c0 + 1 + lane + kWave * bq;
        const float sl = (bq < 0) ? INFINITY : (float)(by * __builtin_amdgcn_rcp(bx));
        const float m = wave_min_f(sl);
        uint64_t con = __ballot(bq >= 0 && sl <= m + fabsf(m) * 0x1p-16f + 0x1p-100f);
        if (!con) con = __ballot(bq >= 0);  // slopes beyond float32's range: compare them all exactly
        int wl = lo_bit(con);
        if (con & (con - 1)) {
            double wx = readlane_d(bx, wl), wy = readlane_d(by, wl);
            int wc = __builtin_amdgcn_readlane(bc, wl);
            for (uint64_t rest = con & (con - 1); rest; rest &= rest - 1) {
                const int q = lo_bit(rest);
                const double qx = readlane_d(bx, q), qy = readlane_d(by, q);
                const int qc = __builtin_amdgcn_readlane(bc, q);
                const double lhs = qy * wx, rhs = wy * qx;
                if (lhs < rhs || (lhs == rhs && qc > wc)) {
                    wx = qx;
                    wy = qy;
                    wc = qc;
                    wl = q;
                }
            }
        }
        v = __builtin_amdgcn_readlane(bc, wl);
        xv += readlane_d(bx, wl);
        yv += readlane_d(by, wl);
        if (lane == 0) out[n] = v;
        ++n;
    }
    return n;
}

template <int K, bool ABS, class Cand>
__device__ inline int wave_wrap_any(const Tile& t, int c0, int c1, Cand cand, int* out, int cap) {
    if constexpr (ABS) {
        if (c1 - c0 <= kWave * 2) return wave_wrap_regs<K, 2>(t, c0, c1, cand, out, cap);
        if (c1 - c0 <= kWave * 4) return wave_wrap_regs<K, 4>(t, c0, c1, cand, out, cap);
        if (c1 - c0 <= kWave * 6) return wave_wrap_regs<K, 6>(t, c0, c1, cand, out, cap);
        if (c1 - c0 <= kWave * 8) return wave_wrap_regs<K, 8>(t, c0, c1, cand, out, cap);
    }
    return wave_wrap<K, ABS>(t, c0, c1, cand, out, cap);
}

// The hull of a few candidates C[0..nc) (list entries in increasing order),
// all at once: a middle candidate p is a vertex iff the steepest slope into
// it from an earlier candidate is strictly less than the least slope out of
// it to a later one (both found by cross-multiplied comparisons over every
// other candidate); the first and last are always vertices.
// The same test by the whole workgroup, L consecutive lanes per candidate
// (each over every L-th other candidate, loaded four at a time, then combined
// across the L lanes), for nc <= blockDim.x / L.  The vertices after the first
// are written straight to the front of the list (entries 1..), their number
// returned (the same in every thread) and stored in flag[1] with point 0.
// With absolute coordinates CXY[q] holds candidate q's point (a copy made with
// C).  The list is read before the first barrier and written after it; the
// caller orders the writes before the next reads of the list.
template <int K, bool ABS, int L>
__device__ inline int tile_hull_small(const Tile& t, const int* C, const double2* CXY, int nc) {
    const int tid = threadIdx.x, p = tid / L, part = tid % L, lane = lane_id(), wid = tid >> 6;
    const int nw = blockDim.x >> 6;
    const int pc = min(p, nc - 1);
    const int ep = C[pc];
    const unsigned short pv = t.V[ep];
    const double2 pxy = t.VXY[ep];
    const double2 P = ABS ? CXY[pc] : pxy;
    double lx = 1.0, ly = -INFINITY, rx = 1.0, ry = INFINITY;
    auto cmp = [&](int q, double2 d) {  // d = P_p - P_q
        if (q > p) d = make_double2(-d.x, -d.y);
        if (q < p && d.y * lx >= ly * d.x) {
            lx = d.x;
            ly = d.y;
        }
        if (q > p && d.y * rx <= ry * d.x) {
            rx = d.x;
            ry = d.y;
        }
    };
    for (int q0 = part; q0 < nc; q0 += 4 * L) {
        double2 d[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int q = min(q0 + u * L, nc - 1);
            if constexpr (ABS) {
                d[u] = sub2(P, CXY[q]);
            } else {
                d[u] = vdiff<K, ABS>(t, C[q], ep);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (q0 + u * L < nc) cmp(q0 + u * L, d[u]);
    }
#pragma unroll
    for (int o = 1; o < L; o <<= 1) {
        const double ox = __shfl_xor(lx, o), oy = __shfl_xor(ly, o);
        const double qx = __shfl_xor(rx, o), qy = __shfl_xor(ry, o);
        if (oy * lx > ly * ox) {
            lx = ox;
            ly = oy;
        }
        if (qy * rx < ry * qx) {
            rx = qx;
            ry = qy;
        }
    }
    const bool vert = part == 0 && p < nc && (p == 0 || p == nc - 1 || ly * rx < ry * lx);
    const uint64_t b = __ballot(vert);
    if (lane == 0) t.W[24 + wid] = __popcll(b);
    __syncthreads();
    int before = 0, total = 0;
    for (int k = 0; k < nw; ++k) {
        const int c = t.W[24 + k];
        before += (k < wid) ? c : 0;
        total += c;
    }
    const int rank = before + __popcll(b & bits_upto(lane - 1));
    if (vert && p > 0) {
        t.V[rank] = pv;
        t.VXY[rank] = pxy;
    }
    if (tid == 0) t.flag[1] = total;
    return total - 1;
}

// After tile_compact: the tile's hull by wrapping, waves first (each over its
// lanes' node, no barriers), then one wave over the waves' hull vertices.  On
// success the list holds exactly the hull, flag[1] = its length, and true is
// returned (uniformly); otherwise the list is unchanged.  Ends with a barrier.
template <int K, bool ABS>
__device__ inline bool tile_wrap(const Tile& t) {
    const int used = (t.N + K - 1) / K;
    const int lane = lane_id(), wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int nwu = (used + kWave - 1) / kWave;
    const int nv = t.flag[1];
    int* Rw = t.R + wid * kWrapWave;
    if (wid < nwu) {
        const int w0 = wid * kWave;
        const int s = t.I[w0] - 1;
        const int e = (w0 + kWave < used) ? t.I[w0 + kWave] - 1 : nv - 1;
        const int h = wave_wrap_any<K, ABS>(t, s, e, [](int c) { return c; }, Rw, kWrapWave);
        if (lane == 0) t.W[wid] = h;
    }
    __syncthreads();
    int* C = t.R + nw * kWrapWave;  // nw > 1 only
    int* F = C + 4 + nw * kWrapWave;
    int nf = -1;  // hull entries after point 0, in F (or in wave 0's results)
    const int* fin = Rw;
    bool ok = true;
    for (int q = 0; q < nwu; ++q) ok = ok && t.W[q] >= 0;
    if (ok && nwu == 1) {
        nf = t.W[0];
        fin = t.R;
    } else if (ok) {
        // the candidates: point 0, then every wave's vertices in order (a
        // wave's last vertex is the next wave's first point)
        int base = 1, off = 1;
        for (int q = 0; q < nwu; ++q) {
            off += (q < wid) ? t.W[q] : 0;
            base += t.W[q];
        }
        const bool small = base * 2 <= (int)blockDim.x && base <= kWrapTile + 1;  // uniform
        double2* CXY = (double2*)t.M;  // free until the final masks; holds nl / 2 points
        // every wave copies its own vertices to their place among the candidates
        if (wid < nwu) {
            const int h = t.W[wid];
            for (int k = lane; k < h; k += kWave) {
                const int e = Rw[k];
                C[off + k] = e;
                if (ABS && small) CXY[off + k] = t.VXY[e];
            }
        }
        if (threadIdx.x == 0) {
            C[0] = 0;
            if (ABS && small) CXY[0] = t.VXY[0];
        }
        __syncthreads();
        if (small) {
            // the hull goes straight to the front of the list
            if (base * 4 <= (int)blockDim.x)
                (void)tile_hull_small<K, ABS, 4>(t, C, CXY, base);
            else
                (void)tile_hull_small<K, ABS, 2>(t, C, CXY, base);
            __syncthreads();
            return true;
        }
        if (wid == 0) {
            const int h = wave_wrap_any<K, ABS>(t, 0, base - 1, [C](int c) { return C[c]; }, F, kWrapTile);
            wave_sync();
            for (int k = lane; k < h; k += kWave) F[k] = C[F[k]];
            if (lane == 0) t.W[16] = h;
        }
        __syncthreads();
        nf = t.W[16];
        fin = F;
    }
    if (nf < 0) {  // uniform: the rounds take over
        __syncthreads();
        return false;
    }
    // the hull's entries to the front of the list, 64 at a time: entries only
    // move down, so a batch's writes land below every entry a later batch reads
    if (wid == 0) {
        for (int k0 = 0; k0 < nf; k0 += kWave) {
            const int k = k0 + lane;
            unsigned short pv = 0;
            double2 xy = make_double2(0.0, 0.0);
            if (k < nf) {
                pv = t.V[fin[k]];
                xy = t.VXY[fin[k]];
            }
            wave_sync();
            if (k < nf) {
                t.V[k + 1] = pv;
                t.VXY[k + 1] = xy;
            }
            wave_sync();
        }
        if (lane == 0) t.flag[1] = nf + 1;
    }
    __syncthreads();
    return true;
}

// After tile_compact: whether every lane junction of the list turns strictly
// left (the entry before the shared point, the shared point and the entry
// after it); if so the list is one convex chain, and the lanes' masks are
// stored as compacted (I and flag[1] already are).  Block scope; ends with a
// barrier.
template <int K, bool ABS>
__device__ inline bool tile_junctions_left(const Tile& t, uint64_t mask) {
    const int used = (t.N + K - 1) / K, l = threadIdx.x;
    int left = 1;
    if (l >= 1 && l < used) {
        const int s = t.I[l] - 1;  // lane l - 1's end, shared with lane l
        left = (vturn<K, ABS>(t, s - 1, s, s + 1) > 0.0) ? 1 : 0;
    }
    if (!__syncthreads_and(left)) return false;
    t.M[l] = mask;
    __syncthreads();
    return true;
}

// Steps 3a-3d: merges of the lane hulls into the tile's hull.
//   3a. one block-wide compaction writes the list of every lane hull's
//       vertices in order (the lane's points xs, ys are not needed after it);
//       each lane's node is the index range of its vertices and the point
//       before them;
//   3b. rounds inside each wave (nodes of up to 64 lanes) with node ranges
//       passed between lanes by shuffles;
//   3c. the waves' nodes are merged in a tree, one wave per merge;
//   3d. the final lane masks are rebuilt from the list, and I[l] = index of
//       lane l's first vertex.
// On return the sorted vertex list of the whole tile is V, VXY [0, flag[1]).
// With wrap, the output-sensitive finish (tile_wrap) is tried first when the
// lane hulls kept at most 3/5 of the points, and (wrap_max) at most
// wrap_max candidates.  With junctions (chunk coordinates, not ABS), the
// lanes' chains are first tested for a strict left turn at every lane
// junction: the entry before the shared point, the shared point and the entry
// after it, the very triple that each merge below tests first.  When every
// junction turns left, each merge would find its bridge at the shared point
// and move nothing, so the compacted list and masks are final (every point
// of a convex chunk a vertex, the first page's Sec. 7.5 regime).
template <int K, bool ABS>
__device__ inline void tile_merges(const Tile& t, uint64_t& mask, const double (&xs)[K], const double (&ys)[K],
                                   bool wrap = false, int wrap_max = 1 << 30, bool junctions = false) {
    const int used = (t.N + K - 1) / K;
    const int l = threadIdx.x, lane = lane_id(), wid = l >> 6, nw = blockDim.x >> 6;
    const int nwu = (used + kWave - 1) / kWave;  // waves holding elements
    tile_compact<K, ABS>(t, mask, xs, ys);
    if (!ABS && junctions && tile_junctions_left<K, ABS>(t, mask)) return;
    if (wrap && 5 * t.flag[1] <= 3 * t.N + 5 && t.flag[1] <= wrap_max && tile_wrap<K, ABS>(t)) {
        tile_masks_short<K>(t, mask);
        return;
    }
    const int w0 = wid * kWave, wend = min(w0 + kWave, used);
    int ns = t.I[l] - 1;
    int ne = (l + 1 < used) ? t.I[l + 1] - 1 : t.flag[1] - 1;
    for (int h = 1; h < kWave; h <<= 1) {
        if (w0 + h >= wend) break;  // wave-uniform
        const int nm = (wend - w0 - h + 2 * h - 1) / (2 * h);
        int G = kWave;
        while (G > 1 && G * nm > kWave) G >>= 1;
        const int k = lane / G, g = lane & (G - 1);
        const int la = ((k < nm) ? k : 0) * 2 * h;
        const int a0 = __shfl(ns, la, kWave), a1 = __shfl(ne, la, kWave);
        const int b0 = __shfl(ns, la + h, kWave), b1 = __shfl(ne, la + h, kWave);
        int nend = 0;
        if (k < nm) nend = group_merge<K, ABS>(t, a0, a1, b0, b1, g, G);
        const int km = (l < wend) ? (lane / (2 * h)) : nm;
        const int src = (km < nm) ? km * G : 0;
        const int ns2 = __shfl(a0, src, kWave), ne2 = __shfl(nend, src, kWave);
        if (km < nm) {
            ns = ns2;
            ne = ne2;
        }
        wave_sync();
    }
    if (lane == 0 && w0 < used) {
        t.W[wid] = ns;
        t.W[8 + wid] = ne;
    }
    __syncthreads();
    // 3c: a tree over the waves' nodes; at distance s, wave w (a multiple of
    // 2s) merges its node with wave w + s's, all such merges at once (their
    // list ranges are disjoint).
    for (int s = 1; s < nwu; s <<= 1) {
        if ((wid & (2 * s - 1)) == 0 && wid + s < nwu) {
            const int e = group_merge<K, ABS>(t, t.W[wid], t.W[8 + wid], t.W[wid + s], t.W[8 + wid + s], lane, kWave);
            if (lane == 0) t.W[8 + wid] = e;
        }
        __syncthreads();
    }
    if (l == 0) t.flag[1] = t.W[8] + 1;  // wave 0's node starts at entry 0 (point 0)
    tile_masks<K>(t, mask);
    (void)nw;
}

// Step 3d for a short final list (the wrap's): every lane scans the whole
// list for its own vertices (points lK+1 .. lK+K) and counts the vertices
// before them, so no atomics, scans or barriers are needed.  The list must be
// final (a barrier after its last write); M and I are read by others only
// after the next barrier.
template <int K>
__device__ inline void tile_masks_short(const Tile& t, uint64_t& mask) {
    const int l = threadIdx.x, nv = t.flag[1], lo = l * K;
    uint64_t m = 0ull;
    int before = 0;
#pragma unroll 4
    for (int i = 1; i < nv; ++i) {
        const int p = t.V[i];
        before += (p <= lo) ? 1 : 0;
        m |= (p > lo && p <= lo + K) ? (1ull << ((p - 1 - lo) & 63)) : 0ull;
    }
    mask = m;
    t.M[l] = m;
    t.I[l] = 1 + before;
}

// Step 3d: the final lane masks from the list V[0, flag[1]), and I[l] = index
// of lane l's first vertex.  flag[1] is read after the first barrier.
template <int K>
__device__ inline void tile_masks(const Tile& t, uint64_t& mask) {
    const int l = threadIdx.x, lane = lane_id(), wid = l >> 6;
    t.M[l] = 0ull;
    __syncthreads();
    const int nv = t.flag[1];
    for (int i = l; i < nv; i += blockDim.x) {
        const int p = t.V[i];
        if (p > 0) {
            const int ln = (p - 1) / K;
            atomicOr((unsigned long long*)&t.M[ln], 1ull << ((p - 1) - ln * K));
        }
    }
    __syncthreads();
    mask = t.M[l];
    const int pc = __popcll(mask);
    const int incl = wave_incl_scan_int(pc);
    if (lane == kWave - 1) t.W[16 + wid] = incl;
    __syncthreads();
    int r = 1;
    for (int q = 0; q < wid; ++q) r += t.W[16 + q];
    t.I[l] = r + incl - pc;
}

// ---------------------------------------------------------------------------
// 4. expand (Sec. 3.4).  First every edge of the tile's hull gets its value,
// written over the list: VXY[i] = (the slope of the edge from entry i to
// i+1, oriented and clipped; 1 where clipping changed it, else 0).  Then
// every element takes the value of the edge that starts at the last vertex at
// or before its left point: for element lK + j that is list entry I[l] - 1 +
// (number of lane l's vertices among its local points 1..j).
// ---------------------------------------------------------------------------
template <int K, bool ABS>
__device__ inline void tile_edge_slopes(const Tile& t, int increasing, double clo, double chi) {
    const int nv = t.flag[1];
    double sv[K + 1];
    bool cv[K + 1];
#pragma unroll
    for (int k = 0; k <= K; ++k) {
        const int i = threadIdx.x + k * t.nl;
        sv[k] = 0.0;
        cv[k] = false;
        if (k * t.nl < nv - 1 && i < nv - 1) {  // the first test is uniform
            const double2 d = vdiff<K, ABS>(t, i, i + 1);
            sv[k] = finish(d.y / d.x, increasing, clo, chi, cv[k]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k <= K; ++k) {
        const int i = threadIdx.x + k * t.nl;
        if (k * t.nl < nv - 1 && i < nv - 1) t.VXY[i] = make_double2(sv[k], cv[k] ? 1.0 : 0.0);
    }
    __syncthreads();
}

// Values of the calling lane's elements into vals[0..cnt); clip flags into
// clipm (bit j <-> element lK + j).
template <int K>
__device__ inline void tile_expand(const Tile& t, uint64_t mask, double (&vals)[K], uint64_t& clipm) {
    const int l = threadIdx.x;
    const int cnt = min(max(t.N - l * K, 0), K);
    const int i0 = t.I[l] - 1;
    clipm = 0ull;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        vals[j] = 0.0;
        if (j < cnt) {
            const double2 e = t.VXY[i0 + __popcll(mask & bits_upto(j - 1))];
            vals[j] = e.x;
            if (e.y != 0.0) clipm |= 1ull << j;
        }
    }
}

// Block-start and clip bit words of the tile's elements (the tile starts at
// a multiple of 64 elements).  Element i >= 1 starts a block iff point i is a
// vertex; element 0 always does.  Lane masks are K bits wide: concatenated,
// bit lK + b stands for point lK + b + 1.  Needs M and CM written and a
// barrier.
template <int K>
__device__ inline void tile_bits(const Tile& t, uint64_t* __restrict__ sbits, uint64_t* __restrict__ cbits) {
    const int words = (t.N + 63) / 64;
    for (int q = threadIdx.x; q < words; q += blockDim.x) {
        uint64_t cm = 0ull, vm = 0ull;  // bit j <-> element 64q + j (vm: its right point is a vertex)
        const int e0 = 64 * q;
        const int l1 = min((e0 + 63) / K, t.nl - 1);
        for (int l = e0 / K; l <= l1; ++l) {
            const int off = l * K - e0;  // > -K
            const uint64_t m = t.M[l] & bits_upto(K - 1), c = t.CM[l] & bits_upto(K - 1);
            vm |= (off >= 0) ? (m << off) : (m >> -off);
            cm |= (off >= 0) ? (c << off) : (c >> -off);
        }
        // element i starts a block when its left point P_i is a vertex: the
        // right point of element i-1 (P_0 always)
        const uint64_t carry = (q == 0) ? 1ull : ((t.M[(e0 - 1) / K] >> ((e0 - 1) % K)) & 1ull);
        const uint64_t s = (vm << 1) | carry;
        const int cnt = t.N - e0;
        const uint64_t valid = (cnt >= 64) ? ~0ull : ((1ull << cnt) - 1ull);
        sbits[q] = s & valid;
        cbits[q] = cm & valid;
    }
}

}  // namespace iso
