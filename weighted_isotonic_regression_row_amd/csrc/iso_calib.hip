// Calibration curves (first page, Sec. 7.7; "torchisotonic" PyPI page, "What
// it is for": scikit-learn's IsotonicRegression curve) and their evaluation.
//
// Per row of scores and labels:
//   k_cal_sort     tiles of at most 2048 scores sorted in increasing order by
//                  one workgroup each (the network of iso_sort.hpp over
//                  (key, index) entries, equal scores in index order);
//   k_cal_merge    runs of 2048, 4096, ... merged pairwise until the row is
//                  one run (merge path, one workgroup per 2048 outputs staged
//                  through LDS);
//   k_cal_pool1    per tile of 2048 sorted scores: how many distinct scores
//                  start in it (a score differs from its predecessor), the
//                  double-double sum of its labels, their largest value, NaNs;
//   k_cal_pool2    per row: exclusive scan of those over the tiles, the number
//                  m of distinct scores, a NaN flag;
//   k_cal_pool3    per tile: for every distinct score, where its run of equal
//                  scores starts and the double-double label prefix there;
//   k_cal_pool4    per distinct score: the pooled mean (difference of two
//                  prefixes over the run's length) and the run's length as its
//                  weight; the row is padded to n with its largest label,
//                  which never pools below the data;
//   launch_fit     the non-decreasing weighted fit of the pooled means;
//   k_cal_predict  per query: linear between the curve's points, constant
//                  beyond them.
#include <math.h>

#include "iso_device.hpp"
#include "iso_compose.hpp"
#include "iso_internal.hpp"
#include "iso_sort.hpp"

namespace iso {
namespace {

// Tiles of 2048 (256 threads, 24 KiB of LDS for float64) keep six workgroups
// on a CU; measured on 6.5e6 float64 scores: 1.46 ms per curve against 1.62 ms
// with tiles of 8192 (one workgroup per CU, two fewer merge passes).
constexpr int kCalSortTile = 2048;
constexpr int kPoolTile = 2048;  // 256 threads x 8
constexpr int kMergeOut = 8;     // outputs per thread of a merge pass

// The network sorts in decreasing order of the key.  Scores are sorted in
// increasing order by sorting -score (neg = 1); the soft rank sorts x itself
// (neg = 0).  Equal values, -0 and +0 included, keep index order.
template <typename T>
__device__ __forceinline__ Ent cal_entry(T x, uint32_t idx, int neg) {
    Ent e;
    const T v = neg ? -x : x;
    if constexpr (sizeof(T) == 4) {
        e.k = ((uint64_t)sort_key((float)v) << 32) | (uint32_t)~idx;
        e.i = 0u;
    } else {
        e.k = sort_key((double)v);
        e.i = idx;
    }
    return e;
}

struct CalSortArgs {
    const void* s;
    uint64_t* K;
    uint32_t* I;
    int64_t n;
    int tiles;  // per row
    int P;      // network width of a tile
    int neg;    // sort -x (increasing order of x) instead of x
};

template <typename T, int E>
__global__ __launch_bounds__(1024) void k_cal_sort(CalSortArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int64_t row = blockIdx.x / a.tiles;
    const int tile = blockIdx.x % a.tiles;
    const int64_t t0 = (int64_t)tile * kCalSortTile;
    const int len = (int)min((int64_t)kCalSortTile, a.n - t0);
    const int t = threadIdx.x, p0 = t * E;
    const int cnt = min(max(len - p0, 0), E);
    const int64_t base = row * a.n + t0;
    double xv[E];
    load_lane<T, E>((const T*)a.s + base + p0, cnt, xv);
    Ent v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (e < cnt) {
            v[e] = cal_entry<T>((T)xv[e], (uint32_t)(t0 + p0 + e), a.neg);
        } else {
            v[e].k = 0ull;
            v[e].i = 0xffffffffu;
        }
    }
    sort_entries<T, E>(v, t, a.P, (uint64_t*)smem, (uint32_t*)(smem + 8 * (size_t)a.P));
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (e < cnt) {
            a.K[base + p0 + e] = v[e].k;
            if constexpr (sizeof(T) == 8) a.I[base + p0 + e] = v[e].i;
        }
    }
}

struct CalMergeArgs {
    const uint64_t* Ki;
    const uint32_t* Ii;
    uint64_t* Ko;
    uint32_t* Io;
    int64_t n;
    int64_t L;  // run length of the input
};

template <typename T>
__device__ __forceinline__ Ent ld_ent(const uint64_t* K, const uint32_t* I, int64_t at) {
    Ent e;
    e.k = K[at];
    e.i = sizeof(T) == 4 ? 0u : I[at];
    return e;
}

// How many of the first d outputs of merging A (lenA) and B (lenB) come from A.
template <typename T, typename LdA, typename LdB>
__device__ __forceinline__ int64_t co_rank(int64_t d, int64_t lenA, int64_t lenB, LdA A, LdB B) {
    int64_t lo = d - lenB > 0 ? d - lenB : 0, hi = d < lenA ? d : lenA;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (before<T>(B(d - mid - 1), A(mid)))
            hi = mid;
        else
            lo = mid + 1;
    }
    return lo;
}

// One workgroup per kMergeTile outputs of a pair of runs (2L is a multiple of
// kMergeTile, so a tile never straddles two pairs): the tile's two input
// slices are found by bisection, loaded into LDS with coalesced reads, merged
// there (each thread bisects its own start, then takes eight outputs), and
// stored back through the same LDS with coalesced writes.
constexpr int kMergeTile = 256 * kMergeOut;

template <typename T>
__global__ __launch_bounds__(256) void k_cal_merge(CalMergeArgs a) {
    __shared__ uint64_t SK[kMergeTile];
    __shared__ uint32_t SI[sizeof(T) == 8 ? kMergeTile : 1];
    __shared__ int64_t cr[2];
    const int64_t tiles = (a.n + kMergeTile - 1) / kMergeTile;
    const int64_t row = blockIdx.x / tiles;
    const int64_t o0 = (blockIdx.x % tiles) * kMergeTile;
    const int64_t o1 = min(o0 + (int64_t)kMergeTile, a.n);
    const int64_t b = o0 - o0 % (2 * a.L);
    const int64_t a1 = min(b + a.L, a.n), b1 = min(b + 2 * a.L, a.n);
    const int64_t lenA = a1 - b, lenB = b1 - a1;
    const int64_t rb = row * a.n;
    const uint64_t* KA = a.Ki + rb + b;
    const uint64_t* KB = a.Ki + rb + a1;
    const uint32_t* IA = sizeof(T) == 8 ? a.Ii + rb + b : nullptr;
    const uint32_t* IB = sizeof(T) == 8 ? a.Ii + rb + a1 : nullptr;
    auto gA = [&](int64_t i) { return ld_ent<T>(KA, IA, i); };
    auto gB = [&](int64_t j) { return ld_ent<T>(KB, IB, j); };
    if (threadIdx.x < 2) cr[threadIdx.x] = co_rank<T>((threadIdx.x ? o1 : o0) - b, lenA, lenB, gA, gB);
    __syncthreads();
    const int64_t i0 = cr[0], i1 = cr[1];
    const int64_t j0 = (o0 - b) - i0, j1 = (o1 - b) - i1;
    const int na = (int)(i1 - i0), nb = (int)(j1 - j0), cnt = na + nb;
    for (int q = threadIdx.x; q < cnt; q += 256) {
        const int64_t at = q < na ? i0 + q : j0 + (q - na);
        const uint64_t* K = q < na ? KA : KB;
        SK[q] = K[at];
        if constexpr (sizeof(T) == 8) SI[q] = (q < na ? IA : IB)[at];
    }
    __syncthreads();
    auto lA = [&](int64_t i) {
        Ent e;
        e.k = SK[i];
        e.i = sizeof(T) == 8 ? SI[i] : 0u;
        return e;
    };
    auto lB = [&](int64_t j) {
        Ent e;
        e.k = SK[na + j];
        e.i = sizeof(T) == 8 ? SI[na + j] : 0u;
        return e;
    };
    const int d = threadIdx.x * kMergeOut;
    Ent out[kMergeOut];
    int took = 0;
    if (d < cnt) {
        int i = (int)co_rank<T>(d, na, nb, lA, lB), j = d - i;
#pragma unroll
        for (int s2 = 0; s2 < kMergeOut; ++s2) {
            if (d + s2 < cnt) {
                const bool takeA = j >= nb || (i < na && !before<T>(lB(j), lA(i)));
                out[s2] = takeA ? lA(i) : lB(j);
                i += takeA ? 1 : 0;
                j += takeA ? 0 : 1;
                ++took;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int s2 = 0; s2 < kMergeOut; ++s2) {
        if (s2 < took) {
            SK[d + s2] = out[s2].k;
            if constexpr (sizeof(T) == 8) SI[d + s2] = out[s2].i;
        }
    }
    __syncthreads();
    for (int q = threadIdx.x; q < cnt; q += 256) {
        a.Ko[rb + o0 + q] = SK[q];
        if constexpr (sizeof(T) == 8) a.Io[rb + o0 + q] = SI[q];
    }
}

// The sorted entry at position p of a row: the score's key (equal scores have
// equal keys), its index, and the score.
template <typename T>
__device__ __forceinline__ uint64_t ent_key(const uint64_t* K, int64_t at) {
    return sizeof(T) == 4 ? (K[at] >> 32) : K[at];
}
template <typename T>
__device__ __forceinline__ uint32_t ent_idx(const uint64_t* K, const uint32_t* I, int64_t at) {
    return sizeof(T) == 4 ? ~(uint32_t)K[at] : I[at];
}
template <typename T>
__device__ __forceinline__ double ent_score(const uint64_t* K, int64_t at) {
    if constexpr (sizeof(T) == 4)
        return -(double)key_value((uint32_t)(K[at] >> 32));
    else
        return -key_value(K[at]);
}

struct PoolArgs {
    const uint64_t* K;
    const uint32_t* I;
    const void* labels;
    int64_t n;
    int tiles;        // pool tiles per row
    double4* trec;    // [rows * tiles]: (label sum hi, lo, distinct scores starting, 0), then their exclusive prefix
    double* tmax;     // [rows * tiles]
    int* tnan;        // [rows * tiles]
    double4* rtot;    // [rows]: (label sum hi, lo, m, largest label)
    int* rnan;        // [rows]
    int32_t* m;       // [rows] output
    int32_t* start;   // [rows * n] start of each distinct score's run
    double2* pst;     // [rows * n] label prefix (double-double) at that start
    void* ys;         // [rows * n] labels in score order (written by pool1)
    void* xs;         // [rows * n] output
    void* yp;         // [rows * n] pooled means, padded
    void* wp;         // [rows * n] run lengths, padded
};

// Workgroup reduction of (double-double, double-double) pairs in a fixed order.
__device__ inline double4 block_sum_dd(double4 v, double4* red) {
    const int lane = lane_id(), wid = threadIdx.x >> 6;
    v = wave_scan_incl(v, [](double4 a, double4 b) { return dd4_add(a, b); });
    if (lane == kWave - 1) red[wid] = v;
    __syncthreads();
    double4 s = make_double4(0.0, 0.0, 0.0, 0.0);
    for (int k = 0; k < (int)(blockDim.x >> 6); ++k) s = dd4_add(s, red[k]);
    __syncthreads();
    return s;
}

template <typename T>
__global__ __launch_bounds__(256) void k_cal_pool1(PoolArgs a) {
    __shared__ double4 red[4];
    __shared__ double mred[4];
    __shared__ int nred;
    const int64_t row = blockIdx.x / a.tiles;
    const int tile = blockIdx.x % a.tiles;
    const int64_t rb = row * a.n;
    const int64_t p0 = (int64_t)tile * kPoolTile + threadIdx.x * 8;
    const T* lab = (const T*)a.labels + rb;
    if (threadIdx.x == 0) nred = 0;
    double sh = 0.0, sl = 0.0, heads = 0.0, mx = -INFINITY;
    bool bad = false;
    for (int e = 0; e < 8; ++e) {
        const int64_t p = p0 + e;
        if (p >= a.n) break;
        const uint64_t key = ent_key<T>(a.K, rb + p);
        if (p == 0 || key != ent_key<T>(a.K, rb + p - 1)) heads += 1.0;
        const T yv = lab[ent_idx<T>(a.K, a.I, rb + p)];
        ((T*)a.ys)[rb + p] = yv;
        const double y = (double)yv;
        bad |= isnan(y) || isnan(ent_score<T>(a.K, rb + p));
        dd_add(sh, sl, y, 0.0, sh, sl);
        mx = fmax(mx, y);
    }
    const double4 s = block_sum_dd(make_double4(sh, sl, heads, 0.0), red);
    double m = mx;
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) m = fmax(m, __shfl_xor(m, k));
    if (lane_id() == 0) mred[threadIdx.x >> 6] = m;
    if (bad) atomicOr(&nred, 1);
    __syncthreads();
    if (threadIdx.x == 0) {
        double all = mred[0];
        for (int k = 1; k < (int)(blockDim.x >> 6); ++k) all = fmax(all, mred[k]);
        const int64_t at = row * a.tiles + tile;
        a.trec[at] = make_double4(s.x, s.y, s.z, 0.0);
        a.tmax[at] = all;
        a.tnan[at] = nred;
    }
}

// One workgroup per row: exclusive prefix of the tile records, in chunks of
// blockDim.x tiles with a running carry.
__global__ __launch_bounds__(256) void k_cal_pool2(PoolArgs a) {
    __shared__ double4 red[4];
    __shared__ double4 incl[256];
    __shared__ double mred[4];
    __shared__ int nred;
    const int64_t row = blockIdx.x;
    double4* tr = a.trec + row * a.tiles;
    if (threadIdx.x == 0) nred = 0;
    double4 carry = make_double4(0.0, 0.0, 0.0, 0.0);
    double mx = -INFINITY;
    bool bad = false;
    for (int c0 = 0; c0 < a.tiles; c0 += blockDim.x) {
        const int t = c0 + threadIdx.x;
        const bool in = t < a.tiles;
        const double4 v = in ? tr[t] : make_double4(0.0, 0.0, 0.0, 0.0);
        if (in) {
            mx = fmax(mx, a.tmax[row * a.tiles + t]);
            bad |= a.tnan[row * a.tiles + t] != 0;
        }
        const int lane = lane_id(), wid = threadIdx.x >> 6;
        const double4 w = wave_scan_incl(v, [](double4 x, double4 y) { return dd4_add(x, y); });
        if (lane == kWave - 1) red[wid] = w;
        __syncthreads();
        double4 before_w = carry;
        double4 chunk = make_double4(0.0, 0.0, 0.0, 0.0);
        for (int k = 0; k < (int)(blockDim.x >> 6); ++k) {
            if (k < wid) before_w = dd4_add(before_w, red[k]);
            chunk = dd4_add(chunk, red[k]);
        }
        incl[threadIdx.x] = dd4_add(before_w, w);
        __syncthreads();
        if (in) tr[t] = threadIdx.x == 0 ? carry : incl[threadIdx.x - 1];
        carry = dd4_add(carry, chunk);
        __syncthreads();
    }
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) mx = fmax(mx, __shfl_xor(mx, k));
    if (lane_id() == 0) mred[threadIdx.x >> 6] = mx;
    if (bad) atomicOr(&nred, 1);
    __syncthreads();
    if (threadIdx.x == 0) {
        double all = mred[0];
        for (int k = 1; k < (int)(blockDim.x >> 6); ++k) all = fmax(all, mred[k]);
        a.rtot[row] = make_double4(carry.x, carry.y, carry.z, all);
        a.rnan[row] = nred;
        a.m[row] = nred ? 0 : (int32_t)carry.z;
    }
}

template <typename T>
__global__ __launch_bounds__(256) void k_cal_pool3(PoolArgs a) {
    __shared__ double4 red[4];
    const int64_t row = blockIdx.x / a.tiles;
    const int tile = blockIdx.x % a.tiles;
    const int64_t rb = row * a.n;
    const int64_t p0 = (int64_t)tile * kPoolTile + threadIdx.x * 8;
    const T* ys = (const T*)a.ys + rb;
    double y[8];
    bool head[8];
    double sh = 0.0, sl = 0.0, heads = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int64_t p = p0 + e;
        y[e] = 0.0;
        head[e] = false;
        if (p < a.n) {
            const uint64_t key = ent_key<T>(a.K, rb + p);
            head[e] = p == 0 || key != ent_key<T>(a.K, rb + p - 1);
            y[e] = (double)ys[p];
        }
        dd_add(sh, sl, y[e], 0.0, sh, sl);
        heads += head[e] ? 1.0 : 0.0;
    }
    // exclusive prefix of the threads before this one, plus the tile's
    const int lane = lane_id(), wid = threadIdx.x >> 6;
    const double4 own = make_double4(sh, sl, heads, 0.0);
    const double4 w = wave_scan_incl(own, [](double4 x, double4 z) { return dd4_add(x, z); });
    if (lane == kWave - 1) red[wid] = w;
    __syncthreads();
    double4 pre = a.trec[row * a.tiles + tile];
    for (int k = 0; k < wid; ++k) pre = dd4_add(pre, red[k]);
    pre = dd4_add(pre, wave_shift_up1(w));
    double ph = pre.x, pl = pre.y;
    int64_t g = (int64_t)pre.z;  // distinct scores before this thread's first position
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int64_t p = p0 + e;
        if (p < a.n && head[e]) {
            a.start[rb + g] = (int32_t)p;
            a.pst[rb + g] = make_double2(ph, pl);
            ++g;
        }
        dd_add(ph, pl, y[e], 0.0, ph, pl);
    }
}

template <typename T>
__global__ __launch_bounds__(256) void k_cal_pool4(PoolArgs a, int64_t total) {
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total; q += (int64_t)gridDim.x * 256) {
        const int64_t row = q / a.n, g = q - row * a.n, rb = row * a.n;
        const double4 rt = a.rtot[row];
        const int64_t m = (int64_t)rt.z;
        T* xs = (T*)a.xs + rb;
        T* yp = (T*)a.yp + rb;
        T* wp = (T*)a.wp + rb;
        if (a.rnan[row]) {
            xs[g] = (T)NAN;
            yp[g] = (T)NAN;
            wp[g] = (T)1;
        } else if (g < m) {
            const int64_t s = a.start[rb + g];
            const int64_t e = g + 1 < m ? (int64_t)a.start[rb + g + 1] : a.n;
            const double2 ps = a.pst[rb + g];
            const double2 pe = g + 1 < m ? a.pst[rb + g + 1] : make_double2(rt.x, rt.y);
            const double sum = (pe.x - ps.x) + (pe.y - ps.y);
            xs[g] = (T)ent_score<T>(a.K, rb + s);
            yp[g] = (T)(sum / (double)(e - s));
            wp[g] = (T)(double)(e - s);
        } else {
            xs[g] = (T)NAN;
            yp[g] = (T)rt.w;  // the row's largest label: never below a data block's mean
            wp[g] = (T)1;
        }
    }
}

struct PredArgs {
    const void* xs;
    const void* fit;
    const int32_t* m;
    const void* q;
    void* out;
    int64_t n, k, total;
};

template <typename T>
__global__ __launch_bounds__(256) void k_cal_predict(PredArgs a) {
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < a.total; e += (int64_t)gridDim.x * 256) {
        const int64_t row = e / a.k;
        const int64_t mr = a.m[row];
        const int64_t m = mr < 0 ? 0 : (mr > a.n ? a.n : mr);  // a caller's m never reads past the row
        const double q = (double)((const T*)a.q)[e];
        const T* x = (const T*)a.xs + row * a.n;
        const T* f = (const T*)a.fit + row * a.n;
        double r;
        if (m == 0 || isnan(q)) {
            r = NAN;
        } else if (m == 1) {
            r = (double)f[0];
        } else {
            int64_t lo = 0, hi = m;  // first i with x[i] >= q
            while (lo < hi) {
                const int64_t mid = (lo + hi) >> 1;
                if ((double)x[mid] < q)
                    lo = mid + 1;
                else
                    hi = mid;
            }
            const int64_t i = lo < 1 ? 1 : (lo > m - 1 ? m - 1 : lo);
            const double x0 = (double)x[i - 1], x1 = (double)x[i];
            double t = (q - x0) / (x1 - x0);
            t = t < 0.0 ? 0.0 : (t > 1.0 ? 1.0 : t);
            const double f0 = (double)f[i - 1];
            r = f0 + t * ((double)f[i] - f0);
        }
        ((T*)a.out)[e] = (T)r;
    }
}

unsigned grid_of(int64_t threads) {
    const int64_t b = (threads + 255) / 256;
    return (unsigned)(b < 65536 ? b : 65536);
}

template <typename T, int E>
hipError_t launch_cal_sort(const CalSortArgs& s, int64_t rows, hipStream_t stream) {
    const int nt = s.P / E;
    const size_t lds = nt > 64 ? (size_t)s.P * (sizeof(T) == 4 ? 8 : 12) : 0;
    static size_t seen[kMaxDevices];
    if (lds > 0) {
        const hipError_t e = ensure_lds((const void*)k_cal_sort<T, E>, lds, seen);
        if (e != hipSuccess) return e;
    }
    k_cal_sort<T, E><<<dim3((unsigned)(rows * s.tiles)), dim3(nt), lds, stream>>>(s);
    return hipGetLastError();
}

// Every row sorted by tiles and merge passes into K[cur], I[cur] (indices
// within the row; float32 keeps them in the key's low word).
template <typename T>
hipError_t sort_rows_t(const void* x, int64_t rows, int64_t n, int neg, uint64_t* const K[2], uint32_t* const I[2],
                       hipStream_t stream, int& cur) {
    // 1. sorted tiles
    CalSortArgs s{};
    s.s = x;
    s.K = K[0];
    s.I = I[0];
    s.n = n;
    s.tiles = (int)((n + kCalSortTile - 1) / kCalSortTile);
    s.neg = neg;
    int P = 64;
    while (P < n && P < kCalSortTile) P <<= 1;
    s.P = P;
    hipError_t e;
    switch (P) {
        case 64:
            e = launch_cal_sort<T, 1>(s, rows, stream);
            break;
        case 128:
            e = launch_cal_sort<T, 2>(s, rows, stream);
            break;
        case 256:
            e = launch_cal_sort<T, 4>(s, rows, stream);
            break;
        default:
            e = launch_cal_sort<T, 8>(s, rows, stream);
    }
    if (e != hipSuccess) return e;
    // 2. merges
    cur = 0;
    for (int64_t L = kCalSortTile; L < n; L *= 2) {
        CalMergeArgs m{};
        m.Ki = K[cur];
        m.Ii = sizeof(T) == 8 ? I[cur] : nullptr;
        m.Ko = K[cur ^ 1];
        m.Io = sizeof(T) == 8 ? I[cur ^ 1] : nullptr;
        m.n = n;
        m.L = L;
        const int64_t tiles = (n + kMergeTile - 1) / kMergeTile;
        k_cal_merge<T><<<dim3((unsigned)(rows * tiles)), dim3(256), 0, stream>>>(m);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        cur ^= 1;
    }
    return hipSuccess;
}

template <typename T>
hipError_t cal_fit_t(const CalLaunch& l) {
    const int64_t rows = l.rows, n = l.n;
    char* ws = l.ws;
    uint64_t* const K[2] = {(uint64_t*)(ws + l.C.k0), (uint64_t*)(ws + l.C.k1)};
    uint32_t* const I[2] = {(uint32_t*)(ws + l.C.i0), (uint32_t*)(ws + l.C.i1)};
    int cur = 0;
    hipError_t e = sort_rows_t<T>(l.scores, rows, n, 1, K, I, l.stream, cur);
    if (e != hipSuccess) return e;
    // 3. pooling of equal scores
    PoolArgs p{};
    p.K = K[cur];
    p.I = I[cur];
    p.labels = l.labels;
    p.n = n;
    p.tiles = (int)((n + kPoolTile - 1) / kPoolTile);
    p.trec = (double4*)(ws + l.C.trec);
    p.tmax = (double*)(ws + l.C.tmax);
    p.tnan = (int*)(ws + l.C.tnan);
    p.rtot = (double4*)(ws + l.C.rtot);
    p.rnan = (int*)(ws + l.C.rnan);
    p.m = l.m;
    p.start = (int32_t*)(ws + l.C.start);
    p.pst = (double2*)(ws + l.C.pst);
    p.ys = ws + l.C.ys;
    p.xs = l.xs;
    p.yp = ws + l.C.yp;
    p.wp = ws + l.C.wp;
    const unsigned ptiles = (unsigned)(rows * p.tiles);
    k_cal_pool1<T><<<dim3(ptiles), dim3(256), 0, l.stream>>>(p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_cal_pool2<<<dim3((unsigned)rows), dim3(256), 0, l.stream>>>(p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_cal_pool3<T><<<dim3(ptiles), dim3(256), 0, l.stream>>>(p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_cal_pool4<T><<<dim3(grid_of(rows * n)), dim3(256), 0, l.stream>>>(p, rows * n);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // 4. the curve: non-decreasing fit of the pooled means, run lengths as weights
    FitLaunch f{};
    f.y = ws + l.C.yp;
    f.w = ws + l.C.wp;
    f.fit = l.fit;
    f.rows = rows;
    f.n = n;
    f.increasing = 1;
    f.dtype = l.dtype;
    f.lo = -INFINITY;
    f.hi = INFINITY;
    f.words = (n + 63) / 64;
    f.ws = ws;
    f.L = l.C.L;
    f.epoch = 0;
    f.stream = l.stream;
    return launch_fit(f);
}

template <typename T>
hipError_t cal_predict_t(const CalPredictLaunch& l) {
    PredArgs a{};
    a.xs = l.xs;
    a.fit = l.fit;
    a.m = l.m;
    a.q = l.q;
    a.out = l.out;
    a.n = l.n;
    a.k = l.k;
    a.total = l.rows * l.k;
    k_cal_predict<T><<<dim3(grid_of(a.total)), dim3(256), 0, l.stream>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_calibration_fit(const CalLaunch& l) {
    return l.dtype == 0 ? cal_fit_t<float>(l) : cal_fit_t<double>(l);
}

hipError_t launch_sort_rows(int dtype, const void* x, int64_t rows, int64_t n, int neg, uint64_t* const K[2],
                           uint32_t* const I[2], hipStream_t stream, int& cur) {
    return dtype == 0 ? sort_rows_t<float>(x, rows, n, neg, K, I, stream, cur)
                      : sort_rows_t<double>(x, rows, n, neg, K, I, stream, cur);
}

hipError_t launch_calibrate(const CalPredictLaunch& l) {
    return l.dtype == 0 ? cal_predict_t<float>(l) : cal_predict_t<double>(l);
}

}  // namespace iso
