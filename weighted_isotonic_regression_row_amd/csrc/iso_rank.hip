// Soft rank with quadratic regularization and its vector-Jacobian product
// (first page, Sec. 7.9, after Blondel et al.).
//
// Forward, per row: theta = x / eps is sorted in decreasing order into s;
// z = s - (n, n-1, ..., 1) is fitted non-increasing with unit weights by the
// library's own solver, and the element at sorted position i gets the rank
// s_i - v_i, written back in the original order.  Rows of 65 to 512 elements
// run all of it in one kernel (k_rank_fused); other rows take these steps:
//   k_rank_sort    one workgroup per row: a bitonic network over (key, index)
//                  pairs in LDS, where key is an order-preserving unsigned image
//                  of x (theta has the order of x as eps > 0), ties broken by the
//                  lower index first; writes perm, its inverse rank, and z in the
//                  data type, into the sorted order;
//   launch_fit     the fit of z and its block bits (the partition the backward
//                  pass uses), over the sorted order;
//   k_rank_finish  r[k] = x[k] / eps - v[rank[k]], element-wise.
// Rows longer than one workgroup sorts (8192) are sorted like the calibration
// scores (tiles of 2048 and merge passes, launch_sort_rows), and k_rank_long_z
// then forms perm, rank and z from the sorted entries.
// Backward, with g_s the upstream gradient in sorted order and A the block
// averaging of the fit: d/dx = P^T (g_s - A g_s) / eps.
//   k_rank_gather      g_s[i] = g[perm[i]];
//   launch_vjp         A g_s over the fit's blocks;
//   k_rank_vjp_finish  grad[k] = (g[k] - (A g_s)[rank[k]]) / eps.
#include <math.h>

#include "iso_compose.hpp"
#include "iso_device.hpp"
#include "iso_internal.hpp"
#include "iso_sort.hpp"
#include "iso_tile.hpp"

namespace iso {
namespace {

struct SortArgs {
    const void* x;
    int32_t* perm;
    int32_t* rank;
    void* z;
    int n;
    int P;  // power of two >= n, at least 64; P / E threads
    double eps;
};

template <typename T, int E>
__global__ __launch_bounds__(1024) void k_rank_sort(SortArgs a) {
    extern __shared__ __align__(32) char smem[];
    const int n = a.n, P = a.P, t = threadIdx.x;
    const int64_t row0 = (int64_t)blockIdx.x * n;
    const int p0 = t * E;
    const int cnt = min(max(n - p0, 0), E);
    double xv[E];
    load_lane<T, E>((const T*)a.x + row0 + p0, cnt, xv);
    Ent v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const bool real = e < cnt;
        const T x = (T)xv[e];
        if constexpr (sizeof(T) == 4) {
            v[e].k = real ? (((uint64_t)sort_key(x) << 32) | (uint32_t)~(uint32_t)(p0 + e)) : 0ull;
            v[e].i = 0u;
        } else {
            v[e].k = real ? sort_key(x) : 0ull;
            v[e].i = real ? (uint32_t)(p0 + e) : 0xffffffffu;
        }
    }
    sort_entries<T, E>(v, t, P, (uint64_t*)smem, (uint32_t*)(smem + 8 * (size_t)P));
    // thread t now holds sorted positions p0 .. p0+E-1; padding sorts last,
    // so every position below n holds an element of the row
    int32_t* perm = a.perm + row0;
    int32_t* rank = a.rank + row0;
    double zv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        int idx;
        double x;
        if constexpr (sizeof(T) == 4) {
            idx = (int)~(uint32_t)v[e].k;
            x = (double)key_value((uint32_t)(v[e].k >> 32));
        } else {
            idx = (int)v[e].i;
            x = key_value(v[e].k);
        }
        zv[e] = x / a.eps - (double)(n - (p0 + e));
        if (e < cnt) {
            perm[p0 + e] = idx;
            if ((unsigned)idx < (unsigned)n) rank[idx] = p0 + e;
        }
    }
    store_lane<T, E>((T*)a.z + row0 + p0, cnt, zv);
}

// Rows of 65 to 512 elements in one kernel, one wave per row.  After the
// sort, lane l holds sorted positions lE .. lE+E-1, which is the layout of
// the one-wave fit tile with E points per lane: z = s - (n..1) goes from the
// sort's registers into the lane hulls, the tile keeps every vertex in LDS
// (no overflow pass), and each element's rank s - v is stored straight to its
// original position.
struct FusedArgs {
    const void* x;
    void* r;
    int32_t* perm;
    int32_t* rank;
    uint64_t* start_bits;
    uint64_t* clip_bits;
    uint32_t* row_nan;
    int64_t words;
    int n;
    double eps;
};

template <typename T, int E>
__global__ __launch_bounds__(64) void k_rank_fused(FusedArgs a) {
    extern __shared__ __align__(32) char smem[];
    const int n = a.n, t = threadIdx.x, p0 = t * E;
    const int64_t row = blockIdx.x;
    const int64_t row0 = row * n;
    const int cnt = min(max(n - p0, 0), E);
    double xv[E];
    load_lane<T, E>((const T*)a.x + row0 + p0, cnt, xv);
    Ent v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const bool real = e < cnt;
        const T x = (T)xv[e];
        if constexpr (sizeof(T) == 4) {
            v[e].k = real ? (((uint64_t)sort_key(x) << 32) | (uint32_t)~(uint32_t)(p0 + e)) : 0ull;
            v[e].i = 0u;
        } else {
            v[e].k = real ? sort_key(x) : 0ull;
            v[e].i = real ? (uint32_t)(p0 + e) : 0xffffffffu;
        }
    }
    sort_entries<T, E>(v, t, 64 * E, nullptr, nullptr);  // every partner is inside the wave
    int idx[E];
    double sv[E], z[E];
    int32_t* perm = a.perm + row0;
    int32_t* rank = a.rank + row0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        double x;
        if constexpr (sizeof(T) == 4) {
            idx[e] = (int)~(uint32_t)v[e].k;
            x = (double)key_value((uint32_t)(v[e].k >> 32));
        } else {
            idx[e] = (int)v[e].i;
            x = key_value(v[e].k);
        }
        sv[e] = x / a.eps;
        z[e] = sv[e] - (double)(n - (p0 + e));
        if (e < cnt) {
            perm[p0 + e] = idx[e];
            if ((unsigned)idx[e] < (unsigned)n) rank[idx[e]] = p0 + e;
        }
    }
    // the non-increasing fit of z over the sorted positions (tile pipeline)
    constexpr bool ABS = sizeof(T) == 4;
    const Tile tl = tile_carve(smem, 64, n, E, n);
    double xs[E], ys[E];
    int f = 0;
    uint64_t mask = lane_hull_vals<E>(z, cnt, 1, xs, ys, f);
    (void)tile_lane_starts<!ABS>(tl, make_double2(xs[E - 1], ys[E - 1]), f, __popcll(mask));
    uint64_t* sb = a.start_bits + row * a.words;
    uint64_t* cb = a.clip_bits + row * a.words;
    T* r = (T*)a.r + row0;
    if (tl.flag[0]) {  // a NaN in the row
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (e < cnt && (unsigned)idx[e] < (unsigned)n) r[idx[e]] = (T)NAN;
        for (int q = t; q < (int)a.words; q += 64) {
            sb[q] = 0ull;
            cb[q] = 0ull;
        }
        if (t == 0) a.row_nan[row] = 1u;
        return;
    }
    tile_merges<E, ABS>(tl, mask, xs, ys, true);
    tile_edge_slopes<E, ABS>(tl, 0, -INFINITY, INFINITY);
    double vals[E];
    uint64_t clipm;
    tile_expand<E>(tl, mask, vals, clipm);
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (e < cnt && (unsigned)idx[e] < (unsigned)n) r[idx[e]] = (T)(sv[e] - vals[e]);
    tl.CM[t] = clipm;
    __syncthreads();
    tile_bits<E>(tl, sb, cb);
    if (t == 0) a.row_nan[row] = 0u;
}

// Element-wise passes over rows x n, grid-stride; `narrow` says that every
// flat index fits 32 bits (cheaper division by n).
struct EwArgs {
    const void* a;       // x (finish) or g (gather, vjp finish)
    const void* b;       // v (finish) or A g_s (vjp finish)
    const int32_t* idx;  // rank (finish, vjp finish) or perm (gather)
    void* out;
    int64_t total;
    int n;
    int narrow;
    double eps;
};

__device__ __forceinline__ int64_t row_base(int64_t e, int n, int narrow) {
    return narrow ? (int64_t)(((uint32_t)e / (uint32_t)n) * (uint32_t)n) : (e / n) * n;
}

// The index stored at e (a position within its row), clamped into the row so
// that a corrupted permutation could never address outside it.
__device__ __forceinline__ int64_t row_at(const EwArgs& a, int64_t e) {
    const uint32_t p = (uint32_t)a.idx[e];
    return row_base(e, a.n, a.narrow) + (p < (uint32_t)a.n ? p : (uint32_t)a.n - 1u);
}

template <typename T>
__global__ __launch_bounds__(256) void k_rank_finish(EwArgs a) {
    const T* x = (const T*)a.a;
    const T* v = (const T*)a.b;
    T* r = (T*)a.out;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < a.total; e += (int64_t)gridDim.x * 256) {
        r[e] = (T)((double)x[e] / a.eps - (double)v[row_at(a, e)]);
    }
}

template <typename T>
__global__ __launch_bounds__(256) void k_rank_gather(EwArgs a) {
    const T* g = (const T*)a.a;
    T* gs = (T*)a.out;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < a.total; e += (int64_t)gridDim.x * 256)
        gs[e] = g[row_at(a, e)];
}

template <typename T>
__global__ __launch_bounds__(256) void k_rank_vjp_finish(EwArgs a) {
    const T* g = (const T*)a.a;
    const T* ag = (const T*)a.b;
    T* out = (T*)a.out;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < a.total; e += (int64_t)gridDim.x * 256) {
        out[e] = (T)(((double)g[e] - (double)ag[row_at(a, e)]) / a.eps);
    }
}

// Rows sorted by launch_sort_rows: the entry at sorted position p of a row is
// the element of index idx and value x; z[p] = x / eps - (n - p).
struct LongZArgs {
    const uint64_t* K;
    const uint32_t* I;
    int32_t* perm;
    int32_t* rank;
    void* z;
    int64_t total;
    int n;
    int narrow;
    double eps;
};

template <typename T>
__global__ __launch_bounds__(256) void k_rank_long_z(LongZArgs a) {
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < a.total; e += (int64_t)gridDim.x * 256) {
        const int64_t base = row_base(e, a.n, a.narrow);
        const int p = (int)(e - base);
        uint32_t idx;
        double x;
        if constexpr (sizeof(T) == 4) {
            idx = ~(uint32_t)a.K[e];
            x = (double)key_value((uint32_t)(a.K[e] >> 32));
        } else {
            idx = a.I[e];
            x = key_value(a.K[e]);
        }
        ((T*)a.z)[e] = (T)(x / a.eps - (double)(a.n - p));
        a.perm[e] = (int32_t)idx;
        if (idx < (uint32_t)a.n) a.rank[base + idx] = p;
    }
}

int sort_width(int64_t n) {
    int P = 64;
    while (P < n) P <<= 1;
    return P;
}

EwArgs ew_args(const RankLaunch& l) {
    EwArgs e{};
    e.total = l.rows * l.n;
    e.n = (int)l.n;
    e.narrow = e.total <= (int64_t)UINT32_MAX ? 1 : 0;
    e.eps = l.eps;
    return e;
}

unsigned ew_grid(int64_t total) {
    const int64_t b = (total + 255) / 256;
    return (unsigned)(b < 65536 ? b : 65536);
}

// Entries per thread of the sort: one wave of E entries each up to 512, then
// eight per thread (at most 1024 threads for 8192 entries).
template <typename T, int E>
hipError_t launch_sort(const SortArgs& s, int64_t rows, hipStream_t stream) {
    const int nt = s.P / E;
    const size_t lds = nt > 64 ? (size_t)s.P * (sizeof(T) == 4 ? 8 : 12) : 0;
    static size_t seen[kMaxDevices];
    if (lds > 0) {
        const hipError_t e = ensure_lds((const void*)k_rank_sort<T, E>, lds, seen);
        if (e != hipSuccess) return e;
    }
    k_rank_sort<T, E><<<dim3((unsigned)rows), dim3(nt), lds, stream>>>(s);
    return hipGetLastError();
}

template <typename T, int E>
hipError_t launch_fused(const RankLaunch& l) {
    FusedArgs f{};
    f.x = l.in;
    f.r = l.out;
    f.perm = l.perm;
    f.rank = l.rank;
    f.start_bits = l.start_bits;
    f.clip_bits = l.clip_bits;
    f.row_nan = l.row_nan;
    f.words = l.words;
    f.n = (int)l.n;
    f.eps = l.eps;
    k_rank_fused<T, E><<<dim3((unsigned)l.rows), dim3(64), tile_smem_bytes(64, (int)l.n, E), l.stream>>>(f);
    return hipGetLastError();
}

template <typename T>
hipError_t soft_rank_t(const RankLaunch& l) {
    if (l.n > 64 && l.n <= 512) {
        if (l.n <= 128) return launch_fused<T, 2>(l);
        if (l.n <= 256) return launch_fused<T, 4>(l);
        return launch_fused<T, 8>(l);
    }
    hipError_t e;
    if (l.n > kRankMaxN) {
        const RankSortAreas A = rank_sort_areas(l.rows, l.n, l.voff, sizeof(T));
        uint64_t* const K[2] = {(uint64_t*)(l.ws + A.k0), (uint64_t*)(l.ws + A.k1)};
        uint32_t* const I[2] = {(uint32_t*)(l.ws + A.i0), (uint32_t*)(l.ws + A.i1)};
        int cur = 0;
        if ((e = launch_sort_rows(sizeof(T) == 4 ? 0 : 1, l.in, l.rows, l.n, 0, K, I, l.stream, cur)) != hipSuccess)
            return e;
        LongZArgs z{};
        z.K = K[cur];
        z.I = I[cur];
        z.perm = l.perm;
        z.rank = l.rank;
        z.z = l.ws + l.zoff;
        z.total = l.rows * l.n;
        z.n = (int)l.n;
        z.narrow = z.total <= (int64_t)UINT32_MAX ? 1 : 0;
        z.eps = l.eps;
        k_rank_long_z<T><<<dim3(ew_grid(z.total)), dim3(256), 0, l.stream>>>(z);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else {
        SortArgs s{};
        s.x = l.in;
        s.perm = l.perm;
        s.rank = l.rank;
        s.z = l.ws + l.zoff;
        s.n = (int)l.n;
        s.P = sort_width(l.n);
        s.eps = l.eps;
        switch (s.P) {
            case 64:
                e = launch_sort<T, 1>(s, l.rows, l.stream);
                break;
            case 128:
                e = launch_sort<T, 2>(s, l.rows, l.stream);
                break;
            case 256:
                e = launch_sort<T, 4>(s, l.rows, l.stream);
                break;
            default:
                e = launch_sort<T, 8>(s, l.rows, l.stream);
        }
        if (e != hipSuccess) return e;
    }

    FitLaunch f{};
    f.y = l.ws + l.zoff;
    f.w = nullptr;
    f.fit = l.ws + l.voff;
    f.rows = l.rows;
    f.n = l.n;
    f.increasing = 0;
    f.dtype = l.dtype;
    f.lo = -INFINITY;
    f.hi = INFINITY;
    f.start_bits = l.start_bits;
    f.clip_bits = l.clip_bits;
    f.row_nan = l.row_nan;
    f.words = l.words;
    f.ws = l.ws;
    f.L = l.L;
    f.epoch = 0;
    f.stream = l.stream;
    if ((e = launch_fit(f)) != hipSuccess) return e;

    EwArgs a = ew_args(l);
    a.a = l.in;
    a.b = l.ws + l.voff;
    a.idx = l.rank;
    a.out = l.out;
    k_rank_finish<T><<<dim3(ew_grid(a.total)), dim3(256), 0, l.stream>>>(a);
    return hipGetLastError();
}

template <typename T>
hipError_t soft_rank_vjp_t(const RankLaunch& l) {
    EwArgs a = ew_args(l);
    a.a = l.in;
    a.idx = l.perm;
    a.out = l.ws + l.zoff;
    k_rank_gather<T><<<dim3(ew_grid(a.total)), dim3(256), 0, l.stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    VjpLaunch v{};
    v.g = l.ws + l.zoff;
    v.w = nullptr;
    v.y = nullptr;
    v.out = l.ws + l.voff;
    v.out_w = nullptr;
    v.rows = l.rows;
    v.n = l.n;
    v.words = l.words;
    v.dtype = l.dtype;
    v.start_bits = l.start_bits;
    v.clip_bits = l.clip_bits;
    v.row_nan = l.row_nan;
    v.ws = l.ws;
    v.L = l.L;
    v.stream = l.stream;
    if ((e = launch_vjp(v)) != hipSuccess) return e;

    EwArgs b = ew_args(l);
    b.a = l.in;
    b.b = l.ws + l.voff;
    b.idx = l.rank;
    b.out = l.out;
    k_rank_vjp_finish<T><<<dim3(ew_grid(b.total)), dim3(256), 0, l.stream>>>(b);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_soft_rank(const RankLaunch& l) {
    return l.dtype == 0 ? soft_rank_t<float>(l) : soft_rank_t<double>(l);
}

hipError_t launch_soft_rank_vjp(const RankLaunch& l) {
    return l.dtype == 0 ? soft_rank_vjp_t<float>(l) : soft_rank_vjp_t<double>(l);
}

}  // namespace iso
