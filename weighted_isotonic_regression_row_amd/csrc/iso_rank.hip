// Soft rank with quadratic regularization and its vector-Jacobian product
// (first page, Sec. 7.9, after Blondel et al.).
//
// Forward, per row: theta = x / eps is sorted in decreasing order into s;
// z = s - (n, n-1, ..., 1) is fitted non-increasing with unit weights by the
// library's own solver (launch_fit), and the element at sorted position i gets
// the rank s_i - v_i, written back in the original order.
//   k_rank_sort    one workgroup per row: a bitonic network over (key, index)
//                  pairs in LDS, where key is an order-preserving unsigned image
//                  of x (theta has the order of x as eps > 0), ties broken by the
//                  lower index first; writes perm, its inverse rank, and z in the
//                  data type, into the sorted order;
//   launch_fit     the fit of z and its block bits (the partition the backward
//                  pass uses), over the sorted order;
//   k_rank_finish  r[k] = x[k] / eps - v[rank[k]], element-wise.
// Backward, with g_s the upstream gradient in sorted order and A the block
// averaging of the fit: d/dx = P^T (g_s - A g_s) / eps.
//   k_rank_gather      g_s[i] = g[perm[i]];
//   launch_vjp         A g_s over the fit's blocks;
//   k_rank_vjp_finish  grad[k] = (g[k] - (A g_s)[rank[k]]) / eps.
#include "iso_device.hpp"
#include "iso_internal.hpp"

namespace iso {
namespace {

// Order-preserving unsigned images of the bits (after -0 is folded into +0):
// a > b as numbers iff key(a) > key(b); NaNs land beyond the infinities.
__device__ __forceinline__ uint32_t sort_key(float v) {
    const uint32_t b = __float_as_uint(v + 0.0f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ uint64_t sort_key(double v) {
    const uint64_t b = (uint64_t)__double_as_longlong(v + 0.0);
    return (b >> 63) ? ~b : (b | (1ull << 63));
}
__device__ __forceinline__ float key_value(uint32_t u) {
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}
__device__ __forceinline__ double key_value(uint64_t u) {
    return __longlong_as_double((long long)((u >> 63) ? (u & ~(1ull << 63)) : ~u));
}

struct SortArgs {
    const void* x;
    int32_t* perm;
    int32_t* rank;
    void* z;
    int n;
    int P;  // power of two >= n, at least 64; P / E threads
    double eps;
};

// A sort entry.  A float32 entry packs (key << 32) | ~index into k, so that one
// unsigned comparison orders by key and then by the lower index; a float64
// entry keeps the index in i.  Padding entries (k = 0, index all ones) come
// after every element.
struct Ent {
    uint64_t k;
    uint32_t i;
};

template <typename T>
__device__ __forceinline__ bool before(const Ent& a, const Ent& b) {
    if constexpr (sizeof(T) == 4)
        return a.k > b.k;
    else
        return a.k > b.k || (a.k == b.k && a.i < b.i);
}

template <typename T>
__device__ __forceinline__ Ent shfl_xor_ent(const Ent& a, int m) {
    Ent r;
    const int lo = __shfl_xor((int)(uint32_t)a.k, m), hi = __shfl_xor((int)(uint32_t)(a.k >> 32), m);
    r.k = ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
    r.i = sizeof(T) == 4 ? 0u : (uint32_t)__shfl_xor((int)a.i, m);
    return r;
}

// The entry of lane (this lane ^ M) for the masks DPP reaches inside a row of
// 16 lanes (quad permutations, the row and half-row mirrors, a rotation by 8;
// xor 4 is the half-row mirror followed by the quad reversal); M == 0 takes
// any mask m through the LDS crossbar.
template <typename T, int CTRL>
__device__ __forceinline__ Ent dpp_ent(const Ent& a) {
    Ent r;
    const unsigned lo = (unsigned)dpp_move<CTRL, 0xf>((int)(uint32_t)a.k);
    const unsigned hi = (unsigned)dpp_move<CTRL, 0xf>((int)(uint32_t)(a.k >> 32));
    r.k = ((uint64_t)hi << 32) | lo;
    r.i = sizeof(T) == 4 ? 0u : (uint32_t)dpp_move<CTRL, 0xf>((int)a.i);
    return r;
}

template <typename T, int M>
__device__ __forceinline__ Ent lanes_xor(const Ent& a, int m) {
    if constexpr (M == 1) return dpp_ent<T, 0xB1>(a);  // quad_perm [1,0,3,2]
    if constexpr (M == 2) return dpp_ent<T, 0x4E>(a);  // quad_perm [2,3,0,1]
    if constexpr (M == 3) return dpp_ent<T, 0x1B>(a);  // quad_perm [3,2,1,0]
    if constexpr (M == 4) return dpp_ent<T, 0x1B>(dpp_ent<T, 0x141>(a));
    if constexpr (M == 7) return dpp_ent<T, 0x141>(a);   // row_half_mirror
    if constexpr (M == 8) return dpp_ent<T, 0x128>(a);   // row_ror:8
    if constexpr (M == 15) return dpp_ent<T, 0x140>(a);  // row_mirror
    if constexpr (M == 0) return shfl_xor_ent<T>(a, m);
    return a;
}

template <typename T>
__device__ __forceinline__ Ent sel(bool c, const Ent& a, const Ent& b) {
    Ent r;
    r.k = c ? a.k : b.k;
    r.i = sizeof(T) == 4 ? 0u : (c ? a.i : b.i);
    return r;
}

// The network sorts P entries in decreasing order, every comparison in the
// same direction: phase k (k = 2, 4, ..., P) first compares position p with
// its mirror p ^ (k-1) inside its block of k, then p with p ^ j for
// j = k/4, ..., 1; of each pair the lower position keeps the entry that comes
// first.  Thread t holds positions tE .. tE+E-1, so distances below E stay in
// the thread, partners up to 64E away are lanes of the same wave (shuffles; a
// mirror partner holds the entries in reverse), farther ones go through LDS.
template <typename T, int E>
__device__ __forceinline__ void cas(Ent (&v)[E], int a, int b) {
    const bool sw = before<T>(v[b], v[a]);
    const Ent x = v[a], y = v[b];
    v[a] = sel<T>(sw, y, x);
    v[b] = sel<T>(sw, x, y);
}

template <typename T, int E, int KK>
__device__ __forceinline__ void mirror_in_thread(Ent (&v)[E]) {
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (!(e & (KK / 2))) cas<T, E>(v, e, e ^ (KK - 1));
}

template <typename T, int E, int J>
__device__ __forceinline__ void half_in_thread(Ent (&v)[E]) {
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (!(e & J)) cas<T, E>(v, e, e | J);
}

// partner lane t ^ mask; `bit` (>= E) of the position says whether this lane
// holds the lower positions of its pairs
template <typename T, int E, bool MIRROR, int M>
__device__ __forceinline__ void stage_in_wave_m(Ent (&v)[E], bool first, int mask) {
    Ent o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = lanes_xor<T, M>(v[MIRROR ? E - 1 - e : e], mask);
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = sel<T>(first == before<T>(o[e], v[e]), o[e], v[e]);
}

template <typename T, int E, bool MIRROR>
__device__ __forceinline__ void stage_in_wave(Ent (&v)[E], int t, int mask, int bit) {
    const bool first = ((t * E) & bit) == 0;
    switch (mask) {
        case 1:
            stage_in_wave_m<T, E, MIRROR, 1>(v, first, mask);
            break;
        case 2:
            stage_in_wave_m<T, E, MIRROR, 2>(v, first, mask);
            break;
        case 3:
            stage_in_wave_m<T, E, MIRROR, 3>(v, first, mask);
            break;
        case 4:
            stage_in_wave_m<T, E, MIRROR, 4>(v, first, mask);
            break;
        case 7:
            stage_in_wave_m<T, E, MIRROR, 7>(v, first, mask);
            break;
        case 8:
            stage_in_wave_m<T, E, MIRROR, 8>(v, first, mask);
            break;
        case 15:
            stage_in_wave_m<T, E, MIRROR, 15>(v, first, mask);
            break;
        default:
            stage_in_wave_m<T, E, MIRROR, 0>(v, first, mask);
    }
}

// partner position p ^ xr through LDS (K, I: P entries)
template <typename T, int E>
__device__ __forceinline__ void stage_in_lds(Ent (&v)[E], int t, int xr, int bit, uint64_t* K, uint32_t* I) {
    const int p = t * E;
    const bool first = (p & bit) == 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        K[p + e] = v[e].k;
        if constexpr (sizeof(T) == 8) I[p + e] = v[e].i;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e) {
        Ent o;
        o.k = K[(p + e) ^ xr];
        o.i = sizeof(T) == 4 ? 0u : I[(p + e) ^ xr];
        v[e] = sel<T>(first == before<T>(o, v[e]), o, v[e]);
    }
    __syncthreads();
}

template <typename T, int E>
__global__ __launch_bounds__(1024) void k_rank_sort(SortArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
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
    uint64_t* K = (uint64_t*)smem;
    uint32_t* I = (uint32_t*)(smem + 8 * (size_t)P);
    for (int k = 2; k <= P; k <<= 1) {
        if (k <= E) {
            if constexpr (E >= 2)
                if (k == 2) mirror_in_thread<T, E, 2>(v);
            if constexpr (E >= 4)
                if (k == 4) mirror_in_thread<T, E, 4>(v);
            if constexpr (E >= 8)
                if (k == 8) mirror_in_thread<T, E, 8>(v);
        } else if (k <= 64 * E) {
            stage_in_wave<T, E, true>(v, t, k / E - 1, k >> 1);
        } else {
            stage_in_lds<T, E>(v, t, k - 1, k >> 1, K, I);
        }
        for (int j = k >> 2; j > 0; j >>= 1) {
            if (j >= 64 * E) {
                stage_in_lds<T, E>(v, t, j, j, K, I);
            } else if (j >= E) {
                stage_in_wave<T, E, false>(v, t, j / E, j);
            } else {
                if constexpr (E >= 8)
                    if (j == 4) half_in_thread<T, E, 4>(v);
                if constexpr (E >= 4)
                    if (j == 2) half_in_thread<T, E, 2>(v);
                if constexpr (E >= 2)
                    if (j == 1) half_in_thread<T, E, 1>(v);
            }
        }
    }
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

template <typename T>
hipError_t soft_rank_t(const RankLaunch& l) {
    SortArgs s{};
    s.x = l.in;
    s.perm = l.perm;
    s.rank = l.rank;
    s.z = l.ws + l.zoff;
    s.n = (int)l.n;
    s.P = sort_width(l.n);
    s.eps = l.eps;
    hipError_t e;
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
