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
    int P;  // power of two >= n, at least 64
    double eps;
};

// One compare-exchange stage of the network at distance j inside blocks of
// size k; a block with (i & k) == 0 is put in decreasing order.  A float32
// entry packs (key << 32) | ~index, so that one unsigned comparison orders by
// key and then by the lower index; padding entries are 0 and sort last.
template <typename T>
__device__ __forceinline__ void sort_stage(uint64_t* K, uint32_t* I, int half, int k, int j) {
    for (int q = threadIdx.x; q < half; q += blockDim.x) {
        const int i = 2 * q - (q & (j - 1));
        const int l = i + j;
        const bool dec = (i & k) == 0;
        const uint64_t u = K[i], v = K[l];
        if constexpr (sizeof(T) == 4) {
            if (dec ? (v > u) : (u > v)) {
                K[i] = v;
                K[l] = u;
            }
        } else {
            const uint32_t a = I[i], b = I[l];
            const bool l_first = v > u || (v == u && b < a);  // the entry at l comes first
            if (dec == l_first) {
                K[i] = v;
                K[l] = u;
                I[i] = b;
                I[l] = a;
            }
        }
    }
}

template <typename T>
__global__ __launch_bounds__(1024) void k_rank_sort(SortArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int n = a.n, P = a.P;
    const int64_t row0 = (int64_t)blockIdx.x * n;
    const T* x = (const T*)a.x + row0;
    uint64_t* K = (uint64_t*)smem;
    uint32_t* I = (uint32_t*)(smem + 8 * (size_t)P);
    for (int i = threadIdx.x; i < P; i += blockDim.x) {
        if constexpr (sizeof(T) == 4) {
            K[i] = i < n ? (((uint64_t)sort_key(x[i]) << 32) | (uint32_t)~(uint32_t)i) : 0ull;
        } else {
            K[i] = i < n ? sort_key(x[i]) : 0ull;
            I[i] = i < n ? (uint32_t)i : 0xffffffffu;
        }
    }
    // Stages at distance <= 64 keep every wave inside its own 128 entries (the
    // pairs of a wave are 64 consecutive q), so between two such stages a wave
    // only waits for itself; any stage at a larger distance, before or after,
    // needs the whole workgroup.
    const int half = P / 2;
    int jprev = P;
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            if (j >= 128 || jprev >= 128)
                __syncthreads();
            else
                wave_sync();
            jprev = j;
            sort_stage<T>(K, I, half, k, j);
        }
    }
    __syncthreads();
    T* z = (T*)a.z + row0;
    int32_t* perm = a.perm + row0;
    int32_t* rank = a.rank + row0;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const uint64_t e = K[i];
        int p;
        double xv;
        if constexpr (sizeof(T) == 4) {
            p = (int)~(uint32_t)e;
            xv = (double)key_value((uint32_t)(e >> 32));
        } else {
            p = (int)I[i];
            xv = key_value(e);
        }
        perm[i] = p;
        if ((unsigned)p < (unsigned)n) rank[p] = i;  // always true once sorted: padding sorts last
        z[i] = (T)(xv / a.eps - (double)(n - i));
    }
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

template <typename T>
hipError_t soft_rank_t(const RankLaunch& l) {
    const int P = sort_width(l.n);
    const int nt = P / 2 < 64 ? 64 : (P / 2 > 1024 ? 1024 : P / 2);
    const size_t lds = (size_t)P * (sizeof(T) == 4 ? 8 : 12);
    static size_t seen[kMaxDevices];
    hipError_t e = ensure_lds((const void*)k_rank_sort<T>, lds, seen);
    if (e != hipSuccess) return e;
    SortArgs s{};
    s.x = l.in;
    s.perm = l.perm;
    s.rank = l.rank;
    s.z = l.ws + l.zoff;
    s.n = (int)l.n;
    s.P = P;
    s.eps = l.eps;
    k_rank_sort<T><<<dim3((unsigned)l.rows), dim3(nt), lds, l.stream>>>(s);
    if ((e = hipGetLastError()) != hipSuccess) return e;

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
