// Backward kernels: vector-Jacobian product of the fit with respect to y.
//
// Page "Merge Hulls Without Copying Vertices: GPU Isotonic Regression",
// Appendix C: the product of the isotonic step is A g, A averaging over the
// solver's blocks (and Sec. 7.8 for its cost).  With weights, differentiating
// a block's value sum_B w y / sum_B w gives, for j in block B,
//     grad_y[j] = w_j * sum_{i in B} g'_i / sum_{i in B} w_i,
// where g'_i = g_i unless the clip was active at i (then 0).  The partition is
// the forward pass's own (its block-start bits), as the page's tests require.
//
// A tile of up to 8192 elements is one workgroup: a segmented inclusive scan
// of (g', w) inside each 64-element group (wave64 shuffles), a carry across
// groups, then every element reads its block's total at the block's last
// element.  Rows longer than one tile go through three launches: per-tile
// partial sums, a per-row carry pass, and the tile pass with those carries.
#include <math.h>

#include "iso_device.hpp"
#include "iso_internal.hpp"

namespace iso {

struct VjpArgs {
    const void* g;
    const void* w;
    void* out;
    int64_t n, words;
    int T;       // elements per tile
    int ntiles;  // tiles per row
    const uint64_t* sb;
    const uint64_t* cb;
    const uint32_t* row_nan;
    double2* head;   // [rows * ntiles] sum from the tile start to its first block start
    double2* tail;   // [rows * ntiles] sum from the tile's last block start to its end
    int* has;        // [rows * ntiles] tile holds a block start
    double2* carry;  // [rows * ntiles] open block's sum before the tile
    double2* tot;    // [rows * ntiles] total of the block open at the tile's end
    int mode;        // 0: whole row in one tile; 1: partial sums; 2: tile pass of a long row
};

__host__ __device__ inline size_t vjp_smem_bytes(int T) {
    const int G = (T + 63) / 64;
    return sizeof(double2) * (size_t)T + (size_t)G * (sizeof(double2) * 2 + sizeof(int) * 3) + 64;
}

template <typename T>
__global__ __launch_bounds__(512) void k_vjp_tile(VjpArgs a) {
    extern __shared__ __align__(32) char smem[];
    const int64_t bid = blockIdx.x;
    const int64_t row = bid / a.ntiles;
    const int tile = (int)(bid % a.ntiles);
    const int64_t t0 = (int64_t)tile * a.T;
    const int N = (int)((a.n - t0) < a.T ? (a.n - t0) : a.T);
    const int G = (N + 63) / 64;
    double2* F = (double2*)smem;
    double2* gtail = F + a.T;
    double2* gcarry = gtail + G;
    int* ghas = (int*)(gcarry + G);
    int* gfirst = ghas + G;
    int* gnext = gfirst + G;

    const T* g = (const T*)a.g + row * a.n + t0;
    const T* w = a.w ? (const T*)a.w + row * a.n + t0 : nullptr;
    T* out = (T*)a.out + row * a.n + t0;
    const uint64_t* sb = a.sb + row * a.words + t0 / 64;
    const uint64_t* cb = a.cb + row * a.words + t0 / 64;
    const int64_t ti = row * a.ntiles + tile;

    if (a.row_nan[row]) {
        if (a.mode != 1)
            for (int i = threadIdx.x; i < N; i += blockDim.x) out[i] = (T)NAN;
        else if (threadIdx.x == 0) {
            a.head[ti] = make_double2(0.0, 1.0);
            a.tail[ti] = make_double2(0.0, 1.0);
            a.has[ti] = 1;
        }
        return;
    }

    const int lane = lane_id();
    const int wid = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    // phase 1: segmented scan inside each group
    for (int q = wid; q < G; q += nw) {
        const int e = q * 64 + lane;
        const bool valid = e < N;
        const uint64_t vmask = (N - q * 64 >= 64) ? ~0ull : ((1ull << (N - q * 64)) - 1ull);
        const uint64_t sw = sb[q] & vmask;
        const uint64_t cw = cb[q];
        double gv = 0.0, wv = 0.0;
        if (valid) {
            gv = ((cw >> lane) & 1ull) ? 0.0 : (double)g[e];
            wv = w ? (double)w[e] : 1.0;
        }
        int fl = (int)((sw >> lane) & 1ull);
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const double og = __shfl_up(gv, d, 64);
            const double ow = __shfl_up(wv, d, 64);
            const int of = __shfl_up(fl, d, 64);
            if (lane >= d) {
                if (!fl) {
                    gv = og + gv;
                    wv = ow + wv;
                }
                fl |= of;
            }
        }
        if (valid) F[e] = make_double2(gv, wv);
        if (lane == 63) {
            gtail[q] = make_double2(gv, wv);
            ghas[q] = sw != 0ull;
            gfirst[q] = sw ? lo_bit(sw) : 64;
        }
    }
    __syncthreads();
    // phase 2: carries across groups and the next block start after each group
    if (threadIdx.x == 0) {
        double2 c = (a.mode == 2) ? a.carry[ti] : make_double2(0.0, 0.0);
        for (int q = 0; q < G; ++q) {
            gcarry[q] = c;
            const double2 t = gtail[q];
            c = ghas[q] ? t : make_double2(c.x + t.x, c.y + t.y);
        }
        int nx = N;
        for (int q = G - 1; q >= 0; --q) {
            gnext[q] = nx;
            if (ghas[q]) nx = q * 64 + gfirst[q];
        }
        if (a.mode == 1) {
            // tail: the open block at the tile's end (no carry in this pass);
            // the head is read after the carries are added below
            a.tail[ti] = c;
            a.has[ti] = (nx < N) ? 1 : 0;
            if (nx >= N) a.head[ti] = c;  // no start: the whole tile
            gfirst[0] = nx;               // group 0's first start is no longer needed
        }
    }
    __syncthreads();
    // phase 3: add the carry where no block starts between the group start and e
    for (int q = wid; q < G; q += nw) {
        const int e = q * 64 + lane;
        if (e < N) {
            const uint64_t sw = sb[q];
            if ((sw & bits_upto(lane)) == 0ull) {
                const double2 c = gcarry[q];
                const double2 v = F[e];
                F[e] = make_double2(v.x + c.x, v.y + c.y);
            }
        }
    }
    __syncthreads();
    if (a.mode == 1) {
        // head: the tile's prefix before its first block start
        if (threadIdx.x == 0) {
            const int nx = gfirst[0];
            if (nx < N) a.head[ti] = (nx > 0) ? F[nx - 1] : make_double2(0.0, 0.0);
        }
        return;
    }
    // phase 4: every element takes its block's total, found at the block's end
    const double2 open_total = (a.mode == 2) ? a.tot[ti] : make_double2(0.0, 0.0);
    for (int q = wid; q < G; q += nw) {
        const int e = q * 64 + lane;
        if (e < N) {
            const uint64_t vmask = (N - q * 64 >= 64) ? ~0ull : ((1ull << (N - q * 64)) - 1ull);
            const uint64_t later = sb[q] & vmask & bits_from(lane + 1);
            const int nxt = later ? q * 64 + lo_bit(later) : gnext[q];
            double2 tot;
            if (nxt < N)
                tot = F[nxt - 1];
            else
                tot = (a.mode == 2) ? open_total : F[N - 1];
            const double wv = w ? (double)w[e] : 1.0;
            out[e] = (T)(wv * (tot.x / tot.y));
        }
    }
}

// per-row carries across tiles (one thread per row)
__global__ void k_vjp_carry(VjpArgs a, int64_t rows) {
    const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= rows) return;
    const int64_t b = row * a.ntiles;
    double2 c = make_double2(0.0, 0.0);
    for (int t = 0; t < a.ntiles; ++t) {
        a.carry[b + t] = c;
        const double2 hd = a.head[b + t], tl = a.tail[b + t];
        c = a.has[b + t] ? tl : make_double2(c.x + hd.x, c.y + hd.y);
    }
    double2 after = c;
    a.tot[b + a.ntiles - 1] = after;
    for (int t = a.ntiles - 2; t >= 0; --t) {
        if (a.has[b + t + 1]) {
            const double2 ci = a.carry[b + t + 1], hd = a.head[b + t + 1];
            after = make_double2(ci.x + hd.x, ci.y + hd.y);
        }
        a.tot[b + t] = after;
    }
}

template <typename T>
static hipError_t launch_vjp_t(const VjpLaunch& l) {
    VjpArgs a{};
    a.g = l.g;
    a.w = l.w;
    a.out = l.out;
    a.n = l.n;
    a.words = l.words;
    a.sb = l.start_bits;
    a.cb = l.clip_bits;
    a.row_nan = l.row_nan;
    static bool attr_set = false;
    if (!attr_set) {
        (void)hipFuncSetAttribute((const void*)k_vjp_tile<T>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)vjp_smem_bytes((int)kSingleMax));
        attr_set = true;
    }
    if (l.n <= kSingleMax) {
        a.T = (int)l.n;
        a.ntiles = 1;
        a.mode = 0;
        const int G = (a.T + 63) / 64;
        const int nt = G >= 32 ? 512 : (G >= 8 ? 256 : 64);
        hipLaunchKernelGGL(k_vjp_tile<T>, dim3((unsigned)l.rows), dim3(nt), vjp_smem_bytes(a.T), l.stream, a);
        return hipGetLastError();
    }
    a.T = kVjpTile;
    a.ntiles = (int)((l.n + kVjpTile - 1) / kVjpTile);
    const size_t tiles = (size_t)l.rows * (size_t)a.ntiles;
    char* p = l.ws + l.L.vjp;
    a.head = (double2*)p;
    a.tail = a.head + tiles;
    a.carry = a.tail + tiles;
    a.tot = a.carry + tiles;
    a.has = (int*)(a.tot + tiles);
    a.mode = 1;
    hipLaunchKernelGGL(k_vjp_tile<T>, dim3((unsigned)tiles), dim3(512), vjp_smem_bytes(a.T), l.stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_vjp_carry, dim3((unsigned)((l.rows + 63) / 64)), dim3(64), 0, l.stream, a, l.rows);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.mode = 2;
    hipLaunchKernelGGL(k_vjp_tile<T>, dim3((unsigned)tiles), dim3(512), vjp_smem_bytes(a.T), l.stream, a);
    return hipGetLastError();
}

hipError_t launch_vjp(const VjpLaunch& l) {
    if (l.dtype == 0) return launch_vjp_t<float>(l);
    return launch_vjp_t<double>(l);
}

}  // namespace iso
