// Backward kernels: vector-Jacobian products of the fit with respect to y
// and to the weights.
//
// Page "Merge Hulls Without Copying Vertices: GPU Isotonic Regression",
// Appendix C: the product of the isotonic step is A g, A averaging over the
// solver's blocks (and Sec. 7.8 for its cost).  With weights, a block B takes
// the value mean_B = sum_B w y / sum_B w; differentiating it gives, for j in B,
//     grad_y[j] = w_j * G_B / W_B,
//     grad_w[j] = G_B * (y_j - mean_B) / W_B        (page "torchisotonic",
//                 "Semantics": the fit is differentiable in y and in w),
// where G_B = sum_{i in B} g'_i, g'_i = g_i unless the clip was active at i
// (then 0), and W_B = sum_B w.  The partition is the forward pass's own (its
// block-start bits), as the page's tests require.
//
// Rows of up to 6144 elements are one workgroup, kVjpK elements per lane: each
// lane sums its elements' blocks in registers, a segmented scan over the
// lanes carries the sums of the block open at each lane's start, and every
// element then takes its block's totals, found where the block ends.  Longer
// rows are cut into tiles of kVjpTile elements and take three launches: the
// sums of each tile's head (before its first block start) and tail (from its
// last block start), which reads only those elements; a per-row carry pass
// over the tiles; and the same per-lane kernel on every tile, given the
// totals of the blocks open at its start and at its end, so that it reads g
// only between its first and last block start and every g is read once.
#include <math.h>

#include "iso_device.hpp"
#include "iso_internal.hpp"

namespace iso {

// Running block sums: (g', w) or (g', w, w y).
template <int NF>
struct Acc {
    double v[NF];
};
template <int NF>
__host__ __device__ __forceinline__ Acc<NF> acc_zero() {
    Acc<NF> r;
#pragma unroll
    for (int k = 0; k < NF; ++k) r.v[k] = 0.0;
    return r;
}
template <int NF>
__device__ __forceinline__ Acc<NF> acc_sum(const Acc<NF>& a, const Acc<NF>& b) {
    Acc<NF> r;
#pragma unroll
    for (int k = 0; k < NF; ++k) r.v[k] = a.v[k] + b.v[k];
    return r;
}
// p ? a : b field by field (a select of whole structs would go through memory)
template <int NF>
__device__ __forceinline__ Acc<NF> acc_pick(bool p, const Acc<NF>& a, const Acc<NF>& b) {
    Acc<NF> r;
#pragma unroll
    for (int k = 0; k < NF; ++k) r.v[k] = p ? a.v[k] : b.v[k];
    return r;
}

struct VjpArgs {
    const void* g;
    const void* w;
    const void* y;  // the fit's input, for the weight product
    void* out;      // grad_y, or nullptr
    void* out_w;    // grad_w, or nullptr
    int64_t n, words;
    int ntiles;  // tiles per row
    const uint64_t* sb;
    const uint64_t* cb;
    const uint32_t* row_nan;
    void* head;   // Acc [rows * ntiles] sums from the tile start to its first block start
    void* tail;   // Acc [rows * ntiles] sums from the tile's last block start to its end
    int* has;     // [rows * ntiles] tile holds a block start
    void* carry;  // Acc [rows * ntiles] open block's sums before the tile
    void* tot;    // Acc [rows * ntiles] totals of the block open at the tile's end
};

template <int NF>
struct SegSum {
    int f;  // a block starts inside the span
    Acc<NF> a;
};
// (earlier, later): the later span's sums restart if a block starts in it
template <int NF>
__device__ __forceinline__ SegSum<NF> seg_op(const SegSum<NF>& x, const SegSum<NF>& y) {
    SegSum<NF> r;
    r.f = x.f | y.f;
#pragma unroll
    for (int k = 0; k < NF; ++k) r.a.v[k] = y.f ? y.a.v[k] : x.a.v[k] + y.a.v[k];
    return r;
}
template <int CTRL, int ROWS, int NF>
__device__ __forceinline__ SegSum<NF> seg_move(const SegSum<NF>& x) {
    SegSum<NF> r;
    r.f = dpp_move<CTRL, ROWS>(x.f);
#pragma unroll
    for (int k = 0; k < NF; ++k) r.a.v[k] = dpp_move<CTRL, ROWS>(x.a.v[k]);
    return r;
}
template <int NF>
__device__ __forceinline__ SegSum<NF> seg_scan_wave(SegSum<NF> x) {
    x = seg_op(seg_move<0x111, 0xf>(x), x);
    x = seg_op(seg_move<0x112, 0xf>(x), x);
    x = seg_op(seg_move<0x114, 0xf>(x), x);
    x = seg_op(seg_move<0x118, 0xf>(x), x);
    x = seg_op(seg_move<0x142, 0xa>(x), x);
    x = seg_op(seg_move<0x143, 0xc>(x), x);
    return x;
}
// Rows of at most kLaneRow elements, one row per lane: running block sums
// forward, then each block's totals handed back to its elements.  Whole,
// aligned rows are read and written with 16-byte accesses.
template <typename T, int NF, int K>
__global__ __launch_bounds__(256) void k_vjp_lane(VjpArgs a, int64_t rows) {
    using A = Acc<NF>;
    const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= rows) return;
    const int N = (int)a.n;
    const T* g = (const T*)a.g + row * a.n;
    const T* w = a.w ? (const T*)a.w + row * a.n : nullptr;
    const T* y = (NF == 3) ? (const T*)a.y + row * a.n : nullptr;
    T* out = a.out ? (T*)a.out + row * a.n : nullptr;
    T* out_w = (NF == 3) ? (T*)a.out_w + row * a.n : nullptr;
    if (a.row_nan[row]) {
        for (int j = 0; j < N; ++j) {
            if (out) out[j] = (T)NAN;
            if (NF == 3) out_w[j] = (T)NAN;
        }
        return;
    }
    const uint64_t sw = a.sb[row * a.words], cw = a.cb[row * a.words];
    A run[K];
    {
        double gv[K], wv[K], yv[K];
        load_lane<T, K>(g, N, gv);
        if (w) {
            load_lane<T, K>(w, N, wv);
        } else {
#pragma unroll
            for (int j = 0; j < K; ++j) wv[j] = 1.0;
        }
        if (NF == 3) load_lane<T, K>(y, N, yv);
        A c = acc_zero<NF>();
#pragma unroll
        for (int j = 0; j < K; ++j) {
            if (j < N) {
                if ((sw >> j) & 1ull) c = acc_zero<NF>();
                c.v[0] += ((cw >> j) & 1ull) ? 0.0 : gv[j];
                c.v[1] += wv[j];
                if (NF == 3) c.v[NF - 1] += wv[j] * yv[j];
            }
            run[j] = c;
        }
    }
    double gw[K];  // G_B / W_B of each element's block, then the products
    double mean[K];
    A tot = acc_zero<NF>();
#pragma unroll
    for (int j = K - 1; j >= 0; --j) {
        // element j closes its block when it is the last or the next starts one
        if (j < N && (j == N - 1 || ((sw >> (j + 1)) & 1ull))) tot = run[j];
        gw[j] = tot.v[0] / tot.v[1];
        mean[j] = (NF == 3) ? tot.v[NF - 1] / tot.v[1] : 0.0;
    }
    if (out) {
        double v[K];
        if (w) load_lane<T, K>(w, N, v);
#pragma unroll
        for (int j = 0; j < K; ++j) v[j] = (w ? v[j] : 1.0) * gw[j];
        store_lane<T, K>(out, N, v);
    }
    if (NF == 3) {
        double v[K];
        load_lane<T, K>(y, N, v);
#pragma unroll
        for (int j = 0; j < K; ++j) v[j] = gw[j] * (v[j] - mean[j]);
        store_lane<T, K>(out_w, N, v);
    }
}

// Rows of 17 to 64 elements, two lanes of K = 16 or 32 elements per row (the
// fit takes one lane up to 32 and two above; the block bits are the same
// word): each lane runs the block sums of its elements; the block open at the end of the left
// lane carries its sums into the right lane's elements before the right lane's
// first block start, and the right lane's first block total flows back to the
// left lane's last block when that block continues across element 32.
template <int NF>
__device__ __forceinline__ Acc<NF> shfl_xor_acc(const Acc<NF>& a, int m) {
    Acc<NF> r;
#pragma unroll
    for (int k = 0; k < NF; ++k) r.v[k] = __shfl_xor(a.v[k], m);
    return r;
}

template <typename T, int NF, int K>
__global__ __launch_bounds__(64) void k_vjp_pair(VjpArgs a, int64_t rows) {
    using A = Acc<NF>;
    const int h = threadIdx.x & 1;
    const int64_t row = ((int64_t)blockIdx.x * 64 + threadIdx.x) >> 1;
    if (row >= rows) return;  // both lanes of a pair leave together
    const int N = (int)a.n;   // K + 1 .. 2K
    const int cnt = h ? N - K : K;
    const int64_t e0 = row * a.n + h * K;
    const T* g = (const T*)a.g + e0;
    const T* w = a.w ? (const T*)a.w + e0 : nullptr;
    const T* y = (NF == 3) ? (const T*)a.y + e0 : nullptr;
    T* out = a.out ? (T*)a.out + e0 : nullptr;
    T* out_w = (NF == 3) ? (T*)a.out_w + e0 : nullptr;
    if (a.row_nan[row]) {
        for (int j = 0; j < cnt; ++j) {
            if (out) out[j] = (T)NAN;
            if (NF == 3) out_w[j] = (T)NAN;
        }
        return;
    }
    const uint64_t swr = a.sb[row * a.words], cwr = a.cb[row * a.words];
    const uint64_t sw = h ? (swr >> K) : swr;  // bit j <-> element hK + j (the left lane also sees element 32's)
    const uint64_t cw = h ? (cwr >> K) : cwr;
    const bool cont = !((swr >> K) & 1ull);  // the block open at element 31 continues into element 32
    A run[K];
    {
        double gv[K], wv[K], yv[K];
        load_lane<T, K>(g, cnt, gv);
        if (w) {
            load_lane<T, K>(w, cnt, wv);
        } else {
#pragma unroll
            for (int j = 0; j < K; ++j) wv[j] = 1.0;
        }
        if (NF == 3) load_lane<T, K>(y, cnt, yv);
        A c = acc_zero<NF>();
#pragma unroll
        for (int j = 0; j < K; ++j) {
            if (j < cnt) {
                if ((sw >> j) & 1ull) c = acc_zero<NF>();
                c.v[0] += ((cw >> j) & 1ull) ? 0.0 : gv[j];
                c.v[1] += wv[j];
                if (NF == 3) c.v[NF - 1] += wv[j] * yv[j];
            }
            run[j] = c;
        }
    }
    // the left lane's open block into the right lane, up to its first start
    const A end0 = shfl_xor_acc<NF>(run[K - 1], 1);
    if (h == 1 && cont) {
        const int fs = sw ? lo_bit(sw) : K;
#pragma unroll
        for (int j = 0; j < K; ++j) run[j] = acc_pick(j < fs, acc_sum(end0, run[j]), run[j]);
    }
    // the right lane's first block total back to the left lane
    const uint64_t ends = (h ? bits_upto(cnt - 1) & ((sw >> 1) | (1ull << (cnt - 1))) : 0ull);
    const int jf = h ? lo_bit(ends) : 0;
    A first = acc_zero<NF>();
#pragma unroll
    for (int j = 0; j < K; ++j) first = acc_pick(j == jf, run[j], first);
    const A from1 = shfl_xor_acc<NF>(first, 1);
    double gw[K];
    double mean[K];
    A tot = (h == 0 && cont) ? from1 : acc_zero<NF>();
#pragma unroll
    for (int j = K - 1; j >= 0; --j) {
        // element j closes its block when the next element starts one (or it is the row's last)
        if (j < cnt && ((h == 1 && j == cnt - 1) || ((sw >> (j + 1)) & 1ull))) tot = run[j];
        gw[j] = tot.v[0] / tot.v[1];
        mean[j] = (NF == 3) ? tot.v[NF - 1] / tot.v[1] : 0.0;
    }
    if (out) {
        double v[K];
        if (w) load_lane<T, K>(w, cnt, v);
#pragma unroll
        for (int j = 0; j < K; ++j) v[j] = (w ? v[j] : 1.0) * gw[j];
        store_lane<T, K>(out, cnt, v);
    }
    if (NF == 3) {
        double v[K];
        load_lane<T, K>(y, cnt, v);
#pragma unroll
        for (int j = 0; j < K; ++j) v[j] = gw[j] * (v[j] - mean[j]);
        store_lane<T, K>(out_w, cnt, v);
    }
}

// Rows of kLaneRow < n <= kSingleMax elements, one workgroup per row, and the
// kVjpTile-element tiles of longer rows, one workgroup per tile, all sums in
// registers (kVjpK elements per lane):
//   1. each lane forms the segmented prefix sums of its elements (reset at
//      every block start);
//   2. a segmented scan over the lanes (DPP inside each wave, the waves'
//      aggregates through LDS) gives every lane the sums of the block that is
//      open when the lane begins, and a max-scan gives, for the block open at
//      each lane's end, the lane where that block began;
//   3. the lane where a block that began in an earlier lane ends writes the
//      block's totals to that lane's LDS slot (in a tile, the blocks open at
//      its start and at its end take their totals from the carry pass: the
//      first has a slot of its own); after one barrier the lanes that the
//      block spans read them;
//   4. a backward pass over each lane's elements hands every element its
//      block's totals and writes the products.
constexpr int kVjpK = 8;

__device__ __forceinline__ int max_scan_wave(int v) {
    return wave_scan_incl(v, [](int a, int b) { return a > b ? a : b; });
}

// Per-row carries across tiles, one workgroup per row.  Tile t hands on the
// sums of the block open at its end: its tail when a block starts in it, else
// the carry into it plus its head, so the carries are an exclusive segmented
// scan of (block starts in t, t's tail or head) over the tiles: each thread
// composes a run of tiles, the threads' compositions are scanned (DPP in each
// wave, then the waves' totals in order), and each thread replays its run.
// tot[t] is the total of the block open at t's end: the carry into the next
// tile with a block start plus that tile's head, or the row's final sums; a
// suffix minimum over the threads' first such tiles finds the next one.
constexpr int kCarryThreads = 256;
template <int NF>
__global__ __launch_bounds__(kCarryThreads) void k_vjp_carry(VjpArgs a, int64_t rows) {
    using A = Acc<NF>;
    __shared__ SegSum<NF> wpart[kCarryThreads / kWave];
    __shared__ int nxt[kCarryThreads];
    __shared__ A fin;
    const int64_t row = blockIdx.x;
    if (row >= rows) return;  // uniform
    A* head = (A*)a.head;
    A* tail = (A*)a.tail;
    A* carry = (A*)a.carry;
    A* tot = (A*)a.tot;
    const int nt = a.ntiles, tid = threadIdx.x, lane = lane_id(), wid = tid >> 6;
    const int per = (nt + kCarryThreads - 1) / kCarryThreads;
    const int t0 = min(nt, tid * per), t1 = min(nt, t0 + per);
    const int64_t b = row * nt;
    // 1. the thread's run of tiles composed
    SegSum<NF> loc;
    loc.f = 0;
    loc.a = acc_zero<NF>();
    int first = INT_MAX;  // the run's first tile with a block start
    for (int t = t0; t < t1; ++t) {
        SegSum<NF> e;
        e.f = a.has[b + t] != 0 ? 1 : 0;
        e.a = e.f ? tail[b + t] : head[b + t];
        loc = seg_op(loc, e);
        if (e.f && first == INT_MAX) first = t;
    }
    // 2. exclusive scan of the compositions
    const SegSum<NF> inc = seg_scan_wave(loc);
    if (lane == kWave - 1) wpart[wid] = inc;
    nxt[tid] = first;
    __syncthreads();
    SegSum<NF> ex = seg_move<0x138, 0xf>(inc);  // the previous lane's (nothing in lane 0)
    SegSum<NF> pre;
    pre.f = 0;
    pre.a = acc_zero<NF>();
    for (int k = 0; k < wid; ++k) pre = seg_op(pre, wpart[k]);
    ex = seg_op(pre, ex);
    // 3. the carries into the run's tiles (the scan starts from zero sums)
    A c = ex.a;
    for (int t = t0; t < t1; ++t) {
        carry[b + t] = c;
        c = acc_pick(a.has[b + t] != 0, tail[b + t], acc_sum(c, head[b + t]));
    }
    if (t0 < nt && t1 == nt) fin = c;  // the thread holding the last tile
    // 4. the first tile with a block start after each thread's run: suffix
    // minimum over the threads (every run's carries written before it is read)
    for (int d = 1; d < kCarryThreads; d <<= 1) {
        __syncthreads();
        const int v = (tid + d < kCarryThreads) ? min(nxt[tid], nxt[tid + d]) : nxt[tid];
        __syncthreads();
        nxt[tid] = v;
    }
    __syncthreads();
    const int s = (tid + 1 < kCarryThreads) ? nxt[tid + 1] : INT_MAX;
    A after = (s < nt) ? acc_sum(carry[b + s], head[b + s]) : fin;
    for (int t = t1 - 1; t >= t0; --t) {
        tot[b + t] = after;
        if (a.has[b + t]) after = acc_sum(carry[b + t], head[b + t]);
    }
}

template <int NF>
__host__ __device__ inline size_t vjp_row_smem_bytes(int nl) {
    // slots [nl + 1] + per wave (flag, sums) and max-scan values
    return sizeof(Acc<NF>) * (size_t)(nl + 1) + 16 * (sizeof(Acc<NF>) + 2 * sizeof(int)) + 64;
}

// The first and last block starts (fs, ls) of a tile of N <= 64 * 64
// elements from its start words sb[0 .. (N + 63) / 64), found by every wave
// on its own (N, N without a start).
__device__ __forceinline__ void tile_start_span(const uint64_t* sb, int N, int& fs, int& ls) {
    const int lane = lane_id();
    uint64_t word = 0ull;
    if (lane < (N + 63) / 64) {
        word = sb[lane];
        const int rem = N - lane * 64;
        if (rem < 64) word &= (1ull << rem) - 1ull;
    }
    const uint64_t nz = __ballot(word != 0ull);
    fs = N;
    ls = N;
    if (nz != 0ull) {
        const int fw = lo_bit(nz), lw = hi_bit(nz);
        fs = fw * 64 + lo_bit(__shfl(word, fw, kWave));
        ls = lw * 64 + hi_bit(__shfl(word, lw, kWave));
    }
}

// NaN products over [t0, t0 + N) of a row whose fit was NaN.
template <typename T, int NF>
__device__ __forceinline__ void vjp_nan_span(const VjpArgs& a, int64_t row, int64_t t0, int N) {
    T* out = a.out ? (T*)a.out + row * a.n + t0 : nullptr;
    T* out_w = (NF == 3) ? (T*)a.out_w + row * a.n + t0 : nullptr;
    for (int i = threadIdx.x; i < N; i += blockDim.x) {
        if (out) out[i] = (T)NAN;
        if (NF == 3) out_w[i] = (T)NAN;
    }
}

// The products over [t0, t0 + N) of one row, kVjpK elements per lane.  In a
// tile (TILE) of a longer row, the block open at the tile's start (ending at
// fs - 1, fs the tile's first block start) has the totals head_total, and
// the block open at its end (from ls, its last block start, or the whole
// tile without a start) has open_total; both come from the carry pass, so
// the tile reads g only in [fs, ls), where its other blocks lie.
template <typename T, int NF, bool TILE>
__device__ __forceinline__ void vjp_span(const VjpArgs& a, int64_t row, int64_t t0, int N, int fs, int ls,
                                         const Acc<NF>& head_total, const Acc<NF>& open_total, char* smem) {
    using A = Acc<NF>;
    constexpr int K = kVjpK;
    const int l = threadIdx.x, lane = lane_id(), wid = l >> 6;
    // slot b + 1: the totals of a block that began in lane b; slot 0: of the
    // block open at the span's start
    A* slot = (A*)smem;
    A* wsum = slot + blockDim.x + 1;
    int* wflag = (int*)(wsum + 16);
    int* wmax = wflag + 16;
    const int64_t base = row * a.n + t0;
    const T* g = (const T*)a.g + base;
    const T* w = a.w ? (const T*)a.w + base : nullptr;
    const T* y = (NF == 3) ? (const T*)a.y + base : nullptr;
    T* out = a.out ? (T*)a.out + base : nullptr;
    T* out_w = (NF == 3) ? (T*)a.out_w + base : nullptr;
    const int e0 = l * K;
    const int cnt = min(max(N - e0, 0), K);
    // start bits of elements e0 .. e0 + K (one past the lane), clip bits of the
    // lane's; t0 and e0 are multiples of K, so a lane's bits sit in one word
    uint32_t sbit = 0, cbit = 0;
    if (cnt > 0) {
        const int64_t pos = t0 + e0;
        const int64_t q = pos >> 6;
        const int off = (int)(pos & 63);
        const uint64_t* sb = a.sb + row * a.words;
        const uint64_t* cb = a.cb + row * a.words;
        const uint64_t s0 = sb[q], s1 = (q + 1 < a.words) ? sb[q + 1] : 0ull;
        const uint64_t win = (s0 >> off) | (off ? (s1 << (64 - off)) : 0ull);
        sbit = (uint32_t)(win & ((1ull << (K + 1)) - 1ull));
        cbit = (uint32_t)((cb[q] >> off) & ((1ull << K) - 1ull));
    }
    // 1. in-lane segmented prefix sums
    double gv[K], wv[K], yv[K];
#pragma unroll
    for (int j = 0; j < K; ++j) gv[j] = wv[j] = yv[j] = 0.0;
    // a tile's lane reads g only where it meets [fs, ls); the clip bits mask
    // the rest, whose sums no block uses
    const bool need_g = !TILE || (e0 < ls && e0 + cnt > fs);
    if (TILE) cbit |= ~(uint32_t)(bits_range(max(fs - e0, 0), ls - 1 - e0) & 0xFFFFFFFFull);
    if (cnt > 0) {
        if (need_g) load_lane<T, K>(g + e0, cnt, gv);
        if (w) {
            load_lane<T, K>(w + e0, cnt, wv);
        } else {
#pragma unroll
            for (int j = 0; j < K; ++j) wv[j] = 1.0;
        }
        if (NF == 3) load_lane<T, K>(y + e0, cnt, yv);
    }
    A P[K];
    {
        A c = acc_zero<NF>();
#pragma unroll
        for (int j = 0; j < K; ++j) {
            if ((sbit >> j) & 1u) c = acc_zero<NF>();
            if (j < cnt) {
                c.v[0] += ((cbit >> j) & 1u) ? 0.0 : gv[j];
                c.v[1] += wv[j];
                if (NF == 3) c.v[NF - 1] += wv[j] * yv[j];
            }
            P[j] = c;
        }
    }
    const uint32_t own = sbit & ((1u << K) - 1u) & ((cnt >= K) ? 0xFFFFFFFFu : ((1u << cnt) - 1u));
    // 2. carries: segmented scan of (block starts in the lane, sums since its last start)
    SegSum<NF> me;
    me.f = own ? 1 : 0;
    me.a = P[K - 1];
    SegSum<NF> inc = seg_scan_wave(me);
    int mx = max_scan_wave(own ? l + 1 : 0);
    if (lane == kWave - 1) {
        wsum[wid] = inc.a;
        wflag[wid] = inc.f;
        wmax[wid] = mx;
    }
    __syncthreads();
    SegSum<NF> pre;
    pre.f = 0;
    pre.a = acc_zero<NF>();
    int pmax = 0;
    for (int k = 0; k < wid; ++k) {
        SegSum<NF> o;
        o.f = wflag[k];
        o.a = wsum[k];
        pre = seg_op(pre, o);
        pmax = max(pmax, wmax[k]);
    }
    SegSum<NF> ex;  // exclusive within the wave
    ex.f = dpp_move<0x138, 0xf>(inc.f);
#pragma unroll
    for (int k = 0; k < NF; ++k) ex.a.v[k] = dpp_move<0x138, 0xf>(inc.a.v[k]);
    const SegSum<NF> cin = seg_op(pre, ex);  // sums of the block open when the lane begins
    // lanes (+1) where blocks began (0: before the span): the last one before
    // the lane holds the block open at its start, the last one up to it the
    // block open at its end
    const int begin_open = max(pmax, dpp_move<0x138, 0xf>(mx));
    const int end_open = max(pmax, mx);
    // the carry reaches the elements before the lane's first start
    const int first = own ? (__ffs((int)own) - 1) : K;
#pragma unroll
    for (int j = 0; j < K; ++j) P[j] = acc_pick(j < first, acc_sum(cin.a, P[j]), P[j]);
    if (TILE) {
#pragma unroll
        for (int j = 0; j < K; ++j) {
            P[j] = acc_pick(e0 + j == fs - 1, head_total, P[j]);
            P[j] = acc_pick(e0 + j == N - 1, open_total, P[j]);
        }
    }
    // 3. a block that began in an earlier lane and ends here: totals to its slot
    //    (element j ends a block when it is the span's last or j + 1 starts one)
    int last_end = -1, first_end = K;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const bool end = (j < cnt) && ((e0 + j == N - 1) || ((sbit >> (j + 1)) & 1u));
        if (end) {
            last_end = j;
            if (first_end == K) first_end = j;
        }
    }
    if (first_end < K && first_end < first) {
        A v = acc_zero<NF>();
#pragma unroll
        for (int j = 0; j < K; ++j) v = acc_pick(j == first_end, P[j], v);  // no indexed access to registers
        slot[begin_open] = v;
    }
    __syncthreads();
    // 4. totals per element, backward; elements after the lane's last block end
    //    belong to the block open at its end
    //    The quotients change only where a block ends, so they are formed
    //    there (a branch that a wave skips unless one of its lanes takes it).
    A tot = acc_zero<NF>();
    if (cnt > 0 && last_end < cnt - 1) tot = slot[end_open];
    double gw = tot.v[0] / tot.v[1], mean = (NF == 3) ? tot.v[NF - 1] / tot.v[1] : 0.0;
#pragma unroll
    for (int j = K - 1; j >= 0; --j) {
        if (j == last_end || (j < last_end && ((sbit >> (j + 1)) & 1u))) {
            tot = P[j];
            gw = tot.v[0] / tot.v[1];
            if (NF == 3) mean = tot.v[NF - 1] / tot.v[1];
        }
        gv[j] = wv[j] * gw;
        if (NF == 3) yv[j] = gw * (yv[j] - mean);
    }
    if (cnt > 0) {
        if (out) store_lane<T, K>(out + e0, cnt, gv);
        if (NF == 3) store_lane<T, K>(out_w + e0, cnt, yv);
    }
}

template <typename T, int NF>
__global__ __launch_bounds__(1024) void k_vjp_row(VjpArgs a) {
    extern __shared__ __align__(32) char smem[];
    const int64_t row = blockIdx.x;
    if (a.row_nan[row]) {  // uniform: before any barrier
        vjp_nan_span<T, NF>(a, row, 0, (int)a.n);
        return;
    }
    vjp_span<T, NF, false>(a, row, 0, (int)a.n, 0, 0, acc_zero<NF>(), acc_zero<NF>(), smem);
}

// One tile of a long row, after the carry pass.  Capped at four waves per
// SIMD (two workgroups per CU): the weight product's registers would otherwise
// leave room for one.
template <typename T, int NF>
__global__ __launch_bounds__(kVjpTile / kVjpK) __attribute__((amdgpu_waves_per_eu(4))) void k_vjp_tile(VjpArgs a) {
    extern __shared__ __align__(32) char smem[];
    const int64_t row = blockIdx.x / a.ntiles;
    const int tile = (int)(blockIdx.x % a.ntiles);
    const int64_t t0 = (int64_t)tile * kVjpTile;
    const int N = (int)((a.n - t0) < kVjpTile ? (a.n - t0) : kVjpTile);
    if (a.row_nan[row]) {  // uniform: before any barrier
        vjp_nan_span<T, NF>(a, row, t0, N);
        return;
    }
    const int64_t ti = row * a.ntiles + tile;
    int fs, ls;
    tile_start_span(a.sb + row * a.words + t0 / 64, N, fs, ls);
    const Acc<NF> ht = acc_sum(((const Acc<NF>*)a.carry)[ti], ((const Acc<NF>*)a.head)[ti]);
    vjp_span<T, NF, true>(a, row, t0, N, fs, ls, ht, ((const Acc<NF>*)a.tot)[ti], smem);
}

// Sums of the tile's elements [lo, hi), kPartThreads apart per thread.  Each
// round issues kPartUnroll loads of every input before using any (the index
// clamped into the range, the value masked after).
constexpr int kPartThreads = 256;
constexpr int kPartUnroll = 4;
template <typename T, int NF>
__device__ __forceinline__ Acc<NF> part_sum(const T* g, const T* w, const T* y, const uint64_t* cb, int lo, int hi) {
    constexpr int U = kPartUnroll;
    Acc<NF> s = acc_zero<NF>();
    for (int b = lo + (int)threadIdx.x; b < hi; b += U * kPartThreads) {
        double gv[U], wv[U], yv[U];
        uint64_t cw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = min(b + u * kPartThreads, hi - 1);
            gv[u] = (double)g[e];
            wv[u] = w ? (double)w[e] : 1.0;
            yv[u] = 0.0;
            if constexpr (NF == 3) yv[u] = (double)y[e];
            cw[u] = cb[e >> 6];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = b + u * kPartThreads;
            const bool in = e < hi;
            const bool clip = ((cw[u] >> (e & 63)) & 1ull) != 0ull;
            s.v[0] += (in && !clip) ? gv[u] : 0.0;
            s.v[1] += in ? wv[u] : 0.0;
            if (NF == 3) s.v[NF - 1] += in ? wv[u] * yv[u] : 0.0;
        }
    }
    return s;
}

// The carry pass's input for one tile: the sums before its first block start
// (head), from its last block start to its end (tail), and whether it holds a
// start; without a start both are the whole tile's sums.  The start bits give
// the two positions, so only the head's and the tail's elements are read.
template <typename T, int NF>
__global__ __launch_bounds__(kPartThreads) void k_vjp_part(VjpArgs a) {
    using A = Acc<NF>;
    __shared__ A part[2][kPartThreads / kWave];
    const int64_t row = blockIdx.x / a.ntiles;
    const int tile = (int)(blockIdx.x % a.ntiles);
    const int64_t t0 = (int64_t)tile * kVjpTile;
    const int N = (int)((a.n - t0) < kVjpTile ? (a.n - t0) : kVjpTile);
    const int64_t ti = row * a.ntiles + tile;
    A* head = (A*)a.head;
    A* tail = (A*)a.tail;
    if (a.row_nan[row]) {
        if (threadIdx.x == 0) {
            A u = acc_zero<NF>();
            u.v[1] = 1.0;
            head[ti] = u;
            tail[ti] = u;
            a.has[ti] = 1;
        }
        return;
    }
    const uint64_t* cb = a.cb + row * a.words + t0 / 64;
    static_assert(kVjpTile <= 64 * kWave, "one start word per lane");
    const int lane = lane_id(), wid = threadIdx.x >> 6;
    int fs, ls;
    tile_start_span(a.sb + row * a.words + t0 / 64, N, fs, ls);
    const bool has = fs < N;
    const int64_t base = row * a.n + t0;
    const T* g = (const T*)a.g + base;
    const T* w = a.w ? (const T*)a.w + base : nullptr;
    const T* y = (NF == 3) ? (const T*)a.y + base : nullptr;
    A h = part_sum<T, NF>(g, w, y, cb, 0, fs);
    A t = acc_zero<NF>();
    if (has) t = part_sum<T, NF>(g, w, y, cb, ls, N);
#pragma unroll
    for (int m = kWave / 2; m >= 1; m >>= 1) {
        h = acc_sum(h, shfl_xor_acc(h, m));
        t = acc_sum(t, shfl_xor_acc(t, m));
    }
    if (lane == 0) {
        part[0][wid] = h;
        part[1][wid] = t;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        A hs = part[0][0], ts = part[1][0];
#pragma unroll
        for (int k = 1; k < kPartThreads / kWave; ++k) {
            hs = acc_sum(hs, part[0][k]);
            ts = acc_sum(ts, part[1][k]);
        }
        head[ti] = hs;
        tail[ti] = acc_pick(has, ts, hs);
        a.has[ti] = has ? 1 : 0;
    }
}

template <typename T, int NF>
static hipError_t launch_vjp_t(const VjpLaunch& l) {
    VjpArgs a{};
    a.g = l.g;
    a.w = l.w;
    a.y = l.y;
    a.out = l.out;
    a.out_w = l.out_w;
    a.n = l.n;
    a.words = l.words;
    a.sb = l.start_bits;
    a.cb = l.clip_bits;
    a.row_nan = l.row_nan;
    if (l.n <= 16) {
        hipLaunchKernelGGL((k_vjp_lane<T, NF, 16>), dim3((unsigned)((l.rows + 255) / 256)), dim3(256), 0, l.stream, a,
                           l.rows);
        return hipGetLastError();
    }
    if (l.n <= 2 * kLaneRow) {
        const dim3 grid((unsigned)((2 * l.rows + 63) / 64));
        if (l.n <= 32)
            hipLaunchKernelGGL((k_vjp_pair<T, NF, 16>), grid, dim3(64), 0, l.stream, a, l.rows);
        else
            hipLaunchKernelGGL((k_vjp_pair<T, NF, 32>), grid, dim3(64), 0, l.stream, a, l.rows);
        return hipGetLastError();
    }
    if (l.n <= kSingleMax) {
        const int nl = (int)(((l.n + kVjpK - 1) / kVjpK + 63) / 64 * 64);
        hipLaunchKernelGGL((k_vjp_row<T, NF>), dim3((unsigned)l.rows), dim3(nl), vjp_row_smem_bytes<NF>(nl), l.stream,
                           a);
        return hipGetLastError();
    }
    a.ntiles = (int)((l.n + kVjpTile - 1) / kVjpTile);
    const size_t tiles = (size_t)l.rows * (size_t)a.ntiles;
    Acc<NF>* p = (Acc<NF>*)(l.ws + l.L.vjp);
    a.head = p;
    a.tail = p + tiles;
    a.carry = p + 2 * tiles;
    a.tot = p + 3 * tiles;
    a.has = (int*)(p + 4 * tiles);
    hipLaunchKernelGGL((k_vjp_part<T, NF>), dim3((unsigned)tiles), dim3(kPartThreads), 0, l.stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_vjp_carry<NF>, dim3((unsigned)l.rows), dim3(kCarryThreads), 0, l.stream, a, l.rows);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int nl = kVjpTile / kVjpK;
    hipLaunchKernelGGL((k_vjp_tile<T, NF>), dim3((unsigned)tiles), dim3(nl), vjp_row_smem_bytes<NF>(nl), l.stream, a);
    return hipGetLastError();
}

hipError_t launch_vjp(const VjpLaunch& l) {
    if (l.out_w) return (l.dtype == 0) ? launch_vjp_t<float, 3>(l) : launch_vjp_t<double, 3>(l);
    return (l.dtype == 0) ? launch_vjp_t<float, 2>(l) : launch_vjp_t<double, 2>(l);
}

}  // namespace iso
