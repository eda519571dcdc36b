// Rows of 33 to 128 elements, several to a wave (first page, Sec. 3.5: short
// rows are packed several to a warp, each on the fewest lanes that hold it).
// The kernels take rows of up to 512 elements (32 lanes of 16 points, two rows
// a wave); the launcher sends rows of kPackedMin to kPackedMax here.
//
// A wave of 64 lanes takes R = floor(64 / L) consecutive rows, each on L =
// ceil(n / K) consecutive lanes of K points (K = 16, or 8 in the second
// pass).  Lane i of row r holds the row's elements Ki .. Ki + K - 1.
//
// The wave runs the one-tile pipeline of iso_tile.hpp over all of its lanes
// at once, as if its rows were one sequence: the lane starts are one scan over
// the wave, so row r's points sit in coordinates translated by the totals of
// the rows before it (the hull, and every slope, is unchanged by a
// translation), and row r's first point is row r-1's last, which is a vertex
// of both hulls.  What differs from one tile:
//   - the merge rounds pair nodes within a row only (node i with node i + h
//     of the same row, i a multiple of 2h), so they end with one node per
//     row, its hull;
//   - those nodes are then moved together into one list (each row's entries
//     after its first point, which is the previous row's last), on which the
//     edge values and the expansion run as for one tile;
//   - a row holding a NaN or a weight <= 0 is given flat points (unit
//     weights, zero values) so that the others' coordinates stay finite, and
//     comes back NaN;
//   - inputs and outputs go through LDS (the wave's rows are one contiguous
//     span of memory, read and written with consecutive lanes on consecutive
//     16-byte pieces), and each row's bit words are gathered by shuffles.
// Two passes, as for the chunks of long rows.  The first, with 16 points per
// lane, gives each wave a list of kPackCap entries (noise rows keep about 5
// of a lane's 16 points as lane-hull vertices), which leaves room for about
// 13 waves on a CU.  A wave with more vertices (dense rows: up to all 1024)
// is appended to one of 16 lists (by its index mod 16, the counters in
// separate 256-byte blocks, so that appends from many waves do not contend
// for one address) and writes nothing.  The second kernel fits the listed
// waves' rows with 8 points per lane, whose list holds every point of a wave
// (513 entries) at the same LDS size: dense rows run faster that way (a lane
// hull of 8 points costs a quarter of the comparisons of one of 16, and no
// wave can overflow), noisy rows slower (more lanes, rounds and waves per row).
#include <math.h>

#include "iso_device.hpp"
#include "iso_internal.hpp"
#include "iso_pack.hpp"
#include "iso_tile.hpp"

namespace iso {
namespace {

constexpr int kPackK = 16;     // points per lane, first pass
constexpr int kPackK2 = 8;     // points per lane, second pass
constexpr int kPackCap = 448;  // first-pass list entries besides point 0
constexpr int kPackAll2 = kWave * kPackK2;  // every point of a second-pass wave
constexpr int kPackLists = 16;
constexpr int kPackCtrStride = 64;  // ints between counters: each in its own 256-byte block

struct PackArgs {
    const void* y;
    const void* w;
    void* fit;
    int64_t rows;
    int n;
    int L;  // lanes per row, first pass
    int R;  // rows per wave, first pass
    int increasing;
    double lo, hi;
    uint64_t* start_bits;
    uint64_t* clip_bits;
    uint32_t* row_nan;
    int64_t words;
    unsigned long long* status;
    unsigned long long epoch;
    int* cover;   // [kPackLists][lcap] the waves left to the second pass
    int* ncover;  // [kPackLists] their counts, kPackCtrStride ints apart
    int lcap;     // entries of each list
};

// LDS of a pass: the tile with its list, or the stage of one input, whichever
// is larger (they are not in use at once).
template <typename T, int K>
constexpr size_t pack_smem_bytes(int cap) {
    const size_t tile = tile_smem_bytes(kWave, cap, K, sizeof(T) == 4);
    const size_t stage = (size_t)kWave * K * sizeof(T);
    return tile > stage ? tile : stage;
}

__global__ void k_pack_zero(int* p) {
    if (threadIdx.x < kPackLists) p[threadIdx.x * kPackCtrStride] = 0;
}

// The wave's span of `avail` elements written from LDS to out with
// consecutive lanes on consecutive elements (16-byte pieces when out is
// aligned to them).
template <typename T>
__device__ __forceinline__ void store_span(T* __restrict__ out, const T* stage, int avail) {
    constexpr int VW = 16 / (int)sizeof(T);
    const int lane = lane_id();
    if ((((uintptr_t)out) & 15) == 0) {
        const int nv = avail / VW;
        for (int q = lane; q < nv; q += kWave) ((uint4*)out)[q] = *(const uint4*)(stage + q * VW);
        for (int e = nv * VW + lane; e < avail; e += kWave) out[e] = stage[e];
    } else {
        for (int e = lane; e < avail; e += kWave) out[e] = stage[e];
    }
}

// Rows row0 .. row0 + nrows - 1 on one wave of K points per lane, with a list
// of cap entries besides point 0; a first-pass wave (wave >= 0) whose
// vertices exceed the list is listed for the second pass instead.
template <typename T, int K>
__device__ inline void packed_wave(const PackArgs& a, int64_t row0, int nrows, int cap, int64_t wave) {
    constexpr bool ABS = sizeof(T) == 4;
    extern __shared__ __align__(32) char smem[];
    const int lane = threadIdx.x;
    const int n = a.n, L = (n + K - 1) / K;
    const int r = lane / L, i = lane - r * L;                  // the lane's row in the wave, its lane in the row
    const bool live = r < nrows;
    const int cnt = live ? min(max(n - i * K, 0), K) : 0;
    const int span = nrows * n;  // the wave's elements, contiguous in memory
    const int off = live ? r * n + i * K : 0;
    const Tile t = tile_carve(smem, kWave, cap, K, kWave * K, ABS);

    // 1. inputs through LDS (the weights first, kept in registers, then the
    // values in the same space), the lane's points and hull
    T* stage = (T*)smem;
    T wv[K];
    const T* yb = (const T*)a.y + row0 * n;
    const T* wb = a.w ? (const T*)a.w + row0 * n : nullptr;
    if ((((uintptr_t)yb) & 15) == 0 && (wb == nullptr || (((uintptr_t)wb) & 15) == 0)) {
        // both inputs' loads in flight together
        StagePieces<T, K> PW, PY;
        if (wb) stage_fetch<T, K>(wb, span, PW);
        stage_fetch<T, K>(yb, span, PY);
        if (wb) {
            stage_put<T, K>(PW, stage);
            wave_sync();
#pragma unroll
            for (int j = 0; j < K; ++j) wv[j] = (j < cnt) ? stage[off + j] : (T)0;
            wave_sync();  // every lane has its weights before the values replace them
        }
        stage_put<T, K>(PY, stage);
        wave_sync();
    } else {
        if (wb) {
            stage_wave<T, K>(wb, span, stage);
#pragma unroll
            for (int j = 0; j < K; ++j) wv[j] = (j < cnt) ? stage[off + j] : (T)0;
            wave_sync();  // every lane has its weights before the values replace them
        }
        stage_wave<T, K>(yb, span, stage);
    }
    double xs[K], ys[K];
    int f = 0;
    {
        // the sums as lane_hull forms them: float32 without branches (products
        // of two floats are exact in float64; a non-finite input leaves a
        // total non-finite, the least weight finds a weight <= 0), float64
        // checked element by element
        double X = 0.0, Y = 0.0;
        const double sg = a.increasing ? 1.0 : -1.0;
        float wmin = INFINITY;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const bool in = j < cnt;
            const double yi = in ? (double)stage[off + j] : 0.0;
            const double wi = in ? (a.w ? (double)wv[j] : 1.0) : 0.0;
            if constexpr (ABS) {
                X += wi;
                Y = fma(wi * sg, yi, Y);
                wmin = fminf(wmin, in ? (float)wi : 1.f);
            } else if (in) {
                if (!isfinite(yi) || !isfinite(wi))
                    f |= 1;
                else if (!(wi > 0.0))
                    f |= 2;
                double ti = wi * yi;
                if (!a.increasing) ti = -ti;
                X += wi;
                Y += ti;
            }
            xs[j] = X;
            ys[j] = Y;
        }
        if constexpr (ABS) {
            if (!isfinite(X) || !isfinite(Y)) f |= 1;
            if (!(wmin > 0.f)) f |= 2;
        }
    }
    wave_sync();  // the stage is read; the tile takes its space
    uint64_t mask = lane_gift_wrap<K>(xs, ys, cnt);
    // a row holding a NaN (bit 0) or a weight <= 0 (bit 1) anywhere
    const uint64_t rbits = live ? (bits_upto(L - 1) << (r * L)) : 0ull;
    const bool rnan = (__ballot((f & 1) != 0) & rbits) != 0ull;
    const bool rwerr = !rnan && (__ballot((f & 2) != 0) & rbits) != 0ull;
    const bool bad = rnan || rwerr;
    if (bad) {
#pragma unroll
        for (int j = 0; j < K; ++j) {
            xs[j] = (double)min(j + 1, cnt);
            ys[j] = 0.0;
        }
        mask = cnt > 0 ? (1ull << (cnt - 1)) : 0ull;
    }
    const int nvert = tile_lane_starts<!ABS>(t, make_double2(xs[K - 1], ys[K - 1]), 0, __popcll(mask));
    if (wave >= 0 && nvert > cap + 1) {  // uniform
        if (lane == 0) {
            const int k = (int)(wave % kPackLists);
            a.cover[k * a.lcap + atomicAdd(a.ncover + k * kPackCtrStride, 1)] = (int)wave;
        }
        return;  // nothing written: the second pass fits the wave
    }

    // 2. the list of every lane's vertices, then merge rounds within each row
    tile_compact<K, ABS>(t, mask, xs, ys);
    int ns = t.I[lane] - 1;
    int ne = (lane + 1 < kWave) ? t.I[lane + 1] - 1 : t.flag[1] - 1;
    for (int h = 1; h < L; h <<= 1) {
        const int m = (L - h + 2 * h - 1) / (2 * h);  // merges per row
        const int M = nrows * m;
        int G = kWave;
        while (G > 1 && G * M > kWave) G >>= 1;
        const int k = lane / G, g = lane & (G - 1);
        const int kr = k / m, la = (k < M) ? kr * L + (k - kr * m) * 2 * h : 0;
        const int a0 = __shfl(ns, la, kWave), a1 = __shfl(ne, la, kWave);
        const int b0 = __shfl(ns, la + h, kWave), b1 = __shfl(ne, la + h, kWave);
        int nend = 0;
        if (k < M) nend = group_merge<K, ABS>(t, a0, a1, b0, b1, g, G);
        const bool owner = live && (i % (2 * h)) == 0 && i + h < L;
        const int src = owner ? (r * m + i / (2 * h)) * G : 0;
        const int ns2 = __shfl(a0, src, kWave), ne2 = __shfl(nend, src, kWave);
        if (owner) {
            ns = ns2;
            ne = ne2;
        }
        wave_sync();
    }

    // 3. the rows' hulls into one list: row q's entries after its first point
    // (the previous row's last) follow row q-1's.  Every entry moves to a
    // place at or before its own, and the moves go in order of destination,
    // 64 at a time, each batch read before it is written: no entry is
    // overwritten before it is read.
    {
        int tot = 1;
        for (int q = 0; q < nrows; ++q) tot += __shfl(ne, q * L, kWave) - __shfl(ns, q * L, kWave);
        for (int d0 = 1; d0 < tot; d0 += kWave) {
            const int d = d0 + lane;
            int src = -1, P = 1;
            for (int q = 0; q < nrows; ++q) {
                const int s = __shfl(ns, q * L, kWave), c = __shfl(ne, q * L, kWave) - s;
                if (d >= P && d < P + c) src = s + 1 + (d - P);
                P += c;
            }
            unsigned short pv = 0;
            double2 xy = make_double2(0.0, 0.0);
            if (src >= 0) {
                pv = t.V[src];
                xy = t.VXY[src];
            }
            wave_sync();
            if (src >= 0) {
                t.V[d] = pv;
                t.VXY[d] = xy;
            }
            wave_sync();
        }
        if (lane == 0) t.flag[1] = tot;
        __syncthreads();
    }
    tile_masks<K>(t, mask);

    // 4. edge values, expansion, stores
    tile_edge_slopes<K, ABS>(t, a.increasing, a.lo, a.hi);
    double vals[K];
    uint64_t clipm;
    tile_expand<K>(t, mask, vals, clipm);
    __syncthreads();  // the list is read; the stage's space takes the outputs
    T* so = (T*)smem;
    if (live) {
#pragma unroll
        for (int j = 0; j < K; ++j)
            if (j < cnt) so[off + j] = bad ? (T)NAN : (T)vals[j];
    }
    __syncthreads();
    store_span<T>((T*)a.fit + row0 * n, so, span);

    // 5. bits: element 16i + j starts a block iff its left point is a vertex
    // (point 0 of the lane: the previous lane's last point; of the row: always)
    if (a.start_bits) {
        const uint64_t prev = __shfl_up(mask, 1, kWave);
        const uint64_t carry = (i == 0) ? 1ull : ((prev >> (K - 1)) & 1ull);
        const uint64_t own = bits_upto(cnt - 1);
        uint64_t sv = bad ? 0ull : (((mask << 1) | carry) & own);
        uint64_t cv = bad ? 0ull : (clipm & own);
        // four lanes to a 64-bit word; the word's first lane gathers it
        constexpr int LPW = 64 / K;
#pragma unroll
        for (int d = 1; d < LPW; ++d) {
            const uint64_t s2 = __shfl_down(sv, d, kWave), c2 = __shfl_down(cv, d, kWave);
            if (i + d < L) {
                sv |= s2 << (d * K);
                cv |= c2 << (d * K);
            }
        }
        if (live && (i % LPW) == 0) {
            const int64_t at = (row0 + r) * a.words + i / LPW;
            a.start_bits[at] = sv;
            a.clip_bits[at] = cv;
        }
    }
    if (live && i == 0) {
        if (a.row_nan) a.row_nan[row0 + r] = bad ? 1u : 0u;
        if (rwerr) report_weight_error(a.status, a.epoch);
    }
}

template <typename T>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4))) void k_rows_packed(PackArgs a) {
    mark_epoch(a.status, a.epoch);
    const int64_t row0 = (int64_t)blockIdx.x * a.R;
    packed_wave<T, kPackK>(a, row0, (int)min((int64_t)a.R, a.rows - row0), kPackCap, blockIdx.x);
}

// The second pass: a grid of workgroups (a multiple of kPackLists) over the
// listed first-pass waves, read after the first pass has completed, in stream
// order.  A first-pass wave's rows take `sub` waves of 8 points per lane.
template <typename T>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3))) void k_rows_packed_cover(PackArgs a) {
    const int L2 = (a.n + kPackK2 - 1) / kPackK2, R2 = kWave / L2, sub = (a.R + R2 - 1) / R2;
    const int k = blockIdx.x % kPackLists, per = gridDim.x / kPackLists;
    const int items = a.ncover[k * kPackCtrStride] * sub;
    for (int it = blockIdx.x / kPackLists; it < items; it += per) {
        const int64_t wave = a.cover[k * a.lcap + it / sub];
        const int64_t w0 = wave * a.R, wend = min(w0 + a.R, a.rows);
        const int64_t row0 = w0 + (int64_t)(it % sub) * R2;
        const int nrows = (int)min((int64_t)R2, wend - row0);
        if (nrows > 0) packed_wave<T, kPackK2>(a, row0, nrows, kPackAll2, -1);
        __syncthreads();  // the next wave reuses the LDS
    }
}

template <typename T>
hipError_t launch_t(const PackedLaunch& l) {
    PackArgs a{};
    a.y = l.y;
    a.w = l.w;
    a.fit = l.fit;
    a.rows = l.rows;
    a.n = (int)l.n;
    a.L = (int)((l.n + kPackK - 1) / kPackK);
    a.R = kWave / a.L;
    a.increasing = l.increasing;
    a.lo = l.lo;
    a.hi = l.hi;
    a.start_bits = l.start_bits;
    a.clip_bits = l.clip_bits;
    a.row_nan = l.row_nan;
    a.words = l.words;
    a.status = l.status;
    a.epoch = l.epoch;
    a.ncover = l.cover;
    a.cover = l.cover + kPackLists * kPackCtrStride;
    const int64_t waves = (l.rows + a.R - 1) / a.R;
    a.lcap = (int)((waves + kPackLists - 1) / kPackLists);
    const size_t smem0 = pack_smem_bytes<T, kPackK>(kPackCap), smem1 = pack_smem_bytes<T, kPackK2>(kPackAll2);
    static size_t seen0[kMaxDevices] = {}, seen1[kMaxDevices] = {};
    hipError_t e = ensure_lds((const void*)k_rows_packed<T>, smem0, seen0);
    if (e == hipSuccess) e = ensure_lds((const void*)k_rows_packed_cover<T>, smem1, seen1);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_pack_zero, dim3(1), dim3(kPackLists), 0, l.stream, a.ncover);
    hipLaunchKernelGGL(k_rows_packed<T>, dim3((unsigned)waves), dim3(kWave), smem0, l.stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // about 13 second-pass waves fit on a CU
    const int L2 = (int)((l.n + kPackK2 - 1) / kPackK2), R2 = kWave / L2;
    const int64_t items = (int64_t)a.lcap * ((a.R + R2 - 1) / R2);
    const int64_t per = items < 208 ? items : 208;
    const unsigned grid = (unsigned)(per * kPackLists);
    hipLaunchKernelGGL(k_rows_packed_cover<T>, dim3(grid), dim3(kWave), smem1, l.stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rows_packed(const PackedLaunch& l) {
    return l.dtype == 0 ? launch_t<float>(l) : launch_t<double>(l);
}

}  // namespace iso
