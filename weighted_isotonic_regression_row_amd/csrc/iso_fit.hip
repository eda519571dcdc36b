// Forward kernels of the isotonic fit for gfx950.
//
// Page "Merge Hulls Without Copying Vertices: GPU Isotonic Regression":
//   k_row_fit      rows of at most 8192 elements: one workgroup per row builds
//                  the row's hull in LDS and writes the fit (Sec. 3: "a row that
//                  fits in one chunk is finished at the second level").
//   k_chunk_hull   longer rows: one workgroup per chunk of 4096 elements builds
//                  the chunk's hull once, stores its vertices (chunk-relative
//                  coordinates, Sec. 3.3), the chunk totals, and a tentative fit
//                  from the chunk's own hull.
//   k_merge_tree   one workgroup per long row: double-double chunk starts
//                  (exclusive scan of the chunk totals, Sec. 3.3 and App. B),
//                  then every level of the merge tree on segment lists, at most
//                  one segment per chunk (Sec. 3.3, Theorem 4.4), then per-chunk
//                  records of the root list (Sec. 3.4).
//   k_fixup        per chunk, rewrites only the elements that lie outside the
//                  chunk's surviving segment (the edge rule after Theorem 4.4:
//                  they lie under the edge entering or leaving the segment, or
//                  a chunk without a segment lies under one edge).
#include <math.h>

#include "iso_device.hpp"
#include "iso_internal.hpp"

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
};

// Every writer of one call stores the same value, so a plain exchange is
// enough; the epoch tells iso_status whether the word belongs to the latest
// call (the word is never cleared, and may hold garbage before a first error).
__device__ inline void report_weight_error(unsigned long long* status, unsigned long long epoch) {
    atomicExch(status, (epoch << 8) | 3ull);
}

// Expand (Sec. 3.4) over the workgroup's range: fit, block-start and clip bits.
template <typename T>
__device__ inline void wg_expand(int N, HullSmem s, T* out, int increasing, double lo, double hi,
                                 uint64_t* sbits, uint64_t* cbits) {
    const int lane = lane_id();
    const int wid = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    const int G = hull_groups(N);
    for (int g = wid; g < G; g += nw) {
        uint64_t word;
        const double sl = group_edge_slope(N, g, s, word);
        const int i = g * kWave + lane;
        bool clipped = false;
        const double v = finish(sl, increasing, lo, hi, clipped);
        if (i < N) out[i] = (T)v;
        const uint64_t cb = __ballot(i < N && clipped);
        if (sbits && lane == 0) {
            const int cnt = N - g * kWave;
            const uint64_t valid = (cnt >= 64) ? ~0ull : ((1ull << cnt) - 1ull);
            sbits[g] = word & valid;
            cbits[g] = cb;
        }
    }
}

template <typename T>
__device__ inline void wg_write_nan_row(int64_t N, T* out, uint64_t* sbits, uint64_t* cbits) {
    for (int64_t i = threadIdx.x; i < N; i += blockDim.x) out[i] = (T)NAN;
    if (sbits) {
        const int64_t words = (N + 63) / 64;
        for (int64_t q = threadIdx.x; q < words; q += blockDim.x) {
            sbits[q] = 0ull;
            cbits[q] = 0ull;
        }
    }
}

// ---------------------------------------------------------------------------
// one workgroup per row
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(512) void k_row_fit(RowArgs a) {
    extern __shared__ __align__(32) char smem[];
    const int64_t row = blockIdx.x;
    const int N = (int)a.n;
    HullSmem s = hull_smem_carve(smem, N);
    const T* y = (const T*)a.y + row * a.n;
    const T* w = a.w ? (const T*)a.w + row * a.n : nullptr;
    T* out = (T*)a.fit + row * a.n;
    uint64_t* sb = a.start_bits ? a.start_bits + row * a.words : nullptr;
    uint64_t* cb = a.clip_bits ? a.clip_bits + row * a.words : nullptr;
    if (threadIdx.x == 0) s.flag[0] = 0;
    __syncthreads();
    wg_load_prefix<T, 4>(y, w, N, a.increasing, s);
    __syncthreads();
    const int flag = s.flag[0];
    if (flag) {
        wg_write_nan_row<T>(N, out, sb, cb);
        if (threadIdx.x == 0) {
            if (a.row_nan) a.row_nan[row] = 1u;
            if (flag == 2) report_weight_error(a.status, a.epoch);
        }
        return;
    }
    wg_group_starts(N, s);
    wg_group_hulls(N, s);
    wg_group_merges(N, s);
    wg_expand<T>(N, s, out, a.increasing, a.lo, a.hi, sb, cb);
    if (a.row_nan && threadIdx.x == 0) a.row_nan[row] = 0u;
}

// ---------------------------------------------------------------------------
// chunk hulls of long rows
// ---------------------------------------------------------------------------
struct ChunkArgs {
    RowArgs r;
    int64_t m;  // chunks per row
    double4* totals;  // chunk totals, double-double (xh, xl, yh, yl)
    int* nv;
    int* cflag;
    double4* vxy;     // chunk hull vertices, chunk-relative double-double
    int* vidx;
};

template <typename T>
__global__ __launch_bounds__(512) void k_chunk_hull(ChunkArgs a) {
    extern __shared__ __align__(32) char smem[];
    const int64_t bid = blockIdx.x;
    const int64_t row = bid / a.m, c = bid % a.m;
    const int64_t e0 = c * kChunk;
    const int N = (int)((a.r.n - e0) < kChunk ? (a.r.n - e0) : kChunk);
    HullSmem s = hull_smem_carve(smem, N);
    const T* y = (const T*)a.r.y + row * a.r.n + e0;
    const T* w = a.r.w ? (const T*)a.r.w + row * a.r.n + e0 : nullptr;
    T* out = (T*)a.r.fit + row * a.r.n + e0;
    uint64_t* sb = a.r.start_bits ? a.r.start_bits + row * a.r.words + e0 / 64 : nullptr;
    uint64_t* cb = a.r.clip_bits ? a.r.clip_bits + row * a.r.words + e0 / 64 : nullptr;
    if (threadIdx.x == 0) s.flag[0] = 0;
    __syncthreads();
    wg_load_prefix<T, 4>(y, w, N, a.r.increasing, s);
    __syncthreads();
    const int flag = s.flag[0];
    if (flag) {
        // the whole row comes back NaN; k_fixup writes it
        if (threadIdx.x == 0) {
            a.cflag[bid] = flag;
            a.nv[bid] = 0;
        }
        return;
    }
    wg_group_starts(N, s);
    wg_group_hulls(N, s);
    wg_group_merges(N, s);

    // vertex ranks: exclusive scan of the popcounts of the vertex words
    const int nwords = hull_words(N);
    const int lane = lane_id();
    if ((threadIdx.x >> 6) == 0) {
        const int k = (nwords + kWave - 1) / kWave;
        int cnt = 0;
        for (int j = 0; j < k; ++j) {
            const int q = lane * k + j;
            if (q < nwords) cnt += __popcll(s.Mk[q]);
        }
        const int incl = wave_incl_scan_int(cnt);
        int ex = incl - cnt;
        for (int j = 0; j < k; ++j) {
            const int q = lane * k + j;
            if (q < nwords) {
                s.WO[q] = ex;
                ex += __popcll(s.Mk[q]);
            }
        }
        if (lane == kWave - 1) s.flag[1] = incl;
    }
    __syncthreads();
    double4* V = a.vxy + bid * kVSlot;
    int* VI = a.vidx + bid * kVSlot;
    for (int k = threadIdx.x; k <= N; k += blockDim.x) {
        const uint64_t word = s.Mk[k >> 6];
        if ((word >> (k & 63)) & 1ull) {
            const int rank = s.WO[k >> 6] + __popcll(word & ((1ull << (k & 63)) - 1ull));
            V[rank] = pabs(s, k);
            VI[rank] = k;
        }
    }
    if (threadIdx.x == 0) {
        a.nv[bid] = s.flag[1];
        a.cflag[bid] = 0;
        a.totals[bid] = pabs(s, N);
    }
    // tentative fit from the chunk's own hull; k_fixup corrects the elements
    // outside the chunk's surviving segment
    wg_expand<T>(N, s, out, a.r.increasing, a.r.lo, a.r.hi, sb, cb);
}

// ---------------------------------------------------------------------------
// merge tree of one long row
// ---------------------------------------------------------------------------
struct MergeArgs {
    int64_t m;
    const double4* totals;
    const int* nv;
    const int* cflag;
    const double4* vxy;
    const int* vidx;
    double4* starts;
    Desc* gdesc;
    int* gnc;
    double* gso;
    Rec* rec;
    uint32_t* row_nan;
    unsigned long long* status;
    unsigned long long epoch;
    int use_lds;
};

// a point of the row: chunk start + chunk-relative vertex, both double-double
struct PtD {
    double4 c;  // chunk start (xh, xl, yh, yl)
    double4 v;  // vertex relative to the chunk start
};

struct MCtx {
    Desc* D;
    int* NC;
    const double4* st;
    const double4* V;
};

struct VR {
    int s;  // descriptor slot
    int k;  // vertex rank in the chunk hull
};

__device__ __forceinline__ PtD ptd(const MCtx& X, int c, int k) {
    PtD p;
    p.c = X.st[c];
    p.v = X.V[(int64_t)c * kVSlot + k];
    return p;
}
__device__ __forceinline__ PtD ptv(const MCtx& X, VR v) { return ptd(X, X.D[v.s].c, v.k); }

// differences formed part by part (first page, App. B, "Merge levels": the
// turn is computed from differences of the hi, lo and chunk-relative parts)
__device__ __forceinline__ double pdx(const PtD& a, const PtD& b) {
    return ((b.c.x - a.c.x) + (b.c.y - a.c.y)) + ((b.v.x - a.v.x) + (b.v.y - a.v.y));
}
__device__ __forceinline__ double pdy(const PtD& a, const PtD& b) {
    return ((b.c.z - a.c.z) + (b.c.w - a.c.w)) + ((b.v.z - a.v.z) + (b.v.w - a.v.w));
}
__device__ __forceinline__ double turnD(const PtD& a, const PtD& b, const PtD& d) {
    return pdx(a, b) * pdy(a, d) - pdy(a, b) * pdx(a, d);
}
__device__ __forceinline__ double slopeD(const PtD& a, const PtD& b) { return pdy(a, b) / pdx(a, b); }

// successor of v in the list whose last slot is s1
__device__ __forceinline__ bool vsucc(const MCtx& X, VR v, int s1, VR& n) {
    if (v.k < X.D[v.s].h) {
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
    if (v.k > X.D[v.s].l) {
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

// First vertex of the view (slots s0..s1, last slot ending at lastH) for which
// a monotone predicate (false ... false true ... true) holds; the view's last
// vertex must satisfy it.  Bisection first over segments, then within one
// (first page, Sec. 3.3).
template <class Pred>
__device__ inline VR first_true(const MCtx& X, int s0, int s1, int lastH, Pred pred) {
    int lo = s0, hi = s1 + 1;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (pred(VR{mid, X.D[mid].l}))
            hi = mid;
        else
            lo = mid + 1;
    }
    if (lo == s0) return VR{s0, X.D[s0].l};
    const int sg = lo - 1;
    const int hv = (sg == s1) ? lastH : X.D[sg].h;
    int rlo = X.D[sg].l + 1, rhi = hv + 1;
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
    return VR{lo, X.D[lo].l};
}

// Lower tangent from p (left of every vertex of B) to B = slots jB..sB1: the
// vertex minimising the slope from p, the farthest one on ties.
__device__ inline VR tangent_b(const MCtx& X, const PtD& p, int jB, int sB1) {
    return first_true(X, jB, sB1, X.D[sB1].h, [&](VR v) -> bool {
        VR nx;
        if (!vsucc(X, v, sB1, nx)) return true;
        return turnD(p, ptv(X, v), ptv(X, nx)) > 0.0;
    });
}

constexpr int kWalkCap = 48;

// Merge the node at j0 (slots j0..) with its right neighbour at jB (Sec. 3.3,
// Lemma 4.2, Theorem 4.4).  The result overwrites the left node's slots.
__device__ inline void merge_pair(const MCtx& X, int j0, int jB) {
    Desc* D = X.D;
    int cntA = X.NC[j0];
    const int cntB = X.NC[jB];
    const int la = j0 + cntA - 1;
    const int sB1 = jB + cntB - 1;
    const Desc dA = D[la];
    const Desc dB = D[jB];
    // s: the last vertex of A and the first of B (chunk jB's point 0)
    const VR sA{la, dA.h};
    const VR sB{jB, dB.l};
    VR pA, nB;
    vpred(X, sA, j0, pA);  // A has at least two vertices
    vsucc(X, sB, sB1, nB); // and so has B
    PtD PA = ptv(X, pA), PS = ptv(X, sB), PB = ptv(X, nB);
    if (turnD(PA, PS, PB) > 0.0) {
        // convex at s: keep s once, in B's first segment
        if (dA.h - 1 < dA.l) {
            cntA -= 1;
        } else {
            D[la].h = dA.h - 1;
        }
        for (int i = 0; i < cntB; ++i) D[j0 + cntA + i] = D[jB + i];
        X.NC[j0] = cntA + cntB;
        return;
    }
    // walk from the neighbours of s (Sec. 4, after Lemma 4.2), capped
    VR al = pA, be = nB;
    bool done = false;
    for (int step = 0; step < kWalkCap; ++step) {
        VR pa, nb;
        const bool canA = vpred(X, al, j0, pa);
        const bool canB = vsucc(X, be, sB1, nb);
        const PtD Pp = canA ? ptv(X, pa) : PA;
        const PtD Pn = canB ? ptv(X, nb) : PB;
        const bool mA = canA && !(turnD(Pp, PA, PB) > 0.0);
        if (mA) {
            al = pa;
            PA = Pp;
        }
        const bool mB = canB && !(turnD(PA, PB, Pn) > 0.0);
        if (mB) {
            be = nb;
            PB = Pn;
        }
        if (!mA && !mB) {
            done = true;
            break;
        }
    }
    if (!done) {
        // nested bisection (Sec. 3.3, Thm. 5.2): a candidate a of A is tested
        // against its tangent to B; a is left of the bridge while A's next
        // vertex lies strictly below the line from a to its tangent point.
        // Candidates end at the predecessor of s.
        int aS1 = la, aLastH = dA.h - 1;
        if (aLastH < dA.l) {
            aS1 = la - 1;
            aLastH = D[la - 1].h;
        }
        al = first_true(X, j0, aS1, aLastH, [&](VR a) -> bool {
            VR an;
            vsucc(X, a, la, an);
            const PtD Pa = ptv(X, a);
            const VR b = tangent_b(X, Pa, jB, sB1);
            return !(turnD(Pa, ptv(X, an), ptv(X, b)) > 0.0);
        });
        be = tangent_b(X, ptv(X, al), jB, sB1);
    }
    // cut A at alpha and B at beta, move B's tail down behind A's head
    D[al.s].h = al.k;
    const int newA = al.s - j0 + 1;
    D[be.s].l = be.k;
    const int nBk = sB1 - be.s + 1;
    for (int i = 0; i < nBk; ++i) D[j0 + newA + i] = D[be.s + i];
    X.NC[j0] = newA + nBk;
}

constexpr int kMergeThreads = 1024;

__global__ __launch_bounds__(kMergeThreads) void k_merge_tree(MergeArgs a) {
    extern __shared__ __align__(32) char smem[];
    const int64_t row = blockIdx.x;
    const int m = (int)a.m;
    const int tid = threadIdx.x;
    const int NT = blockDim.x;
    const int64_t base = row * a.m;
    double4* sbuf = (double4*)smem;                     // [NT]
    int* sflag = (int*)(smem + sizeof(double4) * NT);  // [4]
    Desc* D;
    int* NC;
    if (a.use_lds) {
        D = (Desc*)(smem + sizeof(double4) * NT + 16);
        NC = (int*)(smem + sizeof(double4) * NT + 16 + sizeof(Desc) * (size_t)m);
    } else {
        D = a.gdesc + base;
        NC = a.gnc + base;
    }
    Rec* rec = a.rec + base;

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
    for (int c = c0; c < c1; ++c) loc = dd4_add(loc, a.totals[base + c]);
    double4 v = loc;
    sbuf[tid] = v;
    __syncthreads();
    for (int d = 1; d < NT; d <<= 1) {
        double4 o = make_double4(0.0, 0.0, 0.0, 0.0);
        if (tid >= d) o = sbuf[tid - d];
        __syncthreads();
        if (tid >= d) v = dd4_add(o, v);
        sbuf[tid] = v;
        __syncthreads();
    }
    double4 ex = make_double4(0.0, 0.0, 0.0, 0.0);
    if (tid > 0) ex = sbuf[tid - 1];
    for (int c = c0; c < c1; ++c) {
        a.starts[base + c] = ex;
        ex = dd4_add(ex, a.totals[base + c]);
    }
    // 3. leaves: one segment per chunk, its whole hull
    for (int c = tid; c < m; c += NT) {
        Desc d;
        d.c = c;
        d.l = 0;
        d.h = a.nv[base + c] - 1;
        d.pad = 0;
        D[c] = d;
        NC[c] = 1;
    }
    __threadfence_block();
    __syncthreads();

    MCtx X;
    X.D = D;
    X.NC = NC;
    X.st = a.starts + base;
    X.V = a.vxy + base * kVSlot;

    // 4. merge levels
    for (int h = 1; h < m; h <<= 1) {
        const int nm = (m - h + 2 * h - 1) / (2 * h);
        for (int k = tid; k < nm; k += NT) {
            const int j0 = k * 2 * h;
            merge_pair(X, j0, j0 + h);
        }
        __threadfence_block();
        __syncthreads();
    }

    // 5. per-chunk records of the root list
    const int K = NC[0];
    double* so = a.gso + base;
    for (int k = tid; k < K - 1; k += NT) {
        const Desc d0 = D[k], d1 = D[k + 1];
        so[k] = slopeD(ptd(X, d0.c, d0.h), ptd(X, d1.c, d1.l));
    }
    __threadfence();
    __syncthreads();
    const int* VI = a.vidx + base * kVSlot;
    for (int c = tid; c < m; c += NT) {
        // last root segment whose chunk is <= c
        int lo = 0, hi = K;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (D[mid].c <= c)
                lo = mid;
            else
                hi = mid;
        }
        const Desc d = D[lo];
        Rec r{};
        if (d.c == c) {
            r.mode = 0;
            r.lo = VI[(int64_t)c * kVSlot + d.l];
            r.hi = VI[(int64_t)c * kVSlot + d.h];
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
static int pick_threads(int N) {
    const int G = hull_groups(N);
    if (G >= 32) return 512;
    if (G >= 8) return 256;
    return 64 * ((G + 1) / 2 > 0 ? (G + 1) / 2 : 1);
}

template <typename T>
static hipError_t launch_fit_t(const FitLaunch& a) {
    unsigned long long* status = (unsigned long long*)(a.ws + a.L.status);
    if (a.n <= kSingleMax) {
        RowArgs r{a.y, a.w, a.fit, a.n, a.increasing, a.lo, a.hi, a.start_bits, a.clip_bits, a.row_nan,
                  a.words, status, a.epoch};
        const int N = (int)a.n;
        const size_t smem = hull_smem_bytes(N);
        const int nt = pick_threads(N);
        static bool attr_set = false;
        if (!attr_set) {
            (void)hipFuncSetAttribute((const void*)k_row_fit<T>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)hull_smem_bytes((int)kSingleMax));
            attr_set = true;
        }
        hipLaunchKernelGGL(k_row_fit<T>, dim3((unsigned)a.rows), dim3(nt), smem, a.stream, r);
        return hipGetLastError();
    }
    const int64_t m = a.L.m;
    ChunkArgs ca;
    ca.r = RowArgs{a.y, a.w, a.fit, a.n, a.increasing, a.lo, a.hi, a.start_bits, a.clip_bits, a.row_nan,
                   a.words, status, a.epoch};
    ca.m = m;
    ca.totals = (double4*)(a.ws + a.L.totals);
    ca.nv = (int*)(a.ws + a.L.nv);
    ca.cflag = (int*)(a.ws + a.L.cflag);
    ca.vxy = (double4*)(a.ws + a.L.vxy);
    ca.vidx = (int*)(a.ws + a.L.vidx);
    {
        static bool attr_set = false;
        if (!attr_set) {
            (void)hipFuncSetAttribute((const void*)k_chunk_hull<T>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)hull_smem_bytes(kChunk));
            attr_set = true;
        }
        hipLaunchKernelGGL(k_chunk_hull<T>, dim3((unsigned)(a.rows * m)), dim3(512), hull_smem_bytes(kChunk),
                           a.stream, ca);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    MergeArgs ma;
    ma.m = m;
    ma.totals = ca.totals;
    ma.nv = ca.nv;
    ma.cflag = ca.cflag;
    ma.vxy = ca.vxy;
    ma.vidx = ca.vidx;
    ma.starts = (double4*)(a.ws + a.L.starts);
    ma.gdesc = (Desc*)(a.ws + a.L.desc);
    ma.gnc = (int*)(a.ws + a.L.nc);
    ma.gso = (double*)(a.ws + a.L.so);
    ma.rec = (Rec*)(a.ws + a.L.rec);
    ma.row_nan = a.row_nan;
    ma.status = status;
    ma.epoch = a.epoch;
    ma.use_lds = (m <= kMergeLdsChunks) ? 1 : 0;
    size_t msmem = sizeof(double4) * kMergeThreads + 16;
    if (ma.use_lds) msmem += (sizeof(Desc) + sizeof(int)) * (size_t)m;
    {
        static bool attr_set = false;
        if (!attr_set) {
            (void)hipFuncSetAttribute((const void*)k_merge_tree, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)(sizeof(double4) * kMergeThreads + 16 + (sizeof(Desc) + sizeof(int)) * kMergeLdsChunks));
            attr_set = true;
        }
        hipLaunchKernelGGL(k_merge_tree, dim3((unsigned)a.rows), dim3(kMergeThreads), msmem, a.stream, ma);
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
