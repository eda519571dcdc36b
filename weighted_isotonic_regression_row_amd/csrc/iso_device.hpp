// Device-side building blocks shared by the fit kernels (gfx950, wave64).
//
// A workgroup builds the lower convex hull of the cumulative sum diagram of
// N consecutive elements (page "Merge Hulls Without Copying Vertices: GPU
// Isotonic Regression", Sec. 2.1 Eq. (2) and Sec. 3.1-3.2), here as:
//
//   1. load + weighted prefix sums in float64: one element per lane, 64
//      consecutive elements per "group", a wave-wide inclusive scan inside the
//      group, and a double-double exclusive scan of the group totals;
//   2. group hulls: the 64 points of a group are merged in six pairwise
//      rounds, all merges of a round at once, one lane per merge walking to
//      the bridge (Sec. 4, Lemma 4.2 and the walk that follows it).  The hull
//      is a 64-bit vertex mask held in scalar registers;
//   3. group merges: the group hulls are merged in log2(groups) rounds, one
//      thread per merge walking over a two-level vertex bit set in LDS
//      (one word per group plus a summary word of non-empty groups), the
//      paper's "merge lane hulls by walking, skipping empty lanes" with wave64
//      words.
//
// Coordinates (a hierarchy in the spirit of the first page's Appendix B,
// "Merge levels"): point k is X_k = D[k / 64] + L_k, where L_k is the sum of
// the elements of k's group before k (group-local, at most 64 terms) and
// D[g] is the group's start relative to the workgroup's first point, kept as
// a double-double.  Differences of two points are formed part by part, so a
// difference is accurate to the rounding of the 64-element group sums around
// it rather than of the whole range's sums.
//
// Point k (k = 0..N) is P_k of the range; element i lies between P_i and
// P_{i+1}.  Bit k of the vertex set is point k.  A turn of zero is treated as
// non-convex, so collinear middle points are dropped (Sec. 2.1 and 4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iso {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// (b - a) x (d - a) from the two differences u = b - a and v = d - a:
// positive iff d lies strictly above the line through a and b (x increasing),
// i.e. the chain a -> b -> d turns left and b is a strict lower-hull vertex of
// {a, b, d}.  The "turn" of the first page, Appendix B.
__device__ __forceinline__ double cross2(double2 u, double2 v) { return u.x * v.y - u.y * v.x; }

__device__ __forceinline__ double2 sub2(double2 b, double2 a) { return make_double2(b.x - a.x, b.y - a.y); }

__device__ __forceinline__ double turn3(double2 a, double2 b, double2 d) { return cross2(sub2(b, a), sub2(d, a)); }

// Orientation of the output, clipping after the fit, and the clip flag.  NaN
// passes through unchanged.
__device__ __forceinline__ double finish(double slope, int increasing, double lo, double hi, bool& clipped) {
    double v = increasing ? slope : -slope;
    clipped = (v < lo) || (v > hi);
    v = (v < lo) ? lo : v;
    v = (v > hi) ? hi : v;
    return v;
}

__device__ __forceinline__ double wave_incl_scan(double v) {
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        double t = __shfl_up(v, d, kWave);
        if (lane >= d) v += t;
    }
    return v;
}

__device__ __forceinline__ int wave_incl_scan_int(int v) {
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int t = __shfl_up(v, d, kWave);
        if (lane >= d) v += t;
    }
    return v;
}

__device__ __forceinline__ int hi_bit(uint64_t m) { return 63 - __clzll((long long)m); }
__device__ __forceinline__ int lo_bit(uint64_t m) { return __ffsll((long long)m) - 1; }

// bits [0, b] set (b in [0, 63])
__device__ __forceinline__ uint64_t bits_upto(int b) { return (b >= 63) ? ~0ull : ((2ull << b) - 1ull); }
// bits [b, 63] set (b in [0, 64])
__device__ __forceinline__ uint64_t bits_from(int b) { return (b >= 64) ? 0ull : (~0ull << b); }

// ---------------------------------------------------------------------------
// double-double arithmetic (error-free transformations; no multiplications,
// so no contraction into fused multiply-adds can change them)
// ---------------------------------------------------------------------------
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
    s = a + b;
    const double bb = s - a;
    e = (a - (s - bb)) + (b - bb);
}
__device__ __forceinline__ void fast_two_sum(double a, double b, double& s, double& e) {
    s = a + b;
    e = b - (s - a);
}
__device__ __forceinline__ void dd_add(double ah, double al, double bh, double bl, double& rh, double& rl) {
    double s, e, t, f;
    two_sum(ah, bh, s, e);
    two_sum(al, bl, t, f);
    e += t;
    fast_two_sum(s, e, s, e);
    e += f;
    fast_two_sum(s, e, rh, rl);
}
// (xh, xl, yh, yl) pairs
__device__ __forceinline__ double4 dd4_add(double4 a, double4 b) {
    double4 r;
    dd_add(a.x, a.y, b.x, b.y, r.x, r.y);
    dd_add(a.z, a.w, b.z, b.w, r.z, r.w);
    return r;
}
// double-double + double
__device__ __forceinline__ double4 dd4_add_d(double4 a, double2 b) {
    double4 r;
    dd_add(a.x, a.y, b.x, 0.0, r.x, r.y);
    dd_add(a.z, a.w, b.y, 0.0, r.z, r.w);
    return r;
}
__device__ __forceinline__ double4 shfl_up4(double4 v, int d) {
    return make_double4(__shfl_up(v.x, d, kWave), __shfl_up(v.y, d, kWave), __shfl_up(v.z, d, kWave),
                        __shfl_up(v.w, d, kWave));
}

// ---------------------------------------------------------------------------
// Workgroup hull state in LDS
// ---------------------------------------------------------------------------

struct HullSmem {
    double2* XY;    // [N + 1] group-local cumulative (W, S): XY[k] for k % 64 != 0, and the
                    // group total at XY[64 (g + 1)]
    double2* GT;    // [groups] group totals
    double4* GD;    // [groups + 1] group starts relative to point 0, double-double (xh, xl, yh, yl)
    uint64_t* Mk;   // [N / 64 + 1] vertex set, bit k = point k
    uint64_t* Sm;   // [(words + 63) / 64] summary: bit g = Mk[g] != 0
    int2* MR;       // [64] (alpha, beta) of each group-level merge of a round
    int* flag;      // [4] row flags: bit 0 non-finite input, bit 1 weight <= 0; [1..3] scratch
    int* WO;        // [words] vertex rank offsets (chunk kernel)
};

__host__ __device__ inline int hull_words(int N) { return N / 64 + 1; }
__host__ __device__ inline int hull_groups(int N) { return (N + 63) / 64; }
__host__ __device__ inline int hull_sum_words(int N) { return (hull_words(N) + 63) / 64; }

// LDS bytes of a HullSmem for N elements.
__host__ __device__ inline size_t hull_smem_bytes(int N) {
    size_t b = 0;
    b += sizeof(double2) * (size_t)(N + 1);
    b += sizeof(double2) * (size_t)hull_groups(N);
    b += sizeof(double4) * (size_t)(hull_groups(N) + 1);
    b += sizeof(uint64_t) * (size_t)hull_words(N);
    b += sizeof(uint64_t) * (size_t)hull_sum_words(N);
    b += sizeof(int2) * 64;
    b += sizeof(int) * 4;
    b += sizeof(int) * (size_t)hull_words(N);
    return b + 96;
}

__device__ inline HullSmem hull_smem_carve(char* base, int N) {
    HullSmem s;
    char* p = base;
    s.XY = (double2*)p;
    p += sizeof(double2) * (size_t)(N + 1);
    s.GT = (double2*)p;
    p += sizeof(double2) * (size_t)hull_groups(N);
    p = (char*)(((uintptr_t)p + 31) & ~(uintptr_t)31);
    s.GD = (double4*)p;
    p += sizeof(double4) * (size_t)(hull_groups(N) + 1);
    s.Mk = (uint64_t*)p;
    p += sizeof(uint64_t) * (size_t)hull_words(N);
    s.Sm = (uint64_t*)p;
    p += sizeof(uint64_t) * (size_t)hull_sum_words(N);
    s.MR = (int2*)p;
    p += sizeof(int2) * 64;
    s.flag = (int*)p;
    p += sizeof(int) * 4;
    s.WO = (int*)p;
    return s;
}

// group-local coordinate of point k (0 at a group's first point)
__device__ __forceinline__ double2 local_pt(const HullSmem& s, int k) {
    return (k & 63) ? s.XY[k] : make_double2(0.0, 0.0);
}

// X_b - X_a, formed part by part from the group starts and local sums
__device__ __forceinline__ double2 pdelta(const HullSmem& s, int a, int b) {
    const double2 La = local_pt(s, a), Lb = local_pt(s, b);
    const int ga = a >> 6, gb = b >> 6;
    if (ga == gb) return sub2(Lb, La);
    const double4 A = s.GD[ga], B = s.GD[gb];
    return make_double2(((B.x - A.x) + (B.y - A.y)) + (Lb.x - La.x), ((B.z - A.z) + (B.w - A.w)) + (Lb.y - La.y));
}

__device__ __forceinline__ double pturn(const HullSmem& s, int a, int b, int d) {
    return cross2(pdelta(s, a, b), pdelta(s, a, d));
}

__device__ __forceinline__ double pslope(const HullSmem& s, int a, int b) {
    const double2 d = pdelta(s, a, b);
    return d.y / d.x;
}

// X_k relative to point 0 as a double-double (xh, xl, yh, yl)
__device__ __forceinline__ double4 pabs(const HullSmem& s, int k) {
    return dd4_add_d(s.GD[k >> 6], local_pt(s, k));
}

// ---------------------------------------------------------------------------
// Phase 1: load and weighted prefix sums (first page, Eq. (2)); float64
// accumulation, t_i = w_i * y_i negated for a non-increasing fit (the
// non-increasing fit of y is minus the non-decreasing fit of -y).
// ---------------------------------------------------------------------------

template <typename T, int U>
__device__ inline void wg_load_prefix(const T* __restrict__ y, const T* __restrict__ w, int N, int increasing,
                                      HullSmem s) {
    const int lane = lane_id();
    const int wid = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    const int G = hull_groups(N);
    int f = 0;
    for (int g0 = wid; g0 < G; g0 += nw * U) {
        double wv[U], tv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int g = g0 + u * nw;
            const int i = g * kWave + lane;
            double yi = 0.0, wi = 0.0;
            if (g < G && i < N) {
                yi = (double)y[i];
                wi = w ? (double)w[i] : 1.0;
            }
            wv[u] = wi;
            tv[u] = yi;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int g = g0 + u * nw;
            const int i = g * kWave + lane;
            if (g < G) {
                double wi = wv[u], yi = tv[u];
                if (i < N) {
                    if (!isfinite(yi) || !isfinite(wi))
                        f |= 1;
                    else if (!(wi > 0.0))
                        f |= 2;
                }
                double ti = wi * yi;
                if (!increasing) ti = -ti;
                double pw = wave_incl_scan(wi);
                double pt = wave_incl_scan(ti);
                if (i < N) s.XY[i + 1] = make_double2(pw, pt);
                if (lane == kWave - 1) s.GT[g] = make_double2(pw, pt);
            }
        }
    }
    uint64_t b1 = __ballot(f & 1), b2 = __ballot(f & 2);
    if (lane == 0 && (b1 | b2)) atomicOr(s.flag, (b1 ? 1 : 0) | (b2 ? 2 : 0));
}

// Phase 1b: double-double exclusive scan of the group totals into the group
// starts GD[0..G] (GD[G] = the range total).  One wave; ends with a barrier.
__device__ inline void wg_group_starts(int N, HullSmem s) {
    const int lane = lane_id();
    const int wid = threadIdx.x >> 6;
    const int G = hull_groups(N);
    if (wid == 0) {
        const int k = (G + kWave - 1) / kWave;  // groups per lane
        double4 v = make_double4(0.0, 0.0, 0.0, 0.0);
        for (int j = 0; j < k; ++j) {
            const int g = lane * k + j;
            if (g < G) v = dd4_add_d(v, s.GT[g]);
        }
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const double4 o = shfl_up4(v, d);
            if (lane >= d) v = dd4_add(o, v);
        }
        double4 ex = shfl_up4(v, 1);
        if (lane == 0) ex = make_double4(0.0, 0.0, 0.0, 0.0);
        for (int j = 0; j < k; ++j) {
            const int g = lane * k + j;
            if (g < G) {
                s.GD[g] = ex;
                ex = dd4_add_d(ex, s.GT[g]);
            }
        }
        if (lane == kWave - 1) s.GD[G] = v;
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Phase 2: hull of one group of 64 points by six rounds of pairwise merges.
// Lane l owns point q = l + 1 of the group (relative to the group's start
// point q = 0); bit l of the returned mask is set iff point q = l + 1 is a
// vertex of the group's hull.  cnt = number of elements in the group (1..64).
// All coordinates are the group-local sums.
// ---------------------------------------------------------------------------

// highest owned point q' in (lo, q) whose bit is set, else lo
__device__ __forceinline__ int grp_prev(uint64_t M, int q, int lo) {
    uint64_t m = M & ((q >= 2) ? bits_upto(q - 2) : 0ull) & bits_from(lo);
    return m ? hi_bit(m) + 1 : lo;
}
// lowest owned point q' in (q, hi] whose bit is set, else hi
__device__ __forceinline__ int grp_next(uint64_t M, int q, int hi) {
    uint64_t m = M & bits_from(q) & bits_upto(hi - 1);
    return m ? lo_bit(m) + 1 : hi;
}

__device__ __forceinline__ double2 grp_pt(const double2* __restrict__ XY, int base, int q) {
    return q ? XY[base + q] : make_double2(0.0, 0.0);
}

__device__ inline uint64_t wave_group_hull(const double2* __restrict__ XY, int base, int cnt) {
    const int lane = lane_id();
    uint64_t M = (cnt >= 64) ? ~0ull : ((1ull << cnt) - 1ull);
#pragma unroll 1
    for (int r = 0; r < 6; ++r) {
        const int h = 1 << r;
        if (h >= cnt) break;
        const int a = lane & ~(2 * h - 1);
        const bool owner = (lane == a + h - 1) && (a + h < cnt);
        int alpha = 0, beta = 0, cut = 0;
        if (owner) {
            const int lo = a, s = a + h, hi = min(a + 2 * h, cnt);
            int pA = grp_prev(M, s, lo), nB = grp_next(M, s, hi);
            double2 PA = grp_pt(XY, base, pA), PS = grp_pt(XY, base, s), PB = grp_pt(XY, base, nB);
            if (!(turn3(PA, PS, PB) > 0.0)) {
                cut = 1;
                alpha = pA;
                beta = nB;
                for (;;) {
                    const bool canA = alpha > lo, canB = beta < hi;
                    const int pa = canA ? grp_prev(M, alpha, lo) : alpha;
                    const int nb = canB ? grp_next(M, beta, hi) : beta;
                    const double2 Pp = grp_pt(XY, base, pa), Pn = grp_pt(XY, base, nb);
                    const bool mA = canA && !(turn3(Pp, PA, PB) > 0.0);
                    if (mA) {
                        alpha = pa;
                        PA = Pp;
                    }
                    const bool mB = canB && !(turn3(PA, PB, Pn) > 0.0);
                    if (mB) {
                        beta = nb;
                        PB = Pn;
                    }
                    if (!mA && !mB) break;
                }
            }
        }
        const int o = a + h - 1;
        const int al = __shfl(alpha, o, kWave);
        const int be = __shfl(beta, o, kWave);
        const int ct = __shfl(cut, o, kWave);
        const int q = lane + 1;
        const bool keep = ((M >> lane) & 1ull) && !(ct && q > al && q < be);
        M = __ballot(keep);
    }
    return M;
}

// Phase 2 driver: every wave builds the hulls of its groups and stores the
// vertex words.  Starts after a barrier; ends with a barrier.
__device__ inline void wg_group_hulls(int N, HullSmem s) {
    const int lane = lane_id();
    const int wid = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    const int G = hull_groups(N);
    for (int g = wid; g < G; g += nw) {
        const int cnt = min(kWave, N - g * kWave);
        uint64_t M = wave_group_hull(s.XY, g * kWave, cnt);
        if (lane == 0) s.Mk[g] = (M << 1) | 1ull;  // point 64g (the group's start) is a vertex here
    }
    if (threadIdx.x == 0 && (N % 64) == 0) s.Mk[N / 64] = 1ull;  // the last point N
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Phase 3: group-level merges over the vertex bit set in LDS.
// ---------------------------------------------------------------------------

// highest vertex point in (lo, p), else lo.  lo must be a vertex.
__device__ inline int set_prev(const uint64_t* Mk, const uint64_t* Sm, int p, int lo) {
    const int k = p - 1;
    if (k <= lo) return lo;
    const int g = k >> 6;
    uint64_t word = Mk[g] & bits_upto(k & 63);
    int res = lo;
    if (word) {
        res = (g << 6) + hi_bit(word);
    } else {
        int gg = -1;
        const int gl = g - 1;  // g >= 1 here since lo's word is not empty
        for (int j = gl >> 6; j >= 0; --j) {
            uint64_t sm = Sm[j];
            if (j == (gl >> 6)) sm &= bits_upto(gl & 63);
            if (sm) {
                gg = (j << 6) + hi_bit(sm);
                break;
            }
        }
        if (gg >= 0) res = (gg << 6) + hi_bit(Mk[gg]);
    }
    return res > lo ? res : lo;
}

// lowest vertex point in (p, hi], else hi.  hi must be a vertex.
__device__ inline int set_next(const uint64_t* Mk, const uint64_t* Sm, int nwords, int p, int hi) {
    const int k = p + 1;
    if (k >= hi) return hi;
    const int g = k >> 6;
    uint64_t word = Mk[g] & bits_from(k & 63);
    int res = hi;
    if (word) {
        res = (g << 6) + lo_bit(word);
    } else {
        const int gh = g + 1;
        const int nsw = (nwords + 63) >> 6;
        int gg = -1;
        for (int j = gh >> 6; j < nsw; ++j) {
            uint64_t sm = Sm[j];
            if (j == (gh >> 6)) sm &= bits_from(gh & 63);
            if (sm) {
                gg = (j << 6) + lo_bit(sm);
                break;
            }
        }
        if (gg >= 0) res = (gg << 6) + lo_bit(Mk[gg]);
    }
    return res < hi ? res : hi;
}

__device__ inline void wg_update_summary(int N, HullSmem s) {
    const int nwords = hull_words(N);
    for (int t0 = 0; t0 < nwords; t0 += blockDim.x) {
        const int t = t0 + threadIdx.x;
        const bool nz = (t < nwords) && (s.Mk[t] != 0ull);
        const uint64_t b = __ballot(nz);
        if (lane_id() == 0 && t - lane_id() < nwords) s.Sm[t >> 6] = b;
    }
}

// Group-level merges.  Starts after wg_group_hulls (barrier done); ends with a
// barrier.  Merges of a round are independent, one thread each (at most 64
// merges per round for N <= 8192, so wave 0 runs them).
__device__ inline void wg_group_merges(int N, HullSmem s) {
    const int G = hull_groups(N);
    const int nwords = hull_words(N);
    wg_update_summary(N, s);
    __syncthreads();
    for (int h = 1; h < G; h <<= 1) {
        const int nm = (G - h + 2 * h - 1) / (2 * h);  // merges with a + h < G
        for (int t = threadIdx.x; t < nm; t += blockDim.x) {
            const int a = t * 2 * h;
            const int lo = a * 64, sp = (a + h) * 64, hi = min((a + 2 * h) * 64, N);
            int alpha = sp, beta = sp;
            const int pA = set_prev(s.Mk, s.Sm, sp, lo);
            const int nB = set_next(s.Mk, s.Sm, nwords, sp, hi);
            if (!(pturn(s, pA, sp, nB) > 0.0)) {
                alpha = pA;
                beta = nB;
                for (;;) {
                    const bool canA = alpha > lo, canB = beta < hi;
                    const int pa = canA ? set_prev(s.Mk, s.Sm, alpha, lo) : alpha;
                    const int nb = canB ? set_next(s.Mk, s.Sm, nwords, beta, hi) : beta;
                    const bool mA = canA && !(pturn(s, pa, alpha, beta) > 0.0);
                    if (mA) alpha = pa;
                    const bool mB = canB && !(pturn(s, alpha, beta, nb) > 0.0);
                    if (mB) beta = nb;
                    if (!mA && !mB) break;
                }
            }
            s.MR[t] = make_int2(alpha, beta);
        }
        __syncthreads();
        // clear the points strictly between alpha and beta, one word per thread
        for (int t = threadIdx.x; t < nwords; t += blockDim.x) {
            const int mi = t / (2 * h);
            if (mi < nm) {
                const int2 ab = s.MR[mi];
                const int p0 = max(ab.x + 1, t * 64), p1 = min(ab.y - 1, t * 64 + 63);
                if (p0 <= p1) {
                    const uint64_t m = bits_from(p0 - t * 64) & bits_upto(p1 - t * 64);
                    s.Mk[t] &= ~m;
                }
            }
        }
        __syncthreads();
        wg_update_summary(N, s);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Phase 4: per element, the slope of the hull edge above it (first page,
// Sec. 3.4): element i lies under the edge from the last vertex <= i to the
// first vertex >= i + 1.  A lane whose left point is a vertex computes its
// edge's slope; lane 0 of a group also computes the edge entering the group;
// every other lane takes the slope of the nearest computing lane to its left.
// Returns the slope for element g*64 + lane (garbage for lanes past N).
// ---------------------------------------------------------------------------

__device__ inline double group_edge_slope(int N, int g, HullSmem s, uint64_t& word_out) {
    const int lane = lane_id();
    const int nwords = hull_words(N);
    const int i = g * kWave + lane;
    const uint64_t word = s.Mk[g];
    word_out = word;
    const bool isv = (word >> lane) & 1ull;
    const bool comp = (i < N) && (isv || lane == 0);
    double sl = 0.0;
    if (comp) {
        const int pv = isv ? i : set_prev(s.Mk, s.Sm, i, 0);
        const int nx = set_next(s.Mk, s.Sm, nwords, i, N);
        sl = pslope(s, pv, nx);
    }
    const uint64_t cm = __ballot(comp);
    const uint64_t below = cm & bits_upto(lane);
    const int src = below ? hi_bit(below) : 0;
    return __shfl(sl, src, kWave);
}

}  // namespace iso
