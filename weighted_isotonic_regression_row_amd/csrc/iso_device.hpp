// Device-side helpers shared by the fit and backward kernels (gfx950, wave64):
// bit operations on 64-bit masks, wave scans, and double-double sums.
//
// Coordinates of the cumulative sum diagram (page "Merge Hulls Without Copying
// Vertices: GPU Isotonic Regression", Sec. 2.1 Eq. (2)) are kept as a
// hierarchy in the spirit of the same page's Appendix B ("Merge levels"): a
// short local sum in float64 plus a start kept as a double-double (hi, lo).
// Differences of two points are formed part by part, so their accuracy is
// that of the short local sums, not of the long running totals.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iso {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Orders the calling wave's LDS accesses: writes by any of its lanes before
// the call are seen by reads of any of its lanes after it.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ int hi_bit(uint64_t m) { return 63 - __clzll((long long)m); }
__device__ __forceinline__ int lo_bit(uint64_t m) { return __ffsll((long long)m) - 1; }

// bits [0, b] set (b in [0, 63]); b < 0 gives 0
__device__ __forceinline__ uint64_t bits_upto(int b) {
    return (b < 0) ? 0ull : ((b >= 63) ? ~0ull : ((2ull << b) - 1ull));
}
// bits [b, 63] set (b in [0, 64])
__device__ __forceinline__ uint64_t bits_from(int b) { return (b >= 64) ? 0ull : (~0ull << b); }
// bits [a, b] set (0 <= a, b <= 63); empty if a > b
__device__ __forceinline__ uint64_t bits_range(int a, int b) { return (a > b) ? 0ull : (bits_upto(b) & bits_from(a)); }

// cross product (b - a) x (d - a) from u = b - a and v = d - a: positive iff d
// lies strictly above the line through a and b (x increasing), i.e. b is a
// strict lower-hull vertex of {a, b, d} (the "turn" of the first page,
// Appendix B).
__device__ __forceinline__ double cross2(double2 u, double2 v) { return u.x * v.y - u.y * v.x; }
__device__ __forceinline__ double2 sub2(double2 b, double2 a) { return make_double2(b.x - a.x, b.y - a.y); }

// Orientation of the output, clipping after the fit, and the clip flag.  NaN
// passes through unchanged.
__device__ __forceinline__ double finish(double slope, int increasing, double lo, double hi, bool& clipped) {
    double v = increasing ? slope : -slope;
    clipped = (v < lo) || (v > hi);
    v = (v < lo) ? lo : v;
    v = (v > hi) ? hi : v;
    return v;
}

// Lane moves by DPP (data-parallel primitives of the gfx9 family: a VALU
// operand read from another lane, no LDS round trip).  A lane whose source
// falls outside the pattern, or whose row is masked off, reads 0.
//   row_shr:n   from lane - n within each row of 16 lanes (0x110 + n)
//   row_bcast15 lane 15 of each row to the next row (0x142; rows 1 and 3)
//   row_bcast31 lane 31 to rows 2 and 3 (0x143)
//   wave_shr1   from lane - 1 across the whole wave (0x138)
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_move(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_move(double v) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    const unsigned lo = (unsigned)dpp_move<CTRL, ROWS>((int)(unsigned)b);
    const unsigned hi = (unsigned)dpp_move<CTRL, ROWS>((int)(unsigned)(b >> 32));
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double4 dpp_move(double4 v) {
    return make_double4(dpp_move<CTRL, ROWS>(v.x), dpp_move<CTRL, ROWS>(v.y), dpp_move<CTRL, ROWS>(v.z),
                        dpp_move<CTRL, ROWS>(v.w));
}

// The same moves, but a lane whose source falls outside the pattern (or whose
// row is masked off) keeps its own value.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_keep(double v) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    const int lo = (int)(unsigned)b, hi = (int)(unsigned)(b >> 32);
    const unsigned rlo = (unsigned)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWS, 0xf, false);
    const unsigned rhi = (unsigned)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWS, 0xf, false);
    return __longlong_as_double((long long)(((unsigned long long)rhi << 32) | rlo));
}
__device__ __forceinline__ double readlane_d(double v, int lane) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)b, lane);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), lane);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
// A value every lane of the wave holds alike, moved to scalar registers.
__device__ __forceinline__ double uniform_d(double v) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)b);
    const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(b >> 32));
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
// Least value over the wave (no NaN), the same in every lane: the scan's
// steps with min, whose result gathers in lane 63.
__device__ __forceinline__ double wave_min(double v) {
    v = fmin(v, dpp_keep<0x111, 0xf>(v));
    v = fmin(v, dpp_keep<0x112, 0xf>(v));
    v = fmin(v, dpp_keep<0x114, 0xf>(v));
    v = fmin(v, dpp_keep<0x118, 0xf>(v));
    v = fmin(v, dpp_keep<0x142, 0xa>(v));
    v = fmin(v, dpp_keep<0x143, 0xc>(v));
    return readlane_d(v, kWave - 1);
}

// Least value over the wave (no NaN), the same in every lane.  The floats are
// mapped to unsigned keys that decrease as the value increases (the sort key
// of the float's bits, complemented), so the least value is the greatest key
// and a lane whose source falls outside a move reads 0, which never wins: the
// moves fold into the maximum instructions.
__device__ __forceinline__ float wave_min_f(float v) {
    const unsigned b = __float_as_uint(v);
    unsigned r = ~(b ^ ((b >> 31) ? 0xffffffffu : 0x80000000u));
    r = max(r, (unsigned)dpp_move<0x111, 0xf>((int)r));
    r = max(r, (unsigned)dpp_move<0x112, 0xf>((int)r));
    r = max(r, (unsigned)dpp_move<0x114, 0xf>((int)r));
    r = max(r, (unsigned)dpp_move<0x118, 0xf>((int)r));
    r = max(r, (unsigned)dpp_move<0x142, 0xa>((int)r));
    r = max(r, (unsigned)dpp_move<0x143, 0xc>((int)r));
    const unsigned u = ~(unsigned)__builtin_amdgcn_readlane((int)r, kWave - 1);
    return __uint_as_float(u ^ ((u >> 31) ? 0x80000000u : 0xffffffffu));
}

// Inclusive scan over the 64 lanes of the wave with op(earlier, later), whose
// identity is the all-zero value: Hillis-Steele steps 1, 2, 4, 8 inside each
// row of 16 lanes, then the rows' totals by two broadcasts.
template <typename V, typename Op>
__device__ __forceinline__ V wave_scan_incl(V v, Op op) {
    v = op(dpp_move<0x111, 0xf>(v), v);
    v = op(dpp_move<0x112, 0xf>(v), v);
    v = op(dpp_move<0x114, 0xf>(v), v);
    v = op(dpp_move<0x118, 0xf>(v), v);
    v = op(dpp_move<0x142, 0xa>(v), v);
    v = op(dpp_move<0x143, 0xc>(v), v);
    return v;
}
// The previous lane's value (0 in lane 0).
template <typename V>
__device__ __forceinline__ V wave_shift_up1(V v) {
    return dpp_move<0x138, 0xf>(v);
}

__device__ __forceinline__ int wave_incl_scan_int(int v) {
    return wave_scan_incl(v, [](int a, int b) { return a + b; });
}

// K values of p[0..cnt) as float64 (0 past cnt); 16-byte vector loads when the
// lane's elements are whole and aligned.
template <typename T, int K>
__device__ __forceinline__ void load_lane(const T* __restrict__ p, int cnt, double (&v)[K]) {
    constexpr int VW = 16 / (int)sizeof(T);
    if constexpr (K % VW == 0) {
        if (cnt == K && (((uintptr_t)p) & 15) == 0) {
            if constexpr (sizeof(T) == 4) {
#pragma unroll
                for (int q = 0; q < K / 4; ++q) {
                    const float4 f = ((const float4*)p)[q];
                    v[4 * q] = f.x;
                    v[4 * q + 1] = f.y;
                    v[4 * q + 2] = f.z;
                    v[4 * q + 3] = f.w;
                }
            } else {
#pragma unroll
                for (int q = 0; q < K / 2; ++q) {
                    const double2 d = ((const double2*)p)[q];
                    v[2 * q] = d.x;
                    v[2 * q + 1] = d.y;
                }
            }
            return;
        }
    }
#pragma unroll
    for (int j = 0; j < K; ++j) v[j] = (j < cnt) ? (double)p[j] : 0.0;
}

template <typename T, int K>
__device__ __forceinline__ void store_lane(T* __restrict__ p, int cnt, const double (&v)[K]) {
    constexpr int VW = 16 / (int)sizeof(T);
    if constexpr (K % VW == 0) {
        if (cnt == K && (((uintptr_t)p) & 15) == 0) {
            if constexpr (sizeof(T) == 4) {
#pragma unroll
                for (int q = 0; q < K / 4; ++q)
                    ((float4*)p)[q] = make_float4((float)v[4 * q], (float)v[4 * q + 1], (float)v[4 * q + 2],
                                                  (float)v[4 * q + 3]);
            } else {
#pragma unroll
                for (int q = 0; q < K / 2; ++q) ((double2*)p)[q] = make_double2(v[2 * q], v[2 * q + 1]);
            }
            return;
        }
    }
#pragma unroll
    for (int j = 0; j < K; ++j)
        if (j < cnt) p[j] = (T)v[j];
}

// ---------------------------------------------------------------------------
// double-double arithmetic (error-free transformations; additions only, so no
// contraction into fused multiply-adds can change them)
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
// double-double pair + double pair
__device__ __forceinline__ double4 dd4_add_d(double4 a, double2 b) {
    double4 r;
    dd_add(a.x, a.y, b.x, 0.0, r.x, r.y);
    dd_add(a.z, a.w, b.y, 0.0, r.z, r.w);
    return r;
}
// B - A of two double-double pairs, rounded to a double pair (part by part)
__device__ __forceinline__ double2 dd4_diff(double4 A, double4 B) {
    return make_double2((B.x - A.x) + (B.y - A.y), (B.z - A.z) + (B.w - A.w));
}

// Status words of a fit call (the workspace's first 16 bytes).
// Every writer of one call stores the same value, so a plain exchange is
// enough.  status[0] is never cleared (it may hold garbage before a first
// error); status[1] holds the epoch of the latest call, written by thread 0 of
// workgroup 0 of the call's first kernel, so after the call iso_status reports
// status[0]'s code only when its epoch is status[1].
__device__ inline void report_weight_error(unsigned long long* status, unsigned long long epoch) {
    atomicExch(status, (epoch << 8) | 3ull);
}

__device__ inline void mark_epoch(unsigned long long* status, unsigned long long epoch) {
    if (blockIdx.x == 0 && threadIdx.x == 0) status[1] = epoch;
}

}  // namespace iso
