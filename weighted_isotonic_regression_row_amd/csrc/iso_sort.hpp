// Sorting network of the soft-rank and calibration kernels (gfx950).
//
// A workgroup sorts P entries (a power of two, P / E threads, thread t holding
// positions tE .. tE+E-1) into the order of `before`: a bitonic network with
// every comparison in the same direction.  Phase k (k = 2, 4, ..., P) first
// compares position p with its mirror p ^ (k-1) inside its block of k, then p
// with p ^ j for j = k/4, ..., 1; of each pair the lower position keeps the
// entry that comes first.  Distances below E stay in the thread, partners up
// to 64E away are lanes of the same wave (DPP where a row-of-16 pattern reaches
// them, else the LDS crossbar; a mirror partner holds its entries in reverse),
// farther ones go through LDS.
#pragma once

#include "iso_device.hpp"

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

// The whole network over the workgroup's P entries (K, I: LDS for P entries,
// used only when P > 64E).
template <typename T, int E>
__device__ __forceinline__ void sort_entries(Ent (&v)[E], int t, int P, uint64_t* K, uint32_t* I) {
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
}

}  // namespace
}  // namespace iso
