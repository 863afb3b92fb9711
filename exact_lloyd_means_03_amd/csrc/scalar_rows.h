// Device helpers shared by the scalar-point (d == 1) kernels with few
// centroids: the per-row thresholds between adjacent distinct centroid
// values, and the element conversions they use.
//
// For scalars, the nearest centroid of x is one of the two distinct centroid
// values that bracket it, because the float32 distance (x - v)^2 is monotone
// in |x - v|.  Between adjacent distinct values v_a < v_b, "x prefers v_a"
// (smaller float32 distance, or equal distance and smaller index) holds up
// to some float and fails from it on; that float is the threshold t_a, and
// the rank of x among the distinct values is the number of thresholds <= x.
// This is the same decision as comparing the two bracketing candidates point
// by point (github LeanModels/LeanQuant issue #1, per-row 1D clustering;
// smallest index on exact ties).
#pragma once

#include "common.h"

namespace km {

constexpr int kFit1DMaxK = 16;  // centroids per row for the threshold kernels

template <typename T>
__device__ __forceinline__ float f1_round(float v) {
    if constexpr (sizeof(T) == 4) return v;
    else if constexpr (__is_same(T, _Float16)) return (float)(_Float16)v;
    else return bf16_to_f32(f32_to_bf16_rne(v));
}

template <typename T>
__device__ __forceinline__ float f1_load(const T* p) {
    if constexpr (sizeof(T) == 4) return *p;
    else if constexpr (__is_same(T, _Float16)) return (float)*p;
    else return bf16_to_f32(*p);
}

// Order-preserving float <-> uint32 maps (-0 is canonicalized to +0 first).
__device__ __forceinline__ uint32_t f1_ord(float f) {
    const uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f1_unord(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// x prefers (va, ia) over (vb, ib): smaller float32 squared distance, or the
// same distance and the smaller index.
__device__ __forceinline__ bool f1_prefers(float x, float va, int ia, float vb, int ib) {
    const float ta = x - va, tb = vb - x;
    const float da = ta * ta, db = tb * tb;
    return da < db || (da == db && ia < ib);
}

// Steps 1-2 for one row, by one wave: from the centroids in s_c, the distinct
// rounded values in ascending order (s_val), the smallest index holding each
// (s_idx) and the thresholds between neighbours (s_thr, +inf past A - 1).
// Returns A, the number of distinct values (the same in every lane).
template <typename T>
__device__ __forceinline__ int f1_thresholds(const float* s_c, int K, int lane, float* s_val, int* s_idx,
                                             float* s_thr) {
    float u[kFit1DMaxK];  // every centroid, rounded (the same in all lanes)
#pragma unroll
    for (int k = 0; k < kFit1DMaxK; ++k) u[k] = k < K ? f1_round<T>(s_c[k]) : INFINITY;
    const float v = lane < K ? f1_round<T>(s_c[lane]) : INFINITY;
    bool first = lane < K;  // no smaller index holds the same value
#pragma unroll
    for (int k = 0; k < kFit1DMaxK; ++k)
        if (k < lane && u[k] == v) first = false;
    const unsigned long long firsts = __ballot(first);
    int a = 0;  // distinct values below v
#pragma unroll
    for (int k = 0; k < kFit1DMaxK; ++k)
        if (((firsts >> k) & 1ull) && u[k] < v) ++a;
    if (first) {
        s_val[a] = v;
        s_idx[a] = lane;
    }
    const int A = __popcll(firsts);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    if (lane < kFit1DMaxK) {
        float thr = INFINITY;
        if (lane < A - 1) {
            const float va = s_val[lane], vb = s_val[lane + 1];
            const int ia = s_idx[lane], ib = s_idx[lane + 1];
            // invariant: x = unord(lo) prefers va, x = unord(hi) does not
            uint32_t lo = f1_ord(va), hi = f1_ord(vb);
            // the switch is within a few floats of the midpoint: probe
            // there, gallop outwards, then bisect the bracket found
            uint32_t probe = f1_ord(va + 0.5f * (vb - va));
            probe = probe <= lo ? lo + 1 : (probe > hi ? hi : probe);
            if (probe < hi) {
                if (f1_prefers(f1_unord(probe), va, ia, vb, ib)) {
                    lo = probe;
                    for (uint32_t step = 1; step < hi - lo; step <<= 1) {  // lo + step < hi
                        if (f1_prefers(f1_unord(lo + step), va, ia, vb, ib)) {
                            lo += step;
                        } else {
                            hi = lo + step;
                            break;
                        }
                    }
                } else {
                    hi = probe;
                    for (uint32_t step = 1; step < hi - lo; step <<= 1) {  // hi - step > lo
                        if (!f1_prefers(f1_unord(hi - step), va, ia, vb, ib)) {
                            hi -= step;
                        } else {
                            lo = hi - step;
                            break;
                        }
                    }
                }
            }
            while (hi - lo > 1) {
                const uint32_t mid = lo + ((hi - lo) >> 1);
                if (f1_prefers(f1_unord(mid), va, ia, vb, ib)) lo = mid;
                else hi = mid;
            }
            thr = f1_unord(hi);
        }
        s_thr[lane] = thr;
    }
    return A;
}

// Makes the LDS writes of a wave visible to all of its lanes.
__device__ __forceinline__ void f1_wave_sync() {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
}

// The first NT thresholds in scalar registers: they are the same in every
// lane, so each compare against one takes a scalar operand.
template <int NT>
__device__ __forceinline__ void f1_scalar_thresholds(const float* s_thr, float (&tr)[NT]) {
#pragma unroll
    for (int a = 0; a < NT; ++a) tr[a] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(s_thr[a])));
}

// Rank of x among the distinct values: the number of thresholds <= x.  Rows
// with at most NT + 1 distinct values need only the first NT thresholds (the
// rest are +inf).  Two forms with the same result for finite x; the
// assignment kernel uses f1_rank_sub and the fused fit f1_rank_cmp, each the
// faster of the two there on MI355X.
//
// f1_rank_cmp counts compares (a compare and an add with carry per
// threshold; each compare mask costs a short wait before its use).
template <int NT>
__device__ __forceinline__ int f1_rank_cmp(float x, const float (&tr)[NT]) {
    int m = 0;
#pragma unroll
    for (int a = 0; a < NT; ++a) m += (x >= tr[a]) ? 1 : 0;
    return m;
}

// f1_rank_sub counts negative differences instead: x >= t exactly when the
// float32 difference x - t is not negative, since a difference of two
// distinct floats is never zero and x - x is +0 (x is first mapped from -0 to
// +0, so that -0 - (+0) does not give -0).  About 2.5 vector operations per
// threshold and no compare masks.
template <int NT>
__device__ __forceinline__ int f1_rank_sub(float x, const float (&tr)[NT]) {
    const float xc = x + 0.0f;
    int m = NT;
#pragma unroll
    for (int a = 0; a < NT; ++a) m -= (int)(__float_as_uint(xc - tr[a]) >> 31);
    return m;
}

// Four consecutive elements from an address aligned to four elements.
template <typename T>
__device__ __forceinline__ void f1_load4(const T* p, float (&v)[4]) {
    if constexpr (sizeof(T) == 4) {
        const f32x4 q = __builtin_nontemporal_load((const f32x4*)p);
        v[0] = q[0], v[1] = q[1], v[2] = q[2], v[3] = q[3];
    } else {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 q = __builtin_nontemporal_load((const u32x2*)p);
        const uint32_t h[4] = {q[0] & 0xffffu, q[0] >> 16, q[1] & 0xffffu, q[1] >> 16};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (__is_same(T, _Float16)) v[e] = (float)__builtin_bit_cast(_Float16, (uint16_t)h[e]);
            else v[e] = bf16_to_f32((uint16_t)h[e]);
        }
    }
}

}  // namespace km
