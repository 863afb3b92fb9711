// Whole Lloyd fits of scalar rows (d == 1) that fit on chip, one block per
// row, every iteration in one launch.
//
// The per-row weighted 1D clustering of LLM weight rows (github
// LeanModels/LeanQuant issue #1 "1D k-means", the kmeans_fit diff: K = 16 or
// 8 clusters per row of a few thousand weights, sample weights, a fixed
// number of iterations) is far too small per row for one kernel per step:
// every iteration would re-read the row's points and weights from device
// memory.  Here a block keeps its row's points and weights in registers for
// all iterations and reads device memory once.
//
// Iteration t (same result as the assignment and update kernels):
//   1. The row's centroids, rounded to the point dtype, are ordered by
//      (value, index); among equal values only the smallest index can win
//      (exact ties go to the smallest index).  Call the distinct values
//      v_0 < v_1 < ... < v_{A-1}.
//   2. The nearest centroid of x is one of the two distinct values that
//      bracket it, because the float32 distance (x - v)^2 is monotone in
//      |x - v|.  Between v_a and v_{a+1}, "x prefers v_a" (smaller float32
//      distance, or equal distance and smaller index) holds up to some float
//      and fails from it on; that float, the threshold t_a, is found by
//      bisection over the ordered float bit patterns in (v_a, v_{a+1}].  The
//      rank of x is then the number of thresholds <= x (a branch-free
//      binary search over the A-1 thresholds in LDS).
//   3. Each thread adds w*x and w of its points, in float64, into its own
//      per-rank bins in LDS (no atomics), and w * (x - v)^2 into its
//      objective partial.
//   4. The bins are reduced per rank in float64; the new centroid of the
//      smallest index of each value is S / W (float64 divide, then float32),
//      a value with no points keeps its centroid, and so does every centroid
//      that duplicates a smaller index's value.
// The last iteration also writes the labels and the counts.
#include "common.h"

namespace km {

constexpr int kFit1DThreads = 256;
constexpr int kFit1DMaxK = 16;
constexpr int kFit1DMaxN = 8192;

bool fit_1d_rows_fits(int64_t N, int64_t K) { return N >= 1 && N <= kFit1DMaxN && K <= kFit1DMaxK; }

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

// PPT: points per thread (N <= PPT * kFit1DThreads).
template <typename T, int PPT>
__global__ __launch_bounds__(kFit1DThreads) void k_fit_1d_rows(
    const T* __restrict__ X, const float* __restrict__ w, int N, const float* __restrict__ init, int K,
    int n_iter, float* __restrict__ centroids, int32_t* __restrict__ labels, int32_t* __restrict__ counts,
    double* __restrict__ objective) {
    constexpr int NT = kFit1DThreads;
    __shared__ float s_c[kFit1DMaxK];       // current centroids (float32 state)
    __shared__ float s_val[kFit1DMaxK];     // distinct rounded values, ascending
    __shared__ int s_idx[kFit1DMaxK];       // smallest index holding each value
    __shared__ float s_thr[kFit1DMaxK];     // thresholds, +inf past A - 1
    __shared__ double2 s_bin[kFit1DMaxK][NT + 1];  // per-thread (sum w*x, sum w) per rank (rows padded)
    __shared__ double s_red[NT / 64][2 * kFit1DMaxK + 1];
    __shared__ int s_cnt[kFit1DMaxK];
    __shared__ int s_A;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t b = blockIdx.x;
    const T* Xb = X + b * (int64_t)N;

    float xs[PPT], ws[PPT];
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
        const int i = p * NT + tid;
        xs[p] = i < N ? f1_load<T>(Xb + i) : 0.f;
        ws[p] = i < N ? (w ? w[b * N + i] : 1.f) : 0.f;
    }
    if (tid < K) s_c[tid] = init[b * K + tid];
    if (tid < kFit1DMaxK) s_cnt[tid] = 0;
    __syncthreads();

    for (int t = 0; t < n_iter; ++t) {
        const bool last = t == n_iter - 1;
        // ---- 1-2: distinct sorted values and thresholds (one wave) ----
        if (wave == 0) {
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
                    uint32_t u = f1_ord(va + 0.5f * (vb - va));
                    u = u <= lo ? lo + 1 : (u > hi ? hi : u);
                    if (u < hi) {
                        if (f1_prefers(f1_unord(u), va, ia, vb, ib)) {
                            lo = u;
                            for (uint32_t step = 1; step < hi - lo; step <<= 1) {  // lo + step < hi
                                if (f1_prefers(f1_unord(lo + step), va, ia, vb, ib)) {
                                    lo += step;
                                } else {
                                    hi = lo + step;
                                    break;
                                }
                            }
                        } else {
                            hi = u;
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
            if (lane == 0) s_A = A;
        }
        // ---- clear this thread's bins ----
#pragma unroll
        for (int r = 0; r < kFit1DMaxK; ++r) s_bin[r][tid] = make_double2(0.0, 0.0);
        __syncthreads();

        // ---- 2-3: rank of every point, bins, objective.  The ranks of all
        // points are found first (independent searches that overlap); points
        // past the row end have weight 0 and change nothing. ----
        int ms[PPT];
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            int m = 0;
#pragma unroll
            for (int step = kFit1DMaxK / 2; step >= 1; step >>= 1)
                if (xs[p] >= s_thr[m + step - 1]) m += step;
            ms[p] = m;
        }
        float jpart = 0.f;
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            const float tv = xs[p] - s_val[ms[p]];
            jpart = fmaf(ws[p], tv * tv, jpart);
            // this thread's own bins: no other lane touches them, and the adds
            // return nothing, so no point waits on another
            atomicAdd(&s_bin[ms[p]][tid].x, (double)ws[p] * (double)xs[p]);
            atomicAdd(&s_bin[ms[p]][tid].y, (double)ws[p]);
        }
        if (last) {
#pragma unroll
            for (int p = 0; p < PPT; ++p) {
                const int i = p * NT + tid;
                if (i < N) {
                    if (labels) labels[b * N + i] = s_idx[ms[p]];
                    atomicAdd(&s_cnt[ms[p]], 1);
                }
            }
        }
        double jd = jpart;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) jd += __shfl_xor(jd, o, 64);
        if (lane == 0) s_red[wave][2 * kFit1DMaxK] = jd;
        __syncthreads();

        // ---- 4: per-rank sums.  Lane (r, part) of wave w adds the bins of
        // rank r of threads w*64 + part*16 .. +16 in float64; two exchanges
        // combine the four parts. ----
        {
            const int r = lane & (kFit1DMaxK - 1), part = lane >> 4;
            double S = 0.0, W = 0.0;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const double2 v = s_bin[r][wave * 64 + part * 16 + q];
                S += v.x;
                W += v.y;
            }
            S += __shfl_xor(S, 16, 64);
            W += __shfl_xor(W, 16, 64);
            S += __shfl_xor(S, 32, 64);
            W += __shfl_xor(W, 32, 64);
            if (part == 0) {
                s_red[wave][2 * r] = S;
                s_red[wave][2 * r + 1] = W;
            }
        }
        __syncthreads();
        const int A = s_A;
        if (tid < A) {
            double S = 0.0, W = 0.0;
#pragma unroll
            for (int q = 0; q < NT / 64; ++q) {
                S += s_red[q][2 * tid];
                W += s_red[q][2 * tid + 1];
            }
            if (W > 0.0) s_c[s_idx[tid]] = (float)(S / W);
        }
        if (tid == 0 && objective) {
            double J = 0.0;
#pragma unroll
            for (int q = 0; q < NT / 64; ++q) J += s_red[q][2 * kFit1DMaxK];
            objective[b * n_iter + t] = J;
        }
        __syncthreads();
    }
    if (tid < K) {
        centroids[b * K + tid] = s_c[tid];
        if (counts && n_iter > 0) {
            // ranks map to the smallest index of each value; other indices are empty
            int c = 0;
            const int A = s_A;
            for (int r = 0; r < A; ++r)
                if (s_idx[r] == tid) c = s_cnt[r];
            counts[b * K + tid] = c;
        }
    }
}

hipError_t launch_fit_1d_rows(DType xt, const void* x, const float* w, int64_t B, int64_t N, const float* init,
                              int64_t K, int n_iter, float* centroids, int32_t* labels, int32_t* counts,
                              double* objective, hipStream_t s) {
    if (B == 0) return hipSuccess;
    if (!fit_1d_rows_fits(N, K)) return hipErrorInvalidValue;
    dim3 grid((unsigned)B);
#define KM_F1(TT, PP)                                                                                   \
    hipLaunchKernelGGL((k_fit_1d_rows<TT, PP>), grid, dim3(kFit1DThreads), 0, s, (const TT*)x, w, (int)N, \
                       init, (int)K, n_iter, centroids, labels, counts, objective)
#define KM_F1_T(TT)                      \
    if (N <= 16 * kFit1DThreads) {       \
        KM_F1(TT, 16);                   \
    } else {                             \
        KM_F1(TT, 32);                   \
    }
    if (xt == DType::F32) { KM_F1_T(float) }
    else if (xt == DType::F16) { KM_F1_T(_Float16) }
    else { KM_F1_T(bf16_t) }
#undef KM_F1_T
#undef KM_F1
    return hipGetLastError();
}

}  // namespace km
