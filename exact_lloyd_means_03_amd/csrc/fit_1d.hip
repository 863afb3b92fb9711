// Whole Lloyd fits of scalar rows (d == 1) that fit on chip, every
// iteration in one launch.
//
// The per-row weighted 1D clustering of LLM weight rows (github
// LeanModels/LeanQuant issue #1 "1D k-means", the kmeans_fit diff: K = 16 or
// 8 clusters per row of a few thousand weights, sample weights, a fixed
// number of iterations) is far too small per row for one kernel per step:
// every iteration would re-read the row's points and weights from device
// memory.  Here the row's points and weights stay in registers for all
// iterations and device memory is read once.  Rows of up to 4096 points get
// one wave each (k_fit_1d_wave: no barriers, so the serial part of one row
// overlaps the point work of the other rows on the CU); longer rows, up to
// 8192 points, get one 256-thread block (k_fit_1d_rows).
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
//      and fails from it on; that float, the threshold t_a, is found by a
//      search over the ordered float bit patterns in (v_a, v_{a+1}].  The
//      rank of x is then the number of thresholds <= x.
//   3. Each thread adds w*x and w of its points, in float64, into its own
//      per-rank bins in LDS (adds that return nothing, on addresses no other
//      lane touches), and w * (x - v)^2 into its objective partial.
//   4. The bins are reduced per rank in float64; the new centroid of the
//      smallest index of each value is S / W (float64 divide, then float32),
//      a value with no points keeps its centroid, and so does every centroid
//      that duplicates a smaller index's value.
// After the last iteration the labels and counts of its assignment are
// written.
#include "scalar_rows.h"

namespace km {

constexpr int kFit1DThreads = 256;
constexpr int kFit1DMaxN = 8192;
constexpr int kFit1DWaveMaxN = 64 * 64;  // rows a single wave keeps in registers

bool fit_1d_rows_fits(int64_t N, int64_t K) { return N >= 1 && N <= kFit1DMaxN && K <= kFit1DMaxK; }

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
            const int A = f1_thresholds<T>(s_c, K, lane, s_val, s_idx, s_thr);
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

// One wave per row (rows of up to 64 * PPT points): the same iteration with
// no block barriers, so the serial step of one row (the thresholds) overlaps
// the point work of the other rows on the CU, and about ten rows share a CU.
template <typename T, int PPT>
__global__ __launch_bounds__(64) void k_fit_1d_wave(
    const T* __restrict__ X, const float* __restrict__ w, int N, const float* __restrict__ init, int K,
    int n_iter, float* __restrict__ centroids, int32_t* __restrict__ labels, int32_t* __restrict__ counts,
    double* __restrict__ objective) {
    __shared__ float s_c[kFit1DMaxK];
    __shared__ float s_val[kFit1DMaxK];
    __shared__ int s_idx[kFit1DMaxK];
    __shared__ float s_thr[kFit1DMaxK];
    __shared__ double2 s_bin[kFit1DMaxK][64 + 1];  // per-lane (sum w*x, sum w) per rank (rows padded)
    __shared__ int s_cnt[kFit1DMaxK];
    const int lane = threadIdx.x;
    const int64_t b = blockIdx.x;
    const T* Xb = X + b * (int64_t)N;
    auto wave_sync = [] {
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    };

    float xs[PPT], ws[PPT];
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
        const int i = p * 64 + lane;
        xs[p] = i < N ? f1_load<T>(Xb + i) : 0.f;
        ws[p] = i < N ? (w ? w[b * N + i] : 1.f) : 0.f;  // past the row end: weight 0, no effect
    }
    if (lane < K) s_c[lane] = init[b * K + lane];
    if (lane < kFit1DMaxK) s_cnt[lane] = 0;
    wave_sync();

    int A = 0;
    for (int t = 0; t < n_iter; ++t) {
        A = f1_thresholds<T>(s_c, K, lane, s_val, s_idx, s_thr);
#pragma unroll
        for (int r = 0; r < kFit1DMaxK; ++r) s_bin[r][lane] = make_double2(0.0, 0.0);
        wave_sync();
        // the thresholds are the same in every lane: held in scalar registers,
        // a point's rank is a branch-free count over them
        float tr[kFit1DMaxK - 1];
        f1_scalar_thresholds(s_thr, tr);
        float jpart = 0.f;
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            // the empty asm hides that x and w do not change between
            // iterations, so their float64 forms are not kept live across them
            float xv = xs[p], wv = ws[p];
            asm volatile("" : "+v"(xv), "+v"(wv));
            const int m = f1_rank_cmp(xv, tr);
            const float tv = xv - s_val[m];
            jpart = fmaf(wv, tv * tv, jpart);
            // this lane's own bins, adds that return nothing: no point waits on another
            atomicAdd(&s_bin[m][lane].x, (double)wv * (double)xv);
            atomicAdd(&s_bin[m][lane].y, (double)wv);
            if (p % 16 == 15) __builtin_amdgcn_sched_barrier(0);  // 16 points in flight at most
        }
        double jd = jpart;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) jd += __shfl_xor(jd, o, 64);
        wave_sync();
        // per-rank sums: lane (r, part) adds the bins of rank r of lanes
        // part*16 .. +16; two exchanges combine the four parts
        const int r = lane & (kFit1DMaxK - 1), part = lane >> 4;
        double S = 0.0, W = 0.0;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const double2 v = s_bin[r][part * 16 + q];
            S += v.x;
            W += v.y;
        }
        S += __shfl_xor(S, 16, 64);
        W += __shfl_xor(W, 16, 64);
        S += __shfl_xor(S, 32, 64);
        W += __shfl_xor(W, 32, 64);
        if (lane < A && W > 0.0) s_c[s_idx[lane]] = (float)(S / W);
        if (lane == 0 && objective) objective[b * n_iter + t] = jd;
        wave_sync();
    }
    // labels and counts of the last assignment: s_thr, s_val and s_idx still
    // hold that iteration's values (only s_c has moved on)
    if (n_iter > 0) {
        float tr[kFit1DMaxK - 1];
        f1_scalar_thresholds(s_thr, tr);
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            const int i = p * 64 + lane;
            if (i < N) {
                const int m = f1_rank_cmp(xs[p], tr);
                if (labels) labels[b * N + i] = s_idx[m];
                atomicAdd(&s_cnt[m], 1);
            }
        }
        wave_sync();
    }
    if (lane < K) {
        centroids[b * K + lane] = s_c[lane];
        if (counts && n_iter > 0) {
            int c = 0;  // ranks map to the smallest index of each value; other indices are empty
            for (int q = 0; q < A; ++q)
                if (s_idx[q] == lane) c = s_cnt[q];
            counts[b * K + lane] = c;
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
#define KM_FW(TT, PP)                                                                                 \
    hipLaunchKernelGGL((k_fit_1d_wave<TT, PP>), grid, dim3(64), 0, s, (const TT*)x, w, (int)N, init,    \
                       (int)K, n_iter, centroids, labels, counts, objective)
#define KM_FW_T(TT)                      \
    if (N <= 16 * 64) {                  \
        KM_FW(TT, 16);                   \
    } else if (N <= 32 * 64) {           \
        KM_FW(TT, 32);                   \
    } else {                             \
        KM_FW(TT, 64);                   \
    }
    if (N <= kFit1DWaveMaxN) {
        if (xt == DType::F32) { KM_FW_T(float) }
        else if (xt == DType::F16) { KM_FW_T(_Float16) }
        else { KM_FW_T(bf16_t) }
    } else {
        if (xt == DType::F32) { KM_F1_T(float) }
        else if (xt == DType::F16) { KM_F1_T(_Float16) }
        else { KM_F1_T(bf16_t) }
    }
#undef KM_FW_T
#undef KM_FW
#undef KM_F1_T
#undef KM_F1
    return hipGetLastError();
}

}  // namespace km
