// e-means steps that follow a mini-batch's assignment and segment sums
// (daily.steinslab.io "e-means" article: the moving-average update of each
// cluster's sum and count in "Breaking 70 Years of Full-Batch Inertia", the
// resurrection of dead clusters by proportional splitting in "Proportional
// Splitting Resurrects Thousands of Dead Centers", and the final move to
// the last epoch's plain mean).  The assignment and the batch's segment
// sums are the Lloyd kernels; the state here is float64 (sum S [K][d],
// count N [K]) and the centroids float32.
#include "common.h"

namespace km {

// S = (1 - a) S + a s, N = (1 - a) N + a n, c = S / N where N > 0.  With
// `final` the batch's sums and counts are also added to the last-epoch
// totals F, G.  One thread per (cluster, coordinate); the count by the
// thread of coordinate 0.
__global__ __launch_bounds__(256) void k_ema(double* __restrict__ S, double* __restrict__ Nc,
                                             const float* __restrict__ s, const int32_t* __restrict__ n,
                                             int64_t K, int d, double a, float* __restrict__ C,
                                             double* __restrict__ F, double* __restrict__ G) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= K * d) return;
    const int64_t j = q / d;
    const double nj = (double)n[j];
    const double Nn = (1.0 - a) * Nc[j] + a * nj;  // every thread of cluster j forms the same value
    const double Sn = (1.0 - a) * S[q] + a * (double)s[q];
    S[q] = Sn;
    if (Nn > 0.0) C[q] = (float)(Sn / Nn);
    if (F) {
        F[q] += (double)s[q];
        if (q % d == 0) G[j] += nj;
    }
}

// The new counts, in a launch of their own: every coordinate thread of
// k_ema reads the old count of its cluster.
__global__ __launch_bounds__(256) void k_ema_counts(double* __restrict__ Nc, const int32_t* __restrict__ n,
                                                    int64_t K, double a) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j < K) Nc[j] = (1.0 - a) * Nc[j] + a * (double)n[j];
}

hipError_t launch_emeans_ema(double* S, double* Nc, const float* s, const int32_t* n, int64_t K, int d, double a,
                             float* C, double* F, double* G, hipStream_t st) {
    const int64_t total = K * d;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(k_ema, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, S, Nc, s, n, K, d, a, C, F,
                       G);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_ema_counts, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st, Nc, n, K, a);
    return hipGetLastError();
}

// Dead clusters (N_j < dead_below after the batch's update, decided before
// any split of the batch) are handled as if one after another in ascending
// order, each with its uniform u_j: the donor k is the first cluster whose
// prefix of N (after the batch's update, before any split) exceeds
// u_j * sum(N); k == j is skipped, and so is a donor whose N is zero when
// its turn comes.  The donor's S and N halve, the dead cluster gets the
// same, and the centroids become c_k (1 + eps sgn) and c_k (1 - eps sgn),
// sgn = +1 on even and -1 on odd coordinates (S rescaled to match).
//
// Since the prefix is taken before any split, every donor can be found at
// once.  Split j touches only rows j and k_j, so splits run in rounds: in a
// round, a split goes ahead when it is the lowest pending split touching
// each of its two rows; splits of one round touch disjoint rows, and every
// lower split that shares a row with it has run in an earlier round, which
// gives the ascending order's result.  One block; P [K+1] and donor [K]
// are scratch in global memory (donor[j] is only ever touched by the thread
// of j), the lowest pending split of every row is kept in LDS.
constexpr int kSplitThreads = 1024;
constexpr int kSplitWaves = kSplitThreads / 64;

__global__ __launch_bounds__(kSplitThreads) void k_split(double* __restrict__ S, double* __restrict__ Nc,
                                                         float* __restrict__ C, int64_t K, int d,
                                                         double dead_below, double eps,
                                                         const float* __restrict__ u, double* __restrict__ P,
                                                         int32_t* __restrict__ donor) {
    extern __shared__ int owner[];  // [K]
    __shared__ double s_part[kSplitWaves];
    __shared__ int s_wcnt[kSplitWaves];
    __shared__ int s_list[kSplitThreads];
    __shared__ int s_donor[kSplitThreads];
    __shared__ int s_n;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // exclusive prefix of N: thread t owns a contiguous range
    const int64_t per = (K + kSplitThreads - 1) / kSplitThreads;
    const int64_t j0 = tid * per < K ? tid * per : K, j1 = j0 + per < K ? j0 + per : K;
    double sum = 0.0;
    for (int64_t j = j0; j < j1; ++j) sum += Nc[j];
    double incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
    }
    if (lane == 63) s_part[wave] = incl;
    __syncthreads();
    double run = incl - sum;
    for (int v = 0; v < wave; ++v) run += s_part[v];
    for (int64_t j = j0; j < j1; ++j) {
        P[j] = run;
        run += Nc[j];
    }
    if (tid == kSplitThreads - 1) P[K] = run;  // the last thread's range ends at K
    __syncthreads();
    const double total = P[K];
    // donors of the dead clusters (-1: nothing to do)
    int pending = 0;
    for (int64_t j = tid; j < K; j += kSplitThreads) {
        int dj = -1;
        if (Nc[j] < dead_below) {
            const double target = (double)u[j] * total;
            int64_t lo = 0, len = K;  // first k with P[k + 1] > target (the last cluster if none)
            while (len > 0) {
                const int64_t h = len >> 1;
                if (!(P[lo + h + 1] > target)) {
                    lo += h + 1;
                    len -= h + 1;
                } else {
                    len = h;
                }
            }
            const int64_t k = lo < K ? lo : K - 1;
            dj = k == j ? -1 : (int)k;
        }
        donor[j] = dj;
        pending |= dj >= 0;
    }
    while (__syncthreads_or(pending)) {
        for (int64_t j = tid; j < K; j += kSplitThreads) owner[j] = 0x7fffffff;
        __syncthreads();
        for (int64_t j = tid; j < K; j += kSplitThreads) {
            const int k = donor[j];
            if (k >= 0) {
                atomicMin(&owner[j], (int)j);
                atomicMin(&owner[k], (int)j);
            }
        }
        __syncthreads();
        pending = 0;
        for (int64_t base = 0; base < K; base += kSplitThreads) {
            const int64_t j = base + tid;
            const int k = j < K ? donor[j] : -1;
            const bool ready = k >= 0 && owner[j] == (int)j && owner[k] == (int)j;
            pending |= k >= 0 && !ready;
            // the window's ready splits, listed in LDS
            const unsigned long long mask = __ballot(ready);
            if (lane == 0) s_wcnt[wave] = __popcll(mask);
            __syncthreads();
            if (ready) {
                int r = __popcll(mask & ((1ull << lane) - 1ull));
                for (int v = 0; v < wave; ++v) r += s_wcnt[v];
                s_list[r] = (int)j;
                s_donor[r] = k;
                donor[j] = -1;
            }
            if (tid == 0) {
                int c = 0;
                for (int v = 0; v < kSplitWaves; ++v) c += s_wcnt[v];
                s_n = c;
            }
            __syncthreads();
            const int n = s_n;
            if (n == 0) continue;  // uniform: s_n is the same for every thread
            for (int q = tid; q < n * d; q += kSplitThreads) {
                const int r = q / d, c = q - r * d;
                const int64_t jd = s_list[r], kd = s_donor[r];
                const double nkc = Nc[kd];
                if (!(nkc > 0.0)) continue;  // an empty donor: nothing moves
                const double nk = nkc * 0.5;
                const double ck = S[kd * d + c] * 0.5 / nk;
                const double sg = (c % 2 == 0) ? 1.0 : -1.0;
                const float cj = (float)(ck * (1.0 + eps * sg));
                const float ckn = (float)(ck * (1.0 - eps * sg));
                C[jd * d + c] = cj;
                C[kd * d + c] = ckn;
                S[jd * d + c] = (double)cj * nk;
                S[kd * d + c] = (double)ckn * nk;
            }
            __syncthreads();  // every coordinate read the donor's old N before it changes
            if (tid < n) {
                const int64_t jd = s_list[tid], kd = s_donor[tid];
                const double nkc = Nc[kd];
                if (nkc > 0.0) {
                    Nc[kd] = nkc * 0.5;
                    Nc[jd] = nkc * 0.5;
                }
            }
            __syncthreads();
        }
    }
}

bool emeans_split_supports(int64_t K) { return K >= 1 && K <= kEmeansMaxK; }

hipError_t launch_emeans_split(double* S, double* Nc, float* C, int64_t K, int d, double dead_below, double eps,
                               const float* u, double* P, int32_t* donor, hipStream_t st) {
    if (!emeans_split_supports(K)) return hipErrorInvalidValue;
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void*)k_split, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)(kEmeansMaxK * sizeof(int)));
        if (e != hipSuccess) return e;
        attr = true;
    }
    hipLaunchKernelGGL(k_split, dim3(1), dim3(kSplitThreads), (size_t)K * sizeof(int), st, S, Nc, C, K, d,
                       dead_below, eps, u, P, donor);
    return hipGetLastError();
}

// After the last epoch: c = F / G where G > 0; counts out = G.
__global__ __launch_bounds__(256) void k_final_mean(const double* __restrict__ F, const double* __restrict__ G,
                                                    int64_t K, int d, float* __restrict__ C,
                                                    int32_t* __restrict__ counts) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= K * d) return;
    const int64_t j = q / d;
    if (G[j] > 0.0) C[q] = (float)(F[q] / G[j]);
    if (counts && q % d == 0) counts[j] = (int32_t)G[j];
}

hipError_t launch_emeans_final(const double* F, const double* G, int64_t K, int d, float* C, int32_t* counts,
                               hipStream_t st) {
    const int64_t total = K * d;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(k_final_mean, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, F, G, K, d, C,
                       counts);
    return hipGetLastError();
}

}  // namespace km
