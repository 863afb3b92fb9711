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
// One block.  Thread t owns the clusters [t*per, t*per + per): it sums
// their N and counts its dead ones, and a block scan gives every range its
// exclusive prefix of N (kept in LDS) and the position of its dead clusters
// in a list that comes out in ascending order.  Since the prefix is taken
// before any split, every donor is found at once: a binary search over the
// ranges' end prefixes in LDS, then the prefix within the range, summed in
// the same order as the scan.  Split j touches only rows j and k_j, so the
// splits run in rounds: in a round, a split goes ahead when it is the lowest
// pending split touching each of its two rows; splits of one round touch
// disjoint rows, and every lower split that shares a row with it has run in
// an earlier round, which gives the ascending order's result.  The list of
// (j, k_j) is scratch in global memory, each entry only ever touched by the
// thread i % 1024 of its position i; the lowest pending split of every row
// is kept in LDS.
constexpr int kSplitThreads = 1024;
constexpr int kSplitWaves = kSplitThreads / 64;
constexpr int kSplitPer = (int)(kEmeansMaxK / kSplitThreads);  // clusters per thread at most

template <typename V>
__device__ __forceinline__ V block_exclusive_scan(V v, V* s_part, V* total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    V incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const V t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
    }
    if (lane == 63) s_part[wave] = incl;
    __syncthreads();
    V run = incl - v;
    V all = 0;
    for (int w = 0; w < kSplitWaves; ++w) {
        if (w < wave) run += s_part[w];
        all += s_part[w];
    }
    *total = all;
    return run;
}

__global__ __launch_bounds__(kSplitThreads) void k_split(double* __restrict__ S, double* __restrict__ Nc,
                                                         float* __restrict__ C, int64_t K, int d,
                                                         double dead_below, double eps,
                                                         const float* __restrict__ u,
                                                         int32_t* __restrict__ list_j, int32_t* __restrict__ list_k) {
    extern __shared__ int owner[];  // [K]
    __shared__ double s_dpart[kSplitWaves];
    __shared__ int s_ipart[kSplitWaves];
    __shared__ double s_start[kSplitThreads], s_end[kSplitThreads];
    __shared__ int s_wcnt[kSplitWaves];
    __shared__ int s_lj[kSplitThreads], s_lk[kSplitThreads];
    __shared__ int s_n;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = (int)((K + kSplitThreads - 1) / kSplitThreads);
    const int64_t j0 = (int64_t)tid * per < K ? (int64_t)tid * per : K;
    const int64_t j1 = j0 + per < K ? j0 + per : K;
    double v[kSplitPer];
    double sum = 0.0;
    int ndead = 0;
#pragma unroll
    for (int i = 0; i < kSplitPer; ++i) {
        v[i] = (i < per && j0 + i < j1) ? Nc[j0 + i] : 0.0;
    }
#pragma unroll
    for (int i = 0; i < kSplitPer; ++i) {
        if (i < per && j0 + i < j1) {
            sum += v[i];
            ndead += v[i] < dead_below;
        }
    }
    double total;
    const double start = block_exclusive_scan(sum, s_dpart, &total);
    __syncthreads();  // s_dpart is reused below
    int ndead_all;
    int pos = block_exclusive_scan(ndead, s_ipart, &ndead_all);
    if (ndead_all == 0) return;  // uniform: the same total in every thread
    // range t's prefix after its last cluster, formed as the searches below form it
    double run = start;
#pragma unroll
    for (int i = 0; i < kSplitPer; ++i) {
        if (i < per && j0 + i < j1) {
            run += v[i];
            if (v[i] < dead_below) list_j[pos++] = (int)(j0 + i);
        }
    }
    s_start[tid] = start;
    s_end[tid] = run;
    __syncthreads();
    // donors (list_k = -1: nothing to do)
    int pending = 0;
    for (int i = tid; i < ndead_all; i += kSplitThreads) {
        const int j = list_j[i];
        const double target = (double)u[j] * total;
        // first range whose end prefix exceeds the target
        int lo = 0, len = kSplitThreads;
        while (len > 0) {
            const int h = len >> 1;
            if (!(s_end[lo + h] > target)) {
                lo += h + 1;
                len -= h + 1;
            } else {
                len = h;
            }
        }
        int64_t k = K - 1;  // the last cluster if no prefix exceeds the target
        if (lo < kSplitThreads) {
            const int64_t a0 = (int64_t)lo * per, a1 = a0 + per < K ? a0 + per : K;
            double r = s_start[lo];
            k = a1 - 1;
            for (int64_t q = a0; q < a1; ++q) {
                r += Nc[q];
                if (r > target) {
                    k = q;
                    break;
                }
            }
        }
        const int dj = k == j ? -1 : (int)k;
        list_k[i] = dj;
        pending |= dj >= 0;
    }
    while (__syncthreads_or(pending)) {
        for (int i = tid; i < ndead_all; i += kSplitThreads) {
            const int k = list_k[i];
            if (k >= 0) {
                owner[list_j[i]] = 0x7fffffff;
                owner[k] = 0x7fffffff;
            }
        }
        __syncthreads();
        for (int i = tid; i < ndead_all; i += kSplitThreads) {
            const int k = list_k[i];
            if (k >= 0) {
                const int j = list_j[i];
                atomicMin(&owner[j], j);
                atomicMin(&owner[k], j);
            }
        }
        __syncthreads();
        pending = 0;
        for (int base = 0; base < ndead_all; base += kSplitThreads) {
            const int i = base + tid;
            const int k = i < ndead_all ? list_k[i] : -1;
            const int j = k >= 0 ? list_j[i] : -1;
            const bool ready = k >= 0 && owner[j] == j && owner[k] == j;
            pending |= k >= 0 && !ready;
            // the window's ready splits, listed in LDS
            const unsigned long long mask = __ballot(ready);
            if (lane == 0) s_wcnt[wave] = __popcll(mask);
            __syncthreads();
            if (ready) {
                int r = __popcll(mask & ((1ull << lane) - 1ull));
                for (int w = 0; w < wave; ++w) r += s_wcnt[w];
                s_lj[r] = j;
                s_lk[r] = k;
                list_k[i] = -1;
            }
            if (tid == 0) {
                int c = 0;
                for (int w = 0; w < kSplitWaves; ++w) c += s_wcnt[w];
                s_n = c;
            }
            __syncthreads();
            const int n = s_n;
            if (n == 0) continue;  // uniform: s_n is the same for every thread
            for (int q = tid; q < n * d; q += kSplitThreads) {
                const int r = q / d, c = q - r * d;
                const int64_t jd = s_lj[r], kd = s_lk[r];
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
                const int64_t jd = s_lj[tid], kd = s_lk[tid];
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
                               const float* u, int32_t* list_j, int32_t* list_k, hipStream_t st) {
    if (!emeans_split_supports(K)) return hipErrorInvalidValue;
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void*)k_split, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)(kEmeansMaxK * sizeof(int)));
        if (e != hipSuccess) return e;
        attr = true;
    }
    hipLaunchKernelGGL(k_split, dim3(1), dim3(kSplitThreads), (size_t)K * sizeof(int), st, S, Nc, C, K, d,
                       dead_below, eps, u, list_j, list_k);
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
