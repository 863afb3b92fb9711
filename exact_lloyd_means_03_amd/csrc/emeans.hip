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
// F and G (the last epoch) the batch's sums and counts are also added to the
// last-epoch totals.  One wave per cluster, lanes over coordinates.  The
// batch's sums and count are cleared once read, ready for the next batch.
// With obj_out, the wave of cluster 0 also sums the batch assignment's
// nobj objective partials into *obj_out (lane-strided sums, then a fixed
// shuffle tree), which saves a launch per step.
__global__ __launch_bounds__(256) void k_ema(double* __restrict__ S, double* __restrict__ Nc,
                                             float* __restrict__ s, int32_t* __restrict__ n, int64_t K, int d,
                                             double a, float* __restrict__ C, double* __restrict__ F,
                                             double* __restrict__ G, const double* __restrict__ obj_part,
                                             int64_t nobj, double* __restrict__ obj_out) {
    const int lane = threadIdx.x & 63;
    const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (j >= K) return;
    if (j == 0 && obj_out) {
        double acc = 0.0;
        for (int64_t i = lane; i < nobj; i += 64) acc += obj_part[i];
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
        if (lane == 0) *obj_out = acc;
    }
    const int32_t nj = n[j];
    const double Nn = (1.0 - a) * Nc[j] + a * (double)nj;
    for (int c = lane; c < d; c += 64) {
        const int64_t q = j * d + c;
        const float sq = s[q];
        const double Sn = (1.0 - a) * S[q] + a * (double)sq;
        S[q] = Sn;
        if (Nn > 0.0) C[q] = (float)(Sn / Nn);
        if (F) F[q] += (double)sq;
        s[q] = 0.f;
    }
    if (lane == 0) {  // every lane has read n[j] and Nc[j] above
        Nc[j] = Nn;
        if (G) G[j] += (double)nj;
        n[j] = 0;
    }
}

hipError_t launch_emeans_ema(double* S, double* Nc, float* s, int32_t* n, int64_t K, int d, double a, float* C,
                             double* F, double* G, const double* obj_part, int64_t nobj, double* obj_out,
                             hipStream_t st) {
    if (K == 0) return hipSuccess;
    hipLaunchKernelGGL(k_ema, dim3((unsigned)((K + 3) / 4)), dim3(256), 0, st, S, Nc, s, n, K, d, a, C, F, G,
                       obj_part, nobj, obj_out);
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
// ranges' start prefixes in LDS, then the prefix within the range.  Split j touches only rows j and k_j, so the
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
constexpr int kSplitU = 8;  // coordinates per thread in flight when splitting
constexpr int kSplitL = 8;  // counts per thread in flight when scanning a range

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
    __shared__ double s_start[kSplitThreads + 1];
    __shared__ int s_wcnt[kSplitWaves];
    __shared__ int s_lj[kSplitThreads], s_lk[kSplitThreads];
    __shared__ double s_nk[kSplitThreads];
    __shared__ int s_n;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = (int)((K + kSplitThreads - 1) / kSplitThreads);
    const int64_t j0 = (int64_t)tid * per < K ? (int64_t)tid * per : K;
    const int64_t j1 = j0 + per < K ? j0 + per : K;
    // every thread loads `per` counts (per is the same for all, so the loads
    // are not predicated and issue together); past K the index is clamped and
    // the value ignored
    static_assert(kSplitPer <= 32 && kSplitPer % kSplitL == 0, "one bit per cluster of a range");
    double sum = 0.0;
    uint32_t deadm = 0;  // bit i: cluster j0 + i is dead
    for (int i0 = 0; i0 < per; i0 += kSplitL) {
        double v[kSplitL];
#pragma unroll
        for (int i = 0; i < kSplitL; ++i) v[i] = Nc[j0 + i0 + i < K ? j0 + i0 + i : K - 1];
#pragma unroll
        for (int i = 0; i < kSplitL; ++i) {
            if (i0 + i < per && j0 + i0 + i < j1) {
                sum += v[i];
                deadm |= (uint32_t)(v[i] < dead_below) << (i0 + i);
            }
        }
    }
    const int ndead = __popc(deadm);
    double total;
    const double start = block_exclusive_scan(sum, s_dpart, &total);
    __syncthreads();  // s_dpart is reused below
    int ndead_all;
    int pos = block_exclusive_scan(ndead, s_ipart, &ndead_all);
    if (ndead_all == 0) return;  // uniform: the same total in every thread
    while (deadm) {  // ascending
        const int i = __ffs(deadm) - 1;
        deadm &= deadm - 1;
        list_j[pos++] = (int)(j0 + i);
    }
    s_start[tid] = start;
    if (tid == 0) s_start[kSplitThreads] = total;
    __syncthreads();
    // donors (list_k = -1: nothing to do)
    int pending = 0;
    for (int i = tid; i < ndead_all; i += kSplitThreads) {
        const int j = list_j[i];
        const double target = (double)u[j] * total;
        // first range whose end (the next range's start) exceeds the target
        int lo = 0, len = kSplitThreads;
        while (len > 0) {
            const int h = len >> 1;
            if (!(s_start[lo + h + 1] > target)) {
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
            bool found = false;
            k = a1 - 1;
            for (int q0 = 0; q0 < per && !found; q0 += kSplitL) {
                double nv[kSplitL];  // kSplitL counts of the range at a time (clamped past K)
#pragma unroll
                for (int q = 0; q < kSplitL; ++q) nv[q] = Nc[a0 + q0 + q < K ? a0 + q0 + q : K - 1];
#pragma unroll
                for (int q = 0; q < kSplitL; ++q) {
                    if (q0 + q < per && a0 + q0 + q < a1 && !found) {
                        r += nv[q];
                        if (r > target) {
                            k = a0 + q0 + q;
                            found = true;
                        }
                    }
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
                s_nk[r] = Nc[k];  // the donor's count before this split
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
            // (split, coordinate) pairs, kSplitU per thread at a time: the
            // donor sums of a batch are loaded before any store
            for (int q0 = tid; q0 < n * d; q0 += kSplitU * kSplitThreads) {
                double sk[kSplitU];
#pragma unroll
                for (int uu = 0; uu < kSplitU; ++uu) {
                    const int q = q0 + uu * kSplitThreads;
                    sk[uu] = 0.0;
                    if (q < n * d) {
                        const int r = q / d, c = q - r * d;
                        sk[uu] = S[(int64_t)s_lk[r] * d + c];
                    }
                }
#pragma unroll
                for (int uu = 0; uu < kSplitU; ++uu) {
                    const int q = q0 + uu * kSplitThreads;
                    if (q >= n * d) break;
                    const int r = q / d, c = q - r * d;
                    const int64_t jd = s_lj[r], kd = s_lk[r];
                    const double nkc = s_nk[r];
                    if (!(nkc > 0.0)) continue;  // an empty donor: nothing moves
                    const double nk = nkc * 0.5;
                    const double ck = sk[uu] * 0.5 / nk;
                    const double sg = (c % 2 == 0) ? 1.0 : -1.0;
                    const float cj = (float)(ck * (1.0 + eps * sg));
                    const float ckn = (float)(ck * (1.0 - eps * sg));
                    C[jd * d + c] = cj;
                    C[kd * d + c] = ckn;
                    S[jd * d + c] = (double)cj * nk;
                    S[kd * d + c] = (double)ckn * nk;
                }
            }
            if (tid < n) {
                const int64_t jd = s_lj[tid], kd = s_lk[tid];
                const double nkc = s_nk[tid];
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
    // set on every call: the attribute belongs to the current device
    hipError_t e = hipFuncSetAttribute((const void*)k_split, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)(kEmeansMaxK * sizeof(int)));
    if (e != hipSuccess) return e;
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
