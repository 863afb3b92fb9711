// Globally optimal weighted 1D k-means of every row (github LeanModels/
// LeanQuant issue #1 "1D k-means": for scalar weights the globally optimal
// centroids can be found, and the diff replaces Lloyd with such a weighted
// 1D clustering that returns the centroids).
//
// Some optimal partition of scalars is a set of runs of consecutive values in
// ascending order, so the optimum is the least-cost cut of the sorted row into
// K non-empty runs.  With prefix sums P0, P1, P2 of w, w*x and w*x^2 over the
// sorted row, the cost of the run of sorted points i .. j-1 is
//     SSE(i, j) = (P2[j] - P2[i]) - (P1[j] - P1[i])^2 / (P0[j] - P0[i]),
// and the least cost of the first j points in k runs is
//     D_k[j] = min over k-1 <= i < j of D_{k-1}[i] + SSE(i, j),   D_1[j] = SSE(0, j).
// In terms of E_k[j] = D_k[j] - P2[j] this is
//     E_k[j] = min over i of E_{k-1}[i] - (P1[j] - P1[i])^2 / (P0[j] - P0[i]),
// E_1[j] = -P1[j]^2 / P0[j], and J* = E_K[N] + P2[N]: P2 is needed only
// through its total.  The least-cost i (the cut) never decreases as j grows
// (the run costs satisfy the quadrangle inequality), so each layer is solved
// by divide and conquer: a j scans only the cuts between those of its two
// nearest j's already solved.  A layer costs O(N log N) evaluations instead
// of O(N^2).
//
// gfx950 layout (ours): one 1024-thread block per row (rows of up to 4096
// points).  LDS holds P0, P1 and E_{k-1} in float64 (the sort keys before
// the dynamic program), the cuts of the current layer, and per-level scratch
// (about 147 KB at N = 4096).  The sort is a bitonic sort of (value, index)
// keys in LDS.  The j's of a layer form a complete binary tree in order:
// level l holds j - k = (2s+1) 2^(L-1-l) - 1, whose nearest solved j's are
// 2^(L-1-l) to either side.  The cut ranges of one level can be very uneven
// (where the optimal cut jumps, one j keeps a long range at every level), so
// a level is balanced by candidates, not by j's: the range lengths are
// prefix-summed, each thread takes an equal slice of all (j, cut) candidates
// and the per-j minimum is taken with 64-bit LDS atomic minimums on
// (cost, cut) keys.  E_k goes to device memory and comes back into LDS after
// the layer; the cuts of every layer stay in device memory (uint16) for the
// backtrack.
//
// A key is the order-preserving 64-bit image of a cost with its low 12 bits
// replaced by the cut: the smaller cost wins, and costs that agree to about
// 2^-40 of their magnitude count as tied, the smaller cut winning.  The
// winner's E is then computed again with an exact divide.
#include "scalar_rows.h"

namespace km {

constexpr int kOpt1DThreads = 1024;
constexpr int kOpt1DWaves = kOpt1DThreads / 64;

bool optimal_1d_supports(int64_t N, int64_t K) {
    return N >= 1 && N <= kOpt1DMaxN && K >= 1 && K <= N && K <= kOpt1DMaxK;
}

static int pow2_at_least(int n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

// Dynamic LDS: P0, P1 [N+1] and E [max(NP, N+1)] (the sort keys before the
// dynamic program) in float64, the per-level minimum keys [NP/2] uint64, the
// cuts [N+1] and the per-level candidate offsets [NP/2 + 1] uint16 (NP: N
// rounded up to a power of two; a level has at most NP/2 nodes).
static size_t opt1d_lds_bytes(int N) {
    const size_t nd = (size_t)N + 1, np = (size_t)pow2_at_least(N);
    const size_t ne = np > nd ? np : nd, nb = np / 2 > 0 ? np / 2 : 1;
    return 2 * nd * sizeof(double) + ne * sizeof(double) + 2 * nb * sizeof(uint64_t) + nd * sizeof(uint16_t) +
           (nb + 1) * sizeof(uint16_t);
}

// Workspace per row: E_k [N+1] double, cuts [K][N+1] uint16, sorted-position
// -> point index [N] int32.
void optimal_1d_workspace(int64_t B, int64_t N, int64_t K, size_t* d_off, size_t* cut_off, size_t* perm_off,
                          size_t* total) {
    auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
    size_t off = 0;
    *d_off = off;
    off += up((size_t)B * (N + 1) * sizeof(double));
    *cut_off = off;
    off += up((size_t)B * K * (N + 1) * sizeof(uint16_t));
    *perm_off = off;
    off += up((size_t)B * N * sizeof(int32_t));
    *total = off;
}

template <typename T>
__global__ __launch_bounds__(kOpt1DThreads) void k_optimal_1d(
    const T* __restrict__ X, const float* __restrict__ w, int N, int K, float* __restrict__ centroids,
    int32_t* __restrict__ labels, int32_t* __restrict__ counts, double* __restrict__ objective,
    double* __restrict__ Eg_all, uint16_t* __restrict__ cut_all, int32_t* __restrict__ perm_all) {
    extern __shared__ double s_dyn[];
    __shared__ int s_bound[kOpt1DMaxK + 1];
    __shared__ double s_tot[kOpt1DWaves][3];
    __shared__ int s_cnt[kOpt1DWaves];
    __shared__ double s_p2;  // total of w*x^2 over the row
    static_assert(kOpt1DMaxN <= 4096, "cuts are packed in 12 bits");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t b = blockIdx.x;
    const int NP = [&] {
        int p = 1;
        while (p < N) p <<= 1;
        return p;
    }();
    const int NB = NP / 2 > 0 ? NP / 2 : 1;
    double* P0 = s_dyn;
    double* P1 = P0 + (N + 1);
    double* E = P1 + (N + 1);
    uint64_t* keys = (uint64_t*)E;
    // per-level minimum keys, two levels' worth: a level's results are
    // written out while the next level's ranges are formed
    uint64_t* s_best_a = (uint64_t*)(E + (NP > N + 1 ? NP : N + 1));
    uint64_t* s_best_b = s_best_a + NB;
    uint16_t* cut = (uint16_t*)(s_best_b + NB);
    uint16_t* s_off = cut + (N + 1);
    double* Eg = Eg_all + b * (N + 1);
    uint16_t* cutg = cut_all + b * (int64_t)K * (N + 1);
    int32_t* perm = perm_all + b * N;
    const T* Xb = X + b * N;
    const float* wb = w ? w + b * N : nullptr;

    // ---- sort the row by (value, index)
    for (int p = tid; p < NP; p += kOpt1DThreads)
        keys[p] = p < N ? ((uint64_t)f1_ord(f1_load<T>(Xb + p)) << 32) | (uint32_t)p : ~(uint64_t)0;
    __syncthreads();
    for (int size = 2; size <= NP; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = tid; t < (NP >> 1); t += kOpt1DThreads) {
                const int i = 2 * t - (t & (stride - 1));
                const int k = i + stride;
                const bool up = (i & size) == 0;
                const uint64_t a = keys[i], c = keys[k];
                if ((a > c) == up) {
                    keys[i] = c;
                    keys[k] = a;
                }
            }
            __syncthreads();
        }
    }

    // ---- prefix sums of w and w*x over the sorted row, and the total of
    // w*x^2 (float64).  Thread t owns sorted positions t*CH .. t*CH+CH-1.
    {
        const int CH = (N + kOpt1DThreads - 1) / kOpt1DThreads;  // <= 4
        double l0[4], l1[4];
        double a0 = 0.0, a1 = 0.0, a2 = 0.0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int p = tid * CH + c;
            if (c < CH && p < N) {
                const uint64_t key = keys[p];
                const int idx = (int)(key & 0xffffffffu);
                const double xv = (double)f1_unord((uint32_t)(key >> 32));
                const double wv = wb ? (double)wb[idx] : 1.0;
                perm[p] = idx;
                a0 += wv;
                a1 += wv * xv;
                a2 += (wv * xv) * xv;
            }
            l0[c] = a0, l1[c] = a1;
        }
        // exclusive scan of the per-thread totals: inside the wave, then across waves
        double i0 = a0, i1 = a1, i2 = a2;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const double u0 = __shfl_up(i0, o, 64), u1 = __shfl_up(i1, o, 64), u2 = __shfl_up(i2, o, 64);
            if (lane >= o) i0 += u0, i1 += u1, i2 += u2;
        }
        if (lane == 63) s_tot[wave][0] = i0, s_tot[wave][1] = i1, s_tot[wave][2] = i2;
        __syncthreads();
        double e0 = i0 - a0, e1 = i1 - a1;
        for (int v = 0; v < wave; ++v) e0 += s_tot[v][0], e1 += s_tot[v][1];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int p = tid * CH + c;
            if (c < CH && p < N) {
                P0[p + 1] = e0 + l0[c];
                P1[p + 1] = e1 + l1[c];
            }
        }
        if (tid == 0) {
            P0[0] = P1[0] = 0.0;
            double t2 = 0.0;
            for (int v = 0; v < kOpt1DWaves; ++v) t2 += s_tot[v][2];
            s_p2 = t2;
        }
    }
    __syncthreads();  // the keys are no longer needed: E takes their place

    // ---- layer 1
    for (int j = tid; j <= N; j += kOpt1DThreads) E[j] = j > 0 ? -(P1[j] * P1[j]) / P0[j] : 0.0;
    __syncthreads();

    // ---- layers 2 .. K
    for (int k = 2; k <= K; ++k) {
        const int n = N - k + 1;  // j - k in [0, n)
        int L = 1;
        while ((1 << L) - 1 < n) ++L;  // a complete tree of 2^L - 1 >= n nodes
        uint64_t* s_best = s_best_a;       // this level's keys
        uint64_t* s_best_prev = s_best_b;  // the previous level's
        // the cut and E_k of node sp of a level with spacing hh, from its key
        auto finish = [&](int hh, int sp, const uint64_t* sb) {
            const int jp = (2 * sp + 1) * hh - 1;
            if (jp >= n) return;
            const int j = k + jp;
            const int bi = (int)(sb[sp] & 0xfff);
            const double s1 = P1[j] - P1[bi];
            Eg[j] = E[bi] - s1 * s1 / (P0[j] - P0[bi]);
            cutg[(int64_t)(k - 1) * (N + 1) + j] = (uint16_t)bi;
            cut[j] = (uint16_t)bi;
        };
        for (int l = 0; l < L; ++l) {
            const int nsub = 1 << l, h = 1 << (L - 1 - l);
            // node s of this level: j = k + (2s+1)h - 1, its range of cuts.  Its
            // parent (node s/2 of the previous level) is its right neighbour
            // for even s and its left one for odd s; the parent's cut is read
            // from the previous level's key, since it is written to cut[] only
            // during this level's first phase.
            auto node = [&](int sn, int& j, int& ilo) -> int {  // returns the range length (0: no node)
                const int jp = (2 * sn + 1) * h - 1;
                if (jp >= n) return 0;
                j = k + jp;
                const int par = l > 0 ? (int)(s_best_prev[sn >> 1] & 0xfff) : 0;
                ilo = jp - h >= 0 ? ((sn & 1) ? par : (int)cut[j - h]) : k - 1;
                const int ihi = jp + h < n ? ((sn & 1) ? (int)cut[j + h] : par) : N - 1;
                int imax = ihi < j - 1 ? ihi : j - 1;
                if (imax < ilo) imax = ilo;  // only where rounding breaks the order of the cuts
                return imax - ilo + 1;
            };
            // (a) range lengths, four consecutive nodes per thread, and their
            // exclusive scan; the left child of every node of the previous
            // level writes that node's cut and E_k
            int len[4], sum = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int sn = 4 * tid + q;
                int j, ilo;
                len[q] = sn < nsub ? node(sn, j, ilo) : 0;
                if (sn < nsub) s_best[sn] = ~(uint64_t)0;
                if (l > 0 && sn < nsub && (sn & 1) == 0) finish(2 * h, sn >> 1, s_best_prev);
                sum += len[q];
            }
            int incl = sum;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int u = __shfl_up(incl, o, 64);
                if (lane >= o) incl += u;
            }
            if (lane == 63) s_cnt[wave] = incl;
            __syncthreads();
            int excl = incl - sum, total = 0;
            for (int v = 0; v < kOpt1DWaves; ++v) {
                total += s_cnt[v];
                if (v < wave) excl += s_cnt[v];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int sn = 4 * tid + q;
                if (sn < nsub) s_off[sn] = (uint16_t)excl;
                excl += len[q];
            }
            if (tid == 0) s_off[nsub] = (uint16_t)total;
            __syncthreads();
            // (b) an equal slice of all (node, cut) candidates per thread
            const int C = (total + kOpt1DThreads - 1) / kOpt1DThreads;
            const int t0 = tid * C, t1 = t0 + C < total ? t0 + C : total;
            if (t0 < t1) {
                int sn = 0, cnt = nsub;  // last node with s_off[sn] <= t0
                while (cnt > 1) {
                    const int half = cnt >> 1;
                    if ((int)s_off[sn + half] <= t0) sn += half, cnt -= half;
                    else cnt = half;
                }
                int j = 0, ilo = 0;
                node(sn, j, ilo);
                double p0j = P0[j], p1j = P1[j];
                uint64_t best = ~(uint64_t)0;
                for (int t = t0; t < t1; ++t) {
                    while (t >= (int)s_off[sn + 1]) {  // the next node with candidates
                        atomicMin(&s_best[sn], best);
                        best = ~(uint64_t)0;
                        ++sn;
                        node(sn, j, ilo);
                        p0j = P0[j], p1j = P1[j];
                    }
                    const int i = ilo + (t - (int)s_off[sn]);
                    const double s0 = p0j - P0[i], s1 = p1j - P1[i];
                    double r = __builtin_amdgcn_rcp(s0);  // refined by one Newton step
                    r = r * fma(-s0, r, 2.0);
                    const uint64_t u = (uint64_t)__double_as_longlong(E[i] - s1 * s1 * r);
                    const uint64_t o = (u >> 63) ? ~u : (u | 0x8000000000000000ull);
                    const uint64_t key = (o & ~(uint64_t)0xfff) | (uint64_t)i;
                    best = key < best ? key : best;
                }
                atomicMin(&s_best[sn], best);
            }
            __syncthreads();
            uint64_t* tmp = s_best;
            s_best = s_best_prev;
            s_best_prev = tmp;
        }
        // (c) the cut and E_k of every node of the last level
        for (int sn = tid; sn < (1 << (L - 1)); sn += kOpt1DThreads) finish(1, sn, s_best_prev);
        __syncthreads();
        // E_k back into LDS (the barrier makes this block's device-memory
        // writes visible to all of its threads)
        for (int j = k + tid; j <= N; j += kOpt1DThreads) E[j] = Eg[j];
        __syncthreads();
    }

    // ---- backtrack the cuts, then the outputs
    if (tid == 0) {
        s_bound[K] = N;
        for (int k = K; k >= 2; --k) s_bound[k - 1] = cutg[(int64_t)(k - 1) * (N + 1) + s_bound[k]];
        s_bound[0] = 0;
        if (objective) {
            const double J = E[N] + s_p2;
            objective[b] = J > 0.0 ? J : 0.0;
        }
    }
    __syncthreads();
    for (int c = tid; c < K; c += kOpt1DThreads) {
        const int lo = s_bound[c], hi = s_bound[c + 1];
        centroids[b * K + c] = hi > lo ? (float)((P1[hi] - P1[lo]) / (P0[hi] - P0[lo])) : 0.0f;
        if (counts) counts[b * K + c] = hi - lo;
    }
    if (labels) {
        for (int p = tid; p < N; p += kOpt1DThreads) {
            int lo = 0, len = K - 1;  // runs 1 .. K-1 start at s_bound[1 .. K-1]: count those <= p
            while (len > 0) {
                const int h = len >> 1;
                if (s_bound[1 + lo + h] <= p) {
                    lo += h + 1;
                    len -= h + 1;
                } else {
                    len = h;
                }
            }
            labels[b * N + perm[p]] = lo;
        }
    }
}

hipError_t launch_optimal_1d(DType xt, const void* x, const float* w, int64_t B, int64_t N, int64_t K,
                             float* centroids, int32_t* labels, int32_t* counts, double* objective, void* ws,
                             hipStream_t s) {
    if (B == 0) return hipSuccess;
    if (!optimal_1d_supports(N, K)) return hipErrorInvalidValue;
    size_t d_off, cut_off, perm_off, total;
    optimal_1d_workspace(B, N, K, &d_off, &cut_off, &perm_off, &total);
    double* Eg = (double*)((char*)ws + d_off);
    uint16_t* cutg = (uint16_t*)((char*)ws + cut_off);
    int32_t* perm = (int32_t*)((char*)ws + perm_off);
    const size_t lds = opt1d_lds_bytes((int)N);
    const void* fn = xt == DType::F32 ? (const void*)k_optimal_1d<float>
                     : xt == DType::F16 ? (const void*)k_optimal_1d<_Float16>
                                        : (const void*)k_optimal_1d<bf16_t>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)B);
    if (xt == DType::F32)
        hipLaunchKernelGGL(k_optimal_1d<float>, grid, dim3(kOpt1DThreads), lds, s, (const float*)x, w, (int)N,
                           (int)K, centroids, labels, counts, objective, Eg, cutg, perm);
    else if (xt == DType::F16)
        hipLaunchKernelGGL(k_optimal_1d<_Float16>, grid, dim3(kOpt1DThreads), lds, s, (const _Float16*)x, w,
                           (int)N, (int)K, centroids, labels, counts, objective, Eg, cutg, perm);
    else
        hipLaunchKernelGGL(k_optimal_1d<bf16_t>, grid, dim3(kOpt1DThreads), lds, s, (const bf16_t*)x, w, (int)N,
                           (int)K, centroids, labels, counts, objective, Eg, cutg, perm);
    return hipGetLastError();
}

}  // namespace km
