// Argsort of the label vector by cluster id: the first half of the
// sort-inverse update (technologypulse.uk "Flash-KMeans" article,
// bottleneck 2; wispaper.ai "Flash-KMeans" blog, "Sort-Inverse Update").
// After it, the indices of the points of cluster j form the contiguous
// segment perm[offsets[j] .. offsets[j+1]); the points themselves are never
// moved.
//
// Labels are small integers (< K), so a counting sort replaces the general
// argsort:
//   1. k_count   -- each block histograms a chunk of labels in LDS and adds
//                   its non-zero bins to counts[b][.] (one global atomic per
//                   non-empty bin per chunk);
//   2. k_scan    -- exclusive prefix of counts -> offsets, and scatter cursors
//                   (and, if asked, whether every cluster is short enough for
//                   the one-segment-per-row-group reduction);
//   3. k_scatter -- each block re-histograms its chunk, reserves one
//                   contiguous run per non-empty bin with a single global
//                   atomic on that bin's cursor, then places its indices in
//                   the run with LDS atomics.
// Chunks are large (about one block per CU over the whole job): the global
// atomics on the cursors of the most popular clusters are serialized by the
// memory system, so their number, blocks x non-empty bins, is what limits
// both passes on skewed label distributions.  The scattered 4-byte index
// stores need no staging: successive stores into a run fill the same cache
// lines, which are merged in L2 before they reach HBM.
// Runs of different chunks land in a segment in arrival order, so the order
// inside a segment is unspecified; the set of indices is exact.
//
// Few labels per cluster (N <= 16 K, as in a mini-batch against many
// clusters) would leave the chunked passes with a handful of blocks, each
// walking all K bins with a chain of dependent atomics.  There every label
// takes its own global atomic instead (k_count_direct, k_scatter_direct),
// one thread per label over the whole grid.
// Labels outside [0, K) are skipped by every pass.
#include "common.h"

namespace km {

constexpr int kSortThreads = 512;

// Labels per block: at least 4096 and K, doubled until the whole job takes
// about 256 blocks.
static int64_t sort_chunk(int64_t B, int64_t N, int64_t K) {
    int64_t ch = 4096;
    while (ch < K) ch *= 2;
    while (ch < N && B * ((N + ch - 1) / ch) > 256) ch *= 2;
    return ch;
}

__device__ __forceinline__ void lds_histogram(const int32_t* __restrict__ L, int64_t i0, int64_t i1,
                                              int K, int32_t* s_h) {
    const int tid = threadIdx.x;
    int64_t i = i0 + tid;
    for (; i + 3 * kSortThreads < i1; i += 4 * kSortThreads) {
        const int32_t l0 = L[i], l1 = L[i + kSortThreads], l2 = L[i + 2 * kSortThreads],
                      l3 = L[i + 3 * kSortThreads];
        if ((uint32_t)l0 < (uint32_t)K) atomicAdd(&s_h[l0], 1);
        if ((uint32_t)l1 < (uint32_t)K) atomicAdd(&s_h[l1], 1);
        if ((uint32_t)l2 < (uint32_t)K) atomicAdd(&s_h[l2], 1);
        if ((uint32_t)l3 < (uint32_t)K) atomicAdd(&s_h[l3], 1);
    }
    for (; i < i1; i += kSortThreads) {
        const int32_t l = L[i];
        if ((uint32_t)l < (uint32_t)K) atomicAdd(&s_h[l], 1);
    }
}

__global__ __launch_bounds__(kSortThreads) void k_count(const int32_t* __restrict__ labels, int64_t N,
                                                        int K, int64_t CH, int32_t* __restrict__ counts) {
    extern __shared__ int32_t s_h[];
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.y;
    const int64_t i0 = (int64_t)blockIdx.x * CH;
    const int64_t i1 = (i0 + CH < N) ? i0 + CH : N;
    for (int j = tid; j < K; j += kSortThreads) s_h[j] = 0;
    __syncthreads();
    lds_histogram(labels + b * N, i0, i1, K, s_h);
    __syncthreads();
    for (int j = tid; j < K; j += kSortThreads) {
        const int32_t v = s_h[j];
        if (v) atomicAdd(&counts[b * K + j], v);
    }
}

// One block per batch: exclusive scan of K counts -> offsets and scatter
// cursors.  The counts are staged in LDS with coalesced loads, eight in
// flight per thread, and zero-padded to Kpad (a multiple of 4096).  Each
// thread then scans a contiguous run of Kpad / 1024 bins with 16-byte LDS
// accesses, and the run totals are scanned with wave shuffles and the 16
// wave totals: one shuffle scan for the whole row.  When piece_seg is given
// it also records, for every reduction piece of TW sorted rows, the segment
// its first row falls in (binary search over the offsets in LDS).
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

static int64_t scan_kpad(int64_t K) { return (K + 4095) / 4096 * 4096; }

__global__ __launch_bounds__(1024) void k_scan(const int32_t* __restrict__ counts, int K,
                                               int32_t* __restrict__ offsets, int32_t* __restrict__ cursor,
                                               int TW, int64_t npieces, int32_t* __restrict__ piece_seg,
                                               int32_t* __restrict__ short_flag) {
    extern __shared__ __attribute__((aligned(16))) int32_t s_off[];  // [Kpad + 1]
    __shared__ int32_t s_wave[16];
    __shared__ int32_t s_wmax[16];
    constexpr int U = 8;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t b = blockIdx.x;
    const int Kpad = (K + 4095) / 4096 * 4096;
    int32_t vmax = 0;  // the largest count (for the short-segment flag)
    for (int j0 = tid; j0 < Kpad; j0 += 1024 * U) {
        int32_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = j0 + u * 1024;
            v[u] = j < K ? counts[b * K + j] : 0;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = j0 + u * 1024;
            if (j < Kpad) s_off[j] = v[u];
            vmax = v[u] > vmax ? v[u] : vmax;
        }
    }
    if (short_flag) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const int32_t t = __shfl_xor(vmax, o, 64);
            vmax = t > vmax ? t : vmax;
        }
        if (lane == 0) s_wmax[wid] = vmax;
    }
    __syncthreads();
    if (short_flag && tid == 0) {
        int32_t m = 0;
        for (int w = 0; w < 16; ++w) m = s_wmax[w] > m ? s_wmax[w] : m;
        short_flag[b] = m <= kShortSegMax ? 1 : 0;
    }
    const int per = Kpad / 1024;  // a multiple of 4
    i32x4* run4 = (i32x4*)(s_off + tid * per);
    int32_t sum = 0;
    for (int q = 0; q < per / 4; ++q) {
        const i32x4 v = run4[q];
        sum += v[0] + v[1] + v[2] + v[3];
    }
    int32_t incl = sum;  // inclusive scan of the run totals within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
    }
    if (lane == 63) s_wave[wid] = incl;
    __syncthreads();
    int32_t run = incl - sum, total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        const int32_t t = s_wave[w];
        run += w < wid ? t : 0;
        total += t;
    }
    for (int q = 0; q < per / 4; ++q) {
        const i32x4 v = run4[q];
        i32x4 o;
        o[0] = run;
        o[1] = run + v[0];
        o[2] = o[1] + v[1];
        o[3] = o[2] + v[2];
        run = o[3] + v[3];
        run4[q] = o;
    }
    __syncthreads();  // the last run's store of s_off[K .. Kpad) before s_off[K] is set
    if (tid == 0) s_off[K] = total;
    __syncthreads();
    for (int j = tid; j <= K; j += 1024) offsets[b * (K + 1) + j] = s_off[j];
    for (int j = tid; j < K; j += 1024) cursor[b * K + j] = s_off[j];
    if (!piece_seg) return;
    // first segment of each piece that holds rows: the last j with offsets[j] <= p * TW
    for (int64_t p = tid; p < npieces && p * TW < total; p += 1024) {
        const int32_t q = (int32_t)(p * TW);
        int lo = 0, hi = K;  // invariant: s_off[lo] <= q < s_off[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_off[mid] <= q) lo = mid;
            else hi = mid;
        }
        piece_seg[b * npieces + p] = lo;
    }
}

__global__ __launch_bounds__(kSortThreads) void k_scatter(const int32_t* __restrict__ labels, int64_t N,
                                                          int K, int64_t CH, int32_t* __restrict__ cursor,
                                                          int32_t* __restrict__ perm) {
    extern __shared__ int32_t s_h[];
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.y;
    const int64_t i0 = (int64_t)blockIdx.x * CH;
    const int64_t i1 = (i0 + CH < N) ? i0 + CH : N;
    const int32_t* L = labels + b * N;
    for (int j = tid; j < K; j += kSortThreads) s_h[j] = 0;
    __syncthreads();
    lds_histogram(L, i0, i1, K, s_h);
    __syncthreads();
    // reserve this chunk's run in every non-empty segment
    for (int j = tid; j < K; j += kSortThreads) {
        const int32_t v = s_h[j];
        if (v) s_h[j] = atomicAdd(&cursor[b * K + j], v);
    }
    __syncthreads();
    int32_t* P = perm + b * N;
    auto place = [&](int64_t i, int32_t l) {
        if ((uint32_t)l < (uint32_t)K) P[atomicAdd(&s_h[l], 1)] = (int32_t)i;
    };
    int64_t i = i0 + tid;
    for (; i + 3 * kSortThreads < i1; i += 4 * kSortThreads) {  // 4 labels in flight
        const int32_t l0 = L[i], l1 = L[i + kSortThreads], l2 = L[i + 2 * kSortThreads],
                      l3 = L[i + 3 * kSortThreads];
        place(i, l0);
        place(i + kSortThreads, l1);
        place(i + 2 * kSortThreads, l2);
        place(i + 3 * kSortThreads, l3);
    }
    for (; i < i1; i += kSortThreads) place(i, L[i]);
}

constexpr int kDirectThreads = 256;

static bool sort_direct(int64_t N, int64_t K) { return N <= 16 * K; }

__global__ __launch_bounds__(kDirectThreads) void k_count_direct(const int32_t* __restrict__ labels, int64_t N,
                                                                 int K, int32_t* __restrict__ counts) {
    const int64_t b = blockIdx.y;
    const int64_t i = (int64_t)blockIdx.x * kDirectThreads + threadIdx.x;
    if (i >= N) return;
    const int32_t l = labels[b * N + i];
    if ((uint32_t)l < (uint32_t)K) atomicAdd(&counts[b * K + l], 1);
}

__global__ __launch_bounds__(kDirectThreads) void k_scatter_direct(const int32_t* __restrict__ labels, int64_t N,
                                                                   int K, int32_t* __restrict__ cursor,
                                                                   int32_t* __restrict__ perm) {
    const int64_t b = blockIdx.y;
    const int64_t i = (int64_t)blockIdx.x * kDirectThreads + threadIdx.x;
    if (i >= N) return;
    const int32_t l = labels[b * N + i];
    if ((uint32_t)l < (uint32_t)K) perm[b * N + atomicAdd(&cursor[b * K + l], 1)] = (int32_t)i;
}

static hipError_t set_lds(const void* f, size_t bytes) {
    if (bytes <= 64 * 1024) return hipSuccess;
    return hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_sort(const int32_t* labels, int64_t B, int64_t N, int64_t K, int32_t* counts,
                       int32_t* offsets, int32_t* cursor, int32_t* perm, int TW, int64_t npieces,
                       int32_t* piece_seg, int32_t* short_flag, hipStream_t s, bool counted) {
    // counts must be zero on entry (the caller clears it with the other accumulators)
    if (B == 0) return hipSuccess;
    const size_t lds = (size_t)K * sizeof(int32_t);
    hipError_t e;
    const bool direct = sort_direct(N, K);
    const dim3 dgrid((unsigned)((N + kDirectThreads - 1) / kDirectThreads), (unsigned)B);
    if (N > 0 && direct && !counted) {
        hipLaunchKernelGGL(k_count_direct, dgrid, dim3(kDirectThreads), 0, s, labels, N, (int)K, counts);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if (N > 0 && !counted) {
        if ((e = set_lds((const void*)k_count, lds)) != hipSuccess) return e;
        const int64_t CH = sort_chunk(B, N, K);
        dim3 grid((unsigned)((N + CH - 1) / CH), (unsigned)B);
        hipLaunchKernelGGL(k_count, grid, dim3(kSortThreads), lds, s, labels, N, (int)K, CH, counts);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const size_t scan_lds = (size_t)(scan_kpad(K) + 1) * sizeof(int32_t);
    if ((e = set_lds((const void*)k_scan, scan_lds)) != hipSuccess) return e;
    hipLaunchKernelGGL(k_scan, dim3((unsigned)B), dim3(1024), scan_lds, s, counts, (int)K, offsets, cursor, TW,
                       npieces, piece_seg, short_flag);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (N > 0 && direct) {
        hipLaunchKernelGGL(k_scatter_direct, dgrid, dim3(kDirectThreads), 0, s, labels, N, (int)K, cursor, perm);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if (N > 0) {
        if ((e = set_lds((const void*)k_scatter, lds)) != hipSuccess) return e;
        const int64_t CH = sort_chunk(B, N, K);
        dim3 grid((unsigned)((N + CH - 1) / CH), (unsigned)B);
        hipLaunchKernelGGL(k_scatter, grid, dim3(kSortThreads), lds, s, labels, N, (int)K, CH, cursor, perm);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace km
