// Argsort of the label vector by cluster id: the first half of the
// sort-inverse update (technologypulse.uk "Flash-KMeans" article,
// bottleneck 2; wispaper.ai "Flash-KMeans" blog, "Sort-Inverse Update").
// After it, the indices of the points of cluster j form the contiguous
// segment perm[offsets[j] .. offsets[j+1]) in ascending order (a stable
// sort); the points themselves are never moved.
//
// Labels are small integers (< K <= 32768), so a counting sort replaces the
// general argsort.  The labels of a problem are cut into chunks of CH
// consecutive points (CH >= K, about 256 chunks over the job):
//   1. k_hist     -- each block histograms one chunk in LDS and stores the
//                    chunk's whole row H[c][0..K) (no atomics in device
//                    memory).  Inside a Lloyd fit the assignment kernel
//                    builds H itself while it writes the labels, and this
//                    pass is skipped.
//   2. k_colscan  -- per bin, the exclusive prefix of H over the chunks ->
//                    P[c][j] (the points of bin j in chunks before c), and
//                    the column totals -> counts; H is cleared for the next
//                    assignment that builds it.
//   3. k_scan     -- exclusive prefix of counts -> offsets (and whether
//                    every cluster is short enough for the one-segment-per-
//                    group reduction).  With 16-byte count and prefix rows
//                    the scatter forms the offsets itself instead (each
//                    block scans the counts row it reads anyway; the block
//                    of chunk 0 stores them and the flag), and this launch
//                    is skipped.
//   4. k_scatter  -- chunk c places its points of bin j from
//                    offsets[j] + P[c][j] on, in index order: each wave of
//                    the block takes a consecutive part of the chunk with its
//                    own cursor per bin in LDS (the wave's histogram gives
//                    the bases of the waves after it), and walks its part 64
//                    labels at a time; lanes holding the same label find each
//                    other with one ballot per label bit, the lower lanes
//                    going first, and the lowest lane of each label advances
//                    the cursor.  The lane that places a point at the first
//                    sorted position of a reduction piece also stores the
//                    point's label as the piece's first segment.
// Every step is a deterministic function of the labels, so the whole sort
// is: run twice on the same labels, it produces the same permutation.
//
// Few labels per cluster (a mini-batch against many clusters) can take an
// unordered variant instead, where every label takes one global atomic
// (k_count_direct, k_scatter_direct); its segments hold the right indices in
// arrival order.
// Labels outside [0, K) are skipped by every pass.
#include "common.h"

namespace km {

constexpr int kHistThreads = 512;

// Labels per chunk: a power of two, at least 512 and K, doubled until the
// whole job takes at most 256 chunks (or one chunk per problem).  A chunk is
// a whole number of every assignment point group (those hold 128..512
// points), so the assignment can add a group's labels to its chunk's row.
// Small jobs thus spread their scatter over more blocks (8192 labels with K
// = 256: 16 chunks of 512 instead of 2 of 4096).
int64_t sort_chunk(int64_t B, int64_t N, int64_t K) {
    int64_t ch = 512;
    while (ch < K) ch *= 2;
    while (ch < N && B * ((N + ch - 1) / ch) > 256) ch *= 2;
    return ch;
}

int64_t sort_chunks(int64_t B, int64_t N, int64_t K) {
    const int64_t ch = sort_chunk(B, N, K);
    return N > 0 ? (N + ch - 1) / ch : 1;
}

// One block per (chunk, problem): LDS histogram of the chunk's labels, then
// the whole row of K bins stored to H.
__global__ __launch_bounds__(kHistThreads) void k_hist(const int32_t* __restrict__ labels, int64_t N, int K,
                                                       int64_t CH, int64_t nch, int32_t* __restrict__ H) {
    extern __shared__ int32_t s_h[];
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.y, c = blockIdx.x;
    const int64_t i0 = c * CH;
    const int64_t i1 = (i0 + CH < N) ? i0 + CH : N;
    const int32_t* L = labels + b * N;
    for (int j = tid; j < K; j += kHistThreads) s_h[j] = 0;
    __syncthreads();
    int64_t i = i0 + tid;
    for (; i + 3 * kHistThreads < i1; i += 4 * kHistThreads) {
        const int32_t l0 = L[i], l1 = L[i + kHistThreads], l2 = L[i + 2 * kHistThreads],
                      l3 = L[i + 3 * kHistThreads];
        if ((uint32_t)l0 < (uint32_t)K) atomicAdd(&s_h[l0], 1);
        if ((uint32_t)l1 < (uint32_t)K) atomicAdd(&s_h[l1], 1);
        if ((uint32_t)l2 < (uint32_t)K) atomicAdd(&s_h[l2], 1);
        if ((uint32_t)l3 < (uint32_t)K) atomicAdd(&s_h[l3], 1);
    }
    for (; i < i1; i += kHistThreads) {
        const int32_t l = L[i];
        if ((uint32_t)l < (uint32_t)K) atomicAdd(&s_h[l], 1);
    }
    __syncthreads();
    int32_t* row = H + (b * nch + c) * (int64_t)K;
    for (int j = tid; j < K; j += kHistThreads) row[j] = s_h[j];
}

// Column prefix of H.  A block takes 64 consecutive bins of one problem; its
// 16 lane groups split the chunks into 16 consecutive ranges (at most 16
// chunks each: nch <= 256).  Each thread keeps its range's counts in
// registers, the range totals are combined in LDS in chunk order, and every
// entry gets the count of its bin in all earlier chunks.  clear: store zeros
// back to H (the assignment of the next iteration adds into it).
constexpr int kColBins = 64, kColQ = 16, kColMaxPer = 16;

// obj_out (may be NULL): one extra block per problem, after the bin blocks,
// sums the assignment's objective partials of the problem (obj_sum_1024),
// which saves the objective's own launch inside a fit; a block of its own
// runs beside the bin blocks instead of lengthening one of them.
static_assert(kColBins * kColQ == 1024, "the objective sum takes a block of 1024 threads");

__global__ __launch_bounds__(kColBins* kColQ) void k_colscan(int32_t* __restrict__ H, int64_t nch, int K,
                                                             int32_t* __restrict__ P, int32_t* __restrict__ counts,
                                                             bool clear, const double* __restrict__ obj_part,
                                                             int64_t obj_nblk, double* __restrict__ obj_out,
                                                             int64_t obj_stride) {
    __shared__ int32_t s_tot[kColQ][kColBins];
    __shared__ double s_red[1024];
    const int jl = threadIdx.x % kColBins, q = threadIdx.x / kColBins;
    const int64_t b = blockIdx.y;
    if ((int)blockIdx.x == (K + kColBins - 1) / kColBins) {  // the objective's block
        if (obj_out) obj_sum_1024(obj_part + b * obj_nblk, obj_nblk, obj_out + b * obj_stride, s_red);
        return;
    }
    const int j = blockIdx.x * kColBins + jl;
    const int64_t per = (nch + kColQ - 1) / kColQ;  // <= kColMaxPer
    const int64_t c0 = q * per;
    int32_t v[kColMaxPer];
    int32_t tot = 0;
#pragma unroll
    for (int u = 0; u < kColMaxPer; ++u) {
        const int64_t c = c0 + u;
        v[u] = (u < per && c < nch && j < K) ? H[(b * nch + c) * K + j] : 0;
        tot += v[u];
    }
    s_tot[q][jl] = tot;
    __syncthreads();
    int32_t run = 0, all = 0;
#pragma unroll
    for (int r = 0; r < kColQ; ++r) {
        const int32_t t = s_tot[r][jl];
        run += r < q ? t : 0;
        all += t;
    }
    if (j >= K) return;
#pragma unroll
    for (int u = 0; u < kColMaxPer; ++u) {
        const int64_t c = c0 + u;
        if (u < per && c < nch) {
            P[(b * nch + c) * K + j] = run;
            if (clear) H[(b * nch + c) * K + j] = 0;
            run += v[u];
        }
    }
    if (q == 0) counts[b * K + j] = all;
}

// One block per problem: exclusive scan of K counts -> offsets.  The counts
// are staged in LDS with coalesced loads, eight in flight per thread, and
// zero-padded to Kpad (a multiple of 4096).  Each thread then scans a
// contiguous run of Kpad / 1024 bins with 16-byte LDS accesses, and the run
// totals are scanned with wave shuffles and the 16 wave totals: one shuffle
// scan for the whole row.  When piece_seg is given it also records, for
// every reduction piece of TW sorted rows, the segment its first row falls
// in (binary search over the offsets in LDS).
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
    if (cursor)
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

// One block per (chunk, problem), WB waves; wave w takes the w-th of WB
// consecutive parts of the chunk.  LDS: WB cursor tables of K bins.  Labels
// are read kScatterR rounds of 64 at a time, the next batch's loads issued
// before the current batch is ranked, so the ranking (a chain of LDS reads
// and writes per round) runs under the loads.  At one or two waves per SIMD
// the fixed work of a block (clearing WB·K table entries, reading K bases)
// costs more than its labels, so it moves 16 bytes per lane per instruction
// where the rows allow (K a multiple of 4, the offsets and prefix rows
// 16-byte aligned), the first bases' loads are issued before the count, and a
// part of at most 2 kScatterR rounds keeps its labels in registers from the
// count to the placement instead of reading them twice.
constexpr int kScatterR = 16;

// piece_seg (or NULL): [B][npieces], the first segment of every reduction
// piece of 2^tw_shift sorted rows, that is the label of the point placed at
// the piece's first position.
//
// SCAN (K a multiple of 4, 16-byte aligned count and prefix rows): the
// offsets are not read but formed by every block from the counts row, the
// exclusive prefix of the counts in bin order, which saves the scan's own
// launch; the block of chunk 0 stores them (offsets[b][0..K]) and the
// problem's short-segment flag.  A pass of the base loop covers 64 WB BU
// groups of 4 bins: thread t holds groups t + 64 WB e, e < BU, so round e of
// a pass is 256 WB consecutive bins, 4 per thread in thread order; one wave
// scan per round (BU at once) and one barrier per pass give each bin its
// prefix.
template <int WB, int NB, bool SCAN>
__global__ __launch_bounds__(64 * WB) void k_scatter(const int32_t* __restrict__ labels, int64_t N, int K,
                                                     int64_t CH, int64_t nch,
                                                     const int32_t* __restrict__ P,
                                                     int32_t* offsets,  // read, or with SCAN written
                                                     int32_t* __restrict__ perm, int32_t* __restrict__ piece_seg,
                                                     int64_t npieces, int tw_shift,
                                                     const int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ short_flag) {
    constexpr int R = kScatterR;
    constexpr int BU = 8;  // bins (or groups of 4 bins) per thread and pass
    extern __shared__ __attribute__((aligned(16))) int32_t s_tab[];  // [WB][K]
    __shared__ int32_t s_ws[SCAN ? BU : 1][WB];  // SCAN: wave totals of each round of a pass
    __shared__ int32_t s_max;                    // SCAN: the largest count
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    // Consecutive blocks go to the 8 XCDs in turn, each with its own L2; the
    // points of one cluster sit in the permutation in chunk order, so with
    // nch a multiple of 8 every XCD takes a contiguous range of chunks, and
    // a 128-byte line of the permutation is written from one or two L2s
    // instead of all eight (1M labels, K = 8192: the scatter's writes went
    // from 7.9 to 1.5 times the bytes of the permutation).
    const int64_t b = blockIdx.y;
    const int64_t c = (nch & 7) == 0 ? (int64_t)(blockIdx.x & 7) * (nch >> 3) + (blockIdx.x >> 3) : blockIdx.x;
    const int64_t i0 = c * CH;
    const int64_t i1 = (i0 + CH < N) ? i0 + CH : N;
    const int64_t part = ((i1 - i0 + WB - 1) / WB + 63) / 64 * 64;  // whole rounds per wave
    const int64_t w0 = i0 + w * part;
    const int64_t w1 = (w0 + part < i1) ? w0 + part : i1;
    const int32_t* L = labels + b * N;
    int32_t* tab = s_tab + w * K;
    auto load_batch = [&](int64_t r0, int32_t (&v)[R]) {
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int64_t i = r0 + u * 64 + lane;
            v[u] = i < w1 ? L[i] : -1;
        }
    };
    // cursor of bin j for wave w: where the chunk's points of bin j start,
    // plus those of the earlier waves
    const int32_t* Pc = P + (b * nch + c) * (int64_t)K;
    // SCAN: the first row loaded with the prefix rows is the counts row
    const int32_t* ob = SCAN ? counts + b * K : offsets + b * (K + 1);
    // 16-byte rows: thread tid takes the groups of 4 bins tid, tid + 64 WB, ...
    const bool vec = SCAN || ((K & 3) == 0 && ((uintptr_t)ob & 15) == 0 && ((uintptr_t)Pc & 15) == 0);  // (block-uniform)
    const int K4 = K >> 2;
    // the two rows are kept apart until the bases are formed, so that the
    // first pass's loads are waited for together with the labels' (after the
    // table clear), not before the clear
    auto load_bases4 = [&](int q0, i32x4 (&ov)[BU], i32x4 (&pv)[BU]) {
#pragma unroll
        for (int e = 0; e < BU; ++e) {
            const int q = q0 + e * 64 * WB;
            ov[e] = q < K4 ? ((const i32x4*)ob)[q] : i32x4{0, 0, 0, 0};
            pv[e] = q < K4 ? ((const i32x4*)Pc)[q] : i32x4{0, 0, 0, 0};
        }
    };
    i32x4 ob0[BU], pc0[BU];
    if (vec) load_bases4(tid, ob0, pc0);
    const bool keep = part <= 2 * 64 * R;  // (a block-uniform choice)
    int32_t kept[2][R];
    if ((K & 3) == 0) {
        i32x4* tab4 = (i32x4*)tab;
        for (int q = lane; q < K4; q += 64) tab4[q] = i32x4{0, 0, 0, 0};
    } else {
        for (int j = lane; j < K; j += 64) tab[j] = 0;
    }
    if (SCAN && tid == 0) s_max = 0;
    __builtin_amdgcn_wave_barrier();
    // this wave's histogram, R labels in flight per lane
    if (keep) {
        load_batch(w0, kept[0]);
        load_batch(w0 + 64 * R, kept[1]);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int u = 0; u < R; ++u)
                if ((uint32_t)kept[h][u] < (uint32_t)K) atomicAdd(&tab[kept[h][u]], 1);
    } else {
        for (int64_t r0 = w0; r0 < w1; r0 += 64 * R) {
            int32_t v[R];
            load_batch(r0, v);
#pragma unroll
            for (int u = 0; u < R; ++u)
                if ((uint32_t)v[u] < (uint32_t)K) atomicAdd(&tab[v[u]], 1);
        }
    }
    __syncthreads();
    if constexpr (SCAN) {
        // passes are block-uniform (every thread reaches every barrier)
        constexpr int NT = 64 * WB;
        int32_t* ob_out = offsets + b * (K + 1);
        int32_t carry = 0, vmax = 0;  // bins of earlier passes; the largest count
        for (int p0 = 0; p0 < K4; p0 += NT * BU) {
            const int q0 = p0 + tid;
            i32x4 cv[BU], pv[BU];
            if (p0 == 0) {
#pragma unroll
                for (int e = 0; e < BU; ++e) {
                    cv[e] = ob0[e];
                    pv[e] = pc0[e];
                }
            } else {
                load_bases4(q0, cv, pv);
            }
            int32_t sum[BU], incl[BU];
#pragma unroll
            for (int e = 0; e < BU; ++e) {
                sum[e] = cv[e][0] + cv[e][1] + cv[e][2] + cv[e][3];
                const int32_t m01 = cv[e][0] > cv[e][1] ? cv[e][0] : cv[e][1];
                const int32_t m23 = cv[e][2] > cv[e][3] ? cv[e][2] : cv[e][3];
                const int32_t m = m01 > m23 ? m01 : m23;
                vmax = m > vmax ? m : vmax;
                incl[e] = sum[e];
            }
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
#pragma unroll
                for (int e = 0; e < BU; ++e) {
                    const int32_t t = __shfl_up(incl[e], o, 64);
                    if (lane >= o) incl[e] += t;
                }
            }
            if (lane == 63) {
#pragma unroll
                for (int e = 0; e < BU; ++e) s_ws[e][w] = incl[e];
            }
            __syncthreads();
            int32_t run = carry;
#pragma unroll
            for (int e = 0; e < BU; ++e) {
                int32_t before = 0, tot = 0;
#pragma unroll
                for (int v = 0; v < WB; ++v) {
                    const int32_t t = s_ws[e][v];
                    before += v < w ? t : 0;
                    tot += t;
                }
                const int q = q0 + e * NT;
                i32x4 o;
                o[0] = run + before + incl[e] - sum[e];
                o[1] = o[0] + cv[e][0];
                o[2] = o[1] + cv[e][1];
                o[3] = o[2] + cv[e][2];
                run += tot;
                if (q < K4) {
                    if (c == 0) {
                        ob_out[4 * q + 0] = o[0];
                        ob_out[4 * q + 1] = o[1];
                        ob_out[4 * q + 2] = o[2];
                        ob_out[4 * q + 3] = o[3];
                    }
                    i32x4 base = o + pv[e];
#pragma unroll
                    for (int v = 0; v < WB; ++v) {
                        i32x4* t4 = (i32x4*)(s_tab + v * K) + q;
                        const i32x4 cnt = *t4;
                        *t4 = base;
                        base += cnt;
                    }
                }
            }
            carry = run;
            __syncthreads();  // s_ws is rewritten by the next pass
        }
        if (c == 0) {
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const int32_t t = __shfl_xor(vmax, o, 64);
                vmax = t > vmax ? t : vmax;
            }
            if (lane == 0) atomicMax(&s_max, vmax);
            if (tid == 0) ob_out[K] = carry;
        }
    } else if (vec) {
        for (int q0 = tid; q0 < K4; q0 += 64 * WB * BU) {
            i32x4 base[BU];
            if (q0 == tid) {
#pragma unroll
                for (int e = 0; e < BU; ++e) base[e] = ob0[e] + pc0[e];
            } else {
                i32x4 ov[BU], pv[BU];
                load_bases4(q0, ov, pv);
#pragma unroll
                for (int e = 0; e < BU; ++e) base[e] = ov[e] + pv[e];
            }
#pragma unroll
            for (int e = 0; e < BU; ++e) {
                const int q = q0 + e * 64 * WB;
                if (q < K4) {
#pragma unroll
                    for (int v = 0; v < WB; ++v) {
                        i32x4* t4 = (i32x4*)(s_tab + v * K) + q;
                        const i32x4 cnt = *t4;
                        *t4 = base[e];
                        base[e] += cnt;
                    }
                }
            }
        }
    } else {
        for (int j0 = tid; j0 < K; j0 += 64 * WB * BU) {
            int32_t base[BU];
#pragma unroll
            for (int e = 0; e < BU; ++e) {
                const int j = j0 + e * 64 * WB;
                base[e] = j < K ? ob[j] + Pc[j] : 0;
            }
#pragma unroll
            for (int e = 0; e < BU; ++e) {
                const int j = j0 + e * 64 * WB;
                if (j < K) {
#pragma unroll
                    for (int v = 0; v < WB; ++v) {
                        const int32_t t = s_tab[v * K + j];
                        s_tab[v * K + j] = base[e];
                        base[e] += t;
                    }
                }
            }
        }
    }
    __syncthreads();
    if (SCAN && c == 0 && tid == 0 && short_flag) short_flag[b] = s_max <= kShortSegMax ? 1 : 0;
    int32_t* Pb = perm + b * N;
    int32_t* psb = piece_seg ? piece_seg + b * npieces : nullptr;
    const int32_t tw_mask = (1 << tw_shift) - 1;
    // one batch of R rounds from r0: every round's grouping first (ballots
    // only, no memory), then the chain of cursor reads and advances
    auto place = [&](int64_t r0, const int32_t (&cur)[R]) {
        int rank[R], cnt[R];
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const bool ok = (uint32_t)cur[u] < (uint32_t)K;
            const uint64_t m = lanes_matching_n<NB>(cur[u], ok);
            rank[u] = ok ? lanes_below(m) : -1;
            cnt[u] = (int)__popcll(m);
        }
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int32_t l = rank[u] >= 0 ? cur[u] : 0;
            const int32_t base = tab[l];
            if (rank[u] >= 0) {
                const int32_t pos = base + rank[u];
                Pb[pos] = (int32_t)(r0 + u * 64 + lane);
                if (psb && (pos & tw_mask) == 0) psb[pos >> tw_shift] = cur[u];
            }
            if (rank[u] == 0) tab[l] = base + cnt[u];
        }
    };
    if (keep) {
        place(w0, kept[0]);
        place(w0 + 64 * R, kept[1]);
        return;
    }
    int32_t nxt[R];
    load_batch(w0, nxt);
    for (int64_t r0 = w0; r0 < w1; r0 += 64 * R) {
        int32_t cur[R];
#pragma unroll
        for (int u = 0; u < R; ++u) cur[u] = nxt[u];
        load_batch(r0 + 64 * R, nxt);
        place(r0, cur);
    }
}

// Unordered variant: one global atomic per label (counts must be zero on
// entry unless already counted).
constexpr int kDirectThreads = 256;

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

static hipError_t launch_scan(const int32_t* counts, int64_t B, int64_t K, int32_t* offsets, int32_t* cursor,
                              int TW, int64_t npieces, int32_t* piece_seg, int32_t* short_flag, hipStream_t s) {
    hipError_t e;
    const size_t scan_lds = (size_t)(scan_kpad(K) + 1) * sizeof(int32_t);
    if ((e = set_lds((const void*)k_scan, scan_lds)) != hipSuccess) return e;
    hipLaunchKernelGGL(k_scan, dim3((unsigned)B), dim3(1024), scan_lds, s, counts, (int)K, offsets, cursor, TW,
                       npieces, piece_seg, short_flag);
    return hipGetLastError();
}

hipError_t launch_sort(const int32_t* labels, int64_t B, int64_t N, int64_t K, const SortBufs& o, int TW,
                       int64_t npieces, hipStream_t s, SortMode mode) {
    if (B == 0) return hipSuccess;
    hipError_t e;
    if (mode == SortMode::Direct || mode == SortMode::DirectCounted) {
        // counts must be zero on entry unless the labels were already counted
        const dim3 dgrid((unsigned)((N + kDirectThreads - 1) / kDirectThreads), (unsigned)B);
        if (N > 0 && mode == SortMode::Direct) {
            hipLaunchKernelGGL(k_count_direct, dgrid, dim3(kDirectThreads), 0, s, labels, N, (int)K, o.counts);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        if ((e = launch_scan(o.counts, B, K, o.offsets, o.cursor, TW, npieces, o.piece_seg, o.short_flag, s)) !=
            hipSuccess)
            return e;
        if (N > 0) {
            hipLaunchKernelGGL(k_scatter_direct, dgrid, dim3(kDirectThreads), 0, s, labels, N, (int)K, o.cursor,
                               o.perm);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        return hipSuccess;
    }
    const int64_t CH = sort_chunk(B, N, K), nch = sort_chunks(B, N, K);
    if (mode == SortMode::Stable && N > 0) {
        const size_t lds = (size_t)K * sizeof(int32_t);
        if ((e = set_lds((const void*)k_hist, lds)) != hipSuccess) return e;
        hipLaunchKernelGGL(k_hist, dim3((unsigned)nch, (unsigned)B), dim3(kHistThreads), lds, s, labels, N, (int)K,
                           CH, nch, o.hist);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // StableCounted with N == 0: the rows are zero already
    if (N > 0) {
        hipLaunchKernelGGL(k_colscan, dim3((unsigned)((K + kColBins - 1) / kColBins + (o.obj_out ? 1 : 0)), (unsigned)B),
                           dim3(kColBins * kColQ), 0, s, o.hist, nch, (int)K, o.prefix, o.counts,
                           mode == SortMode::StableCounted, o.obj_part, o.obj_nblk, o.obj_out, o.obj_stride);
    } else {
        e = launch_zero(o.counts, (size_t)B * K * sizeof(int32_t), s);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // the pieces' first segments come from the scatter where the piece width
    // is a power of two (always, for the widths the reduction picks), else
    // from a search of the offsets in the scan
    int tw_shift = 0;
    while ((1 << tw_shift) < TW) ++tw_shift;
    const bool seg_in_scatter = (1 << tw_shift) == TW;
    // the scatter forms the offsets itself from 16-byte count and prefix rows
    const bool scan_in_scatter = N > 0 && seg_in_scatter && (K & 3) == 0 && ((uintptr_t)o.counts & 15) == 0 &&
                                 ((uintptr_t)o.prefix & 15) == 0;
    if (!scan_in_scatter) {
        if ((e = launch_scan(o.counts, B, K, o.offsets, nullptr, TW, npieces,
                             seg_in_scatter || N == 0 ? nullptr : o.piece_seg, o.short_flag, s)) != hipSuccess)
            return e;
    }
    if (N == 0) return hipSuccess;
    const int nbits = label_bits(K);
    const dim3 grid((unsigned)nch, (unsigned)B);
#define KM_SCATTER_S(WBV, NBV, SC)                                                                            \
    do {                                                                                                      \
        const size_t lds = (size_t)(WBV) * K * sizeof(int32_t);                                               \
        if ((e = set_lds((const void*)k_scatter<WBV, NBV, SC>, lds)) != hipSuccess) return e;                \
        hipLaunchKernelGGL((k_scatter<WBV, NBV, SC>), grid, dim3(64 * WBV), lds, s, labels, N, (int)K, CH, nch, \
                           o.prefix, o.offsets, o.perm, seg_in_scatter ? o.piece_seg : nullptr, npieces,      \
                           tw_shift, o.counts, o.short_flag);                                                 \
    } while (0)
#define KM_SCATTER(WBV, NBV)                        \
    do {                                            \
        if (scan_in_scatter) KM_SCATTER_S(WBV, NBV, true); \
        else KM_SCATTER_S(WBV, NBV, false);         \
    } while (0)
    // waves per block: as many K-bin cursor tables as fit in 128 KB of LDS
    // (K <= 4096: 8, 8192: 4, 16384: 2, 32768: 1); labels of nbits bits
    if (nbits <= 8) KM_SCATTER(8, 8);
    else if (nbits <= 12) KM_SCATTER(8, 12);
    else if (nbits <= 13) KM_SCATTER(4, 13);
    else if (nbits <= 14) KM_SCATTER(2, 14);
    else KM_SCATTER(1, 15);
#undef KM_SCATTER
#undef KM_SCATTER_S
    return hipGetLastError();
}

}  // namespace km
