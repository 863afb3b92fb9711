// Second half of the sort-inverse update: reduce each cluster's contiguous
// segment of perm on chip and write it to the cluster's sums once per
// reduced piece (technologypulse.uk "Flash-KMeans"
// article, bottleneck 2: one atomic per segment, O((K + N/B) d) atomics
// instead of O(N d); wispaper.ai "Flash-KMeans" blog, "Sort-Inverse
// Update": segmented reductions instead of scattered writes).
//
// gfx950 layout (ours): the sorted positions are cut into pieces of TW rows,
// one piece per 64-lane wave.  A point row is read with 16-byte loads by LPR
// lanes (d=128 bf16: 16 lanes), so one wave gathers 64/LPR rows per step and
// keeps two batches of U steps of loads in flight.  At a segment boundary the
// wave reduces its row groups with cross-lane shuffles.  The first segment of
// every piece comes with the sort (the stable scatter stores the label of the
// point it places at a piece's first position; the unordered variant's scan
// searches the offsets for it), and the following segment boundaries come
// from a 64-entry window of offsets held one per lane, so a wave never
// searches device memory serially.
//
// Where the partial sums go: a segment that starts inside a piece is stored
// by that piece with plain stores, since no other piece writes it directly
// (added with atomics instead when the sums accumulate over several
// launches, as in the chunked streaming fit).
// A piece's first segment (which may have begun in earlier pieces) is
// written to the piece's own slot instead.  The Lloyd update adds the slots
// in a fixed order (each block of kFoldG pieces sums its group's first run
// at its end, and the divide adds the rest); sums that accumulate over
// launches take a second, small kernel that adds runs of slots into the
// sums with atomics after the first has finished.
// Without that split, the pieces of a very large cluster (the head of a Zipf
// size distribution spans thousands of pieces) would all finish together and
// serialize on the same addresses; and device-wide float atomics are slow on
// this chip (tens of billions per second), so a batch of short segments
// flushed with atomics would be bound by them.
//
// Scalar points (d == 1) with a row that fits in LDS take a whole-row kernel
// instead: the row's (x, w) pairs are placed in cluster order in LDS and each
// segment is summed by one wave in float64.  Rows with few clusters (K <= 16)
// need no ordering at all: one wave streams the row and adds every point into
// bins of its own lane (float64 sums, integer counts), then combines the
// lanes' bins.
#include "scalar_rows.h"

namespace km {

template <typename T>
__device__ __forceinline__ float ld_elem(const T* p) {
    if constexpr (sizeof(T) == 4) return *p;
    else if constexpr (__is_same(T, _Float16)) return (float)*p;
    else return bf16_to_f32(*p);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16 bytes of a row -> EPL floats.
template <typename T>
__device__ __forceinline__ void unpack(const u32x4 u, float* out) {
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = __uint_as_float(u[e]);
    } else if constexpr (__is_same(T, _Float16)) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            out[2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[e] & 0xffffu));
            out[2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[e] >> 16));
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            out[2 * e] = __uint_as_float(u[e] << 16);
            out[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
        }
    }
}

// VEC: lane li of a row group reads elements [li*EPL, li*EPL + EPL) with one
// 16-byte load; otherwise it reads elements li + LPR*m, m < 4.
//
// A wave walks its piece in chunks of kSegChunk sorted rows.  The chunk's
// point indices are first copied to LDS with coalesced loads, so the row
// gathers that follow depend only on an LDS read, and U row steps (U*64/LPR
// rows) are kept in flight.  The running sums survive chunk boundaries and
// are flushed whenever a segment ends and at the end of the piece.
constexpr int kSegChunk = 512;

// One piece per wave; a block holds the kFoldG pieces of one fold group.
template <typename T, bool VEC, bool WEIGHTED>
__device__ __forceinline__ void segreduce_piece(const T* __restrict__ X, const float* __restrict__ w, int64_t N,
                                                int d, int lpr_shift, const int32_t* __restrict__ perm,
                                                const int32_t* __restrict__ offsets,
                                                const int32_t* __restrict__ piece_seg, int64_t npieces, int K,
                                                int TW, float* __restrict__ sums, float* __restrict__ wsum,
                                                float* __restrict__ slot, float* __restrict__ wslot,
                                                bool accumulate, const int32_t* __restrict__ skip,
                                                int32_t (*s_idx)[kSegChunk]) {
    constexpr int EPL = VEC ? 16 / (int)sizeof(T) : 8;  // non-vector rows: 64 lanes x 8 = 512 elements
    // row steps per batch (two batches in flight); rows read one element per
    // lane hold EPL values per step, and a block of kFoldG waves leaves 128
    // VGPRs per lane
    constexpr int U = VEC ? 8 : (WEIGHTED ? 1 : 2);
    // wv is uniform over the wave: saying so keeps the piece's bounds and
    // every loop over them in scalar registers and scalar branches
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t piece = (int64_t)blockIdx.x * kFoldG + wv;
    const int64_t b = blockIdx.y;
    if (piece >= npieces) return;
    if (skip && skip[b]) return;  // reduced by k_segsum_short
    const int32_t* offb = offsets + b * (K + 1);
    const int32_t total = offb[K];
    const int64_t q0 = piece * (int64_t)TW;
    if (q0 >= total) return;
    const int32_t q1 = (int32_t)((q0 + TW < total) ? q0 + TW : total);
    const int LPR = 1 << lpr_shift, RPW = 64 >> lpr_shift;
    const int gl = lane >> lpr_shift, li = lane & (LPR - 1);
    const int nvec = VEC ? d / EPL : 0;
    const bool active = VEC ? (li < nvec) : true;
    const T* Xb = X + b * N * (int64_t)d;
    const float* wb = WEIGHTED ? w + b * N : nullptr;
    const int32_t* pb = perm + b * N;
    int32_t* sidx = s_idx[wv];

    // A chunk's point indices are staged in LDS: every load of the chunk is
    // issued before the first store, so the staging costs one load latency.
    constexpr int kIdxPerLane = kSegChunk / 64;
    int32_t iv[kIdxPerLane];
    auto load_idx = [&](int32_t c0, int32_t c1) {
#pragma unroll
        for (int i = 0; i < kIdxPerLane; ++i) {
            // written on every path, so no value lives on to the next chunk
            iv[i] = 0;
            if (64 * i < c1 - c0) {
                const int32_t r = c0 + lane + 64 * i;
                iv[i] = pb[r < c1 ? r : c1 - 1];
            }
        }
    };
    auto store_idx = [&](int32_t c0, int32_t c1) {
#pragma unroll
        for (int i = 0; i < kIdxPerLane; ++i)
            if (64 * i < c1 - c0) sidx[lane + 64 * i] = iv[i];
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    };
    const int32_t c1_first = (q0 + kSegChunk < q1) ? (int32_t)q0 + kSegChunk : q1;
    load_idx((int32_t)q0, c1_first);

    // window of offsets: lane l holds offsets[wbase + l] (INT_MAX past K)
    int wbase = piece_seg[b * npieces + piece];
    auto load_win = [&]() {
        const int jw = wbase + lane;
        const int32_t v = offb[jw <= K ? jw : K];
        return jw <= K ? v : 0x7fffffff;
    };
    int32_t win = load_win();
    // segment containing q: the last j with offsets[j] <= q; returns its end
    int j = 0;
    auto locate = [&](int32_t q) -> int32_t {
        unsigned long long m = __ballot(win > q);
        while (m == 0ull) {
            wbase += 63;
            win = load_win();
            m = __ballot(win > q);
        }
        const int l = __ffsll((long long)m) - 1;  // first lane with offsets > q (l >= 1)
        j = wbase + l - 1;
        return __builtin_amdgcn_readfirstlane(__shfl(win, l, 64));
    };
    // whether the piece's first segment began in an earlier piece (then its
    // part here goes to the piece's slot); one that begins exactly at the
    // piece's first row is stored directly, like any later segment
    const bool cont = offb[wbase] < (int32_t)q0;

    float acc[EPL];
#pragma unroll
    for (int t = 0; t < EPL; ++t) acc[t] = 0.f;
    float wacc = 0.f;
    bool first = true;
    auto flush = [&]() {
        for (int o = LPR; o < 64; o <<= 1) {
#pragma unroll
            for (int t = 0; t < EPL; ++t) acc[t] += __shfl_xor(acc[t], o, 64);
            if constexpr (WEIGHTED) wacc += __shfl_xor(wacc, o, 64);
        }
        if (first && cont) {  // a segment begun earlier: its part goes to the piece's slot
            float* sp = slot + (b * npieces + piece) * (int64_t)d;
            if (gl == 0 && active) {
#pragma unroll
                for (int t = 0; t < EPL; ++t) {
                    const int k = VEC ? li * EPL + t : li + LPR * t;
                    if (k < d) sp[k] = acc[t];
                }
            }
            if constexpr (WEIGHTED) {
                if (lane == 0) wslot[b * npieces + piece] = wacc;
            }
        } else {
            // a segment that starts in this piece: no other piece writes it
            // directly (later pieces hold its rest in their slots, which the
            // fold adds after this launch), so a plain store suffices, unless
            // the sums carry earlier launches' contributions
            float* sj = sums + (b * K + j) * (int64_t)d;
            if (gl == 0 && active) {
#pragma unroll
                for (int t = 0; t < EPL; ++t) {
                    const int k = VEC ? li * EPL + t : li + LPR * t;
                    if (k < d) {
                        if (accumulate) unsafeAtomicAdd(sj + k, acc[t]);
                        else sj[k] = acc[t];
                    }
                }
            }
            if constexpr (WEIGHTED) {
                if (lane == 0) {
                    if (accumulate) unsafeAtomicAdd(wsum + b * K + j, wacc);
                    else wsum[b * K + j] = wacc;
                }
            }
        }
        first = false;
#pragma unroll
        for (int t = 0; t < EPL; ++t) acc[t] = 0.f;
        wacc = 0.f;
    };

    // The piece is walked in batches of STEP = RPW*U sorted rows, each row
    // group taking rows bs + u*RPW + gl.  The loads of the next batch are
    // issued before the current one is added, so two batches are in flight
    // whatever the segment lengths; a batch that crosses segment ends is
    // added once per segment it holds, each row masked to its own segment.
    // Every load is issued unconditionally (rows past the chunk read its last
    // row, lanes past the row read its first 16 bytes, and the values are
    // dropped), so the wait before a batch is added never has to cover the
    // batch behind it.
    const int STEP = RPW * U;
    struct Batch {
        u32x4 raw[U];
        float vs[U][VEC ? 1 : EPL];
        float wi[U];
    };
    // an empty asm statement that reads every register of a batch: the
    // point where its loads are waited for.  Each use site passes its own
    // text, so that the compiler cannot merge two of them into one placed
    // after the paths join.
#define KM_TOUCH(B, TAG)                                                                  \
    do {                                                                                  \
        _Pragma("unroll") for (int u_ = 0; u_ < U; ++u_) {                                \
            if constexpr (VEC) asm volatile("; " TAG ::"v"((B).raw[u_]));                \
            else {                                                                        \
                _Pragma("unroll") for (int t_ = 0; t_ < EPL; ++t_)                        \
                    asm volatile("; " TAG ::"v"((B).vs[u_][t_]));                         \
            }                                                                             \
            if constexpr (WEIGHTED) asm volatile("; " TAG ::"v"((B).wi[u_]));             \
        }                                                                                 \
    } while (0)
    auto load_batch = [&](Batch& B, int32_t bs, int32_t c0, int32_t c1) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // row bs + u*RPW + gl, clamped to the chunk's last row; the
            // wave-uniform part stays scalar
            const int32_t sb = __builtin_amdgcn_readfirstlane(bs + u * RPW - c0);
            const int32_t o = gl + sb, last = c1 - 1 - c0;
            const int32_t ix = sidx[o < last ? o : last];
            const T* row = Xb + (int64_t)ix * d;
            if constexpr (VEC) {
                B.raw[u] = __builtin_nontemporal_load((const u32x4*)(row + (active ? li * EPL : 0)));
            } else {
#pragma unroll
                for (int t = 0; t < EPL; ++t) {
                    const int k = li + LPR * t;
                    B.vs[u][t] = ld_elem<T>(row + (k < d ? k : 0));
                }
            }
            if constexpr (WEIGHTED) B.wi[u] = wb[ix];
        }
    };
    int32_t send = 0;
    bool pending = false;  // rows accumulated since the last flush
    auto add_batch = [&](const Batch& B, int32_t bs, int32_t c1) {
        // the batch's registers are read on every path, so no later
        // instruction that reuses them waits on loads issued after them
        KM_TOUCH(B, "batch");
        const int32_t be = (bs + STEP < c1) ? bs + STEP : c1;
        int32_t q = bs;
        while (q < be) {
            const int32_t e = send < be ? send : be;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                // row bs + u*RPW + gl lies in [q, e): bounds on gl are scalar
                const int32_t su = bs + u * RPW;
                const bool in = gl >= q - su && gl < e - su;
                float v[EPL];
                if constexpr (VEC) {
                    const u32x4 r = (in && active) ? B.raw[u] : u32x4{0u, 0u, 0u, 0u};
                    unpack<T>(r, v);
                } else {
#pragma unroll
                    for (int t = 0; t < EPL; ++t) v[t] = (in && li + LPR * t < d) ? B.vs[u][t] : 0.f;
                }
                const float wu = in ? (WEIGHTED ? B.wi[u] : 1.f) : 0.f;
#pragma unroll
                for (int t = 0; t < EPL; ++t) {
                    if constexpr (WEIGHTED) acc[t] = fmaf(wu, v[t], acc[t]);
                    else acc[t] += v[t];
                }
                wacc += wu;
            }
            pending = pending || (e > q);
            q = e;
            if (q == send) {  // the segment ends here
                if (pending) flush();
                pending = false;
                if (q < q1) send = locate(q);
            }
        }
    };
    Batch A, Bn;
    // the first chunk's rows are requested before the segment lookup, whose
    // loads then run under them
    store_idx((int32_t)q0, c1_first);
    load_batch(A, (int32_t)q0, (int32_t)q0, c1_first);
    send = locate((int32_t)q0);
    for (int32_t c0 = (int32_t)q0; c0 < q1; c0 += kSegChunk) {
        const int32_t c1 = (c0 + kSegChunk < q1) ? c0 + kSegChunk : q1;
        if (c0 != (int32_t)q0) {
            load_idx(c0, c1);
            store_idx(c0, c1);
            load_batch(A, c0, c0, c1);
        }
        // one exit, at the top: both adds run in every round (an add of a
        // batch that starts past the chunk only waits for its loads), so no
        // path back into the loop leaves loads pending in either batch.  A
        // batch loaded past the chunk's end repeats its last row, which has
        // just arrived.
        for (int32_t bs = c0; bs < c1; bs += 2 * STEP) {
            load_batch(Bn, bs + STEP, c0, c1);
            add_batch(A, bs, c1);
            load_batch(A, bs + 2 * STEP, c0, c1);
            add_batch(Bn, bs + STEP, c1);
        }
        KM_TOUCH(A, "past end");
        __builtin_amdgcn_wave_barrier();
    }
    if (pending) flush();
#undef KM_TOUCH
}

template <bool WEIGHTED>
__device__ __forceinline__ void fold_group(int64_t g, int64_t b, int lane, const float* __restrict__ slot,
                                           const float* __restrict__ wslot, const int32_t* __restrict__ piece_seg,
                                           const int32_t* __restrict__ offsets, int64_t npieces, int64_t ngroups,
                                           int K, int TW, int d, float* __restrict__ gslot,
                                           float* __restrict__ gwslot);

// The segmented reduction of kFoldG pieces per block, then (gslot set: the
// deterministic Lloyd fold) the fold of the block's own group: once every
// piece of the block has stored its slot, wave 0 adds the slots of the
// group's first run in piece order into the group slot (fold_group below).
template <typename T, bool VEC, bool WEIGHTED>
__global__ __launch_bounds__(64 * kFoldG) void k_segreduce(
    const T* __restrict__ X, const float* __restrict__ w, int64_t N, int d, int lpr_shift,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets, const int32_t* __restrict__ piece_seg,
    int64_t npieces, int K, int TW, float* __restrict__ sums, float* __restrict__ wsum, float* __restrict__ slot,
    float* __restrict__ wslot, bool accumulate, const int32_t* __restrict__ skip, int64_t ngroups,
    float* __restrict__ gslot, float* __restrict__ gwslot) {
    __shared__ int32_t s_idx[kFoldG][kSegChunk];
    segreduce_piece<T, VEC, WEIGHTED>(X, w, N, d, lpr_shift, perm, offsets, piece_seg, npieces, K, TW, sums, wsum,
                                      slot, wslot, accumulate, skip, s_idx);
    if (gslot) {
        // the slots of every piece of the group are stored and visible to
        // the block after the barrier
        __syncthreads();
        if (threadIdx.x < 64 && !(skip && skip[blockIdx.y]))  // (skip: reduced by k_segsum_short)
            fold_group<WEIGHTED>(blockIdx.x, blockIdx.y, threadIdx.x, slot, wslot, piece_seg, offsets, npieces,
                                 ngroups, K, TW, d, gslot, gwslot);
    }
}

// Second pass: fold the per-piece slots into the segment sums.  Pieces are in
// sorted order, so the pieces that share a first segment are consecutive;
// each wave walks kFoldG of them and issues one atomic per coordinate per
// segment change, so even a segment that spans thousands of pieces receives
// only (its pieces / kFoldG) atomic flushes.  The order of those atomics
// varies from run to run; this fold serves the sums that accumulate over
// several launches and the mini-batch steps, the Lloyd update folds
// deterministically (the group fold at the end of each k_segreduce block,
// then the divide).
int64_t fold_groups(int64_t npieces) { return (npieces + kFoldG - 1) / kFoldG; }

template <bool WEIGHTED>
__global__ __launch_bounds__(256) void k_fold_slots(const float* __restrict__ slot, const float* __restrict__ wslot,
                                                    const int32_t* __restrict__ piece_seg,
                                                    const int32_t* __restrict__ offsets, int64_t npieces, int K,
                                                    int TW, int d, float* __restrict__ sums,
                                                    float* __restrict__ wsum, const int32_t* __restrict__ skip) {
    constexpr int U = 8;
    const int lane = threadIdx.x & 63;
    const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t b = blockIdx.y;
    if (skip && skip[b]) return;  // reduced by k_segsum_short
    const int32_t total = offsets[b * (K + 1) + K];
    const int64_t np = ((int64_t)total + TW - 1) / TW;  // pieces that hold rows
    const int64_t p0 = g * kFoldG;
    const int64_t p1 = (p0 + kFoldG < np) ? p0 + kFoldG : np;
    if (p0 >= p1) return;
    const int32_t* ps = piece_seg + b * npieces;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // columns lane + 64 t (d <= 512)
    float wacc = 0.f;
    int cur = ps[p0];
    auto flush = [&]() {
        float* sj = sums + (b * K + cur) * (int64_t)d;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int k = lane + 64 * t;
            if (k < d) unsafeAtomicAdd(sj + k, acc[t]);
            acc[t] = 0.f;
        }
        if constexpr (WEIGHTED) {
            if (lane == 0) unsafeAtomicAdd(wsum + b * K + cur, wacc);
        }
        wacc = 0.f;
    };
    for (int64_t pb = p0; pb < p1; pb += U) {
        float v[U][8];
        float wv[U];
        int sg[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t p = pb + u;
            bool ok = p < p1;
            const int sgp = ok ? ps[p] : 0;
            // a piece whose first segment starts at its first row stored it
            // directly: no slot
            ok = ok && offsets[b * (K + 1) + sgp] < (int32_t)(p * TW);
            sg[u] = ok ? sgp : -1;
            const float* sp = slot + (b * npieces + (ok ? p : p0)) * (int64_t)d;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int k = lane + 64 * t;
                v[u][t] = (ok && k < d) ? sp[k] : 0.f;
            }
            wv[u] = (WEIGHTED && ok) ? wslot[b * npieces + p] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (sg[u] >= 0) {
                if (sg[u] != cur) {
                    flush();
                    cur = sg[u];
                }
#pragma unroll
                for (int t = 0; t < 8; ++t) acc[t] += v[u][t];
                wacc += wv[u];
            }
        }
    }
    flush();
}

// Deterministic fold (sums that do not accumulate over launches): instead of
// atomics, the slots of a segment are added in piece order by the divide.  A
// segment spanning many pieces would make that a long serial walk, so the
// reduction block of every group of kFoldG consecutive pieces first adds, at
// its end, the slots of the group's first run (its first piece and the
// following ones that share that piece's segment), in piece order, into the
// group's own slot.  The divide then adds at most kFoldG piece slots and one
// group slot per further group.  A group whose first piece starts a segment
// holds no slot there and stores nothing (no segment reads it).
template <bool WEIGHTED>
__device__ __forceinline__ void fold_group(int64_t g, int64_t b, int lane, const float* __restrict__ slot,
                                           const float* __restrict__ wslot, const int32_t* __restrict__ piece_seg,
                                           const int32_t* __restrict__ offsets, int64_t npieces, int64_t ngroups,
                                           int K, int TW, int d, float* __restrict__ gslot,
                                           float* __restrict__ gwslot) {
    constexpr int U = 8;
    if (g >= ngroups) return;
    const int32_t* offb = offsets + b * (K + 1);
    const int32_t total = offb[K];
    const int64_t np = ((int64_t)total + TW - 1) / TW;  // pieces that hold rows
    const int64_t p0 = g * kFoldG;
    if (p0 >= np) return;
    const int32_t* ps = piece_seg + b * npieces;
    const int s0 = ps[p0];
    if (offb[s0] >= (int32_t)(p0 * TW)) return;  // the group's first piece starts a segment
    const int64_t pe = (p0 + kFoldG < np) ? p0 + kFoldG : np;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // columns lane + 64 t (d <= 512)
    float wacc = 0.f;
    bool more = true;
    for (int64_t pb = p0; pb < pe && more; pb += U) {
        float v[U][8];
        float wv[U];
        bool in[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t p = pb + u;
            in[u] = p < pe && ps[p < pe ? p : p0] == s0;
            const float* sp = slot + (b * npieces + (in[u] ? p : p0)) * (int64_t)d;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int k = lane + 64 * t;
                v[u][t] = (in[u] && k < d) ? sp[k] : 0.f;
            }
            wv[u] = (WEIGHTED && in[u]) ? wslot[b * npieces + p] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (in[u]) {
#pragma unroll
                for (int t = 0; t < 8; ++t) acc[t] += v[u][t];
                wacc += wv[u];
            } else {
                more = false;
            }
        }
    }
    float* gp = gslot + (b * ngroups + g) * (int64_t)d;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int k = lane + 64 * t;
        if (k < d) gp[k] = acc[t];
    }
    if constexpr (WEIGHTED) {
        if (lane == 0) gwslot[b * ngroups + g] = wacc;
    }
}

// Rows per wave piece: enough pieces to fill the chip, and long pieces when
// there is plenty of work (fewer atomics on the largest clusters).
// Problems whose clusters are all short (at most kShortSegMax points, as a
// mini-batch against many centroids has them: 65536 points in 16384 clusters
// hold 4 on average): one row group of LPR lanes per segment, so a wave
// reduces 64 / LPR segments side by side instead of walking them one after
// another, each with its own load latency.  The group loads its segment's
// point indices and rows kSegShortU at a time, adds the rows in sorted order
// and stores the sum; an empty cluster gets zeros.  Every cluster's sum is
// written exactly once, with plain stores, so there are no slots, no fold and
// no atomics.  The kernel runs only where the sort's flag is set for the
// problem; k_segreduce and k_fold_slots return at once there.
constexpr int kSegShortU = 8;

template <typename T, bool VEC, bool WEIGHTED>
__global__ __launch_bounds__(256) void k_segsum_short(const T* __restrict__ X, const float* __restrict__ w,
                                                      int64_t N, int d, int lpr_shift,
                                                      const int32_t* __restrict__ perm,
                                                      const int32_t* __restrict__ offsets, int K,
                                                      const int32_t* __restrict__ short_flag,
                                                      float* __restrict__ sums, float* __restrict__ wsum) {
    constexpr int EPL = VEC ? 16 / (int)sizeof(T) : 8;
    constexpr int U = kSegShortU;
    const int64_t b = blockIdx.y;
    if (!short_flag[b]) return;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int LPR = 1 << lpr_shift, RPW = 64 >> lpr_shift;
    const int gl = lane >> lpr_shift, li = lane & (LPR - 1);
    const int64_t j = ((int64_t)blockIdx.x * 4 + wv) * RPW + gl;  // this group's cluster
    if (j >= K) return;
    const int nvec = VEC ? d / EPL : 0;
    const bool active = VEC ? (li < nvec) : true;
    const T* Xb = X + b * N * (int64_t)d;
    const float* wb = WEIGHTED ? w + b * N : nullptr;
    const int32_t* pb = perm + b * N;
    const int32_t o0 = offsets[b * (K + 1) + j], o1 = offsets[b * (K + 1) + j + 1];
    float acc[EPL];
#pragma unroll
    for (int t = 0; t < EPL; ++t) acc[t] = 0.f;
    float wacc = 0.f;
    for (int32_t r0 = o0; r0 < o1; r0 += U) {
        int32_t idx[U];
#pragma unroll
        for (int u = 0; u < U; ++u) idx[u] = r0 + u < o1 ? pb[r0 + u] : -1;
        u32x4 raw[U];
        float vs[U][VEC ? 1 : EPL];
        float wi[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = idx[u] >= 0;
            const T* row = Xb + (int64_t)(ok ? idx[u] : 0) * d;
            if constexpr (VEC) {
                raw[u] = (ok && active) ? __builtin_nontemporal_load((const u32x4*)(row + li * EPL))
                                        : u32x4{0u, 0u, 0u, 0u};
            } else {
#pragma unroll
                for (int t = 0; t < EPL; ++t) {
                    const int k = li + LPR * t;
                    vs[u][t] = (ok && k < d) ? ld_elem<T>(row + k) : 0.f;
                }
            }
            if constexpr (WEIGHTED) wi[u] = ok ? wb[idx[u]] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (idx[u] < 0) break;
            float v[EPL];
            if constexpr (VEC) unpack<T>(raw[u], v);
            else {
#pragma unroll
                for (int t = 0; t < EPL; ++t) v[t] = vs[u][t];
            }
#pragma unroll
            for (int t = 0; t < EPL; ++t) {
                if constexpr (WEIGHTED) acc[t] = fmaf(wi[u], v[t], acc[t]);
                else acc[t] += v[t];
            }
            if constexpr (WEIGHTED) wacc += wi[u];
        }
    }
    float* sj = sums + (b * K + j) * (int64_t)d;
    if (active) {
#pragma unroll
        for (int t = 0; t < EPL; ++t) {
            const int k = VEC ? li * EPL + t : li + LPR * t;
            if (k < d) sj[k] = acc[t];
        }
    }
    if constexpr (WEIGHTED) {
        if (li == 0) wsum[b * K + j] = wacc;
    }
}

int segreduce_tw(int64_t B, int64_t N) {
    int64_t tw = 256;
    while (tw < 4096 && B * N / (tw * 2) >= 8192) tw *= 2;
    // small jobs: shorter pieces, so that enough waves share the segments
    while (tw > 32 && B * N / tw < 2048) tw /= 2;
    return (int)tw;
}

// piece_seg: the first segment of every piece, written by the sort.
hipError_t launch_segreduce(DType xt, const void* x, const float* w, int64_t B, int64_t N, int d,
                            const int32_t* perm, const int32_t* offsets, int64_t K, float* sums,
                            float* wsum, const int32_t* piece_seg, float* slot, float* wslot, float* gslot,
                            float* gwslot, const int32_t* short_flag, hipStream_t s) {
    return launch_segreduce_tw(xt, x, w, B, N, d, perm, offsets, K, sums, wsum, piece_seg, slot, wslot, gslot,
                               gwslot, segreduce_tw(B, N), false, short_flag, s);
}

hipError_t launch_segreduce_tw(DType xt, const void* x, const float* w, int64_t B, int64_t N, int d,
                               const int32_t* perm, const int32_t* offsets, int64_t K, float* sums,
                               float* wsum, const int32_t* piece_seg, float* slot, float* wslot, float* gslot,
                               float* gwslot, int TW, bool accumulate, const int32_t* short_flag, hipStream_t s) {
    if (B == 0 || N == 0) return hipSuccess;
    if (accumulate) gslot = nullptr;
    // short segments on average: try the one-segment-per-row-group kernel
    // (it runs where the sort found every cluster short; the piece kernels
    // run elsewhere)
    const int32_t* skip = (short_flag && !accumulate && N <= kShortSegMean * K) ? short_flag : nullptr;
    const int64_t npieces = (N + TW - 1) / TW;
    const int esz = dtype_bytes(xt);
    const int epl = 16 / esz;
    const bool vec = (d % epl == 0) && ((uintptr_t)x % 16 == 0) && (d / epl <= 64);
    int lanes = vec ? d / epl : (d < 64 ? d : 64);
    int shift = 0;
    while ((1 << shift) < lanes) ++shift;
    if (skip) {
        const int64_t per_block = 4 * (64 >> shift);  // clusters per block: one per row group
        dim3 sgrid((unsigned)((K + per_block - 1) / per_block), (unsigned)B);
#define KM_SHORT(T, V, W)                                                                                   \
    hipLaunchKernelGGL((k_segsum_short<T, V, W>), sgrid, dim3(256), 0, s, (const T*)x, w, N, d, shift, perm, \
                       offsets, (int)K, short_flag, sums, wsum)
#define KM_SHORT_T(T)                     \
    if (vec) {                            \
        if (w) KM_SHORT(T, true, true);   \
        else KM_SHORT(T, true, false);    \
    } else {                              \
        if (w) KM_SHORT(T, false, true);  \
        else KM_SHORT(T, false, false);   \
    }
        if (xt == DType::F32) { KM_SHORT_T(float) }
        else if (xt == DType::F16) { KM_SHORT_T(_Float16) }
        else { KM_SHORT_T(bf16_t) }
#undef KM_SHORT_T
#undef KM_SHORT
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t ng = fold_groups(npieces);
    dim3 grid((unsigned)ng, (unsigned)B);
#define KM_SEG(T, V, W)                                                                                        \
    hipLaunchKernelGGL((k_segreduce<T, V, W>), grid, dim3(64 * kFoldG), 0, s, (const T*)x, w, N, d, shift, perm, \
                       offsets, piece_seg, npieces, (int)K, TW, sums, wsum, slot, wslot, accumulate, skip, ng,    \
                       gslot, gwslot)
#define KM_SEG_T(T)                      \
    if (vec) {                           \
        if (w) KM_SEG(T, true, true);    \
        else KM_SEG(T, true, false);     \
    } else {                             \
        if (w) KM_SEG(T, false, true);   \
        else KM_SEG(T, false, false);    \
    }
    if (xt == DType::F32) { KM_SEG_T(float) }
    else if (xt == DType::F16) { KM_SEG_T(_Float16) }
    else { KM_SEG_T(bf16_t) }
#undef KM_SEG_T
#undef KM_SEG
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the deterministic fold's group slots came with the reduction.  The
    // atomic fold stays a launch of its own: without `accumulate` the pieces
    // store the sums of the segments they start with plain stores, and a
    // slot's atomic add must not land before the plain store of its segment,
    // which another block makes (folding each block's slots at its end gave
    // wrong e-means sums in a test for exactly that reason)
    if (gslot) return hipSuccess;
    dim3 fgrid((unsigned)((npieces + 4 * kFoldG - 1) / (4 * kFoldG)), (unsigned)B);
    if (w)
        hipLaunchKernelGGL(k_fold_slots<true>, fgrid, dim3(256), 0, s, slot, wslot, piece_seg, offsets, npieces,
                           (int)K, TW, d, sums, wsum, skip);
    else
        hipLaunchKernelGGL(k_fold_slots<false>, fgrid, dim3(256), 0, s, slot, wslot, piece_seg, offsets, npieces,
                           (int)K, TW, d, sums, wsum, skip);
    return hipGetLastError();
}

int64_t segreduce_pieces(int64_t B, int64_t N) {
    const int TW = segreduce_tw(B, N);
    return (N + TW - 1) / TW;
}

// ---------------------------------------------------------------------------
// d == 1, whole row on chip.
constexpr int kRow1DMaxN = 8192;
constexpr int kRow1DMaxK = 256;

bool update_1d_row_fits(int64_t N, int64_t K) { return N <= kRow1DMaxN && K <= kRow1DMaxK; }

template <typename T>
__global__ __launch_bounds__(256) void k_update_1d_row(const T* __restrict__ X, const float* __restrict__ w,
                                                       int N, const int32_t* __restrict__ labels, int K,
                                                       const float* c_old, float* c_new,
                                                       int32_t* __restrict__ counts) {
    __shared__ int32_t s_cnt[kRow1DMaxK];
    __shared__ int32_t s_off[kRow1DMaxK + 1];
    __shared__ int32_t s_cur[kRow1DMaxK];
    __shared__ float s_x[kRow1DMaxN];
    __shared__ float s_w[kRow1DMaxN];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t b = blockIdx.x;
    const int32_t* L = labels + b * N;
    const T* Xb = X + b * N;
    for (int j = tid; j < K; j += 256) s_cnt[j] = 0;
    __syncthreads();
    for (int i = tid; i < N; i += 256) {
        const int32_t l = L[i];
        if ((uint32_t)l < (uint32_t)K) atomicAdd(&s_cnt[l], 1);
    }
    __syncthreads();
    if (tid == 0) {
        int32_t run = 0;
        for (int j = 0; j < K; ++j) {
            s_off[j] = run;
            s_cur[j] = run;
            run += s_cnt[j];
        }
        s_off[K] = run;
    }
    __syncthreads();
    // place (x, w) in cluster order
    for (int i = tid; i < N; i += 256) {
        const int32_t l = L[i];
        if ((uint32_t)l < (uint32_t)K) {
            const int32_t pos = atomicAdd(&s_cur[l], 1);
            s_x[pos] = ld_elem<T>(Xb + i);
            s_w[pos] = w ? w[b * N + i] : 1.f;
        }
    }
    __syncthreads();
    // one wave per segment: float64 sums (order-insensitive to float32 output precision)
    for (int j = wave; j < K; j += 4) {
        const int32_t lo = s_off[j], hi = s_off[j + 1];
        double S = 0.0, W = 0.0;
        for (int32_t r = lo + lane; r < hi; r += 64) {
            const double wi = s_w[r];
            S += wi * (double)s_x[r];
            W += wi;
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            S += __shfl_xor(S, o, 64);
            W += __shfl_xor(W, o, 64);
        }
        if (lane == 0) {
            const int32_t n = hi - lo;
            c_new[b * K + j] = n > 0 ? (float)(S / W) : c_old[b * K + j];
            if (counts) counts[b * K + j] = n;
        }
    }
}

// d == 1, K <= KC <= 16, rows of up to kUpd1DFewMaxN points with N % 4 == 0
// and four-element-aligned rows: one wave per row.  Each lane adds its points
// into its own bins in LDS (bin j of lane l at [j][l]: the 64 lanes of one
// add cover consecutive 8-byte words, so an add touches every bank the same
// number of times whatever the labels), with adds that return nothing; no
// other lane touches those words, so the adds of one point never wait on
// another's.  Labels outside [0, K) add nothing.
constexpr int kUpd1DFewMaxN = 16384;
constexpr int kUpd1DGroups = 4;

template <typename T, int KC, bool WEIGHTED>
__global__ __launch_bounds__(64) void k_update_1d_few(const T* __restrict__ X, const float* __restrict__ w,
                                                      int N, const int32_t* __restrict__ labels, int K,
                                                      const float* c_old, float* c_new,
                                                      int32_t* __restrict__ counts) {
    constexpr int G = kUpd1DGroups, P = 4 * G;
    __shared__ double s_S[KC][64];                 // sum of w * x
    __shared__ double s_W[WEIGHTED ? KC : 1][64];  // sum of w (weighted rows)
    __shared__ int32_t s_N[KC][64];                // number of points
    const int lane = threadIdx.x;
    const int64_t b = blockIdx.x;
    const T* Xb = X + b * N;
    const int32_t* Lb = labels + b * N;
    const float* wb = WEIGHTED ? w + b * N : nullptr;
#pragma unroll
    for (int j = 0; j < KC; ++j) {
        s_S[j][lane] = 0.0;
        if constexpr (WEIGHTED) s_W[j][lane] = 0.0;
        s_N[j][lane] = 0;
    }

    auto load = [&](int g0, float (&xv)[P], float (&wv)[P], int (&lv)[P]) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int i = g0 + g * 256 + lane * 4;
            float xq[4] = {0.f, 0.f, 0.f, 0.f}, wq[4] = {1.f, 1.f, 1.f, 1.f};
            int lq[4] = {-1, -1, -1, -1};
            if (i < N) {  // N and i are multiples of 4: the four points are in the row
                typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
                const i32x4 l4 = __builtin_nontemporal_load((const i32x4*)(Lb + i));
                lq[0] = l4[0], lq[1] = l4[1], lq[2] = l4[2], lq[3] = l4[3];
                f1_load4<T>(Xb + i, xq);
                if constexpr (WEIGHTED) f1_load4<float>(wb + i, wq);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) xv[4 * g + e] = xq[e], wv[4 * g + e] = wq[e], lv[4 * g + e] = lq[e];
        }
    };

    float xa[P], wa[P];
    int la[P];
    load(0, xa, wa, la);
    f1_wave_sync();  // bins cleared
    for (int g0 = 0; g0 < N; g0 += 256 * G) {
        float xn[P], wn[P];
        int ln[P];
        if (g0 + 256 * G < N) load(g0 + 256 * G, xn, wn, ln);
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const int l = la[j];
            if ((uint32_t)l < (uint32_t)K) {
                if constexpr (WEIGHTED) {
                    atomicAdd(&s_S[l][lane], (double)wa[j] * (double)xa[j]);
                    atomicAdd(&s_W[l][lane], (double)wa[j]);
                } else {
                    atomicAdd(&s_S[l][lane], (double)xa[j]);
                }
                atomicAdd(&s_N[l][lane], 1);
            }
        }
#pragma unroll
        for (int j = 0; j < P; ++j) xa[j] = xn[j], wa[j] = wn[j], la[j] = ln[j];
    }
    f1_wave_sync();
    // lane (r, part) adds the bins of cluster r of lanes part*KC .. +KC (the
    // walk starts at a different lane per r, so the reads spread over the
    // banks), then exchanges combine the parts
    const int r = lane % KC, part = lane / KC;
    double S = 0.0, W = 0.0;
    int n = 0;
#pragma unroll
    for (int q = 0; q < KC; ++q) {
        const int l = part * KC + ((q + r) & (KC - 1));
        S += s_S[r][l];
        if constexpr (WEIGHTED) W += s_W[r][l];
        n += s_N[r][l];
    }
#pragma unroll
    for (int o = KC; o < 64; o <<= 1) {
        S += __shfl_xor(S, o, 64);
        if constexpr (WEIGHTED) W += __shfl_xor(W, o, 64);
        n += __shfl_xor(n, o, 64);
    }
    if constexpr (!WEIGHTED) W = (double)n;
    if (part == 0 && r < K) {
        c_new[b * K + r] = n > 0 ? (float)(S / W) : c_old[b * K + r];
        counts[b * K + r] = n;
    }
}

bool update_1d_few_fits(DType xt, const void* x, const float* w, const int32_t* labels, int64_t N, int64_t K) {
    const size_t eb = xt == DType::F32 ? 16 : 8;
    return N <= kUpd1DFewMaxN && N % 4 == 0 && K <= kFit1DMaxK && (uintptr_t)x % eb == 0 &&
           (uintptr_t)labels % 16 == 0 && (uintptr_t)w % 16 == 0;
}

hipError_t launch_update_1d_row(DType xt, const void* x, const float* w, int64_t B, int64_t N,
                                const int32_t* labels, int64_t K, const float* c_old, float* c_new,
                                int32_t* counts, hipStream_t s) {
    if (B == 0) return hipSuccess;
    if (update_1d_few_fits(xt, x, w, labels, N, K)) {
#define KM_U1F(TT, KK)                                                                                        \
    do {                                                                                                      \
        if (w)                                                                                                \
            hipLaunchKernelGGL((k_update_1d_few<TT, KK, true>), dim3((unsigned)B), dim3(64), 0, s,            \
                               (const TT*)x, w, (int)N, labels, (int)K, c_old, c_new, counts);                \
        else                                                                                                  \
            hipLaunchKernelGGL((k_update_1d_few<TT, KK, false>), dim3((unsigned)B), dim3(64), 0, s,           \
                               (const TT*)x, w, (int)N, labels, (int)K, c_old, c_new, counts);                \
    } while (0)
#define KM_U1F_T(TT)              \
    if (K <= 4) KM_U1F(TT, 4);     \
    else if (K <= 8) KM_U1F(TT, 8); \
    else KM_U1F(TT, 16);
        if (xt == DType::F32) { KM_U1F_T(float) }
        else if (xt == DType::F16) { KM_U1F_T(_Float16) }
        else { KM_U1F_T(bf16_t) }
#undef KM_U1F_T
#undef KM_U1F
        return hipGetLastError();
    }
    if (!update_1d_row_fits(N, K)) return hipErrorInvalidValue;
    if (xt == DType::F32)
        hipLaunchKernelGGL(k_update_1d_row<float>, dim3((unsigned)B), dim3(256), 0, s, (const float*)x, w,
                           (int)N, labels, (int)K, c_old, c_new, counts);
    else if (xt == DType::F16)
        hipLaunchKernelGGL(k_update_1d_row<_Float16>, dim3((unsigned)B), dim3(256), 0, s, (const _Float16*)x,
                           w, (int)N, labels, (int)K, c_old, c_new, counts);
    else
        hipLaunchKernelGGL(k_update_1d_row<bf16_t>, dim3((unsigned)B), dim3(256), 0, s, (const bf16_t*)x, w,
                           (int)N, labels, (int)K, c_old, c_new, counts);
    return hipGetLastError();
}

}  // namespace km
