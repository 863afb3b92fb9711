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
//      lane touches).  The block kernel also adds w * (x - v)^2 into an
//      objective partial; the wave kernel takes the objective from the
//      row's sum of w x^2 and the per-rank sums instead.
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
constexpr int kRankBuckets = 256;         // buckets of the rank table (the values of a byte)

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
// the point work of the other rows on the CU.  KC: the most ranks a row can
// have (K <= KC).
//
// A point's rank comes from a table instead of a compare per threshold:
// kRankBuckets buckets of equal width between the first and the last
// threshold, with bucket(x) monotone in x (float32 multiply-add, then a
// saturating conversion to a byte).  A threshold in a lower bucket than x's is below x and one in a
// higher bucket is above it.  So with c the count of thresholds in buckets
// below x's, the rank of x is c plus one compare with threshold c (the one
// in x's bucket if there is one, else a higher one, or +inf): an entry holds
// threshold c and c.  The table is built from a mark per threshold in its
// bucket and a count of the marks below each bucket (ballots).  An iteration
// whose thresholds put two in one bucket counts compares instead.
//
// Each lane adds w*x and w of its points, in float64, into its own per-rank
// bins ([rank][lane] doubles, so the 64 lanes of one add hit distinct banks
// whatever the ranks).  The objective sum w (x - v)^2 of an assignment is
// sum w x^2 (the same for every assignment) minus sum_r v_r (2 S_r - v_r W_r)
// over the ranks, in float64.
template <typename T, int PPT, int KC>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void k_fit_1d_wave(
    const T* __restrict__ X, const float* __restrict__ w, int N, const float* __restrict__ init, int K,
    int n_iter, float* __restrict__ centroids, int32_t* __restrict__ labels, int32_t* __restrict__ counts,
    double* __restrict__ objective) {
    static_assert(KC >= 2 && KC <= kFit1DMaxK && (KC & (KC - 1)) == 0, "KC: a power of two up to the rank limit");
    static_assert(kRankBuckets == 4 * 64, "each lane builds four consecutive table entries");
    constexpr int NT = KC - 1;                          // thresholds at most
    constexpr int kRow = 64 * (int)sizeof(double);      // bytes of one rank's bins
    __shared__ float s_c[kFit1DMaxK];
    __shared__ float s_val[kFit1DMaxK];
    __shared__ int s_idx[kFit1DMaxK];
    __shared__ float s_thr[kFit1DMaxK];
    // per-lane bins per rank, S_r = sum w x in s_bin[0] and W_r = sum w in
    // s_bin[1]: a row is 64 doubles, so the bank of a bin depends on its lane
    // alone and the lanes' adds never conflict
    __shared__ double s_bin[2][KC][64];
    __shared__ float2 s_tab[kRankBuckets];  // (threshold c, c as the byte offset of its bin row)
    __shared__ uint32_t s_hit[kRankBuckets / 4];  // a byte per bucket: 1 where a threshold falls
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
    s_hit[lane] = 0u;
#pragma unroll
    for (int r = 0; r < KC; ++r) s_bin[0][r][lane] = s_bin[1][r][lane] = 0.0;
    // sum w x^2 over the row
    double qtot = 0.0;
#pragma unroll
    for (int p = 0; p < PPT; ++p) qtot += ((double)ws[p] * (double)xs[p]) * (double)xs[p];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) qtot += __shfl_xor(qtot, o, 64);
    wave_sync();

    int A = 0;
    bool tab_ok = false;  // the table holds the last assignment's ranks
    float scale = 0.f, bias = 0.f;
    // monotone in x (any monotone map serves: the table is built with the
    // same one): the float32 multiply-add, converted to an unsigned byte with
    // rounding to nearest even and saturation (NaN to 0), so every result is
    // an entry of the table
    static_assert(kRankBuckets == 256, "bucket() yields a byte");
    auto bucket = [&](float x) { return (int)__builtin_amdgcn_cvt_pk_u8_f32(fmaf(x, scale, bias), 0, 0); };
    for (int t = 0; t < n_iter; ++t) {
        // the empty asm hides that the points do not change between
        // iterations, so their float64 forms are not kept live across them
#pragma unroll
        for (int p = 0; p < PPT; ++p) asm volatile("" : "+v"(xs[p]), "+v"(ws[p]));
        A = f1_thresholds<T>(s_c, K, lane, s_val, s_idx, s_thr);
        wave_sync();
        // the thresholds are the same in every lane: held in scalar registers
        float tr[NT];
        f1_scalar_thresholds(s_thr, tr);
        const int nt = A - 1;
        const float lo = tr[0], hi = nt >= 1 ? s_thr[nt - 1] : lo;
        scale = (nt >= 2 && hi > lo) ? (float)(kRankBuckets - 1) / (hi - lo) : 0.f;
        bias = -lo * scale;
        // lane a < nt: the bucket of threshold a, and whether threshold a - 1
        // shares it
        const int bt = lane < nt ? bucket(s_thr[lane]) : 0;
        const bool coll = __ballot(lane >= 1 && lane < nt && bt == bucket(s_thr[lane - 1 < 0 ? 0 : lane - 1])) != 0;
        tab_ok = !coll;
        if (!coll) {
            if (lane < nt) ((unsigned char*)s_hit)[bt] = 1;
            wave_sync();
            const uint32_t h = s_hit[lane];  // the marks of buckets 4 lane .. 4 lane + 3
            s_hit[lane] = 0u;                // cleared for the next table
            const uint64_t below_lanes = (1ull << lane) - 1ull;
            int c = 0;  // marks in the buckets of lower lanes
#pragma unroll
            for (int j = 0; j < 4; ++j) c += __popcll(__ballot((h >> (8 * j)) & 1u) & below_lanes);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s_tab[4 * lane + j] = make_float2(s_thr[c], __int_as_float(c * kRow));  // c <= nt: s_thr[nt] is +inf
                c += (h >> (8 * j)) & 1u;
            }
        }
        wave_sync();
        // off: the byte offset of this lane's bin of rank m, m kRow + 8 lane;
        // this lane's own bins, adds that return nothing: no point waits on
        // another
        const int lane8 = lane * (int)sizeof(double);
        auto add = [&](int off, float xv, float wv) {
            const double wd = (double)wv;
            double* bin = (double*)((char*)&s_bin[0][0][0] + off);
            atomicAdd(bin, wd * (double)xv);
            atomicAdd(bin + KC * 64, wd);
        };
        // groups of 16 points: their ranks first (the table reads overlap
        // instead of each waiting in turn), then their adds
        constexpr int G = 16;
#pragma unroll
        for (int p0 = 0; p0 < PPT; p0 += G) {
            int off[G];
            if (!coll) {
                float2 e[G];
#pragma unroll
                for (int j = 0; j < G; ++j) e[j] = s_tab[bucket(xs[p0 + j])];
#pragma unroll
                for (int j = 0; j < G; ++j)
                    off[j] = __float_as_int(e[j].y) + (xs[p0 + j] >= e[j].x ? kRow : 0) + lane8;
            } else {
#pragma unroll
                for (int j = 0; j < G; ++j) off[j] = f1_rank_cmp(xs[p0 + j], tr) * kRow + lane8;
            }
#pragma unroll
            for (int j = 0; j < G; ++j) add(off[j], xs[p0 + j], ws[p0 + j]);
            __builtin_amdgcn_sched_barrier(0);  // one group of points in flight at a time
        }
        wave_sync();
        // per-rank sums: lane (r, part) takes the bins of rank r of lanes
        // part*KC .. +KC, clearing them for the next iteration in the same
        // exchange, and shuffles combine the parts.  Lane r starts at column
        // r of its part, so each exchange of the wave touches 64 distinct
        // columns.
        const int r = lane % KC, part = lane / KC;
        double S = 0.0, W = 0.0;
#pragma unroll
        for (int q = 0; q < KC; ++q) {
            const int c = part * KC + ((q + r) & (KC - 1));
            S += __longlong_as_double((long long)atomicExch((unsigned long long*)&s_bin[0][r][c], 0ull));
            W += __longlong_as_double((long long)atomicExch((unsigned long long*)&s_bin[1][r][c], 0ull));
        }
#pragma unroll
        for (int o = KC; o < 64; o <<= 1) {
            S += __shfl_xor(S, o, 64);
            W += __shfl_xor(W, o, 64);
        }
        // the objective's share of rank r with value v: v (2 S - v W)
        const double v = r < A ? (double)s_val[r] : 0.0;
        double J = r < A ? v * (2.0 * S - v * W) : 0.0;
#pragma unroll
        for (int o = 1; o < KC; o <<= 1) J += __shfl_xor(J, o, 64);
        if (lane < A && W > 0.0) s_c[s_idx[lane]] = (float)(S / W);
        if (lane == 0 && objective) objective[b * n_iter + t] = qtot - J;
        wave_sync();
    }
    // labels and counts of the last assignment: s_thr, s_val, s_idx, s_tab,
    // scale and bias still hold that iteration's values (only s_c has moved
    // on).  The bins are all zero again: per-lane counts go there.
    if (n_iter > 0) {
        int* cbin = (int*)&s_bin[0][0][0];  // [rank][lane]
        float tr[NT];
        f1_scalar_thresholds(s_thr, tr);
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            const int i = p * 64 + lane;
            int m;
            if (tab_ok) {
                const float2 e = s_tab[bucket(xs[p])];
                m = __float_as_int(e.y) / kRow + (xs[p] >= e.x ? 1 : 0);
            } else {
                m = f1_rank_cmp(xs[p], tr);
            }
            if (i < N) {
                if (labels) labels[b * N + i] = s_idx[m];
                atomicAdd(&cbin[m * 64 + lane], 1);
            }
        }
        wave_sync();
        const int r = lane % KC, part = lane / KC;
        int c = 0;
#pragma unroll
        for (int q = 0; q < KC; ++q) c += cbin[r * 64 + part * KC + ((q + r) & (KC - 1))];
#pragma unroll
        for (int o = KC; o < 64; o <<= 1) c += __shfl_xor(c, o, 64);
        if (lane < KC) s_cnt[lane] = c;
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
#define KM_FW(TT, PP)                                                                                     \
    do {                                                                                                      \
        if (K <= 8)                                                                                           \
            hipLaunchKernelGGL((k_fit_1d_wave<TT, PP, 8>), grid, dim3(64), 0, s, (const TT*)x, w, (int)N, init, \
                               (int)K, n_iter, centroids, labels, counts, objective);                         \
        else                                                                                                  \
            hipLaunchKernelGGL((k_fit_1d_wave<TT, PP, 16>), grid, dim3(64), 0, s, (const TT*)x, w, (int)N,     \
                               init, (int)K, n_iter, centroids, labels, counts, objective);                   \
    } while (0)
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
