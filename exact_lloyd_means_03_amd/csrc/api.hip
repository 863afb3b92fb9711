// Host side of the C ABI declared in include/kmeans.h: argument checks,
// the workspace plan and the per-iteration kernel sequence.  Every check
// happens before the first enqueue; nothing here allocates device memory or
// synchronizes the stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>
#include <string>

#include "../../include/kmeans.h"
#include "common.h"

namespace km {

static thread_local std::string g_last_error;

static km_status fail(km_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
static km_status fail(km_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

static km_status hip_fail(hipError_t e, const char* where) {
    return fail(KM_EHIP, "%s: %s", where, hipGetErrorString(e));
}

static size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

static bool use_assign_1d(int64_t d, int64_t K) { return d == 1 && assign_1d_supports(K); }
static bool use_update_1d(DType xt, const void* x, const float* w, const int32_t* labels, int64_t d, int64_t N,
                          int64_t K) {
    return d == 1 && (update_1d_row_fits(N, K) || update_1d_few_fits(xt, x, w, labels, N, K));
}

Workspace plan_workspace(int64_t B, int64_t N, int64_t d, int64_t K, DType xt) {
    Workspace w{};
    w.DP = padded_dim(d, xt != DType::F32);
    w.Kp = padded_k(K);
    const bool a1d = use_assign_1d(d, K);
    w.nblk_assign = a1d ? assign_1d_blocks(N) : assign_mfma_blocks(B, N, w.DP, xt, w.Kp);
    if (w.nblk_assign < 1) w.nblk_assign = 1;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align_up(bytes);
        return at;
    };
    const size_t Bz = (size_t)B;
    w.chat = take(a1d ? 0 : Bz * (w.Kp / tile_rows(w.DP, dtype_bytes(xt))) *
                                (size_t)tile_bytes(w.DP, dtype_bytes(xt)));
    w.obj_part = take(Bz * w.nblk_assign * sizeof(double));
    w.split = take(a1d ? 0 : assign_mfma_scratch_bytes(B, N, w.DP, xt, w.Kp));
    w.seg_short = take(Bz * sizeof(int32_t));
    w.labels = take(Bz * N * sizeof(int32_t));
    w.counts = take(Bz * K * sizeof(int32_t));
    w.sums = take(Bz * K * d * sizeof(float));
    w.wsum = take(Bz * K * sizeof(float));
    w.offsets = take(Bz * (K + 1) * sizeof(int32_t));
    w.cursor = take(Bz * K * sizeof(int32_t));
    w.perm = take(Bz * N * sizeof(int32_t));
    const size_t np = (size_t)segreduce_pieces(B, N);
    w.piece_seg = take(Bz * np * sizeof(int32_t));
    w.slot = take(Bz * np * d * sizeof(float));
    w.wslot = take(Bz * np * sizeof(float));
    const size_t ng = (size_t)fold_groups((int64_t)np);
    w.gslot = take(Bz * ng * d * sizeof(float));
    w.gwslot = take(Bz * ng * sizeof(float));
    const size_t nch = (size_t)sort_chunks(B, N, K);
    w.hist = take(Bz * nch * K * sizeof(int32_t));
    w.prefix = take(Bz * nch * K * sizeof(int32_t));
    w.total = off;
    return w;
}

}  // namespace km

using namespace km;

namespace {

// The code of an enum argument as the caller passed it: a C caller may pass
// any int, and reading a value outside the enumerators through the enum type
// is undefined, so the bytes are read as an int.
template <typename E>
int enum_code(const E& e) {
    static_assert(sizeof(E) == sizeof(int), "enums of the ABI are int-sized");
    int v;
    memcpy(&v, &e, sizeof v);
    return v;
}

constexpr int64_t kMaxD = 512;     // 16-bit points
constexpr int64_t kMaxDF32 = 256;  // float32 points
constexpr int64_t kMaxK = 32768;
constexpr int64_t kMaxB = 65535;
constexpr int64_t kMaxN = 0x7fffffff;

km_status check_shape(int64_t B, int64_t N, int64_t d, int64_t K, int xt) {
    if (B < 0 || N < 0) return fail(KM_EINVAL, "negative size: B=%lld N=%lld", (long long)B, (long long)N);
    if (d < 1 || K < 1) return fail(KM_EINVAL, "d and K must be >= 1 (d=%lld K=%lld)", (long long)d, (long long)K);
    if (xt != KM_F32 && xt != KM_F16 && xt != KM_BF16) return fail(KM_EUNSUPPORTED, "unknown dtype %d", xt);
    if (d > kMaxD) return fail(KM_EUNSUPPORTED, "d=%lld > %lld is not supported", (long long)d, (long long)kMaxD);
    if (xt == KM_F32 && d > kMaxDF32)
        return fail(KM_EUNSUPPORTED, "d=%lld > %lld is not supported for float32 points", (long long)d,
                    (long long)kMaxDF32);
    if (K > kMaxK) return fail(KM_EUNSUPPORTED, "K=%lld > %lld is not supported", (long long)K, (long long)kMaxK);
    if (B > kMaxB) return fail(KM_EUNSUPPORTED, "B=%lld > %lld is not supported", (long long)B, (long long)kMaxB);
    if (N > kMaxN) return fail(KM_EUNSUPPORTED, "N=%lld >= 2^31 is not supported", (long long)N);
    int64_t bn, bnd;
    if (__builtin_mul_overflow(B, N, &bn) || __builtin_mul_overflow(bn, d, &bnd) || bnd > ((int64_t)1 << 46))
        return fail(KM_EUNSUPPORTED, "B*N*d too large");
    return KM_OK;
}

// Scalar points are always assigned by the binary search: the expanded form
// ||x||^2 - 2xc + c^2 cancels catastrophically when many centroids are packed
// closely on a line.
km_status check_scalar_k(int64_t d, int64_t K) {
    if (d == 1 && !assign_1d_supports(K))
        return fail(KM_EUNSUPPORTED, "d=1 assignment supports K <= 16384 (K=%lld)", (long long)K);
    return KM_OK;
}

km_status need(const void* p, int64_t n, const char* name) {
    if (n > 0 && p == nullptr) return fail(KM_EINVAL, "%s is NULL", name);
    return KM_OK;
}

km_status check_ws(const Workspace& w, const void* ws, size_t bytes) {
    if (w.total == 0) return KM_OK;
    if (ws == nullptr) return fail(KM_EINVAL, "workspace is NULL (%zu bytes needed)", w.total);
    if ((uintptr_t)ws % 256 != 0) return fail(KM_EINVAL, "workspace must be 256-byte aligned");
    if (bytes < w.total)
        return fail(KM_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", bytes, w.total);
    return KM_OK;
}

#define KM_TRY(expr)                       \
    do {                                   \
        km_status _st = (expr);            \
        if (_st != KM_OK) return _st;      \
    } while (0)

#define KM_HIP(expr, where)                              \
    do {                                                 \
        hipError_t _e = (expr);                          \
        if (_e != hipSuccess) return hip_fail(_e, where); \
    } while (0)

template <typename P>
P* at(void* ws, size_t off) {
    return (P*)((char*)ws + off);
}

// Assignment of all B*N points against C; optional per-block objective
// partials reduced into obj_out[b * obj_stride].  prep = false: the tile
// blob already holds C (written by the previous update's fused divide).
// ev_begin / ev_end (may be NULL): recorded on s right before and right after
// the assignment kernel launches (after the prep, before the objective
// reduction).  reduce_obj = false: leave the partials in W.obj_part for the
// sort's column scan to sum (matrix-core path with N > 0 only).
km_status run_assign(const void* x, DType xt, int64_t B, int64_t N, int64_t d, const float* C, int64_t K,
                     const float* w, int32_t* labels, float* min_dist, double* obj_out, int64_t obj_stride,
                     const Workspace& W, void* ws, hipStream_t s, bool prep = true, hipEvent_t ev_begin = nullptr,
                     hipEvent_t ev_end = nullptr, int32_t* hist = nullptr, bool reduce_obj = true) {
    double* part = obj_out ? at<double>(ws, W.obj_part) : nullptr;
    if (use_assign_1d(d, K)) {
        if (ev_begin) KM_HIP(hipEventRecord(ev_begin, s), "event");
        if (obj_out && N > 0 && W.nblk_assign == 1) {
            // one partial per row: it is the row's objective, written in place
            KM_HIP(launch_assign_1d(xt, x, B, N, C, K, w, labels, min_dist, obj_out, obj_stride, 1, s),
                   "assign_1d");
            if (ev_end) KM_HIP(hipEventRecord(ev_end, s), "event");
            return KM_OK;
        }
        KM_HIP(launch_assign_1d(xt, x, B, N, C, K, w, labels, min_dist, part, W.nblk_assign, W.nblk_assign, s),
               "assign_1d");
    } else {
        void* blob = at<void>(ws, W.chat);
        if (prep) KM_HIP(launch_prep(xt, C, B, K, (int)d, W.DP, W.Kp, blob, s), "prep");
        if (ev_begin) KM_HIP(hipEventRecord(ev_begin, s), "event");
        KM_HIP(launch_assign_mfma(xt, x, B, N, (int)d, W.DP, blob, W.Kp, w, labels, min_dist, part,
                                  W.nblk_assign, at<void>(ws, W.split), s, nullptr, K, hist),
               "assign_mfma");
    }
    if (ev_end) KM_HIP(hipEventRecord(ev_end, s), "event");
    if (obj_out && reduce_obj) {
        if (N == 0) {
            KM_HIP(launch_zero(part, (size_t)B * W.nblk_assign * sizeof(double), s), "zero");
        }
        KM_HIP(launch_obj_reduce(part, B, W.nblk_assign, obj_out, obj_stride, s), "obj_reduce");
    }
    return KM_OK;
}

// The stable argsort of the labels (histogram rows in W.hist / W.prefix).
// piece_seg (may be NULL): also record the first segment of every reduction
// piece; short_flag (may be NULL): also flag the problems whose clusters are
// all short enough for the one-segment-per-row-group reduction.  counted:
// the assignment already built the histogram rows.
// obj_out (may be NULL): the column scan also sums the assignment's objective
// partials left in W.obj_part into obj_out[b * obj_stride].
km_status run_sort(const int32_t* labels, int64_t B, int64_t N, int64_t K, int32_t* counts, int32_t* offsets,
                   int32_t* perm, int32_t* piece_seg, int32_t* short_flag, const Workspace& W, void* ws,
                   hipStream_t s, bool counted = false, double* obj_out = nullptr, int64_t obj_stride = 0) {
    SortBufs o{counts, offsets, perm, at<int32_t>(ws, W.hist), at<int32_t>(ws, W.prefix), nullptr, piece_seg,
               short_flag};
    if (obj_out) {
        o.obj_part = at<double>(ws, W.obj_part);
        o.obj_nblk = W.nblk_assign;
        o.obj_out = obj_out;
        o.obj_stride = obj_stride;
    }
    KM_HIP(launch_sort(labels, B, N, K, o, segreduce_tw(B, N), segreduce_pieces(B, N), s,
                       counted ? SortMode::StableCounted : SortMode::Stable),
           "sort");
    return KM_OK;
}

// prep_next: also write c_new to the tile blob for the next assignment
// (the divide fused with the prep; matrix-core path only).
km_status run_update(const void* x, DType xt, const float* w, int64_t B, int64_t N, int64_t d,
                     const int32_t* labels, int64_t K, const float* c_old, float* c_new, int32_t* counts,
                     const Workspace& W, void* ws, hipStream_t s, bool prep_next = false, bool counted = false,
                     double* obj_out = nullptr, int64_t obj_stride = 0) {
    int32_t* cnt = counts ? counts : at<int32_t>(ws, W.counts);
    if (use_update_1d(xt, x, w, labels, d, N, K)) {
        KM_HIP(launch_update_1d_row(xt, x, w, B, N, labels, K, c_old, c_new, cnt, s), "update_1d_row");
        return KM_OK;
    }
    // no clearing: every non-empty cluster's sum is stored once before the
    // fold adds its slots, and empty clusters' sums are never read
    float* sums = at<float>(ws, W.sums);
    float* wsum = w ? at<float>(ws, W.wsum) : nullptr;
    int32_t* offsets = at<int32_t>(ws, W.offsets);
    int32_t* perm = at<int32_t>(ws, W.perm);
    int32_t* piece_seg = at<int32_t>(ws, W.piece_seg);
    int32_t* short_flag = at<int32_t>(ws, W.seg_short);
    KM_TRY(run_sort(labels, B, N, K, cnt, offsets, perm, piece_seg, short_flag, W, ws, s, counted, obj_out,
                    obj_stride));
    float* slot = at<float>(ws, W.slot);
    float* wslot = w ? at<float>(ws, W.wslot) : nullptr;
    float* gslot = at<float>(ws, W.gslot);
    float* gwslot = w ? at<float>(ws, W.gwslot) : nullptr;
    KM_HIP(launch_segreduce(xt, x, w, B, N, (int)d, perm, offsets, K, sums, wsum, piece_seg, slot, wslot, gslot,
                            gwslot, short_flag, s),
           "segreduce");
    void* blob = (prep_next && !use_assign_1d(d, K)) ? at<void>(ws, W.chat) : nullptr;
    KM_HIP(launch_fold_divide(xt, sums, wsum, slot, wslot, gslot, gwslot, offsets, cnt,
                              N <= kShortSegMean * K ? short_flag : nullptr, segreduce_pieces(B, N),
                              segreduce_tw(B, N), B, K, (int)d, W.DP, W.Kp, c_old, c_new, blob, s),
           "fold_divide");
    return KM_OK;
}

// ---------------------------------------------------------------------------
// Fits of one problem whose points stay in host memory (technologypulse.uk
// "Flash-KMeans" article, performance section: out-of-core runs in which a
// chunked stream overlap hides the PCIe transfers; wispaper.ai blog,
// performance: up to a billion points by overlapping CPU-to-GPU copies with
// computation).  Every iteration streams the points through two device
// buffers: chunk g is copied on a copy stream while chunk g - 1 is assigned
// and reduced on the caller's stream; sums, weight sums and counts
// accumulate over the chunks and the divide closes the iteration.

constexpr int64_t kStreamAlign = 4096;  // chunk sizes: a multiple of every assignment group size

struct StreamPlan {
    Workspace chunk;  // the per-chunk plan (B = 1, N = chunk points)
    int64_t chunk_n = 0, nchunks = 0, nblk_chunk = 0, nblk_total = 0;
    size_t xbuf[2] = {0, 0}, wbuf[2] = {0, 0}, obj_all = 0, counts_total = 0, split = 0, total = 0;
};

StreamPlan plan_stream(int64_t N, int64_t d, int64_t K, DType xt, int64_t chunk) {
    StreamPlan p;
    int64_t c = (chunk + kStreamAlign - 1) / kStreamAlign * kStreamAlign;
    if (c > N) c = N;
    if (c < 1) c = 1;
    p.chunk_n = c;
    p.nchunks = N > 0 ? (N + c - 1) / c : 0;
    p.chunk = plan_workspace(1, c, d, K, xt);
    p.nblk_chunk = p.chunk.nblk_assign;
    const int64_t last = N - (p.nchunks > 0 ? (p.nchunks - 1) * c : 0);
    const int64_t nblk_last = p.nchunks > 0 ? assign_mfma_blocks(1, last, p.chunk.DP, xt, p.chunk.Kp) : 0;
    p.nblk_total = p.nchunks > 0 ? (p.nchunks - 1) * p.nblk_chunk + nblk_last : 1;
    size_t off = p.chunk.total;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align_up(bytes);
        return at;
    };
    for (int i = 0; i < 2; ++i) p.xbuf[i] = take((size_t)c * d * dtype_bytes(xt));
    for (int i = 0; i < 2; ++i) p.wbuf[i] = take((size_t)c * sizeof(float));
    p.obj_all = take((size_t)p.nblk_total * sizeof(double));
    p.counts_total = take((size_t)K * sizeof(int32_t));
    // assignment scratch of a full and of the last chunk (a short last chunk
    // may cut the centroids into slices where a full one does not)
    const size_t sc = assign_mfma_scratch_bytes(1, c, p.chunk.DP, xt, p.chunk.Kp),
                 sl = p.nchunks > 0 ? assign_mfma_scratch_bytes(1, last, p.chunk.DP, xt, p.chunk.Kp) : 0;
    p.split = take(sc > sl ? sc : sl);
    p.total = off;
    return p;
}

// The copy stream of a device and the events that order its copies against
// the caller's stream (created once per device, default priority).  Calls on
// one device take the lock for as long as they enqueue work.
struct StreamRes {
    hipStream_t copy = nullptr;
    hipEvent_t copied[2] = {nullptr, nullptr}, consumed[2] = {nullptr, nullptr}, start = nullptr;
};
std::mutex g_stream_mu;
std::map<int, StreamRes> g_stream_res;

hipError_t stream_res(int dev, StreamRes** out) {
    auto it = g_stream_res.find(dev);
    if (it != g_stream_res.end()) {
        *out = &it->second;
        return hipSuccess;
    }
    StreamRes r;
    hipError_t e = hipStreamCreateWithFlags(&r.copy, hipStreamNonBlocking);
    for (int i = 0; i < 2 && e == hipSuccess; ++i) e = hipEventCreateWithFlags(&r.copied[i], hipEventDisableTiming);
    for (int i = 0; i < 2 && e == hipSuccess; ++i) e = hipEventCreateWithFlags(&r.consumed[i], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&r.start, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    *out = &(g_stream_res[dev] = r);
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// e-means (daily.steinslab.io "e-means" article): mini-batches of
// consecutive points, each assigned against the current centroids by the
// Lloyd assignment and reduced into per-cluster sums and counts by the
// Lloyd sort and segmented reduction; a float64 moving average of those
// statistics then moves the centroids, dead clusters are split from live
// ones, and after the last epoch every centroid becomes that epoch's plain
// mean.

struct EmeansPlan {
    Workspace batch;  // the per-batch plan (B = 1, N = batch points)
    int64_t mfull = 0, nb = 0, steps = 0;
    size_t S = 0, Nc = 0, F = 0, G = 0, list_j = 0, list_k = 0, obj_part = 0, split = 0, total = 0;
};

EmeansPlan plan_emeans(int64_t N, int64_t d, int64_t K, DType xt, int64_t batch, int32_t epochs) {
    EmeansPlan p;
    p.mfull = batch < N ? batch : N;
    p.nb = N > 0 ? (N + batch - 1) / batch : 0;
    p.steps = p.nb * epochs;
    p.batch = plan_workspace(1, p.mfull > 0 ? p.mfull : 1, d, K, xt);
    size_t off = p.batch.total;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align_up(bytes);
        return at;
    };
    p.S = take((size_t)K * d * sizeof(double));
    p.Nc = take((size_t)K * sizeof(double));
    p.F = take((size_t)K * d * sizeof(double));
    p.G = take((size_t)K * sizeof(double));
    p.list_j = take((size_t)K * sizeof(int32_t));
    p.list_k = take((size_t)K * sizeof(int32_t));
    // objective partials of one batch's assignment: a shorter last batch can
    // have more of them than a full one (fewer points per group when its
    // groups would not fill the chip)
    // (the same for the assignment scratch)
    int64_t nblk = 1;
    size_t split = 0;
    if (p.nb > 0) {
        const int64_t mlast = N - (p.nb - 1) * batch;
        for (const int64_t m : {p.mfull, mlast}) {
            const bool a1d = use_assign_1d(d, K);
            const int64_t n = a1d ? assign_1d_blocks(m) : assign_mfma_blocks(1, m, p.batch.DP, xt, p.batch.Kp);
            if (n > nblk) nblk = n;
            const size_t sb = a1d ? 0 : assign_mfma_scratch_bytes(1, m, p.batch.DP, xt, p.batch.Kp);
            if (sb > split) split = sb;
        }
    }
    p.obj_part = take((size_t)nblk * sizeof(double));
    p.split = take(split);
    p.total = off;
    return p;
}

// The step size of step t of T: cosine decay from alpha0 to floor * alpha0.
double emeans_step_size(double alpha0, double floor_frac, int64_t t, int64_t T) {
    if (T <= 1) return alpha0;
    return alpha0 * floor_frac +
           alpha0 * (1.0 - floor_frac) * 0.5 * (1.0 + cos(acos(-1.0) * (double)t / (double)(T - 1)));
}

km_status check_fit_args(const void* x, int xt, int64_t B, int64_t N, int64_t d, int64_t K, const float* init,
                         int32_t n_iter, const float* centroids) {
    KM_TRY(check_shape(B, N, d, K, enum_code(xt)));
    if (n_iter < 0) return fail(KM_EINVAL, "n_iter=%d < 0", n_iter);
    KM_TRY(check_scalar_k(d, K));
    KM_TRY(need(x, B * N, "x"));
    KM_TRY(need(init, B, "init"));
    KM_TRY(need(centroids, B, "centroids"));
    return KM_OK;
}

km_status run_fit(const void* x, int xt, const float* weights, int64_t B, int64_t N, int64_t d, int64_t K,
                  const float* init, int32_t n_iter, float* centroids, int32_t* labels, int32_t* counts,
                  double* objective, const Workspace& W, void* workspace, hipStream_t s,
                  void* const* assign_events = nullptr);

// ---------------------------------------------------------------------------
// Scratch of kmeans_fit_static: one array per device, in the code object's
// device memory, so that the entry point needs no allocation.  Host code
// never uses the array's name as an address (on the host it is only a
// stand-in symbol): the device address comes from hipGetSymbolAddress, once
// per device with that device current, and is kept per device.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

km_status static_scratch(void** out) {
    int dev = 0;
    KM_HIP(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(KM_EUNSUPPORTED, "kmeans_fit_static: device %d >= %d", dev, kMaxScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        KM_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (p == nullptr || (uintptr_t)p % 256 != 0)
            return fail(KM_EHIP, "kmeans_fit_static: unexpected scratch address %p", p);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KM_OK;
}

}  // namespace

extern "C" {

size_t kmeans_workspace_bytes(int64_t B, int64_t N, int64_t d, int64_t K, km_dtype xt) {
    if (check_shape(B, N, d, K, enum_code(xt)) != KM_OK) return 0;
    return plan_workspace(B, N, d, K, (DType)enum_code(xt)).total;
}

km_status kmeans_assign(const void* x, km_dtype xt, int64_t B, int64_t N, int64_t d, const float* centroids,
                        int64_t K, const float* weights, int32_t* labels, float* min_dist, double* objective,
                        void* workspace, size_t workspace_bytes, km_stream stream) {
    KM_TRY(check_shape(B, N, d, K, enum_code(xt)));
    KM_TRY(check_scalar_k(d, K));
    KM_TRY(need(x, B * N, "x"));
    KM_TRY(need(centroids, B, "centroids"));
    KM_TRY(need(labels, B * N, "labels"));
    const Workspace W = plan_workspace(B, N, d, K, (DType)enum_code(xt));
    KM_TRY(check_ws(W, workspace, workspace_bytes));
    return run_assign(x, (DType)enum_code(xt), B, N, d, centroids, K, weights, labels, min_dist, objective, 1, W,
                      workspace, (hipStream_t)stream);
}

km_status kmeans_sort_labels(const int32_t* labels, int64_t B, int64_t N, int64_t K, int32_t* counts,
                             int32_t* offsets, int32_t* perm, void* workspace, size_t workspace_bytes,
                             km_stream stream) {
    KM_TRY(check_shape(B, N, 2, K, KM_F32));
    KM_TRY(need(labels, B * N, "labels"));
    // histogram rows and their prefix, then whichever outputs the caller left
    // to the workspace; this never exceeds kmeans_workspace_bytes() of the
    // same B, N, K for any d
    Workspace W{};
    size_t off = 0;
    const size_t rows = (size_t)B * sort_chunks(B, N, K) * K * sizeof(int32_t);
    W.hist = off;
    off += align_up(rows);
    W.prefix = off;
    off += align_up(rows);
    if (!counts) { W.counts = off; off += align_up((size_t)B * K * sizeof(int32_t)); }
    if (!offsets) { W.offsets = off; off += align_up((size_t)B * (K + 1) * sizeof(int32_t)); }
    if (!perm) { W.perm = off; off += align_up((size_t)B * N * sizeof(int32_t)); }
    W.total = off;
    KM_TRY(check_ws(W, workspace, workspace_bytes));
    int32_t* cnt = counts ? counts : at<int32_t>(workspace, W.counts);
    int32_t* ofs = offsets ? offsets : at<int32_t>(workspace, W.offsets);
    int32_t* pm = perm ? perm : at<int32_t>(workspace, W.perm);
    return run_sort(labels, B, N, K, cnt, ofs, pm, nullptr, nullptr, W, workspace, (hipStream_t)stream);
}

km_status kmeans_update(const void* x, km_dtype xt, const float* weights, int64_t B, int64_t N, int64_t d,
                        const int32_t* labels, int64_t K, const float* c_old, float* c_new, int32_t* counts,
                        void* workspace, size_t workspace_bytes, km_stream stream) {
    KM_TRY(check_shape(B, N, d, K, enum_code(xt)));
    KM_TRY(need(x, B * N, "x"));
    KM_TRY(need(labels, B * N, "labels"));
    KM_TRY(need(c_old, B, "c_old"));
    KM_TRY(need(c_new, B, "c_new"));
    const Workspace W = plan_workspace(B, N, d, K, (DType)enum_code(xt));
    KM_TRY(check_ws(W, workspace, workspace_bytes));
    return run_update(x, (DType)enum_code(xt), weights, B, N, d, labels, K, c_old, c_new, counts, W, workspace,
                      (hipStream_t)stream);
}

km_status kmeans_fit(const void* x, km_dtype xt, const float* weights, int64_t B, int64_t N, int64_t d, int64_t K,
                     const float* init, int32_t n_iter, float* centroids, int32_t* labels, int32_t* counts,
                     double* objective, void* workspace, size_t workspace_bytes, km_stream stream) {
    KM_TRY(check_fit_args(x, enum_code(xt), B, N, d, K, init, n_iter, centroids));
    const Workspace W = plan_workspace(B, N, d, K, (DType)enum_code(xt));
    KM_TRY(check_ws(W, workspace, workspace_bytes));
    return run_fit(x, enum_code(xt), weights, B, N, d, K, init, n_iter, centroids, labels, counts, objective, W,
                   workspace, (hipStream_t)stream);
}

km_status kmeans_fit_timed(const void* x, km_dtype xt, const float* weights, int64_t B, int64_t N, int64_t d,
                           int64_t K, const float* init, int32_t n_iter, float* centroids, int32_t* labels,
                           int32_t* counts, double* objective, void* const* assign_events, void* workspace,
                           size_t workspace_bytes, km_stream stream) {
    KM_TRY(check_fit_args(x, enum_code(xt), B, N, d, K, init, n_iter, centroids));
    KM_TRY(need(assign_events, n_iter, "assign_events"));
    for (int32_t i = 0; i < 2 * n_iter; ++i)
        if (assign_events[i] == nullptr) return fail(KM_EINVAL, "assign_events[%d] is NULL", i);
    const Workspace W = plan_workspace(B, N, d, K, (DType)enum_code(xt));
    KM_TRY(check_ws(W, workspace, workspace_bytes));
    return run_fit(x, enum_code(xt), weights, B, N, d, K, init, n_iter, centroids, labels, counts, objective, W,
                   workspace, (hipStream_t)stream, assign_events);
}

size_t kmeans_fit_static_max_bytes(void) { return kStaticScratchBytes; }

km_status kmeans_fit_static(const void* x, km_dtype xt, const float* weights, int64_t B, int64_t N, int64_t d,
                            int64_t K, const float* init, int32_t n_iter, float* centroids, int32_t* labels,
                            int32_t* counts, double* objective, km_stream stream) {
    KM_TRY(check_fit_args(x, enum_code(xt), B, N, d, K, init, n_iter, centroids));
    const Workspace W = plan_workspace(B, N, d, K, (DType)enum_code(xt));
    if (W.total > kStaticScratchBytes)
        return fail(KM_EWORKSPACE,
                    "kmeans_fit_static: these shapes need %zu bytes of scratch, more than the library's static "
                    "%zu bytes (use kmeans_fit with a caller workspace)",
                    W.total, kStaticScratchBytes);
    void* ws = nullptr;
    KM_TRY(static_scratch(&ws));
    return run_fit(x, enum_code(xt), weights, B, N, d, K, init, n_iter, centroids, labels, counts, objective, W, ws,
                   (hipStream_t)stream);
}

}  // extern "C"

namespace {

km_status run_fit(const void* x, int xt, const float* weights, int64_t B, int64_t N, int64_t d, int64_t K,
                  const float* init, int32_t n_iter, float* centroids, int32_t* labels, int32_t* counts,
                  double* objective, const Workspace& W, void* workspace, hipStream_t s,
                  void* const* assign_events) {
    auto ev = [&](int64_t i) { return assign_events ? (hipEvent_t)assign_events[i] : nullptr; };
    if (d == 1 && n_iter > 0 && fit_1d_rows_fits(N, K)) {
        // scalar rows that fit on chip: every iteration in one launch
        for (int32_t t = 0; t < n_iter && assign_events; ++t) KM_HIP(hipEventRecord(ev(2 * t), s), "event");
        KM_HIP(launch_fit_1d_rows((DType)enum_code(xt), x, weights, B, N, init, K, n_iter, centroids, labels, counts,
                                  objective, s),
               "fit_1d_rows");
        for (int32_t t = 0; t < n_iter && assign_events; ++t) KM_HIP(hipEventRecord(ev(2 * t + 1), s), "event");
        return KM_OK;
    }
    if (init != centroids && B > 0)
        KM_HIP(hipMemcpyAsync(centroids, init, (size_t)B * K * d * sizeof(float), hipMemcpyDeviceToDevice, s),
               "copy init");
    int32_t* lab = labels ? labels : at<int32_t>(workspace, W.labels);
    // the matrix-core assignment adds its labels to the sort's histogram rows
    // (cleared here once; every sort clears them again after use), so the
    // update needs no separate pass over the labels
    const bool counted = n_iter > 0 && N > 0 && B > 0 && !use_assign_1d(d, K) &&
                         !assign_mfma_merges(B, N, W.DP, (DType)enum_code(xt), W.Kp);
    int32_t* hist = counted ? at<int32_t>(workspace, W.hist) : nullptr;
    if (counted) KM_HIP(launch_zero(hist, W.prefix - W.hist, s), "zero");
    for (int32_t t = 0; t < n_iter; ++t) {
        // from the second iteration on, the previous update's divide wrote the
        // centroid tiles, unless the update took the scalar-row path
        const bool fused = t > 0 && !use_update_1d((DType)enum_code(xt), x, weights, lab, d, N, K);
        // counted: the sort's column scan also sums the objective partials
        double* obj_t = objective ? objective + t : nullptr;
        KM_TRY(run_assign(x, (DType)enum_code(xt), B, N, d, centroids, K, weights, lab, nullptr, obj_t, n_iter, W,
                          workspace, s, !fused, ev(2 * t), ev(2 * t + 1), hist, !counted));
        KM_TRY(run_update(x, (DType)enum_code(xt), weights, B, N, d, lab, K, centroids, centroids, counts, W, workspace, s,
                          t + 1 < n_iter, counted, counted ? obj_t : nullptr, n_iter));
    }
    return KM_OK;
}

}  // namespace

extern "C" {

size_t kmeans_optimal_1d_workspace_bytes(int64_t B, int64_t N, int64_t K) {
    if (B < 0 || !optimal_1d_supports(N, K)) return 0;
    size_t d_off, cut_off, perm_off, total;
    optimal_1d_workspace(B, N, K, &d_off, &cut_off, &perm_off, &total);
    return total;
}

km_status kmeans_optimal_1d(const void* x, km_dtype xt, const float* weights, int64_t B, int64_t N, int64_t K,
                            float* centroids, int32_t* labels, int32_t* counts, double* objective,
                            void* workspace, size_t workspace_bytes, km_stream stream) {
    if (B < 0 || N < 0) return fail(KM_EINVAL, "negative size: B=%lld N=%lld", (long long)B, (long long)N);
    const int xc = enum_code(xt);
    if (xc != KM_F32 && xc != KM_F16 && xc != KM_BF16) return fail(KM_EUNSUPPORTED, "unknown dtype %d", xc);
    if (K < 1 || K > N)
        return fail(KM_EINVAL, "the optimum needs 1 <= K <= N (K=%lld, N=%lld)", (long long)K, (long long)N);
    if (N > kOpt1DMaxN)
        return fail(KM_EUNSUPPORTED, "the optimum supports rows of N <= %d points (N=%lld)", kOpt1DMaxN,
                    (long long)N);
    if (K > kOpt1DMaxK)
        return fail(KM_EUNSUPPORTED, "the optimum supports K <= %d (K=%lld)", kOpt1DMaxK, (long long)K);
    if (B > kMaxB) return fail(KM_EUNSUPPORTED, "B=%lld > %lld is not supported", (long long)B, (long long)kMaxB);
    KM_TRY(need(x, B * N, "x"));
    KM_TRY(need(centroids, B, "centroids"));
    size_t d_off, cut_off, perm_off, total;
    optimal_1d_workspace(B, N, K, &d_off, &cut_off, &perm_off, &total);
    Workspace W{};
    W.total = total;
    KM_TRY(check_ws(W, workspace, workspace_bytes));
    KM_HIP(launch_optimal_1d((DType)enum_code(xt), x, weights, B, N, K, centroids, labels, counts, objective,
                             workspace, (hipStream_t)stream),
           "optimal_1d");
    return KM_OK;
}

size_t kmeans_stream_workspace_bytes(int64_t N, int64_t d, int64_t K, km_dtype xt, int64_t chunk) {
    if (check_shape(1, N, d, K, enum_code(xt)) != KM_OK || d < 2 || chunk < 1) return 0;
    return plan_stream(N, d, K, (DType)enum_code(xt), chunk).total;
}

km_status kmeans_fit_stream(const void* x_host, km_dtype xt, const float* w_host, int64_t N, int64_t d, int64_t K,
                            const float* init, int32_t n_iter, float* centroids, int32_t* labels, int32_t* counts,
                            double* objective, int64_t chunk, void* workspace, size_t workspace_bytes,
                            km_stream stream) {
    KM_TRY(check_shape(1, N, d, K, enum_code(xt)));
    if (d < 2) return fail(KM_EUNSUPPORTED, "streamed fits need d >= 2 (d=%lld)", (long long)d);
    if (n_iter < 0) return fail(KM_EINVAL, "n_iter=%d < 0", n_iter);
    if (chunk < 1) return fail(KM_EINVAL, "chunk=%lld < 1", (long long)chunk);
    KM_TRY(need(x_host, N, "x_host"));
    KM_TRY(need(init, 1, "init"));
    KM_TRY(need(centroids, 1, "centroids"));
    const DType t = (DType)enum_code(xt);
    const StreamPlan P = plan_stream(N, d, K, t, chunk);
    {
        Workspace W{};
        W.total = P.total;
        KM_TRY(check_ws(W, workspace, workspace_bytes));
    }
    hipStream_t s = (hipStream_t)stream;
    const size_t cbytes = (size_t)K * d * sizeof(float);
    if (init != centroids) KM_HIP(hipMemcpyAsync(centroids, init, cbytes, hipMemcpyDeviceToDevice, s), "copy init");
    if (n_iter == 0) return KM_OK;
    if (N == 0) {
        if (objective) KM_HIP(launch_zero(objective, (size_t)n_iter * sizeof(double), s), "zero");
        if (counts) KM_HIP(launch_zero(counts, (size_t)K * sizeof(int32_t), s), "zero");
        return KM_OK;
    }
    int dev = 0;
    KM_HIP(hipGetDevice(&dev), "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_stream_mu);
    StreamRes* R = nullptr;
    KM_HIP(stream_res(dev, &R), "copy stream");
    const Workspace& W = P.chunk;
    char* ws = (char*)workspace;
    const int64_t c = P.chunk_n, es = dtype_bytes(t);
    float* sums = at<float>(ws, W.sums);
    float* wsum = w_host ? at<float>(ws, W.wsum) : nullptr;
    int32_t* ctot = at<int32_t>(ws, P.counts_total);
    double* obj_all = at<double>(ws, P.obj_all);
    // the first copies must not overwrite buffers that earlier work on the
    // caller's stream may still read
    KM_HIP(hipEventRecord(R->start, s), "event");
    KM_HIP(hipStreamWaitEvent(R->copy, R->start, 0), "event wait");
    int64_t g = 0;  // chunk counter over all iterations: buffer g % 2
    for (int32_t it = 0; it < n_iter; ++it) {
        // later iterations find their centroid tiles written by the previous divide
        if (it == 0) KM_HIP(launch_prep(t, centroids, 1, K, (int)d, W.DP, W.Kp, at<void>(ws, W.chat), s), "prep");
        // sums and wsum are adjacent in the plan: clear both with one fill
        KM_HIP(launch_zero(sums, W.offsets - W.sums, s), "zero");
        KM_HIP(launch_zero(ctot, (size_t)K * sizeof(int32_t), s), "zero");
        for (int64_t ci = 0; ci < P.nchunks; ++ci, ++g) {
            const int buf = (int)(g & 1);
            const int64_t p0 = ci * c, nc = (p0 + c <= N) ? c : N - p0;
            void* xb = at<void>(ws, P.xbuf[buf]);
            float* wb = w_host ? at<float>(ws, P.wbuf[buf]) : nullptr;
            if (g >= 2) KM_HIP(hipStreamWaitEvent(R->copy, R->consumed[buf], 0), "event wait");
            KM_HIP(hipMemcpyAsync(xb, (const char*)x_host + p0 * d * es, (size_t)(nc * d * es),
                                  hipMemcpyHostToDevice, R->copy),
                   "copy points");
            if (w_host)
                KM_HIP(hipMemcpyAsync(wb, w_host + p0, (size_t)nc * sizeof(float), hipMemcpyHostToDevice, R->copy),
                       "copy weights");
            KM_HIP(hipEventRecord(R->copied[buf], R->copy), "event");
            KM_HIP(hipStreamWaitEvent(s, R->copied[buf], 0), "event wait");
            int32_t* lab = labels ? labels + p0 : at<int32_t>(ws, W.labels);
            KM_HIP(launch_assign_mfma(t, xb, 1, nc, (int)d, W.DP, at<void>(ws, W.chat), W.Kp, wb, lab, nullptr,
                                      obj_all + ci * P.nblk_chunk, assign_mfma_blocks(1, nc, W.DP, t, W.Kp),
                                      at<void>(ws, P.split), s),
                   "assign_mfma");
            int32_t* cnt = at<int32_t>(ws, W.counts);
            int32_t* offsets = at<int32_t>(ws, W.offsets);
            int32_t* perm = at<int32_t>(ws, W.perm);
            int32_t* piece_seg = at<int32_t>(ws, W.piece_seg);
            // every chunk uses the piece width of a full chunk, so a shorter
            // last chunk never has more pieces than the plan holds (nor more
            // histogram rows: a shorter chunk has at most as many)
            const int TW = segreduce_tw(1, c);
            SortBufs o{cnt, offsets, perm, at<int32_t>(ws, W.hist), at<int32_t>(ws, W.prefix), nullptr, piece_seg,
                       nullptr};
            KM_HIP(launch_sort(lab, 1, nc, K, o, TW, (nc + TW - 1) / TW, s, SortMode::Stable), "sort");
            KM_HIP(launch_segreduce_tw(t, xb, wb, 1, nc, (int)d, perm, offsets, K, sums, wsum, piece_seg,
                                       at<float>(ws, W.slot), at<float>(ws, W.wslot), nullptr, nullptr, TW, true,
                                       nullptr, s),
                   "segreduce");
            KM_HIP(launch_add_i32(ctot, cnt, K, s), "add counts");
            KM_HIP(hipEventRecord(R->consumed[buf], s), "event");
        }
        if (objective) KM_HIP(launch_obj_reduce(obj_all, 1, P.nblk_total, objective + it, 1, s), "obj_reduce");
        if (it + 1 < n_iter)
            KM_HIP(launch_divide_prep(t, sums, wsum, ctot, 1, K, (int)d, W.DP, W.Kp, centroids, centroids,
                                      at<void>(ws, W.chat), s),
                   "divide");
        else
            KM_HIP(launch_divide(sums, wsum, ctot, 1, K, (int)d, centroids, centroids, s), "divide");
    }
    if (counts) KM_HIP(hipMemcpyAsync(counts, ctot, (size_t)K * sizeof(int32_t), hipMemcpyDeviceToDevice, s), "copy");
    return KM_OK;
}

size_t kmeans_emeans_workspace_bytes(int64_t N, int64_t d, int64_t K, km_dtype xt, int64_t batch) {
    if (check_shape(1, N, d, K, enum_code(xt)) != KM_OK || batch < 1 || !emeans_split_supports(K)) return 0;
    if (d == 1 && !assign_1d_supports(K)) return 0;
    return plan_emeans(N, d, K, (DType)enum_code(xt), batch, 1).total;
}

km_status kmeans_emeans(const void* x, km_dtype xt, int64_t N, int64_t d, int64_t K, const float* init,
                        int64_t batch, int32_t epochs, double alpha0, double floor_frac, double dead_frac,
                        double eps, const float* uniforms, float* centroids, int32_t* labels, int32_t* counts,
                        double* objective, void* workspace, size_t workspace_bytes, km_stream stream) {
    KM_TRY(check_shape(1, N, d, K, enum_code(xt)));
    KM_TRY(check_scalar_k(d, K));
    if (!emeans_split_supports(K))
        return fail(KM_EUNSUPPORTED, "e-means supports K <= %lld (K=%lld)", (long long)kEmeansMaxK, (long long)K);
    if (batch < 1) return fail(KM_EINVAL, "batch=%lld < 1", (long long)batch);
    if (epochs < 1) return fail(KM_EINVAL, "epochs=%d < 1", epochs);
    if (!(alpha0 > 0.0 && alpha0 <= 1.0)) return fail(KM_EINVAL, "alpha0=%g is not in (0, 1]", alpha0);
    if (!(floor_frac >= 0.0 && floor_frac <= 1.0))
        return fail(KM_EINVAL, "floor_frac=%g is not in [0, 1]", floor_frac);
    if (!(dead_frac >= 0.0)) return fail(KM_EINVAL, "dead_frac=%g < 0", dead_frac);
    if (!(eps >= 0.0 && eps < 1.0)) return fail(KM_EINVAL, "eps=%g is not in [0, 1)", eps);
    KM_TRY(need(x, N, "x"));
    KM_TRY(need(init, 1, "init"));
    KM_TRY(need(centroids, 1, "centroids"));
    if (dead_frac > 0.0) KM_TRY(need(uniforms, N, "uniforms"));
    const DType t = (DType)enum_code(xt);
    const EmeansPlan P = plan_emeans(N, d, K, t, batch, epochs);
    {
        Workspace W{};
        W.total = P.total;
        KM_TRY(check_ws(W, workspace, workspace_bytes));
    }
    hipStream_t s = (hipStream_t)stream;
    const size_t cbytes = (size_t)K * d * sizeof(float);
    if (init != centroids) KM_HIP(hipMemcpyAsync(centroids, init, cbytes, hipMemcpyDeviceToDevice, s), "copy init");
    if (N == 0) {
        if (counts) KM_HIP(launch_zero(counts, (size_t)K * sizeof(int32_t), s), "zero");
        return KM_OK;
    }
    const Workspace& W = P.batch;
    char* ws = (char*)workspace;
    double* S = at<double>(ws, P.S);
    double* Nc = at<double>(ws, P.Nc);
    double* F = at<double>(ws, P.F);
    double* G = at<double>(ws, P.G);
    // S, N, F, G are adjacent in the plan: clear them with one fill
    KM_HIP(launch_zero(S, P.list_j - P.S, s), "zero");
    const int64_t es = dtype_bytes(t);
    float* sums = at<float>(ws, W.sums);
    int32_t* cnt = at<int32_t>(ws, W.counts);
    int32_t* offsets = at<int32_t>(ws, W.offsets);
    int32_t* perm = at<int32_t>(ws, W.perm);
    int32_t* piece_seg = at<int32_t>(ws, W.piece_seg);
    double* part = at<double>(ws, P.obj_part);
    // every batch uses the piece width of a full batch, so a shorter last
    // batch never has more pieces than the plan holds
    const int TW = segreduce_tw(1, P.mfull);
    const double dead_below = dead_frac * (double)P.mfull / (double)K;
    // the batch's sums and counts start at zero; the moving average clears
    // them after every batch
    KM_HIP(launch_zero(sums, (size_t)K * d * sizeof(float), s), "zero");
    KM_HIP(launch_zero(cnt, (size_t)K * sizeof(int32_t), s), "zero");
    for (int64_t st = 0; st < P.steps; ++st) {
        const int64_t e = st / P.nb, i0 = (st % P.nb) * batch;
        const int64_t m = (i0 + batch <= N) ? batch : N - i0;
        const bool last = e == epochs - 1;
        const void* xb = (const char*)x + i0 * d * es;
        int32_t* lab = (last && labels) ? labels + i0 : at<int32_t>(ws, W.labels);
        int64_t nblk;
        bool counted = false;
        if (use_assign_1d(d, K)) {
            nblk = assign_1d_blocks(m);
            KM_HIP(launch_assign_1d(t, xb, 1, m, centroids, K, nullptr, lab, nullptr, part, nblk, nblk, s),
                   "assign_1d");
        } else {
            nblk = assign_mfma_blocks(1, m, W.DP, t, W.Kp);
            void* blob = at<void>(ws, W.chat);
            KM_HIP(launch_prep(t, centroids, 1, K, (int)d, W.DP, W.Kp, blob, s), "prep");
            // a sliced launch's merge also counts the labels (cnt is zero here:
            // cleared before the first step and by the moving average after each)
            counted = assign_mfma_merges(1, m, W.DP, t, W.Kp);
            KM_HIP(launch_assign_mfma(t, xb, 1, m, (int)d, W.DP, blob, W.Kp, nullptr, lab, nullptr, part, nblk,
                                      at<void>(ws, P.split), s, counted ? cnt : nullptr, K),
                   "assign_mfma");
        }
        // the batch's objective partials are summed by the moving-average kernel below
        SortBufs o{cnt, offsets, perm, nullptr, nullptr, at<int32_t>(ws, W.cursor), piece_seg,
                   at<int32_t>(ws, W.seg_short)};
        KM_HIP(launch_sort(lab, 1, m, K, o, TW, (m + TW - 1) / TW, s,
                           counted ? SortMode::DirectCounted : SortMode::Direct),
               "sort");
        // the atomic fold completes the sums (the moving average reads them)
        KM_HIP(launch_segreduce_tw(t, xb, nullptr, 1, m, (int)d, perm, offsets, K, sums, nullptr, piece_seg,
                                   at<float>(ws, W.slot), at<float>(ws, W.wslot), nullptr, nullptr, TW, false,
                                   at<int32_t>(ws, W.seg_short), s),
               "segreduce");
        const double a = emeans_step_size(alpha0, floor_frac, st, P.steps);
        KM_HIP(launch_emeans_ema(S, Nc, sums, cnt, K, (int)d, a, centroids, last ? F : nullptr, last ? G : nullptr,
                                 part, nblk, objective ? objective + st : nullptr, s),
               "ema");
        if (dead_frac > 0.0)
            KM_HIP(launch_emeans_split(S, Nc, centroids, K, (int)d, dead_below, eps, uniforms + st * K,
                                       at<int32_t>(ws, P.list_j), at<int32_t>(ws, P.list_k), s),
                   "split");
    }
    KM_HIP(launch_emeans_final(F, G, K, (int)d, centroids, counts, s), "final mean");
    return KM_OK;
}

const char* kmeans_status_str(km_status st) {
    switch (enum_code(st)) {
        case KM_OK: return "ok";
        case KM_EINVAL: return "invalid argument";
        case KM_EUNSUPPORTED: return "unsupported shape or dtype";
        case KM_EWORKSPACE: return "workspace too small";
        case KM_EHIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* kmeans_last_error(void) { return g_last_error.c_str(); }

int kmeans_version(void) { return 100; }

}  // extern "C"
