/*
 * kmeans.h -- C ABI of the MI355X (gfx950) exact Lloyd k-means library.
 *
 * One Lloyd iteration is an assignment stage followed by an update stage
 * (technologypulse.uk "Flash-KMeans" article, section "math unchanged,
 * dataflow changed").  The library computes the textbook result; only the
 * data flow differs:
 *
 *   - assignment: the squared distance ||x||^2 - 2 x.c + ||c||^2 is computed
 *     tile by tile on the matrix cores and reduced on the fly to the running
 *     nearest centroid, so the N x K distance matrix never reaches device
 *     memory (same article, "bottleneck 1"; wispaper.ai "Flash-KMeans" blog,
 *     "FlashAssign: Materialization-Free Assignment").  Scalar points (d = 1)
 *     take a binary search over the sorted centroids instead.
 *   - update: the label vector is argsorted by cluster id (a stable
 *     counting sort) so that each cluster is a contiguous segment, and every
 *     segment is reduced on chip and stored once; the pieces of a cluster
 *     that spans several reduction pieces are added in a fixed order by the
 *     divide, instead of one scattered atomic per point and coordinate.
 *     The point matrix is never permuted in memory
 *     (technologypulse.uk article, "bottleneck 2"; wispaper.ai blog,
 *     "Sort-Inverse Update").  Inside a fit, the assignment also counts its
 *     labels for the sort.  The new centroid is the mean
 *     of its points (daily.steinslab.io "e-means" article, "Breaking 70 Years
 *     of Full-Batch Inertia": centroid = S_j / N_j); a cluster with no points
 *     keeps its previous centroid.
 *   - optional per-point sample weights, as in the per-row weighted 1D
 *     clustering of github LeanModels/LeanQuant issue #1 ("1D k-means"):
 *     the assignment ignores them, the centroid is sum(w x) / sum(w) and the
 *     objective is sum(w * distance).
 *
 * Conventions shared by every entry point:
 *   - Layouts are row-major and contiguous: points x [B, N, d] of dtype xt,
 *     centroids [B, K, d] float32, labels [B, N] int32, counts [B, K] int32,
 *     weights [B, N] float32.  B independent problems are solved in one call.
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library never allocates or frees device memory: scratch space is the
 *     caller's workspace of at least kmeans_workspace_bytes() bytes, aligned
 *     to 256 bytes.  Calls that share one workspace must not overlap in time.
 *   - Calls only enqueue kernels on `stream` (a hipStream_t; NULL is the
 *     default stream) and return without synchronizing.  Arguments are
 *     checked on the host before anything is enqueued; on an error nothing is
 *     enqueued and the status says why (kmeans_last_error() has the detail).
 *     Faults inside kernels surface at the caller's next synchronization.
 *   - Supported shapes: d == 1 (scalar path), or 2 <= d <= 512 for 16-bit
 *     points and 2 <= d <= 256 for float32 points (matrix-core path; d is
 *     zero-padded internally to 16, 32, 64, 128, 256 or 512, which does not
 *     change any distance).  1 <= K <= 32768 (K <= 16384 when d == 1).
 *     N < 2^31, B <= 65535; B and N may be 0.
 *   - Centroids are float32 state.  Distances use the centroids rounded
 *     (IEEE round-to-nearest-even) to the point dtype, because that is the
 *     matrix-core operand; products accumulate in float32.  Ties between
 *     equally near centroids go to the smallest index.
 *   - Inputs must be finite; weights, when given, must be positive.
 */
#ifndef KMEANS_MI355X_H
#define KMEANS_MI355X_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define KM_API __attribute__((visibility("default")))
#else
#define KM_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KM_F32 = 0, KM_F16 = 1, KM_BF16 = 2 } km_dtype;

typedef enum {
    KM_OK = 0,
    KM_EINVAL = 1,        /* null pointer, negative size, misaligned workspace, ... */
    KM_EUNSUPPORTED = 2,  /* a shape or dtype outside the supported set */
    KM_EWORKSPACE = 3,    /* workspace smaller than kmeans_workspace_bytes() */
    KM_EHIP = 4           /* the HIP runtime refused a launch */
} km_status;

typedef void *km_stream; /* hipStream_t */

/* Bytes of workspace any entry point needs for these shapes (0 on invalid
 * shapes).  One workspace of this size serves kmeans_assign, kmeans_update,
 * kmeans_sort_labels and kmeans_fit. */
KM_API size_t kmeans_workspace_bytes(int64_t B, int64_t N, int64_t d, int64_t K, km_dtype xt);

/* Assignment stage (fused distance + running argmin).
 *   x          [B,N,d] points of dtype xt.
 *   centroids  [B,K,d] float32.
 *   weights    [B,N] float32 or NULL; used only for the objective.
 *   labels     out [B,N] int32: index of the nearest centroid.
 *   min_dist   out [B,N] float32 or NULL: squared distance to it, clamped at 0.
 *   objective  out [B] float64 or NULL: sum_i w_i * min_dist_i per batch.
 * Reads x once; writes no N x K data. */
KM_API km_status kmeans_assign(const void *x, km_dtype xt, int64_t B, int64_t N, int64_t d,
                        const float *centroids, int64_t K, const float *weights,
                        int32_t *labels, float *min_dist, double *objective,
                        void *workspace, size_t workspace_bytes, km_stream stream);

/* Argsort step of the update: groups the point indices of each batch by
 * label.
 *   labels   [B,N] int32; a label outside [0, K) belongs to no cluster.
 *   counts   out [B,K] int32: points per cluster.
 *   offsets  out [B,K+1] int32: exclusive prefix of counts; offsets[b][K] is
 *            the number of labelled points.
 *   perm     out [B,N] int32: perm[b][offsets[b][j] .. offsets[b][j+1]) are
 *            the indices i of batch b with labels[b][i] == j, in ascending
 *            order (a stable sort: the result is unique); entries from
 *            offsets[b][K] on are not written.
 * May be NULL: none of counts / offsets / perm (they then live in the
 * workspace, which makes the call a no-op for the caller). */
KM_API km_status kmeans_sort_labels(const int32_t *labels, int64_t B, int64_t N, int64_t K,
                             int32_t *counts, int32_t *offsets, int32_t *perm,
                             void *workspace, size_t workspace_bytes, km_stream stream);

/* Update stage (sort-inverse segmented reduction, then the divide).
 *   x        [B,N,d] points of dtype xt; weights [B,N] float32 or NULL.
 *   labels   [B,N] int32 (labels outside [0, K) are skipped).
 *   c_old    [B,K,d] float32: kept for clusters with no point.
 *   c_new    out [B,K,d] float32; may alias c_old.
 *   counts   out [B,K] int32 or NULL: points per cluster. */
KM_API km_status kmeans_update(const void *x, km_dtype xt, const float *weights,
                        int64_t B, int64_t N, int64_t d, const int32_t *labels, int64_t K,
                        const float *c_old, float *c_new, int32_t *counts,
                        void *workspace, size_t workspace_bytes, km_stream stream);

/* n_iter Lloyd iterations (assignment, then update) from init.  For d >= 2
 * the result is a deterministic function of the inputs: two calls on the
 * same inputs give bit-identical outputs (no floating-point atomics on this
 * path).
 *   init       [B,K,d] float32 (may alias centroids).
 *   centroids  out [B,K,d] float32: after the last update.
 *   labels     out [B,N] int32 or NULL: the last assignment.
 *   counts     out [B,K] int32 or NULL: the last update.
 *   objective  out [B,n_iter] float64 or NULL: objective of assignment t
 *              (computed with the centroids that assignment used).
 * No tolerance, no early stop, no host synchronization.  n_iter == 0 copies
 * init to centroids. */
KM_API km_status kmeans_fit(const void *x, km_dtype xt, const float *weights,
                     int64_t B, int64_t N, int64_t d, int64_t K,
                     const float *init, int32_t n_iter,
                     float *centroids, int32_t *labels, int32_t *counts, double *objective,
                     void *workspace, size_t workspace_bytes, km_stream stream);

/* kmeans_fit that also times the assignment stage of every iteration with
 * the caller's events (the assignment stage dominates an iteration:
 * technologypulse.uk "Flash-KMeans" article, "bottleneck 1").
 *   assign_events  2 * n_iter hipEvent_t handles, created by the caller
 *                  (with timing enabled to read durations): assign_events[2t]
 *                  is recorded on `stream` right before the assignment
 *                  kernels of iteration t are launched (after the centroid
 *                  prep), assign_events[2t + 1] right after them (before the
 *                  objective reduction and the update).  Where all
 *                  iterations run in one launch (scalar rows that fit on
 *                  chip), every even event is recorded before that launch
 *                  and every odd one after it.
 * The rest is kmeans_fit.  KM_EINVAL if any handle is NULL. */
KM_API km_status kmeans_fit_timed(const void *x, km_dtype xt, const float *weights,
                           int64_t B, int64_t N, int64_t d, int64_t K,
                           const float *init, int32_t n_iter,
                           float *centroids, int32_t *labels, int32_t *counts, double *objective,
                           void *const *assign_events,
                           void *workspace, size_t workspace_bytes, km_stream stream);

/* kmeans_fit for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels and results as kmeans_fit, without the workspace:
 * the scratch lives in one static device array of
 * kmeans_fit_static_max_bytes() bytes (64 MiB) per device, held from the
 * first call on that device until the process ends.  The call allocates and
 * frees nothing.  Shapes whose kmeans_workspace_bytes() exceeds that size
 * return KM_EWORKSPACE before anything is enqueued.
 * Every call on one device uses the same array, and each call clears what
 * it needs at the start: calls that may overlap in time on one device (on
 * different streams, or from different threads without ordering) race on
 * it and must not be issued. */
KM_API size_t kmeans_fit_static_max_bytes(void);
KM_API km_status kmeans_fit_static(const void *x, km_dtype xt, const float *weights,
                            int64_t B, int64_t N, int64_t d, int64_t K,
                            const float *init, int32_t n_iter,
                            float *centroids, int32_t *labels, int32_t *counts, double *objective,
                            km_stream stream);

/* Lloyd fit of one problem whose points stay in host memory
 * (technologypulse.uk "Flash-KMeans" article, performance section:
 * out-of-core runs in which a chunked stream overlap hides the PCIe
 * transfers; wispaper.ai blog, performance: CPU-to-GPU copies overlapped
 * with computation).  Every iteration copies the points chunk by chunk into
 * two device buffers on a copy stream the library keeps per device, while
 * the previous chunk is assigned and reduced on `stream`; sums, weight sums
 * and counts accumulate over the chunks, then the divide.  The result is
 * that of kmeans_fit on the same points up to fp32 summation order.
 *   x_host     [N,d] points of dtype xt in host memory.  Pinned memory (e.g.
 *              hipHostMalloc) lets the copies overlap the kernels; pageable
 *              memory works, staged by the runtime.  It must stay valid and
 *              unchanged until the work on `stream` completes.
 *   w_host     [N] float32 in host memory, or NULL (same lifetime).
 *   init       [K,d] float32 device (may alias centroids).
 *   centroids  out [K,d] float32 device.
 *   labels     out [N] int32 device or NULL: the last assignment.
 *   counts     out [K] int32 device or NULL: the last update.
 *   objective  out [n_iter] float64 device or NULL.
 *   chunk      points per copy, rounded up to a multiple of 4096 (at most N).
 * One problem (B = 1) with d >= 2 (KM_EUNSUPPORTED for d = 1).  The
 * workspace must hold kmeans_stream_workspace_bytes(N, d, K, xt, chunk)
 * bytes, 256-byte aligned.  Calls on one device enqueue their work one at a
 * time (they share the device's copy stream). */
KM_API size_t kmeans_stream_workspace_bytes(int64_t N, int64_t d, int64_t K, km_dtype xt, int64_t chunk);
KM_API km_status kmeans_fit_stream(const void *x_host, km_dtype xt, const float *w_host,
                            int64_t N, int64_t d, int64_t K, const float *init, int32_t n_iter,
                            float *centroids, int32_t *labels, int32_t *counts, double *objective,
                            int64_t chunk, void *workspace, size_t workspace_bytes, km_stream stream);

/* Globally optimal weighted 1D k-means of every row (github LeanModels/
 * LeanQuant issue #1 "1D k-means": for scalar data the globally optimal
 * centroids can be found; the issue's diff calls such a weighted 1D
 * clustering in place of Lloyd).  Among all partitions of a row's points
 * into K non-empty groups, one with the least sum_i w_i (x_i - mean_g(i))^2,
 * found exactly (up to float64 rounding) over the cuts of the sorted row
 * into K runs.
 *   x          [B,N] (or [B,N,1]) points of dtype xt.
 *   weights    [B,N] float32 or NULL (all 1); must be positive.
 *   centroids  out [B,K] float32: the runs' weighted means, ascending.
 *   labels     out [B,N] int32 or NULL: the run of every point (0 .. K-1).
 *   counts     out [B,K] int32 or NULL: points per run.
 *   objective  out [B] float64 or NULL: the least cost J*.
 * Needs 1 <= K <= N (KM_EINVAL otherwise); supports N <= 4096 and K <= 256
 * (KM_EUNSUPPORTED beyond).  Equal values may be split between runs only
 * where that does not change J*; ties between cuts go to the earliest cut
 * in (value, index) order, up to float64 rounding.  The workspace must hold
 * kmeans_optimal_1d_workspace_bytes(B, N, K) bytes, 256-byte aligned. */
KM_API size_t kmeans_optimal_1d_workspace_bytes(int64_t B, int64_t N, int64_t K);
KM_API km_status kmeans_optimal_1d(const void *x, km_dtype xt, const float *weights,
                            int64_t B, int64_t N, int64_t K,
                            float *centroids, int32_t *labels, int32_t *counts, double *objective,
                            void *workspace, size_t workspace_bytes, km_stream stream);

/* e-means: mini-batch k-means with moving-average statistics
 * (daily.steinslab.io "e-means" article: the update S_j <- (1 - a) S_j +
 * a s_j of each cluster's sum and count in "Breaking 70 Years of Full-Batch
 * Inertia"; the cosine step decay from alpha0 to a fraction of it, and the
 * move to the last epoch's plain mean, in "Mini-Batch Stochastic Noise" and
 * "Matching 25 Iterations"; proportional splitting of dead clusters in
 * "Proportional Splitting Resurrects Thousands of Dead Centers").  Not
 * Lloyd: a different, approximate algorithm that reuses its kernels.
 *
 * The points are cut into ceil(N / batch) batches of consecutive points
 * (the last one shorter); there are T = epochs * ceil(N / batch) steps.
 * Step t assigns its batch to the nearest current centroid (the Lloyd
 * assignment, ties to the lower index), sums and counts the batch per
 * cluster (s_j, n_j) and sets, in float64, S_j = (1 - a_t) S_j + a_t s_j,
 * N_j = (1 - a_t) N_j + a_t n_j (both start at zero) and c_j = S_j / N_j
 * where N_j > 0, with a_t = alpha0 (floor + (1 - floor) (1 + cos(pi t /
 * (T - 1))) / 2) (a_0 = alpha0 when T = 1).  Then every cluster with
 * N_j < dead_frac * min(batch, N) / K is dead; dead clusters are resolved
 * in ascending order: the donor k is the first cluster whose prefix sum of
 * N (taken before any split of the step) exceeds u_j * sum(N), with u_j =
 * uniforms[t * K + j]; k == j or a donor with N_k == 0 does nothing;
 * otherwise N_k and S_k halve, cluster j takes the same N, and the two
 * centroids become c_k (1 + eps s_c) and c_k (1 - eps s_c) (s_c = +1 on even,
 * -1 on odd coordinates), S rescaled to match.  After the last step every
 * cluster that received points in the last epoch moves to the plain mean of
 * those points.
 *   x          [N,d] device points of dtype xt.
 *   init       [K,d] float32 device (may alias centroids).
 *   batch      points per step (>= 1; min(batch, N) is the full batch).
 *   epochs     passes over the points (>= 1).
 *   alpha0     first step size, in (0, 1]; floor_frac, in [0, 1], is the
 *              last step's fraction of it.
 *   dead_frac  0 turns splitting off.  eps in [0, 1).
 *   uniforms   [T,K] float32 device in [0, 1), or NULL when dead_frac == 0:
 *              the draws of the splits (the caller's random numbers).
 *   centroids  out [K,d] float32 device.
 *   labels     out [N] int32 device or NULL: the last epoch's assignments.
 *   counts     out [K] int32 device or NULL: points per cluster in the last
 *              epoch.
 *   objective  out [T] float64 device or NULL: sum over the batch of step t
 *              of the squared distance to the centroid it was assigned to.
 * One problem (B = 1); d = 1 needs K <= 16384, and K <= 32768 always
 * (KM_EUNSUPPORTED).  The workspace must hold
 * kmeans_emeans_workspace_bytes(N, d, K, xt, batch) bytes, 256-byte
 * aligned. */
KM_API size_t kmeans_emeans_workspace_bytes(int64_t N, int64_t d, int64_t K, km_dtype xt, int64_t batch);
KM_API km_status kmeans_emeans(const void *x, km_dtype xt, int64_t N, int64_t d, int64_t K,
                        const float *init, int64_t batch, int32_t epochs, double alpha0,
                        double floor_frac, double dead_frac, double eps, const float *uniforms,
                        float *centroids, int32_t *labels, int32_t *counts, double *objective,
                        void *workspace, size_t workspace_bytes, km_stream stream);

/* Static description of a status code. */
KM_API const char *kmeans_status_str(km_status status);

/* Message of the last failed call on this thread ("" if none). */
KM_API const char *kmeans_last_error(void);

/* ABI version, major * 10000 + minor * 100 + patch. */
KM_API int kmeans_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KMEANS_MI355X_H */
