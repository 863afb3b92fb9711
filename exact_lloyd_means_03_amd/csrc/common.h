// Internal declarations shared by the kernels and the host entry points of
// the gfx950 k-means library.  Not part of the public ABI (include/kmeans.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace km {

// Storage types of the points.
enum class DType : int { F32 = 0, F16 = 1, BF16 = 2 };

inline int dtype_bytes(DType t) { return t == DType::F32 ? 4 : 2; }

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t bf16_t;  // bfloat16 bits in memory

constexpr int kWave = 64;

// Padded point dimension used by the matrix-core assignment for a given d:
// powers of two, and 96 for 16-bit points (six 16-deep k-steps; the rows of
// 12 16-byte chunks take a rotation swizzle in LDS instead of the XOR one).
inline int padded_dim(int64_t d, bool wide16) {
    if (d <= 16) return 16;
    if (d <= 32) return 32;
    if (d <= 64) return 64;
    if (wide16 && d <= 96) return 96;
    if (d <= 128) return 128;
    if (d <= 256) return 256;
    return 512;
}

// Centroid tiles of the matrix-core assignment: tile_rows() rows in the point
// dtype (the largest of 256, 128, 64 rows that fits in 64 KB), followed by
// -|c|^2/2 of those rows as float32.  Two tiles are double-buffered in LDS.
constexpr int kTileBytesMax = 64 * 1024;
constexpr int kTileRowsMax = 256;
constexpr int tile_rows(int DP, int elem_bytes) {
    return 256 * DP * elem_bytes <= kTileBytesMax ? 256 : (128 * DP * elem_bytes <= kTileBytesMax ? 128 : 64);
}
// Waves per assignment block: rows of up to 256 bytes keep their points in
// few enough registers for 8 waves (two per SIMD); larger rows use 4 waves so
// each wave may use the whole register file.
constexpr int assign_waves(int DP, int elem_bytes) { return DP * elem_bytes <= 256 ? 8 : 4; }
constexpr int tile_bytes(int DP, int elem_bytes) {
    return tile_rows(DP, elem_bytes) * (DP * elem_bytes + 4);
}

// Rows of the padded centroid matrix: K rounded up to the largest tile.
inline int64_t padded_k(int64_t K) { return (K + kTileRowsMax - 1) / kTileRowsMax * kTileRowsMax; }

// Element conversions -------------------------------------------------------
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(_Float16 v) { return (float)v; }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float32 -> bfloat16 bits, round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Lanes of the wave whose v equals this lane's (among the lanes where
// `active` holds): one ballot per bit of the values (0 <= v < 2^nbits).
__device__ __forceinline__ uint64_t lanes_matching(int32_t v, int nbits, bool active) {
    uint64_t m = __ballot(active);
    for (int bit = 0; bit < nbits; ++bit) {
        const bool set = (v >> bit) & 1;
        const uint64_t s = __ballot(active && set);
        m &= set ? s : ~s;
    }
    return m;
}

// The same with the number of bits fixed at compile time (unrolled); bits at
// or above the values' width are zero in every active lane and change
// nothing, so NB may exceed it.
// Per bit: e = 0 or -1 by the lane's bit, s = the lanes whose bit is set, and
// s ^ e the lanes whose bit differs from this lane's; the differing lanes of
// all bits are removed from the active lanes at the end.
template <int NB>
__device__ __forceinline__ uint64_t lanes_matching_n(int32_t v, bool active) {
    uint32_t diff_lo = 0u, diff_hi = 0u;
#pragma unroll
    for (int bit = 0; bit < NB; ++bit) {
        const int32_t e = (int32_t)((uint32_t)v << (31 - bit)) >> 31;
        const uint64_t s = __ballot(e != 0);
        diff_lo |= (uint32_t)s ^ (uint32_t)e;
        diff_hi |= (uint32_t)(s >> 32) ^ (uint32_t)e;
    }
    return __ballot(active) & ~(((uint64_t)diff_hi << 32) | diff_lo);
}

// Set lanes of m below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Bits of the largest label K - 1 (0 for K == 1).
inline int label_bits(int64_t K) {
    int n = 0;
    while ((int64_t(1) << n) < K) ++n;
    return n;
}

// Workspace layout ----------------------------------------------------------
// One layout serves every entry point; all regions are 256-byte aligned.
struct Workspace {
    size_t chat;       // [B][Kp/tile_rows] tiles: rows x DP in the point dtype + -|c|^2/2 segment
    size_t obj_part;   // [B][nblk_assign] double: per-block objective partials
    size_t split;      // matrix-core assignment scratch (centroid slices)
    size_t seg_short;  // [B] int32: the sort's short-segment flags
    size_t labels;     // [B][N] int32: labels of the current assignment (fit)
    size_t counts;     // [B][K] int32
    size_t offsets;    // [B][K+1] int32
    size_t cursor;     // [B][K] int32: scatter cursors
    size_t perm;       // [B][N] int32
    size_t sums;       // [B][K][d] float: segment sums
    size_t wsum;       // [B][K] float: segment weight sums (weighted update)
    size_t piece_seg;  // [B][npieces] int32: first segment of each reduction piece
    size_t slot;       // [B][npieces][d] float: each piece's sum over its first segment
    size_t wslot;      // [B][npieces] float: its weight sum (weighted update)
    size_t gslot;      // [B][fold groups][d] float: group slots of the deterministic fold
    size_t gwslot;     // [B][fold groups] float
    size_t hist;       // [B][sort chunks][K] int32: histogram rows of the label chunks
    size_t prefix;     // [B][sort chunks][K] int32: their column prefix
    size_t total;
    int DP;
    int64_t Kp;
    int64_t nblk_assign;
};

Workspace plan_workspace(int64_t B, int64_t N, int64_t d, int64_t K, DType xt);

// Launchers (one per kernel family).  All take the caller's stream and
// return the launch status.
hipError_t launch_prep(DType xt, const float* C, int64_t B, int64_t K, int d, int DP, int64_t Kp,
                       void* blob, hipStream_t s);

// Matrix-core assignment.  nblk = assign_mfma_blocks(...) point groups per
// problem (one objective partial each); scratch: assign_mfma_scratch_bytes(...)
// bytes (zero unless the launch cuts the centroids into slices).  counts
// (may be NULL, [B][K], zero on entry): where assign_mfma_merges(...), the
// merge also counts the labels; elsewhere it is ignored.
// hist (may be NULL, unless merging): also add every label to the
// histogram row of its sort chunk, hist[b][i / sort_chunk(B, N, K)][label]
// (rows zero on entry), as the stable sort's StableCounted mode expects.
hipError_t launch_assign_mfma(DType xt, const void* x, int64_t B, int64_t N, int d, int DP,
                              const void* blob, int64_t Kp, const float* w, int32_t* labels,
                              float* min_dist, double* obj_part, int64_t nblk, void* scratch, hipStream_t s,
                              int32_t* counts = nullptr, int64_t K = 0, int32_t* hist = nullptr);
int64_t assign_mfma_blocks(int64_t B, int64_t N, int DP, DType xt, int64_t Kp);
bool assign_mfma_merges(int64_t B, int64_t N, int DP, DType xt, int64_t Kp);
size_t assign_mfma_scratch_bytes(int64_t B, int64_t N, int DP, DType xt, int64_t Kp);

// obj_part (may be NULL): the objective partial of block j of row b goes to
// obj_part[b * obj_stride + j].
hipError_t launch_assign_1d(DType xt, const void* x, int64_t B, int64_t N, const float* C,
                            int64_t K, const float* w, int32_t* labels, float* min_dist,
                            double* obj_part, int64_t obj_stride, int64_t nblk, hipStream_t s);
int64_t assign_1d_blocks(int64_t N);
bool assign_1d_supports(int64_t K);

// The sum of one problem's nblk objective partials by a block of 1024
// threads: each sums a fixed strided subset with 8 independent accumulators
// (loads stay in flight), then a fixed-order tree through red[1024] in LDS,
// so the result does not depend on timing.  Every thread of the block calls
// it; thread 0 stores the sum.
__device__ inline void obj_sum_1024(const double* __restrict__ pb, int64_t nblk, double* out, double* red) {
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int64_t i = threadIdx.x;
    for (; i + 7 * 1024 < nblk; i += 8 * 1024) {
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] += pb[i + u * 1024];
    }
#pragma unroll
    for (int u = 0; u < 7; ++u)
        if (i + u * 1024 < nblk) acc[u] += pb[i + u * 1024];
    red[threadIdx.x] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    __syncthreads();
    for (int o = 512; o >= 1; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) *out = red[0];
}

hipError_t launch_obj_reduce(const double* part, int64_t B, int64_t nblk, double* out,
                             int64_t out_stride, hipStream_t s);

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);
// dst[i] += src[i], i < n.
hipError_t launch_add_i32(int32_t* dst, const int32_t* src, int64_t n, hipStream_t s);

// Longest segment (points of one cluster) that the short-segment reduction
// takes, and the largest mean segment length for which it is tried.
constexpr int kShortSegMax = 64;
constexpr int64_t kShortSegMean = 16;

// The argsort.  Stable: labels[perm] ascending, indices ascending within a
// segment, deterministic.  Modes:
//   Stable        -- histogram the labels into hist (rows of K per chunk of
//                    sort_chunk() points), then as StableCounted;
//   StableCounted -- hist already holds the histogram rows (the assignment
//                    built them); they are cleared after use;
//   Direct        -- unordered within a segment: one global atomic per label
//                    (counts must be zero on entry; cursor needed);
//   DirectCounted -- the same with counts already holding the histogram.
enum class SortMode { Stable, StableCounted, Direct, DirectCounted };
struct SortBufs {
    int32_t* counts;      // [B][K]
    int32_t* offsets;     // [B][K+1]
    int32_t* perm;        // [B][N]
    int32_t* hist;        // [B][nch][K] (stable modes)
    int32_t* prefix;      // [B][nch][K] (stable modes)
    int32_t* cursor;      // [B][K] (direct modes)
    int32_t* piece_seg;   // [B][npieces] or NULL: first segment of every reduction piece
    int32_t* short_flag;  // [B] or NULL: 1 when no cluster has more than kShortSegMax points
    // optional: the assignment's objective partials [B][obj_nblk], summed by
    // the column scan into obj_out[b * obj_stride] (stable modes only)
    const double* obj_part = nullptr;
    int64_t obj_nblk = 0;
    double* obj_out = nullptr;
    int64_t obj_stride = 0;
};
int64_t sort_chunk(int64_t B, int64_t N, int64_t K);
int64_t sort_chunks(int64_t B, int64_t N, int64_t K);
hipError_t launch_sort(const int32_t* labels, int64_t B, int64_t N, int64_t K, const SortBufs& bufs, int TW,
                       int64_t npieces, hipStream_t s, SortMode mode);

// Segment sums of the sorted points.  Each non-empty segment is stored once,
// by the piece of TW sorted rows where it begins; the parts of a segment in
// later pieces go to those pieces' slots.  Then either
//   gslot == NULL: the slots are added into sums / wsum with atomics (sums
//                  complete afterwards; order of the adds varies), or
//   gslot != NULL: group slots are formed deterministically and
//                  launch_fold_divide() adds them in a fixed order.
// Empty clusters get nothing (their sums are not read).  short_flag (may be
// NULL): the sort's flags; problems whose clusters are all short are reduced
// one segment per row group instead (every cluster stored, empty ones 0).
hipError_t launch_segreduce(DType xt, const void* x, const float* w, int64_t B, int64_t N, int d,
                            const int32_t* perm, const int32_t* offsets, int64_t K,
                            float* sums, float* wsum, const int32_t* piece_seg, float* slot, float* wslot,
                            float* gslot, float* gwslot, const int32_t* short_flag, hipStream_t s);
// The same with a given piece width TW (the sort must have used the same).
// accumulate: add every segment into sums / wsum, which hold earlier
// contributions (the atomic fold; gslot is ignored).
hipError_t launch_segreduce_tw(DType xt, const void* x, const float* w, int64_t B, int64_t N, int d,
                               const int32_t* perm, const int32_t* offsets, int64_t K, float* sums,
                               float* wsum, const int32_t* piece_seg, float* slot, float* wslot, float* gslot,
                               float* gwslot, int TW, bool accumulate, const int32_t* short_flag, hipStream_t s);
int64_t segreduce_pieces(int64_t B, int64_t N);
int segreduce_tw(int64_t B, int64_t N);
constexpr int kFoldG = 16;  // pieces per group slot
int64_t fold_groups(int64_t npieces);

// The deterministic fold fused with the divide: per cluster, the stored sum,
// then its piece slots, then its group slots, added in that fixed order;
// then c_new = S / W (or c_old for an empty cluster).  blob (may be NULL):
// also write c_new in the tile layout of launch_prep for the next
// assignment (xt, DP, Kp describe it).
hipError_t launch_fold_divide(DType xt, const float* sums, const float* wsum, const float* slot, const float* wslot,
                              const float* gslot, const float* gwslot, const int32_t* offsets,
                              const int32_t* counts, const int32_t* short_flag, int64_t npieces, int TW, int64_t B,
                              int64_t K, int d, int DP, int64_t Kp, const float* c_old, float* c_new, void* blob,
                              hipStream_t s);

hipError_t launch_divide(const float* sums, const float* wsum, const int32_t* counts,
                         int64_t B, int64_t K, int d, const float* c_old, float* c_new,
                         hipStream_t s);
// The divide fused with the prep of the next assignment (the tile layout of
// launch_prep, from the new centroids).
hipError_t launch_divide_prep(DType xt, const float* sums, const float* wsum, const int32_t* counts, int64_t B,
                              int64_t K, int d, int DP, int64_t Kp, const float* c_old, float* c_new, void* blob,
                              hipStream_t s);

// Whole fits of scalar rows kept on chip (one block per row, all iterations).
bool fit_1d_rows_fits(int64_t N, int64_t K);
hipError_t launch_fit_1d_rows(DType xt, const void* x, const float* w, int64_t B, int64_t N, const float* init,
                              int64_t K, int n_iter, float* centroids, int32_t* labels, int32_t* counts,
                              double* objective, hipStream_t s);
// Scalar points: whole-row on-chip update (sort-inverse in LDS).
bool update_1d_row_fits(int64_t N, int64_t K);
// Few clusters (K <= 16): one wave per row, N % 4 == 0, aligned rows.
bool update_1d_few_fits(DType xt, const void* x, const float* w, const int32_t* labels, int64_t N, int64_t K);
hipError_t launch_update_1d_row(DType xt, const void* x, const float* w, int64_t B, int64_t N,
                                const int32_t* labels, int64_t K, const float* c_old,
                                float* c_new, int32_t* counts, hipStream_t s);

// Globally optimal 1D k-means (one block per row).
constexpr int kOpt1DMaxN = 4096;  // points per row
constexpr int kOpt1DMaxK = 256;   // runs per row
bool optimal_1d_supports(int64_t N, int64_t K);
void optimal_1d_workspace(int64_t B, int64_t N, int64_t K, size_t* d_off, size_t* cut_off, size_t* perm_off,
                          size_t* total);
hipError_t launch_optimal_1d(DType xt, const void* x, const float* w, int64_t B, int64_t N, int64_t K,
                             float* centroids, int32_t* labels, int32_t* counts, double* objective, void* ws,
                             hipStream_t s);

// e-means state updates (float64 sums S [K][d] and counts N [K]).
constexpr int64_t kEmeansMaxK = 32768;  // the split keeps one int per cluster in LDS
// Clears s and n after reading them.  obj_out (may be NULL): also the sum
// of the nobj objective partials obj_part.
hipError_t launch_emeans_ema(double* S, double* Nc, float* s, int32_t* n, int64_t K, int d, double a, float* C,
                             double* F, double* G, const double* obj_part, int64_t nobj, double* obj_out,
                             hipStream_t st);
bool emeans_split_supports(int64_t K);
hipError_t launch_emeans_split(double* S, double* Nc, float* C, int64_t K, int d, double dead_below, double eps,
                               const float* u, int32_t* list_j, int32_t* list_k, hipStream_t st);
hipError_t launch_emeans_final(const double* F, const double* G, int64_t K, int d, float* C, int32_t* counts,
                               hipStream_t st);

}  // namespace km
