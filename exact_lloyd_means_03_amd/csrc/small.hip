// Small per-centroid kernels of the Lloyd iteration on gfx950:
//   - centroid prep: round the float32 centroids to the point dtype (the
//     matrix-core operand) and precompute -||c_hat||^2 / 2, the centroid term
//     of ||x||^2 - 2 x.c + ||c||^2 (technologypulse.uk "Flash-KMeans"
//     article, bottleneck 1: distances fused with the argmin);
//   - the divide: centroid = segment sum / segment weight, and an empty
//     cluster keeps its previous centroid (daily.steinslab.io "e-means"
//     article, "Breaking 70 Years of Full-Batch Inertia": centroid S_j / N_j);
//   - the deterministic per-batch sum of the per-block objective partials;
//   - a fill kernel (used instead of memset so the enqueued work can be
//     captured into a graph).
#include "common.h"

namespace km {

// One element of a tile row: the centroid coordinate rounded to the point
// dtype (IEEE round to nearest even), stored; returns the rounded value.
template <typename T>
__device__ __forceinline__ float tile_elem(float v, T* out) {
    if constexpr (sizeof(T) == 4) {
        *out = v;
        return v;
    } else if constexpr (__is_same(T, _Float16)) {
        const _Float16 h = (_Float16)v;  // v_cvt_f16_f32: round to nearest even
        *out = h;
        return (float)h;
    } else {
        const uint16_t h = f32_to_bf16_rne(v);
        *out = h;
        return bf16_to_f32(h);
    }
}

// Where padded centroid row `row` of [B][Kp] lives in the tile layout: its
// elements, and the slot of its -|c|^2/2.
template <typename T>
__device__ __forceinline__ void tile_row(char* blob, int64_t row, int DP, T** out, float** hn) {
    const int TR = tile_rows(DP, (int)sizeof(T));
    const int64_t tile = row / TR;  // batches hold whole tiles (Kp is a multiple of every tile size)
    const int i = (int)(row % TR);
    char* tbase = blob + tile * tile_bytes(DP, (int)sizeof(T));
    *out = (T*)(tbase + (int64_t)i * DP * (int)sizeof(T));
    *hn = (float*)(tbase + (int64_t)TR * DP * (int)sizeof(T)) + i;
}

// One wave per padded centroid row; 4 rows per 256-thread block.  Writes the
// tile layout the matrix-core assignment copies to LDS: per tile, the rows in
// the point dtype (zero padded to DP), then -|c|^2/2 of each row (-inf for
// the padding rows K..Kp-1, which never win).
template <typename T>
__global__ __launch_bounds__(256) void k_prep(const float* __restrict__ C, int64_t BKp, int64_t K,
                                              int64_t Kp, int d, int DP, char* __restrict__ blob) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= BKp) return;
    const int64_t b = row / Kp, j = row - b * Kp;
    const bool real = j < K;
    const float* c = C + (b * K + j) * (int64_t)d;
    T* out;
    float* hn;
    tile_row<T>(blob, row, DP, &out, &hn);
    float ss = 0.f;
    for (int k = lane; k < DP; k += 64) {
        const float r = tile_elem<T>((real && k < d) ? c[k] : 0.f, out + k);
        ss = fmaf(r, r, ss);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    if (lane == 0) *hn = real ? -0.5f * ss : -INFINITY;
}

// The divide of an update fused with the prep of the next assignment: per
// padded row, c_new = S / W where the cluster has points (IEEE float32
// division), c_old otherwise, and the same row written to the tile layout as
// k_prep writes it.  c_new may alias c_old (each element is read, then
// written, by one lane).
template <typename T>
__global__ __launch_bounds__(256) void k_divide_prep(const float* __restrict__ sums,
                                                     const float* __restrict__ wsum,
                                                     const int32_t* __restrict__ counts, int64_t BKp,
                                                     int64_t K, int64_t Kp, int d, int DP, const float* c_old,
                                                     float* c_new, char* __restrict__ blob) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= BKp) return;
    const int64_t b = row / Kp, j = row - b * Kp;
    const bool real = j < K;
    const int64_t bj = b * K + j;
    const int32_t n = real ? counts[bj] : 0;
    const float W = n > 0 ? (wsum ? wsum[bj] : (float)n) : 1.f;
    T* out;
    float* hn;
    tile_row<T>(blob, row, DP, &out, &hn);
    float ss = 0.f;
    for (int k = lane; k < DP; k += 64) {
        float v = 0.f;
        if (real && k < d) {
            const int64_t i = bj * d + k;
            v = n > 0 ? sums[i] / W : c_old[i];
            c_new[i] = v;
        }
        const float r = tile_elem<T>(v, out + k);
        ss = fmaf(r, r, ss);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    if (lane == 0) *hn = real ? -0.5f * ss : -INFINITY;
}

// The deterministic fold of a Lloyd update fused with its divide (and, with
// PREP, with the prep of the next assignment).  One wave per padded centroid
// row (b, j); lane l holds coordinates l + 64 t.  For a cluster with points,
// its sum is the value its first piece stored, then the slots of the pieces
// after it that hold parts of it (the ones up to the end of the first piece's
// group of kFoldG pieces), then the group slots of the following groups,
// added in that order; the divide follows (IEEE float32, c_old for an empty
// cluster).  Problems reduced one segment per row group (skip set) have
// complete sums and no slots.
template <typename T, bool WEIGHTED, bool PREP, int DT>
__global__ __launch_bounds__(256) void k_fold_divide(
    const float* __restrict__ sums, const float* __restrict__ wsum, const float* __restrict__ slot,
    const float* __restrict__ wslot, const float* __restrict__ gslot, const float* __restrict__ gwslot,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ counts, const int32_t* __restrict__ skip,
    int64_t npieces, int64_t ngroups, int TW, int64_t BKp, int64_t K, int64_t Kp, int d, int DP,
    const float* c_old, float* c_new, char* __restrict__ blob) {
    constexpr int U = 16;  // slots in flight (a cluster of millions of points has ~100 group slots)
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= BKp) return;
    const int64_t b = row / Kp, j = row - b * Kp;
    const bool real = j < K;
    const int64_t bj = b * K + j;
    const int32_t n = real ? counts[bj] : 0;
    float acc[DT];  // coordinates lane + 64 t, t < DT (d <= 64 DT)
    float wacc = 0.f;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
        const int k = lane + 64 * t;
        acc[t] = (n > 0 && k < d) ? sums[bj * d + k] : 0.f;
    }
    if (WEIGHTED && n > 0) wacc = wsum[bj];
    if (n > 0 && !(skip && skip[b])) {
        const int32_t o0 = offsets[b * (K + 1) + j], o1 = offsets[b * (K + 1) + j + 1];
        const int64_t p_lo = o0 / TW + 1, p_hi = (o1 - 1) / TW;  // pieces holding a slot of this cluster
        const int64_t g_lo = p_lo / kFoldG, g_hi = p_hi / kFoldG;
        const int64_t ph = p_hi < (g_lo + 1) * kFoldG - 1 ? p_hi : (g_lo + 1) * kFoldG - 1;
        // piece slots up to the end of the first group, then one group slot per group
        auto add_run = [&](const float* base, const float* wbase, int64_t q0, int64_t q1) {
            for (int64_t q = q0; q <= q1; q += U) {
                float v[U][DT], wv[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const bool ok = q + u <= q1;
                    const float* sp = base + (ok ? q + u : q0) * (int64_t)d;
#pragma unroll
                    for (int t = 0; t < DT; ++t) {
                        const int k = lane + 64 * t;
                        v[u][t] = (ok && k < d) ? sp[k] : 0.f;
                    }
                    wv[u] = (WEIGHTED && ok) ? wbase[q + u] : 0.f;
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (q + u <= q1) {
#pragma unroll
                        for (int t = 0; t < DT; ++t) acc[t] += v[u][t];
                        if constexpr (WEIGHTED) wacc += wv[u];
                    }
                }
            }
        };
        if (p_lo <= p_hi) {
            add_run(slot + b * npieces * (int64_t)d, WEIGHTED ? wslot + b * npieces : nullptr, p_lo, ph);
            if (g_hi > g_lo)
                add_run(gslot + b * ngroups * (int64_t)d, WEIGHTED ? gwslot + b * ngroups : nullptr, g_lo + 1, g_hi);
        }
    }
    const float W = n > 0 ? (WEIGHTED ? wacc : (float)n) : 1.f;
    float ss = 0.f;
    T* out = nullptr;
    float* hn = nullptr;
    if constexpr (PREP) tile_row<T>(blob, row, DP, &out, &hn);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int k = lane + 64 * t;
        float v = 0.f;
        if (t < DT && real && k < d) {
            const int64_t i = bj * d + k;
            v = n > 0 ? acc[t < DT ? t : 0] / W : c_old[i];
            c_new[i] = v;
        }
        if constexpr (PREP) {
            if (k < DP) {
                const float r = tile_elem<T>(v, out + k);
                ss = fmaf(r, r, ss);
            }
        }
    }
    if constexpr (PREP) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
        if (lane == 0) *hn = real ? -0.5f * ss : -INFINITY;
    }
}

hipError_t launch_fold_divide(DType xt, const float* sums, const float* wsum, const float* slot, const float* wslot,
                              const float* gslot, const float* gwslot, const int32_t* offsets,
                              const int32_t* counts, const int32_t* short_flag, int64_t npieces, int TW, int64_t B,
                              int64_t K, int d, int DP, int64_t Kp, const float* c_old, float* c_new, void* blob,
                              hipStream_t s) {
    const bool prep = blob != nullptr;
    const int64_t Kr = prep ? Kp : K;  // rows: padded ones only to write the tile padding
    const int64_t rows = B * Kr;
    if (rows == 0) return hipSuccess;
    const int64_t ng = fold_groups(npieces);
    dim3 grid((unsigned)((rows + 3) / 4));
    char* p = (char*)blob;
#define KM_FD(TT, WW, PP, DD)                                                                               \
    hipLaunchKernelGGL((k_fold_divide<TT, WW, PP, DD>), grid, dim3(256), 0, s, sums, wsum, slot, wslot, gslot, \
                       gwslot, offsets, counts, short_flag, npieces, ng, TW, rows, K, Kr, d, DP, c_old, c_new, p)
#define KM_FD_D(TT, WW, PP)             \
    if (d <= 128) KM_FD(TT, WW, PP, 2); \
    else KM_FD(TT, WW, PP, 8);
#define KM_FD_T(TT)                           \
    if (wsum) {                               \
        if (prep) { KM_FD_D(TT, true, true) } \
        else { KM_FD_D(TT, true, false) }     \
    } else {                                  \
        if (prep) { KM_FD_D(TT, false, true) } \
        else { KM_FD_D(TT, false, false) }    \
    }
    if (xt == DType::F32) { KM_FD_T(float) }
    else if (xt == DType::F16) { KM_FD_T(_Float16) }
    else { KM_FD_T(bf16_t) }
#undef KM_FD_T
#undef KM_FD_D
#undef KM_FD
    return hipGetLastError();
}

hipError_t launch_divide_prep(DType xt, const float* sums, const float* wsum, const int32_t* counts, int64_t B,
                              int64_t K, int d, int DP, int64_t Kp, const float* c_old, float* c_new, void* blob,
                              hipStream_t s) {
    const int64_t rows = B * Kp;
    if (rows == 0) return hipSuccess;
    dim3 grid((unsigned)((rows + 3) / 4));
    char* p = (char*)blob;
    if (xt == DType::F32)
        hipLaunchKernelGGL(k_divide_prep<float>, grid, dim3(256), 0, s, sums, wsum, counts, rows, K, Kp, d, DP,
                           c_old, c_new, p);
    else if (xt == DType::F16)
        hipLaunchKernelGGL(k_divide_prep<_Float16>, grid, dim3(256), 0, s, sums, wsum, counts, rows, K, Kp, d, DP,
                           c_old, c_new, p);
    else
        hipLaunchKernelGGL(k_divide_prep<bf16_t>, grid, dim3(256), 0, s, sums, wsum, counts, rows, K, Kp, d, DP,
                           c_old, c_new, p);
    return hipGetLastError();
}

hipError_t launch_prep(DType xt, const float* C, int64_t B, int64_t K, int d, int DP, int64_t Kp,
                       void* blob, hipStream_t s) {
    const int64_t rows = B * Kp;
    if (rows == 0) return hipSuccess;
    dim3 grid((unsigned)((rows + 3) / 4));
    char* p = (char*)blob;
    if (xt == DType::F32)
        hipLaunchKernelGGL(k_prep<float>, grid, dim3(256), 0, s, C, rows, K, Kp, d, DP, p);
    else if (xt == DType::F16)
        hipLaunchKernelGGL(k_prep<_Float16>, grid, dim3(256), 0, s, C, rows, K, Kp, d, DP, p);
    else
        hipLaunchKernelGGL(k_prep<bf16_t>, grid, dim3(256), 0, s, C, rows, K, Kp, d, DP, p);
    return hipGetLastError();
}

// c_new = S / W for non-empty clusters, c_old otherwise.  W is the weight sum
// (weighted) or the count.  IEEE float32 division (no fast-math).
__global__ __launch_bounds__(256) void k_divide(const float* __restrict__ sums,
                                                const float* __restrict__ wsum,
                                                const int32_t* __restrict__ counts, int64_t BK, int d,
                                                const float* c_old, float* c_new) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = BK * d;
    if (i >= total) return;
    const int64_t bj = i / d;
    const int32_t n = counts[bj];
    float v;
    if (n > 0) {
        const float W = wsum ? wsum[bj] : (float)n;
        v = sums[i] / W;
    } else {
        v = c_old[i];
    }
    c_new[i] = v;
}

hipError_t launch_divide(const float* sums, const float* wsum, const int32_t* counts, int64_t B,
                         int64_t K, int d, const float* c_old, float* c_new, hipStream_t s) {
    const int64_t total = B * K * d;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(k_divide, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, sums, wsum,
                       counts, B * K, d, c_old, c_new);
    return hipGetLastError();
}

// One block per batch (obj_sum_1024).
__global__ __launch_bounds__(1024) void k_obj_reduce(const double* __restrict__ part, int64_t nblk,
                                                     double* __restrict__ out, int64_t out_stride) {
    __shared__ double red[1024];
    const int64_t b = blockIdx.x;
    obj_sum_1024(part + b * nblk, nblk, out + b * out_stride, red);
}

// Few partials per row (many short rows): one wave per row, four rows per block.
__global__ __launch_bounds__(256) void k_obj_reduce_rows(const double* __restrict__ part, int64_t B,
                                                         int64_t nblk, double* __restrict__ out,
                                                         int64_t out_stride) {
    const int lane = threadIdx.x & 63;
    const int64_t b = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (b >= B) return;
    const double* pb = part + b * nblk;
    double acc = 0.0;
    for (int64_t i = lane; i < nblk; i += 64) acc += pb[i];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0) out[b * out_stride] = acc;
}

hipError_t launch_obj_reduce(const double* part, int64_t B, int64_t nblk, double* out,
                             int64_t out_stride, hipStream_t s) {
    if (B == 0) return hipSuccess;
    if (nblk <= 256)
        hipLaunchKernelGGL(k_obj_reduce_rows, dim3((unsigned)((B + 3) / 4)), dim3(256), 0, s, part, B, nblk, out,
                           out_stride);
    else
        hipLaunchKernelGGL(k_obj_reduce, dim3((unsigned)B), dim3(1024), 0, s, part, nblk, out, out_stride);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_add_i32(int32_t* __restrict__ dst, const int32_t* __restrict__ src,
                                                 int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] += src[i];
}

hipError_t launch_add_i32(int32_t* dst, const int32_t* src, int64_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_add_i32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dst, src, n);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_zero(uint32_t* __restrict__ p, int64_t n_words) {
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (; i < n_words; i += stride) p[i] = 0u;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
    const int64_t words = (int64_t)(bytes / 4);
    if (words == 0) return hipSuccess;
    int64_t blocks = (words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(256), 0, s, (uint32_t*)p, words);
    return hipGetLastError();
}

}  // namespace km
