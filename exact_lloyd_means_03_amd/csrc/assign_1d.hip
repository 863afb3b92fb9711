// Assignment for scalar points (d == 1): binary search over sorted centroids.
//
// The per-row weighted 1D clustering of LLM weight rows (github
// LeanModels/LeanQuant issue #1 "1D k-means", the kmeans_fit diff) has d = 1
// and small K (16 for 4-bit, 8 for 3-bit).  There is no dot product to put on
// the matrix cores: the nearest centroid of x is one of the two centroids
// that bracket x in sorted order, because (x - c)^2 grows with |x - c| (and
// float rounding is monotone, so the same holds for the float32 distances).
//
// Each block sorts its row's K centroids in LDS by (value, index).  Runs of
// equal centroid values are represented by their smallest index, so exact
// ties keep the smallest index as in the matrix-core path.
#include "common.h"

namespace km {

constexpr int kMaxK1D = 1024;
constexpr int kPts1D = 4096;  // points per block

template <typename T>
__device__ __forceinline__ float round_as_point(float v) {
    if constexpr (sizeof(T) == 4) return v;
    else if constexpr (__is_same(T, _Float16)) return (float)(_Float16)v;
    else return bf16_to_f32(f32_to_bf16_rne(v));
}

template <typename T>
__device__ __forceinline__ float load_point(const T* p) {
    if constexpr (sizeof(T) == 4) return *p;
    else if constexpr (__is_same(T, _Float16)) return (float)*p;
    else return bf16_to_f32(*p);
}

__device__ __forceinline__ int lower_bound(const float* v, int n, float x) {
    int lo = 0, len = n;
    while (len > 0) {
        const int h = len >> 1;
        if (v[lo + h] < x) {
            lo += h + 1;
            len -= h + 1;
        } else {
            len = h;
        }
    }
    return lo;
}

template <typename T>
__global__ __launch_bounds__(256) void k_assign_1d(const T* __restrict__ X, int64_t N,
                                                   const float* __restrict__ C, int K,
                                                   const float* __restrict__ w,
                                                   int32_t* __restrict__ labels,
                                                   float* __restrict__ min_dist,
                                                   double* __restrict__ obj_part) {
    __shared__ float s_raw[kMaxK1D];
    __shared__ float s_v[kMaxK1D];
    __shared__ int32_t s_i[kMaxK1D];
    __shared__ int32_t s_rep[kMaxK1D];
    __shared__ double s_obj[4];
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.y;

    for (int j = tid; j < K; j += 256) s_raw[j] = round_as_point<T>(C[b * K + j]);
    __syncthreads();
    // rank of each centroid under (value, index) order
    for (int j = tid; j < K; j += 256) {
        const float v = s_raw[j];
        int rank = 0;
        for (int i = 0; i < K; ++i) {
            const float u = s_raw[i];
            rank += (u < v) || (u == v && i < j);
        }
        s_v[rank] = v;
        s_i[rank] = j;
    }
    __syncthreads();
    for (int p = tid; p < K; p += 256) s_rep[p] = s_i[lower_bound(s_v, K, s_v[p])];
    __syncthreads();

    const T* Xb = X + b * N;
    const int64_t i0 = (int64_t)blockIdx.x * kPts1D;
    const int64_t i1 = (i0 + kPts1D < N) ? i0 + kPts1D : N;
    double obj = 0.0;
    for (int64_t i = i0 + tid; i < i1; i += 256) {
        const float x = load_point<T>(Xb + i);
        const int m = lower_bound(s_v, K, x);
        float dl = INFINITY, dh = INFINITY;
        int32_t il = 0x7fffffff, ih = 0x7fffffff;
        if (m > 0) {
            const float t = x - s_v[m - 1];
            dl = t * t;
            il = s_rep[m - 1];
        }
        if (m < K) {
            const float t = s_v[m] - x;
            dh = t * t;
            ih = s_rep[m];
        }
        const bool lo = (dl < dh) || (dl == dh && il < ih);
        const float dist = lo ? dl : dh;
        labels[b * N + i] = lo ? il : ih;
        if (min_dist) min_dist[b * N + i] = dist;
        obj += (double)(w ? w[b * N + i] : 1.f) * (double)dist;
    }
    if (obj_part) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) obj += __shfl_xor(obj, o, 64);
        if ((tid & 63) == 0) s_obj[tid >> 6] = obj;
        __syncthreads();
        if (tid == 0) obj_part[b * gridDim.x + blockIdx.x] = s_obj[0] + s_obj[1] + s_obj[2] + s_obj[3];
    }
}

int64_t assign_1d_blocks(int64_t N) { return (N + kPts1D - 1) / kPts1D; }

bool assign_1d_supports(int64_t K) { return K <= kMaxK1D; }

hipError_t launch_assign_1d(DType xt, const void* x, int64_t B, int64_t N, const float* C,
                            int64_t K, const float* w, int32_t* labels, float* min_dist,
                            double* obj_part, int64_t nblk, hipStream_t s) {
    if (B == 0 || N == 0) return hipSuccess;
    if (K > kMaxK1D) return hipErrorInvalidValue;
    dim3 grid((unsigned)nblk, (unsigned)B);
    if (xt == DType::F32)
        hipLaunchKernelGGL(k_assign_1d<float>, grid, dim3(256), 0, s, (const float*)x, N, C, (int)K, w,
                           labels, min_dist, obj_part);
    else if (xt == DType::F16)
        hipLaunchKernelGGL(k_assign_1d<_Float16>, grid, dim3(256), 0, s, (const _Float16*)x, N, C, (int)K,
                           w, labels, min_dist, obj_part);
    else
        hipLaunchKernelGGL(k_assign_1d<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)x, N, C, (int)K, w,
                           labels, min_dist, obj_part);
    return hipGetLastError();
}

}  // namespace km
