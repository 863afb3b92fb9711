// Assignment for scalar points (d == 1): binary search over sorted centroids.
//
// The per-row weighted 1D clustering of LLM weight rows (github
// LeanModels/LeanQuant issue #1 "1D k-means", the kmeans_fit diff) has d = 1
// and small K (16 for 4-bit, 8 for 3-bit).  There is no dot product to put on
// the matrix cores: the nearest centroid of x is one of the two centroids
// that bracket x in sorted order, because (x - c)^2 grows with |x - c| (and
// float rounding is monotone, so the same holds for the float32 distances).
//
// Each block sorts its row's K centroids in LDS by (value, index) with a
// bitonic network.  The first centroid of a run of equal values carries the
// smallest index of that value, so exact ties keep the smallest index as in
// the matrix-core path.  The distance (x - c)^2 is formed directly, with no
// cancellation, which is why every scalar problem stays on this path.
#include "common.h"

namespace km {

constexpr int kMaxK1D = 16384;  // (value, index) keys of a row fit in 128 KB of LDS
constexpr int kPts1D = 4096;    // points per block

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

// Order-preserving map of a float to uint32 (-0 is canonicalized to +0 first,
// so values that compare equal get equal keys).
__device__ __forceinline__ uint32_t orderable(float f) {
    const uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// First position p in keys[0, n) with keys[p] >= k.
__device__ __forceinline__ int lower_bound_u64(const uint64_t* keys, int n, uint64_t k) {
    int lo = 0, len = n;
    while (len > 0) {
        const int h = len >> 1;
        if (keys[lo + h] < k) {
            lo += h + 1;
            len -= h + 1;
        } else {
            len = h;
        }
    }
    return lo;
}

// keys: (orderable(value) << 32) | index, sorted ascending, so equal values
// are ordered by index and the first key of a run of equal values carries
// the smallest index of that value.
template <typename T>
__global__ __launch_bounds__(256) void k_assign_1d(const T* __restrict__ X, int64_t N,
                                                   const float* __restrict__ C, int K, int Kpow2,
                                                   const float* __restrict__ w,
                                                   int32_t* __restrict__ labels,
                                                   float* __restrict__ min_dist,
                                                   double* __restrict__ obj_part) {
    extern __shared__ uint64_t s_key[];
    __shared__ double s_obj[4];
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.y;

    for (int j = tid; j < Kpow2; j += 256) {
        s_key[j] = j < K ? ((uint64_t)orderable(round_as_point<T>(C[b * K + j])) << 32) | (uint32_t)j
                         : ~(uint64_t)0;
    }
    __syncthreads();
    // bitonic sort of Kpow2 keys
    for (int size = 2; size <= Kpow2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = tid; t < (Kpow2 >> 1); t += 256) {
                const int i = 2 * t - (t & (stride - 1));  // first element of the pair
                const int k = i + stride;
                const bool up = (i & size) == 0;
                const uint64_t a = s_key[i], c = s_key[k];
                if ((a > c) == up) {
                    s_key[i] = c;
                    s_key[k] = a;
                }
            }
            __syncthreads();
        }
    }

    const T* Xb = X + b * N;
    const int64_t i0 = (int64_t)blockIdx.x * kPts1D;
    const int64_t i1 = (i0 + kPts1D < N) ? i0 + kPts1D : N;
    double obj = 0.0;
    for (int64_t i = i0 + tid; i < i1; i += 256) {
        const float x = load_point<T>(Xb + i);
        const int m = lower_bound_u64(s_key, K, (uint64_t)orderable(x) << 32);
        float dl = INFINITY, dh = INFINITY;
        int32_t il = 0x7fffffff, ih = 0x7fffffff;
        if (m > 0) {
            // first key of the run holding the largest value below x
            const uint64_t kl = s_key[m - 1] & 0xffffffff00000000ull;
            const uint64_t first = s_key[lower_bound_u64(s_key, m, kl)];
            const float t = x - __uint_as_float(((uint32_t)(kl >> 32) & 0x80000000u)
                                                    ? ((uint32_t)(kl >> 32) & 0x7fffffffu)
                                                    : ~(uint32_t)(kl >> 32));
            dl = t * t;
            il = (int32_t)(first & 0xffffffffu);
        }
        if (m < K) {
            const uint64_t kh = s_key[m];
            const uint32_t o = (uint32_t)(kh >> 32);
            const float v = __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
            const float t = v - x;
            dh = t * t;
            ih = (int32_t)(kh & 0xffffffffu);
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
    int kp = 1;
    while (kp < K) kp <<= 1;
    const size_t lds = (size_t)kp * sizeof(uint64_t);
    if (lds > 64 * 1024) {
        hipError_t e = hipSuccess;
        if (xt == DType::F32)
            e = hipFuncSetAttribute((const void*)k_assign_1d<float>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        else if (xt == DType::F16)
            e = hipFuncSetAttribute((const void*)k_assign_1d<_Float16>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        else
            e = hipFuncSetAttribute((const void*)k_assign_1d<bf16_t>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    dim3 grid((unsigned)nblk, (unsigned)B);
    if (xt == DType::F32)
        hipLaunchKernelGGL(k_assign_1d<float>, grid, dim3(256), lds, s, (const float*)x, N, C, (int)K, kp, w,
                           labels, min_dist, obj_part);
    else if (xt == DType::F16)
        hipLaunchKernelGGL(k_assign_1d<_Float16>, grid, dim3(256), lds, s, (const _Float16*)x, N, C, (int)K,
                           kp, w, labels, min_dist, obj_part);
    else
        hipLaunchKernelGGL(k_assign_1d<bf16_t>, grid, dim3(256), lds, s, (const bf16_t*)x, N, C, (int)K, kp,
                           w, labels, min_dist, obj_part);
    return hipGetLastError();
}

}  // namespace km
