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
//
// Rows with few centroids (K <= 16, the quantization case) take a second
// kernel, one wave per chunk of a row: the wave turns the row's centroids
// into thresholds between adjacent distinct values (scalar_rows.h), keeps
// them in scalar registers, and a point's nearest centroid is its rank among
// them looked up in a table of (value, smallest index).  Both kernels give
// the same labels and distances.
#include "scalar_rows.h"

namespace km {

constexpr int kMaxK1D = 16384;  // (value, index) keys of a row fit in 128 KB of LDS
constexpr int kPts1D = 4096;    // points per block (and per wave in the few-centroid kernel)

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

// keys: (f1_ord(value) << 32) | index, sorted ascending, so equal values
// are ordered by index and the first key of a run of equal values carries
// the smallest index of that value.
template <typename T>
__global__ __launch_bounds__(256) void k_assign_1d(const T* __restrict__ X, int64_t N,
                                                   const float* __restrict__ C, int K, int Kpow2,
                                                   const float* __restrict__ w,
                                                   int32_t* __restrict__ labels,
                                                   float* __restrict__ min_dist,
                                                   double* __restrict__ obj_part, int64_t obj_stride) {
    extern __shared__ uint64_t s_key[];
    __shared__ double s_obj[4];
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.y;

    for (int j = tid; j < Kpow2; j += 256) {
        s_key[j] = j < K ? ((uint64_t)f1_ord(f1_round<T>(C[b * K + j])) << 32) | (uint32_t)j
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
        const float x = f1_load<T>(Xb + i);
        const int m = lower_bound_u64(s_key, K, (uint64_t)f1_ord(x) << 32);
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
        if (tid == 0) obj_part[b * obj_stride + blockIdx.x] = s_obj[0] + s_obj[1] + s_obj[2] + s_obj[3];
    }
}

// Few centroids (K <= KC <= 16): one wave per chunk of kPts1D points of a
// row.  Requires N % 4 == 0 and four-element-aligned rows: each lane takes
// four consecutive points per 16-byte (8-byte for 16-bit points) load, a
// wave 256 points per group, kGroups1D groups per batch; the next batch is
// loaded while the current one is assigned.
constexpr int kGroups1D = 4;

template <typename T, int KC, bool OBJ>
__global__ __launch_bounds__(64) void k_assign_1d_few(const T* __restrict__ X, int64_t N,
                                                      const float* __restrict__ C, int K,
                                                      const float* __restrict__ w,
                                                      int32_t* __restrict__ labels,
                                                      float* __restrict__ min_dist,
                                                      double* __restrict__ obj_part, int64_t obj_stride) {
    constexpr int G = kGroups1D, P = 4 * G;  // points per lane per batch
    __shared__ float s_c[kFit1DMaxK];
    __shared__ float s_val[kFit1DMaxK];
    __shared__ int s_idx[kFit1DMaxK];
    __shared__ float s_thr[kFit1DMaxK];
    const int lane = threadIdx.x;
    const int64_t b = blockIdx.y;
    const int64_t i0 = (int64_t)blockIdx.x * kPts1D;
    const int64_t i1 = (i0 + kPts1D < N) ? i0 + kPts1D : N;
    const T* Xb = X + b * N;
    const float* wb = OBJ && w ? w + b * N : nullptr;

    // point j of a batch at g0: group j / 4, element j % 4
    auto load = [&](int64_t g0, float (&xv)[P], float (&wv)[P]) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int64_t i = g0 + g * 256 + lane * 4;
            float xq[4] = {0.f, 0.f, 0.f, 0.f}, wq[4] = {0.f, 0.f, 0.f, 0.f};
            if (i < i1) {  // i1 and i are multiples of 4: the four points are in the row
                f1_load4<T>(Xb + i, xq);
                if (wb) {
                    f1_load4<float>(wb + i, wq);
                } else {
                    wq[0] = wq[1] = wq[2] = wq[3] = 1.f;
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) xv[4 * g + e] = xq[e], wv[4 * g + e] = wq[e];
        }
    };

    float xa[P], wa[P];
    load(i0, xa, wa);  // in flight while the thresholds are formed
    if (lane < K) s_c[lane] = C[b * K + lane];
    f1_wave_sync();
    const int A = f1_thresholds<T>(s_c, K, lane, s_val, s_idx, s_thr);
    f1_wave_sync();
    // ranks past A - 1 (only x = +inf reaches one) read the last real entry
    if (lane >= A && lane < kFit1DMaxK) {
        s_val[lane] = s_val[A - 1];
        s_idx[lane] = s_idx[A - 1];
    }
    f1_wave_sync();
    float tr[KC - 1];
    f1_scalar_thresholds(s_thr, tr);

    double obj = 0.0;
    for (int64_t g0 = i0; g0 < i1; g0 += 256 * G) {
        float xn[P], wn[P];
        if (g0 + 256 * G < i1) load(g0 + 256 * G, xn, wn);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int64_t i = g0 + g * 256 + lane * 4;
            int lq[4];
            float dq[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = xa[4 * g + e];
                const int m = f1_rank_sub(x, tr);
                const float t = x - s_val[m];
                dq[e] = t * t;
                lq[e] = s_idx[m];
                if constexpr (OBJ) obj += (double)wa[4 * g + e] * (double)dq[e];  // weight 0 past the end
            }
            if (i < i1) {
                typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
                const i32x4 lv = {lq[0], lq[1], lq[2], lq[3]};
                __builtin_nontemporal_store(lv, (i32x4*)(labels + b * N + i));
                if (min_dist) {
                    const f32x4 dv = {dq[0], dq[1], dq[2], dq[3]};
                    __builtin_nontemporal_store(dv, (f32x4*)(min_dist + b * N + i));
                }
            }
        }
#pragma unroll
        for (int j = 0; j < P; ++j) xa[j] = xn[j], wa[j] = wn[j];
    }
    if constexpr (OBJ) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) obj += __shfl_xor(obj, o, 64);
        if (lane == 0) obj_part[b * obj_stride + blockIdx.x] = obj;
    }
}

int64_t assign_1d_blocks(int64_t N) { return (N + kPts1D - 1) / kPts1D; }

bool assign_1d_supports(int64_t K) { return K <= kMaxK1D; }

hipError_t launch_assign_1d(DType xt, const void* x, int64_t B, int64_t N, const float* C,
                            int64_t K, const float* w, int32_t* labels, float* min_dist,
                            double* obj_part, int64_t obj_stride, int64_t nblk, hipStream_t s) {
    if (B == 0 || N == 0) return hipSuccess;
    if (K > kMaxK1D) return hipErrorInvalidValue;
    const size_t eb = xt == DType::F32 ? 16 : 8;
    const bool aligned4 = N % 4 == 0 && (uintptr_t)x % eb == 0 && (uintptr_t)labels % 16 == 0 &&
                          (uintptr_t)w % 16 == 0 && (uintptr_t)min_dist % 16 == 0;
    if (K <= kFit1DMaxK && aligned4) {
        dim3 grid((unsigned)nblk, (unsigned)B);
#define KM_A1F(TT, KK)                                                                                    \
    do {                                                                                                  \
        if (obj_part)                                                                                     \
            hipLaunchKernelGGL((k_assign_1d_few<TT, KK, true>), grid, dim3(64), 0, s, (const TT*)x, N, C, \
                               (int)K, w, labels, min_dist, obj_part, obj_stride);                        \
        else                                                                                              \
            hipLaunchKernelGGL((k_assign_1d_few<TT, KK, false>), grid, dim3(64), 0, s, (const TT*)x, N,   \
                               C, (int)K, w, labels, min_dist, obj_part, obj_stride);                     \
    } while (0)
#define KM_A1F_T(TT)              \
    if (K <= 4) KM_A1F(TT, 4);     \
    else if (K <= 8) KM_A1F(TT, 8); \
    else KM_A1F(TT, 16);
        if (xt == DType::F32) { KM_A1F_T(float) }
        else if (xt == DType::F16) { KM_A1F_T(_Float16) }
        else { KM_A1F_T(bf16_t) }
#undef KM_A1F_T
#undef KM_A1F
        return hipGetLastError();
    }
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
                           labels, min_dist, obj_part, obj_stride);
    else if (xt == DType::F16)
        hipLaunchKernelGGL(k_assign_1d<_Float16>, grid, dim3(256), lds, s, (const _Float16*)x, N, C, (int)K,
                           kp, w, labels, min_dist, obj_part, obj_stride);
    else
        hipLaunchKernelGGL(k_assign_1d<bf16_t>, grid, dim3(256), lds, s, (const bf16_t*)x, N, C, (int)K, kp,
                           w, labels, min_dist, obj_part, obj_stride);
    return hipGetLastError();
}

}  // namespace km
