// Fused assignment on the gfx950 matrix cores: distance + running argmin,
// with no N x K distance matrix in device memory.
//
// Technologypulse.uk "Flash-KMeans" article, bottleneck 1, and wispaper.ai
// "Flash-KMeans" blog, "FlashAssign": point and centroid tiles are streamed
// on chip, the distance is fused with an online argmin, and the running best
// index lives in registers, so device-memory traffic is O(Nd + Kd) instead
// of O(NK).
//
// gfx950 design (ours, not the pages'):
//   * one 64-lane wave owns NCB column blocks of 32 points; their coordinates
//     stay in VGPRs for the whole kernel as the B operand of
//     v_mfma_f32_32x32x16_{f16,bf16} (v_mfma_f32_32x32x2_f32 for float32);
//   * centroid tiles of TK rows are double buffered in LDS and shared by the
//     4 waves of the block; rows are padded by 16 bytes so the 32 A-operand
//     rows read by one instruction fall in distinct banks;
//   * the accumulator starts at -||c||^2 / 2 (precomputed per centroid), so
//     the matrix core produces x.c - ||c||^2 / 2 = (||x||^2 - D(x,c)) / 2 and
//     the nearest centroid is the running MAXIMUM -- no VALU work per
//     distance besides the compare and two selects;
//   * each lane holds 16 centroid rows of one point per 32x32 block and
//     scans them in ascending index order with a strict '>', so ties keep the
//     smallest index; the two half-waves that share a point merge at the end
//     by (value, then smaller index);
//   * padding centroids (K..Kp-1) start at -inf and never win.
#include "common.h"

namespace km {

template <typename T>
struct Mf;

template <>
struct Mf<_Float16> {
    static constexpr int KS = 16;  // reduction depth of one MFMA
    static constexpr int EPL = 8;  // elements per lane per MFMA operand
    typedef f16x8 frag;
    static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Mf<bf16_t> {
    static constexpr int KS = 16;
    static constexpr int EPL = 8;
    typedef bf16x8 frag;
    static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Mf<float> {
    static constexpr int KS = 2;
    static constexpr int EPL = 1;
    typedef float frag;
    static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

template <typename T>
__device__ __forceinline__ float elem_f32(T v) {
    if constexpr (sizeof(T) == 4) return v;
    else if constexpr (__is_same(T, _Float16)) return (float)v;
    else return bf16_to_f32(v);
}

// Sum of squares of a fragment's elements, float32.
template <typename T>
__device__ __forceinline__ float frag_sq(typename Mf<T>::frag f) {
    if constexpr (sizeof(T) == 4) {
        return f * f;
    } else {
        u16x8 u = __builtin_bit_cast(u16x8, f);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v;
            if constexpr (__is_same(T, _Float16)) v = (float)__builtin_bit_cast(_Float16, (uint16_t)u[e]);
            else v = bf16_to_f32((uint16_t)u[e]);
            s = fmaf(v, v, s);
        }
        return s;
    }
}

// Load EPL consecutive elements starting at element k of a point row.
// VEC: the row is fully inside [0, d) and 16-byte aligned.
template <typename T, bool VEC>
__device__ __forceinline__ typename Mf<T>::frag load_point_frag(const T* row, int k, int d, bool valid) {
    typedef typename Mf<T>::frag F;
    if constexpr (sizeof(T) == 4) {
        return (valid && k < d) ? row[k] : 0.f;
    } else {
        if constexpr (VEC) {
            if (valid) return __builtin_bit_cast(F, *(const u32x4*)(row + k));
            return __builtin_bit_cast(F, u32x4{0u, 0u, 0u, 0u});
        } else {
            u16x8 u;
            const uint16_t* r16 = (const uint16_t*)row;
#pragma unroll
            for (int e = 0; e < 8; ++e) u[e] = (valid && k + e < d) ? r16[k + e] : (uint16_t)0;
            return __builtin_bit_cast(F, u);
        }
    }
}

template <typename T, int DP>
struct AssignCfg {
    static constexpr int NCB = (DP * (int)sizeof(T) <= 512) ? 2 : 1;   // 32-point blocks per wave
    static constexpr int WAVES = 4;
    static constexpr int PTS = WAVES * NCB * 32;                         // points per block
    static constexpr int TK = (DP * (int)sizeof(T) <= 256) ? 64 : 32;    // centroid rows per tile
    static constexpr int PAD = sizeof(T) == 4 ? 1 : 8;                   // LDS row padding (elements)
    static constexpr int LDR = DP + PAD;                                  // LDS row stride (elements)
    static constexpr int KSTEPS = DP / Mf<T>::KS;
    static constexpr int CH_PER_ROW = DP * (int)sizeof(T) / 16;          // 16-byte chunks per row
    static constexpr int TILE_CH = TK * CH_PER_ROW;                       // 16-byte chunks per tile
    static constexpr int CH_PER_THR = (TILE_CH + 255) / 256;
};

template <typename T, int DP, bool VEC>
__global__ __launch_bounds__(256) void k_assign_mfma(
    const T* __restrict__ X, int64_t N, int d, const T* __restrict__ chat,
    const float* __restrict__ hnorm, int64_t Kp, const float* __restrict__ w,
    int32_t* __restrict__ labels, float* __restrict__ min_dist, double* __restrict__ obj_part) {
    typedef AssignCfg<T, DP> Cfg;
    typedef Mf<T> M;
    typedef typename M::frag F;
    constexpr int NCB = Cfg::NCB, TK = Cfg::TK, LDR = Cfg::LDR, KSTEPS = Cfg::KSTEPS;

    __shared__ __attribute__((aligned(16))) T s_c[2][TK * LDR];
    __shared__ __attribute__((aligned(16))) float s_hn[2][TK];
    __shared__ double s_obj[Cfg::WAVES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, col = lane & 31;
    const int64_t b = blockIdx.y;
    const T* Xb = X + b * N * (int64_t)d;
    const T* Cb = chat + b * Kp * (int64_t)DP;
    const float* Hb = hnorm + b * Kp;

    // ---- points of this wave: B operand fragments + squared norms -------
    F bx[NCB][KSTEPS];
    float xx[NCB];
    int64_t pidx[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int64_t p = (int64_t)blockIdx.x * Cfg::PTS + (wave * NCB + cb) * 32 + col;
        pidx[cb] = p;
        const bool valid = p < N;
        const T* row = Xb + (valid ? p : 0) * (int64_t)d;
        float s = 0.f;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            bx[cb][ks] = load_point_frag<T, VEC>(row, ks * M::KS + half * M::EPL, d, valid);
            s += frag_sq<T>(bx[cb][ks]);
        }
        xx[cb] = s + __shfl_xor(s, 32, 64);
    }

    float best[NCB];
    int32_t bidx[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        best[cb] = -INFINITY;
        bidx[cb] = 0;
    }

    // ---- centroid tile pipeline (global -> registers -> LDS) ------------
    const int64_t ntiles = Kp / TK;
    u32x4 pre[Cfg::CH_PER_THR];
    float pre_hn = 0.f;
    auto gload = [&](int64_t t) {
        const u32x4* src = (const u32x4*)(Cb + t * TK * (int64_t)DP);
#pragma unroll
        for (int i = 0; i < Cfg::CH_PER_THR; ++i) {
            const int c = tid + i * 256;
            if (c < Cfg::TILE_CH) pre[i] = src[c];
        }
        if (tid < TK) pre_hn = Hb[t * TK + tid];
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < Cfg::CH_PER_THR; ++i) {
            const int c = tid + i * 256;
            if (c < Cfg::TILE_CH) {
                const int r = c / Cfg::CH_PER_ROW, q = c % Cfg::CH_PER_ROW;
                T* dst = &s_c[buf][r * LDR] + q * (16 / (int)sizeof(T));
                if constexpr (sizeof(T) == 4) {
                    // padded float rows are only 4-byte aligned
                    float* df = (float*)dst;
                    df[0] = __uint_as_float(pre[i][0]);
                    df[1] = __uint_as_float(pre[i][1]);
                    df[2] = __uint_as_float(pre[i][2]);
                    df[3] = __uint_as_float(pre[i][3]);
                } else {
                    *(u32x4*)dst = pre[i];
                }
            }
        }
        if (tid < TK) s_hn[buf][tid] = pre_hn;
    };

    gload(0);
    lstore(0);
    __syncthreads();

    for (int64_t t = 0; t < ntiles; ++t) {
        const int buf = (int)(t & 1);
        if (t + 1 < ntiles) gload(t + 1);

#pragma unroll
        for (int rb = 0; rb < TK / 32; ++rb) {
            // accumulator init: -||c||^2/2 of this lane's 16 rows
            f32x16 cinit;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 h = *(const f32x4*)&s_hn[buf][rb * 32 + 8 * g + 4 * half];
                cinit[4 * g + 0] = h[0];
                cinit[4 * g + 1] = h[1];
                cinit[4 * g + 2] = h[2];
                cinit[4 * g + 3] = h[3];
            }
            f32x16 acc[NCB];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) acc[cb] = cinit;
            const T* arow = &s_c[buf][(rb * 32 + col) * LDR + half * M::EPL];
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                F a;
                if constexpr (sizeof(T) == 4) a = arow[ks * M::KS];
                else a = __builtin_bit_cast(F, *(const u32x4*)(arow + ks * M::KS));
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) acc[cb] = M::mma(a, bx[cb][ks], acc[cb]);
            }
            const int32_t jbase = (int32_t)(t * TK) + rb * 32 + 4 * half;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float v = acc[cb][r];
                    const int32_t j = jbase + 8 * (r >> 2) + (r & 3);
                    const bool gt = v > best[cb];
                    best[cb] = gt ? v : best[cb];
                    bidx[cb] = gt ? j : bidx[cb];
                }
            }
        }

        if (t + 1 < ntiles) lstore(buf ^ 1);
        __syncthreads();
    }

    // ---- merge the two half-waves that share a point; write results ----
    double obj = 0.0;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const float ob = __shfl_xor(best[cb], 32, 64);
        const int32_t oi = __shfl_xor(bidx[cb], 32, 64);
        if (ob > best[cb] || (ob == best[cb] && oi < bidx[cb])) {
            best[cb] = ob;
            bidx[cb] = oi;
        }
        const int64_t p = pidx[cb];
        if (half == 0 && p < N) {
            const float dist = fmaxf(xx[cb] - 2.f * best[cb], 0.f);
            labels[b * N + p] = bidx[cb];
            if (min_dist) min_dist[b * N + p] = dist;
            obj += (double)(w ? w[b * N + p] : 1.f) * (double)dist;
        }
    }
    if (obj_part) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) obj += __shfl_xor(obj, o, 64);
        if (lane == 0) s_obj[wave] = obj;
        __syncthreads();
        if (tid == 0) {
            double s = 0.0;
#pragma unroll
            for (int i = 0; i < Cfg::WAVES; ++i) s += s_obj[i];
            obj_part[b * gridDim.x + blockIdx.x] = s;
        }
    }
}

template <typename T>
static int64_t blocks_for(int64_t N, int DP) {
    int pts = 0;
    switch (DP) {
        case 16: pts = AssignCfg<T, 16>::PTS; break;
        case 32: pts = AssignCfg<T, 32>::PTS; break;
        case 64: pts = AssignCfg<T, 64>::PTS; break;
        case 128: pts = AssignCfg<T, 128>::PTS; break;
        default: pts = AssignCfg<T, 256>::PTS; break;
    }
    return (N + pts - 1) / pts;
}

int64_t assign_mfma_blocks(int64_t N, int DP, DType xt) {
    if (xt == DType::F32) return blocks_for<float>(N, DP);
    if (xt == DType::F16) return blocks_for<_Float16>(N, DP);
    return blocks_for<bf16_t>(N, DP);
}

template <typename T, int DP>
static hipError_t launch_t(const void* x, int64_t B, int64_t N, int d, const void* chat,
                           const float* hnorm, int64_t Kp, const float* w, int32_t* labels,
                           float* min_dist, double* obj_part, int64_t nblk, hipStream_t s) {
    dim3 grid((unsigned)nblk, (unsigned)B);
    const bool vec = (d == DP) && ((uintptr_t)x % 16 == 0);
    if (vec)
        hipLaunchKernelGGL((k_assign_mfma<T, DP, true>), grid, dim3(256), 0, s, (const T*)x, N, d,
                           (const T*)chat, hnorm, Kp, w, labels, min_dist, obj_part);
    else
        hipLaunchKernelGGL((k_assign_mfma<T, DP, false>), grid, dim3(256), 0, s, (const T*)x, N, d,
                           (const T*)chat, hnorm, Kp, w, labels, min_dist, obj_part);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_dp(int DP, const void* x, int64_t B, int64_t N, int d, const void* chat,
                            const float* hnorm, int64_t Kp, const float* w, int32_t* labels,
                            float* min_dist, double* obj_part, int64_t nblk, hipStream_t s) {
    switch (DP) {
        case 16: return launch_t<T, 16>(x, B, N, d, chat, hnorm, Kp, w, labels, min_dist, obj_part, nblk, s);
        case 32: return launch_t<T, 32>(x, B, N, d, chat, hnorm, Kp, w, labels, min_dist, obj_part, nblk, s);
        case 64: return launch_t<T, 64>(x, B, N, d, chat, hnorm, Kp, w, labels, min_dist, obj_part, nblk, s);
        case 128: return launch_t<T, 128>(x, B, N, d, chat, hnorm, Kp, w, labels, min_dist, obj_part, nblk, s);
        case 256: return launch_t<T, 256>(x, B, N, d, chat, hnorm, Kp, w, labels, min_dist, obj_part, nblk, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_assign_mfma(DType xt, const void* x, int64_t B, int64_t N, int d, int DP,
                              const void* chat, const float* hnorm, int64_t K, int64_t Kp,
                              const float* w, int32_t* labels, float* min_dist, double* obj_part,
                              int64_t nblk, hipStream_t s) {
    (void)K;
    if (B == 0 || N == 0) return hipSuccess;
    if (xt == DType::F32)
        return launch_dp<float>(DP, x, B, N, d, chat, hnorm, Kp, w, labels, min_dist, obj_part, nblk, s);
    if (xt == DType::F16)
        return launch_dp<_Float16>(DP, x, B, N, d, chat, hnorm, Kp, w, labels, min_dist, obj_part, nblk, s);
    return launch_dp<bf16_t>(DP, x, B, N, d, chat, hnorm, Kp, w, labels, min_dist, obj_part, nblk, s);
}

}  // namespace km
