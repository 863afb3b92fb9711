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
//   * centroid tiles of up to 256 rows (64 KB, followed by their -|c|^2/2
//     values) move from device memory to LDS by direct DMA
//     (global_load_lds_dwordx4), double-buffered, and are shared by the 8 (or
//     4) waves of the block; rows are swizzled in 16-byte chunks (XOR, or a
//     rotation for 96-wide rows) so the A-operand rows read together fall in
//     distinct banks;
//   * software pipeline over 32-row blocks: the MFMAs of block s are issued
//     next to the epilogue of block s-1, so the matrix core and the vector
//     ALU work at the same time;
//   * the accumulator starts at -||c||^2 / 2 (precomputed per centroid), so
//     the matrix core produces x.c - ||c||^2 / 2 = (||x||^2 - D(x,c)) / 2 and
//     the nearest centroid is the running MAXIMUM;
//   * online argmax at block granularity: each lane holds 16 centroid rows of
//     one point per 32x32 block; it reduces them with a v_max3 chain, compares
//     once against its running best (strict '>', so the earliest block wins
//     ties) and keeps the winning block's 16 values, from which the smallest
//     row holding the maximum is recovered after the last tile.  About 1.6
//     VALU instructions per distance instead of a compare and two selects
//     each;
//   * the two half-waves that share a point merge at the end by (value, then
//     smaller index);
//   * padding centroids (K..Kp-1) start at -inf and never win;
//   * persistent blocks: the grid holds as many blocks as the device runs at
//     once, and each walks groups of points i, i + grid, ...; the tile
//     pipeline runs on from one group into the next (the next group's first
//     tile loads during the current group's last tile), which matters when
//     K is small and a group walks few tiles;
//   * a launch with fewer groups than compute units (a mini-batch against
//     many centroids) cuts the centroid tiles into slices of at least 8
//     tiles: each (group, slice) unit writes its points' best value and
//     index to scratch, and k_assign_merge keeps, per point, the best over
//     the slices (the earlier slice on equal values, so the smallest index
//     still wins ties).  Groups keep their full width, so every A fragment
//     read from LDS still feeds two matrix-core instructions.  With too few
//     tiles to slice, one column block per wave doubles the groups instead.
#include <atomic>

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

// 32-point column blocks per wave: two where rows are short (each A fragment
// read from LDS feeds two MFMAs), one for long rows.
constexpr int default_ncb(int DP, int elem_bytes) { return DP * elem_bytes <= 512 ? 2 : 1; }

template <typename T, int DP, int NCBT = default_ncb(DP, sizeof(T)), int WAVEST = assign_waves(DP, sizeof(T))>
struct AssignCfg {
    static constexpr int NCB = NCBT;                                      // 32-point blocks per wave
    static constexpr int WAVES = WAVEST;
    static constexpr int PTS = WAVES * NCB * 32;                         // points per block
    static constexpr int TK = tile_rows(DP, sizeof(T));                   // centroid rows per tile
    static_assert(TK % 64 == 0, "tiles hold an even number of 32-row blocks");
    static constexpr int NRB = TK / 32;                                  // 32-row blocks per tile
    static constexpr int RB = DP * (int)sizeof(T);                       // bytes per centroid row
    static constexpr int CPR = RB / 16;                                   // 16-byte chunks per row
    static constexpr int SW = CPR < 32 ? CPR : 32;                        // XOR swizzle period (rows)
    static constexpr bool XOR = (CPR & (CPR - 1)) == 0;                   // else the rotation swizzle
    static constexpr int TILE = tile_bytes(DP, sizeof(T));                // rows + the -|c|^2/2 floats
    static constexpr int NR = TK * RB / 1024;                             // 1 KB DMA instructions of rows
    static constexpr int HN_LANES = TK * 4 / 16;                          // lanes of the -|c|^2/2 instruction
    static constexpr int NI = NR + 1;                                     // DMA instructions per tile
    static constexpr int NIW = (NI + WAVES - 1) / WAVES;                  // ... at most per wave
    static constexpr int KSTEPS = DP / Mf<T>::KS;
    static_assert(TK * RB % 1024 == 0 && HN_LANES <= 64, "tile rows split into whole 1 KB DMA instructions");
    static_assert(2 * TILE <= 150 * 1024, "two tile buffers fit in LDS");
};

constexpr uint32_t vmcnt_imm(int n) {  // s_waitcnt with only vmcnt <= n
    return (uint32_t)((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One global_load_lds_dwordx4: lane l copies 16 bytes from sbase + voff to
// LDS byte lds + 16 l (sbase and lds are wave-uniform: an SGPR pair and M0).
// Written as a one-instruction asm statement so the compiler does not treat
// the in-flight LDS write as aliasing every later LDS read (it would wait for
// the copy right after issuing it); the kernel waits on vmcnt explicitly
// before the barrier that publishes a tile.  The instruction has no register
// results.
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, const void* lds) {
    const uint32_t l = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
                 "{m0}"(__builtin_amdgcn_readfirstlane(l))
                 : "memory");
}

// LDS chunk position of global 16-byte chunk c of tile row r.  Rows of a
// power-of-two number of chunks are XOR-swizzled, c ^ (r % SW) with SW =
// min(chunks per row, 32), so the 32 rows read by one A-operand instruction
// hit distinct banks without padding.  Rows of 12 chunks (96 16-bit
// elements, 192 bytes) start on banks that repeat every 4 rows; they are
// rotated by (r % 32) / 4 chunks, which puts the 16 rows read in one LDS
// phase (4 row starts x 4 rotations) on distinct 16-byte bank groups.
// Either way the swizzle of row r depends only on r % 32.
template <typename Cfg>
__device__ __forceinline__ int lds_chunk(int c, int r) {
    if constexpr (Cfg::XOR) return c ^ (r % Cfg::SW);
    else return (c + ((r & 31) >> 2)) % Cfg::CPR;
}

// The global chunk that LDS chunk position q of row r holds (the inverse).
template <typename Cfg>
__device__ __forceinline__ int global_chunk(int q, int r) {
    if constexpr (Cfg::XOR) return q ^ (r % Cfg::SW);
    else return (q + Cfg::CPR - ((r & 31) >> 2)) % Cfg::CPR;
}

// Source offset (within a tile) of the 16 bytes lane `lane` copies with the
// DMA instruction i (the LDS side is contiguous).  Bytes past the rows (the
// -|c|^2/2 segment and padding) are copied unchanged.
template <typename Cfg>
__device__ __forceinline__ uint32_t dma_src(int i, int lane) {
    const int p = i * 1024 + lane * 16;
    if (p >= Cfg::TK * Cfg::RB) return (uint32_t)p;
    const int r = p / Cfg::RB, q = (p % Cfg::RB) / 16;
    return (uint32_t)(r * Cfg::RB + global_chunk<Cfg>(q, r) * 16);
}

// Copy one tile (global bytes tile_g) into LDS buffer dst: wave w issues the
// instructions i = n * WAVES + w < NI with precomputed source offsets; the
// last instruction (i = NR) carries the -|c|^2/2 floats on its first
// HN_LANES lanes only.  Waves may issue different numbers of instructions;
// each waits for all of its own before the barrier that publishes the tile.
template <typename Cfg>
__device__ __forceinline__ void dma_tile(const char* tile_g, char* dst, int wave, int lane, const uint32_t* voff) {
#pragma unroll
    for (int n = 0; n < Cfg::NIW; ++n) {
        const int i = n * Cfg::WAVES + wave;
        if (i < Cfg::NR) dma16(tile_g, voff[n], dst + i * 1024);
        else if (i == Cfg::NR && lane < Cfg::HN_LANES) dma16(tile_g, voff[n], dst + i * 1024);
    }
}

template <typename T, int DP, bool VEC, int NCBT, int WAVEST>
__global__ __launch_bounds__(64 * WAVEST) void k_assign_mfma(
    const T* __restrict__ X, int64_t N, int d, const char* __restrict__ blob, int ntiles, int tps,
    const float* __restrict__ w, int32_t* __restrict__ labels, float* __restrict__ min_dist,
    double* __restrict__ obj_part, int64_t gpb, int64_t bgroups, int64_t ngroups, float* __restrict__ split,
    int32_t* __restrict__ hist, int64_t hist_ch, int64_t hist_nch, int K, int nbits) {
    typedef AssignCfg<T, DP, NCBT, WAVEST> Cfg;
    typedef Mf<T> M;
    typedef typename M::frag F;
    constexpr int NCB = Cfg::NCB, TK = Cfg::TK, RB = Cfg::RB, KSTEPS = Cfg::KSTEPS, NRB = Cfg::NRB;

    __shared__ __attribute__((aligned(1024))) char s_tile[2][Cfg::TILE];
    __shared__ double s_obj[Cfg::WAVES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, col = lane & 31;
    // Work units: group pg of PTS points of problem b against centroid slice
    // sl (tiles [sl * tps, sl * tps + tps) of the problem's ntiles), unit
    // g = sl * bgroups + b * gpb + pg; block i takes units i, i + gridDim.x, ...
    // With one slice (tps = ntiles) a unit is a whole point group.
    int64_t g = blockIdx.x;
    if (g >= ngroups) return;
    int64_t b, pg;
    int t0;
    auto decode = [&](int64_t u, int64_t& bb, int64_t& pgg, int& tt) {
        const int sl = (int)(u / bgroups);
        const int64_t r = u - sl * bgroups;
        bb = r / gpb;
        pgg = r - bb * gpb;
        tt = sl * tps;
    };
    decode(g, b, pg, t0);
    int nt = ntiles - t0 < tps ? ntiles - t0 : tps;  // tiles of this unit's slice
    const char* Bb = blob + (b * ntiles + t0) * (int64_t)Cfg::TILE;

    // per-lane DMA source offsets (the same for every tile)
    uint32_t voff[Cfg::NIW];
#pragma unroll
    for (int n = 0; n < Cfg::NIW; ++n) voff[n] = dma_src<Cfg>(n * Cfg::WAVES + wave, lane);
    // start the first tile's DMA before the point loads
    dma_tile<Cfg>(Bb, s_tile[0], wave, lane, voff);
    int par = 0;  // the buffer that holds a group's first tile

    // ---- points of this wave: B operand fragments + squared norms -------
    F bx[NCB][KSTEPS];
    float xx[NCB];
    auto load_points = [&](int64_t bb, int64_t pgg) {
        const T* Xb = X + bb * N * (int64_t)d;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int64_t p = pgg * Cfg::PTS + (wave * NCB + cb) * 32 + col;
            const bool valid = p < N;
            const T* row = Xb + (valid ? p : 0) * (int64_t)d;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
                bx[cb][ks] = load_point_frag<T, VEC>(row, ks * M::KS + half * M::EPL, d, valid);
        }
    };
    auto point_norms = [&]() {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            float s = 0.f;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) s += frag_sq<T>(bx[cb][ks]);
            xx[cb] = s + __shfl_xor(s, 32, 64);
        }
    };
    load_points(b, pg);
    point_norms();

    // running best per point: value, 32-row block that holds it, and that
    // block's 16 values of this lane (to recover the row at the end)
    float best[NCB];
    int32_t bblk[NCB];
    f32x16 saved[NCB];

    // per-lane byte offsets of the A operand in a tile (row col of block 0)
    int aoff[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
        const int ob = (ks * M::KS + half * M::EPL) * (int)sizeof(T);
        aoff[ks] = col * RB + lds_chunk<Cfg>(ob / 16, col) * 16 + (ob % 16);
    }

    // Epilogue of a finished 32-row block, cut into 8 pieces of 3-4 VALU
    // instructions per column block: max of the lane's 16 rows (v_max3
    // chain), one compare against the running best (strict '>', so the
    // earliest block wins ties), and a select that keeps the winning block's
    // 16 values (the row is recovered from them after the last tile).
    float pm[NCB];
    bool pimp[NCB];
    auto epi_piece = [&](int piece, const f32x16* v, int32_t blk) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const f32x16& a = v[cb];
            switch (piece) {
                case 0:
                    pm[cb] = fmaxf(fmaxf(a[0], a[1]), a[2]);
                    pm[cb] = fmaxf(fmaxf(pm[cb], a[3]), a[4]);
                    pm[cb] = fmaxf(fmaxf(pm[cb], a[5]), a[6]);
                    break;
                case 1:
                    pm[cb] = fmaxf(fmaxf(pm[cb], a[7]), a[8]);
                    pm[cb] = fmaxf(fmaxf(pm[cb], a[9]), a[10]);
                    pm[cb] = fmaxf(fmaxf(pm[cb], a[11]), a[12]);
                    break;
                case 2:
                    pm[cb] = fmaxf(fmaxf(pm[cb], a[13]), a[14]);
                    pm[cb] = fmaxf(pm[cb], a[15]);
                    pimp[cb] = pm[cb] > best[cb];
                    break;
                case 3: case 4: case 5: case 6: {
                    const int r0 = 4 * (piece - 3);
#pragma unroll
                    for (int r = r0; r < r0 + 4; ++r) saved[cb][r] = pimp[cb] ? a[r] : saved[cb][r];
                    break;
                }
                default:
                    best[cb] = pimp[cb] ? pm[cb] : best[cb];
                    bblk[cb] = pimp[cb] ? blk : bblk[cb];
                    break;
            }
        }
    };

    // LDS operand reads: the A fragment of k-step ks of 32-row block rb, and
    // the -|c|^2/2 values of the lane's 16 rows of block rb.
    auto lda_at = [&](const char* tile, int rb, int ks) -> F {
        const char* arow = tile + rb * 32 * RB;
        if constexpr (sizeof(T) == 4) return *(const float*)(arow + aoff[ks]);
        else return __builtin_bit_cast(F, *(const u32x4*)(arow + aoff[ks]));
    };
    auto ldh_at = [&](const char* tile, int rb) -> f32x16 {
        const float* hn = (const float*)(tile + TK * RB);
        f32x16 h;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 v = *(const f32x4*)&hn[rb * 32 + 8 * g + 4 * half];
            h[4 * g + 0] = v[0];
            h[4 * g + 1] = v[1];
            h[4 * g + 2] = v[2];
            h[4 * g + 3] = v[3];
        }
        return h;
    };

    // One 32-row block.  On entry a0, a1 hold the A fragments of its first two
    // k-steps and h the -|c|^2/2 values of its rows, which the first MFMA of
    // each column block takes as its C operand.  The A stream runs two
    // k-steps ahead across block boundaries within the tile and the next
    // block's h is read early, so LDS latency is exposed only at the start of
    // a tile.  After the MFMAs of each k-step comes one piece of the previous
    // block's epilogue, and a scheduling fence keeps that order, so the
    // matrix core and the vector ALU are busy at the same time.
    auto mma_block = [&](const char* tile, int rb, f32x16* acc, const f32x16* prev, int32_t pblk, F& a0, F& a1,
                         f32x16& h) {
        f32x16 hnext;
        constexpr int PER = (KSTEPS + 7) / 8;  // k-steps per epilogue piece
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const F a = a0;
            a0 = a1;
            const int g = rb * KSTEPS + ks + 2;  // the fragment two k-steps ahead
            if (g < NRB * KSTEPS) a1 = lda_at(tile, g / KSTEPS, g % KSTEPS);
            if (ks == (KSTEPS > 1 ? 1 : 0) && rb + 1 < NRB) hnext = ldh_at(tile, rb + 1);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) acc[cb] = M::mma(a, bx[cb][ks], ks == 0 ? h : acc[cb]);
            if (ks % PER == PER - 1 || ks == KSTEPS - 1) {
                // pieces not reached by short blocks are finished on the last k-step
                const int piece = ks / PER;
                if (ks == KSTEPS - 1) {
#pragma unroll
                    for (int pc = piece; pc < 8; ++pc) epi_piece(pc, prev, pblk);
                }
                else
                    epi_piece(piece, prev, pblk);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (rb + 1 < NRB) h = hnext;
    };
    auto epilogue = [&](const f32x16* v, int32_t blk) {
#pragma unroll
        for (int pc = 0; pc < 8; ++pc) epi_piece(pc, v, blk);
    };

    for (;;) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            best[cb] = -INFINITY;
            bblk[cb] = 0;
#pragma unroll
            for (int r = 0; r < 16; ++r) saved[cb][r] = -INFINITY;
        }
        // wait for the group's first tile, then make it visible
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();

        // the next group of this block: its first tile is loaded during this
        // group's last tile, its points while this group's outputs are written
        const int64_t gn = g + gridDim.x;
        const bool has_next = gn < ngroups;
        int64_t bn = b, pgn = pg;
        int t0n = t0;
        if (has_next) decode(gn, bn, pgn, t0n);
        const char* Bn = blob + (bn * ntiles + t0n) * (int64_t)Cfg::TILE;

        // Software pipeline over 32-row blocks (acc0 / acc1 alternate).  The loop
        // body is one basic block: every iteration issues one tile DMA (the next
        // tile, the next group's first tile, or past the end a re-read of the
        // last tile into the buffer no one reads), so the vmcnt bookkeeping is
        // the same on every iteration.
        f32x16 acc0[NCB], acc1[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc1[cb][r] = -INFINITY;
        int32_t blk1 = 0;
        for (int t = 0; t < nt; ++t) {
            const char* tile = s_tile[(par + t) & 1];
            F a0 = lda_at(tile, 0, 0);
            F a1 = KSTEPS > 1 ? lda_at(tile, 0, 1) : lda_at(tile, 1, 0);
            f32x16 h = ldh_at(tile, 0);
            const char* src = t + 1 < nt ? Bb + (t + 1) * (int64_t)Cfg::TILE
                              : has_next ? Bn
                                         : Bb + t * (int64_t)Cfg::TILE;
            dma_tile<Cfg>(src, s_tile[(par + t + 1) & 1], wave, lane, voff);
#pragma unroll
            for (int rb = 0; rb < NRB; rb += 2) {
                const int32_t blk0 = (t0 + t) * NRB + rb;
                mma_block(tile, rb, acc0, acc1, blk1, a0, a1, h);
                mma_block(tile, rb + 1, acc1, acc0, blk0, a0, a1, h);
                blk1 = blk0 + 1;
            }
            // tile t+1 must have landed before the barrier that publishes it
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            __syncthreads();
        }
        par = (par + nt) & 1;
        epilogue(acc1, blk1);

        // ---- recover the row, merge the two half-waves that share a point ----
        int32_t bidx[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            int rs = 15;
#pragma unroll
            for (int r = 15; r >= 0; --r) rs = (saved[cb][r] == best[cb]) ? r : rs;  // first (smallest) row
            bidx[cb] = bblk[cb] * 32 + 8 * (rs >> 2) + 4 * half + (rs & 3);
            const float ob = __shfl_xor(best[cb], 32, 64);
            const int32_t oi = __shfl_xor(bidx[cb], 32, 64);
            if (ob > best[cb] || (ob == best[cb] && oi < bidx[cb])) {
                best[cb] = ob;
                bidx[cb] = oi;
            }
        }
        // the next group's points load while this group's outputs are written
        // (xx keeps this group's norms until then)
        if (has_next) load_points(bn, pgn);
        double obj = 0.0;
        if (split) {
            // one slice of the centroids: its best value and centroid per
            // point (and, from the first slice, the point's squared norm) for
            // k_assign_merge; split holds [nslice][B*N] values, then as many
            // indices, then [B*N] norms
            const int64_t BN = bgroups / gpb * N, sl = t0 / tps, ns = (ntiles + tps - 1) / tps;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const int64_t p = pg * Cfg::PTS + (wave * NCB + cb) * 32 + col;
                if (half == 0 && p < N) {
                    split[sl * BN + b * N + p] = best[cb];
                    ((int32_t*)split)[(ns + sl) * BN + b * N + p] = bidx[cb];
                    if (sl == 0) split[2 * ns * BN + b * N + p] = xx[cb];
                }
            }
        } else {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const int64_t p = pg * Cfg::PTS + (wave * NCB + cb) * 32 + col;
                if (half == 0 && p < N) {
                    const float dist = fmaxf(xx[cb] - 2.f * best[cb], 0.f);
                    labels[b * N + p] = bidx[cb];
                    if (min_dist) min_dist[b * N + p] = dist;
                    obj += (double)(w ? w[b * N + p] : 1.f) * (double)dist;
                }
            }
            if (hist) {
                // the histogram row of the sort chunk that holds this group
                // (a chunk is a whole number of groups): lanes with the same
                // label add together, through their lowest lane
                int32_t* row = hist + (b * hist_nch + (pg * Cfg::PTS) / hist_ch) * (int64_t)K;
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    const int64_t p = pg * Cfg::PTS + (wave * NCB + cb) * 32 + col;
                    const bool act = half == 0 && p < N;
                    const uint64_t m = lanes_matching(bidx[cb], nbits, act);
                    if (act && lanes_below(m) == 0) atomicAdd(&row[bidx[cb]], (int32_t)__popcll(m));
                }
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
                obj_part[b * gpb + pg] = s;
            }
        }
        if (!has_next) break;
        g = gn;
        b = bn;
        pg = pgn;
        t0 = t0n;
        nt = ntiles - t0 < tps ? ntiles - t0 : tps;
        Bb = Bn;
        point_norms();
    }
    // no DMA may still be writing this block's LDS when it exits
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// Work units of a launch.  A point group is WAVES waves of NCB 32-point
// column blocks.  With at least as many groups as the chip has compute units
// a unit is a group against all centroid tiles.  With fewer (a mini-batch
// against many centroids) the tiles are cut into slices of at least
// kMinSliceTiles tiles, so that groups x slices reach the compute units while
// each group keeps its full width (every A fragment read from LDS still feeds
// NCB matrix-core instructions); k_assign_merge then picks each point's best
// over the slices.  Too few tiles to slice: one column block per wave, which
// doubles the groups, each reading the tiles for half as many points.
constexpr int64_t kFewGroups = 256;
constexpr int64_t kMinSliceTiles = 8;

struct GroupShape {
    int ncb, waves;
    int64_t nslice, tps;  // centroid slices, tiles per slice (the last one may hold fewer)
};

template <typename T>
static GroupShape group_shape(int64_t B, int64_t N, int DP, int64_t ntiles) {
    const int def = default_ncb(DP, sizeof(T)), wv = assign_waves(DP, sizeof(T));
    const int64_t pts = (int64_t)wv * def * 32;
    const int64_t groups = B * ((N + pts - 1) / pts);
    if (groups >= kFewGroups || groups == 0) return {def, wv, 1, ntiles};
    int64_t ns = (kFewGroups + groups - 1) / groups;
    if (ns > ntiles / kMinSliceTiles) ns = ntiles / kMinSliceTiles;
    if (ns >= 2) {
        const int64_t tps = (ntiles + ns - 1) / ns;
        return {def, wv, (ntiles + tps - 1) / tps, tps};
    }
    // two column blocks on half the waves (the same points per group) timed
    // the same within noise on batches of 32768..100000 points
    return {1, wv, 1, ntiles};
}

template <typename T>
static GroupShape shape_for(int64_t B, int64_t N, int DP, int64_t Kp) {
    return group_shape<T>(B, N, DP, Kp / tile_rows(DP, sizeof(T)));
}

static int64_t groups_per_problem(const GroupShape& g, int64_t N) {
    const int64_t pts = (int64_t)g.waves * g.ncb * 32;
    return (N + pts - 1) / pts;
}

static GroupShape shape_of(int64_t B, int64_t N, int DP, DType xt, int64_t Kp) {
    if (xt == DType::F32) return shape_for<float>(B, N, DP, Kp);
    if (xt == DType::F16) return shape_for<_Float16>(B, N, DP, Kp);
    return shape_for<bf16_t>(B, N, DP, Kp);
}

int64_t assign_mfma_blocks(int64_t B, int64_t N, int DP, DType xt, int64_t Kp) {
    return groups_per_problem(shape_of(B, N, DP, xt, Kp), N);
}

bool assign_mfma_merges(int64_t B, int64_t N, int DP, DType xt, int64_t Kp) {
    return shape_of(B, N, DP, xt, Kp).nslice > 1;
}

size_t assign_mfma_scratch_bytes(int64_t B, int64_t N, int DP, DType xt, int64_t Kp) {
    const GroupShape g = shape_of(B, N, DP, xt, Kp);
    if (g.nslice < 2) return 0;
    return (size_t)(2 * g.nslice + 1) * (size_t)(B * N) * 4;
}

// One block per point group: the best (largest x.c - |c|^2/2) over the
// slices, the earlier slice on equal values (its centroid indices are the
// smaller ones, and within a slice the unit already kept the smallest index),
// then the outputs as the one-slice kernel writes them.  counts (may be
// NULL, [B][K], zero on entry): also count the labels, one atomic each.
__global__ __launch_bounds__(256) void k_assign_merge(const float* __restrict__ sv, const int32_t* __restrict__ si,
                                                      const float* __restrict__ sxx, int64_t nslice, int64_t BN,
                                                      int64_t N, int pts, int64_t gpb, const float* __restrict__ w,
                                                      int32_t* __restrict__ labels, float* __restrict__ min_dist,
                                                      double* __restrict__ obj_part, int32_t* __restrict__ counts,
                                                      int64_t K) {
    __shared__ double s_obj[4];
    const int64_t grp = blockIdx.x, b = grp / gpb, pg = grp - b * gpb;
    double obj = 0.0;
    for (int q = threadIdx.x; q < pts; q += 256) {
        const int64_t p = pg * pts + q;
        if (p >= N) break;
        const int64_t i = b * N + p;
        float bv = sv[i];
        int32_t bi = si[i];
        for (int64_t sl = 1; sl < nslice; ++sl) {
            const float v = sv[sl * BN + i];
            if (v > bv) {
                bv = v;
                bi = si[sl * BN + i];
            }
        }
        const float dist = fmaxf(sxx[i] - 2.f * bv, 0.f);
        labels[i] = bi;
        if (counts && (uint64_t)bi < (uint64_t)K) atomicAdd(&counts[b * K + bi], 1);
        if (min_dist) min_dist[i] = dist;
        obj += (double)(w ? w[i] : 1.f) * (double)dist;
    }
    if (obj_part) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) obj += __shfl_xor(obj, o, 64);
        if ((threadIdx.x & 63) == 0) s_obj[threadIdx.x >> 6] = obj;
        __syncthreads();
        if (threadIdx.x == 0) obj_part[grp] = s_obj[0] + s_obj[1] + s_obj[2] + s_obj[3];
    }
}

// Persistent blocks: as many as the device holds at once (compute units x
// resident blocks per unit), each walking groups i, i + grid, ...  Cached
// per device and kernel; concurrent first calls compute the same value.
constexpr int kMaxDevices = 64;

template <typename T, int DP, bool VEC, int NCBT, int WV>
static int64_t resident_blocks() {
    static std::atomic<int64_t> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    const bool cached = dev >= 0 && dev < kMaxDevices;
    if (cached) {
        const int64_t n = cache[dev].load(std::memory_order_relaxed);
        if (n > 0) return n;
    }
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, (const void*)k_assign_mfma<T, DP, VEC, NCBT, WV>,
                                                     64 * WV, 0) != hipSuccess ||
        cus <= 0 || per <= 0)
        return 256;
    const int64_t n = (int64_t)cus * per;
    if (cached) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

template <typename T, int DP, int NCBT, int WV>
static hipError_t launch_n(const void* x, int64_t B, int64_t N, int d, const void* blob, int64_t ntiles,
                           const GroupShape& gs, const float* w, int32_t* labels, float* min_dist,
                           double* obj_part, int64_t nblk, void* scratch, int32_t* counts, int64_t K,
                           int32_t* hist, hipStream_t s) {
    const int64_t bgroups = B * nblk, ngroups = bgroups * gs.nslice;
    const bool vec = (d == DP) && ((uintptr_t)x % 16 == 0);
    const int64_t P = vec ? resident_blocks<T, DP, true, NCBT, WV>() : resident_blocks<T, DP, false, NCBT, WV>();
    dim3 grid((unsigned)(ngroups < P ? ngroups : P));
    const bool split = gs.nslice > 1;
    const int64_t BN = B * N;
    float* sv = split ? (float*)scratch : nullptr;
    const int32_t* si = split ? (const int32_t*)scratch + gs.nslice * BN : nullptr;
    const float* sxx = split ? (const float*)scratch + 2 * gs.nslice * BN : nullptr;
    double* part = split ? nullptr : obj_part;
    int32_t* hrow = split ? nullptr : hist;  // (the merge path does not build rows)
    const int64_t hch = hrow ? sort_chunk(B, N, K) : 1, hnch = hrow ? sort_chunks(B, N, K) : 1;
    const int nbits = label_bits(K);
    if (vec)
        hipLaunchKernelGGL((k_assign_mfma<T, DP, true, NCBT, WV>), grid, dim3(64 * WV), 0, s, (const T*)x, N, d,
                           (const char*)blob, (int)ntiles, (int)gs.tps, w, labels, min_dist, part, nblk, bgroups,
                           ngroups, sv, hrow, hch, hnch, (int)K, nbits);
    else
        hipLaunchKernelGGL((k_assign_mfma<T, DP, false, NCBT, WV>), grid, dim3(64 * WV), 0, s, (const T*)x, N, d,
                           (const char*)blob, (int)ntiles, (int)gs.tps, w, labels, min_dist, part, nblk, bgroups,
                           ngroups, sv, hrow, hch, hnch, (int)K, nbits);
    if (!split) return hipGetLastError();
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_assign_merge, dim3((unsigned)bgroups), dim3(256), 0, s, sv, si, sxx, gs.nslice, BN, N,
                       WV * NCBT * 32, nblk, w, labels, min_dist, obj_part, counts, K);
    return hipGetLastError();
}

// nblk: point groups per problem, as assign_mfma_blocks(B, N, DP, xt, Kp)
// gives them (the group shape follows from the same rule); scratch: at least
// assign_mfma_scratch_bytes(B, N, DP, xt, Kp) bytes (4-byte aligned).
template <typename T, int DP>
static hipError_t launch_t(const void* x, int64_t B, int64_t N, int d, const void* blob,
                           int64_t ntiles, const float* w, int32_t* labels, float* min_dist,
                           double* obj_part, int64_t nblk, void* scratch, int32_t* counts, int64_t K,
                           int32_t* hist, hipStream_t s) {
    const GroupShape g = group_shape<T>(B, N, DP, ntiles);
    if (nblk != groups_per_problem(g, N)) return hipErrorInvalidValue;
    if (g.nslice > 1 && scratch == nullptr) return hipErrorInvalidValue;
    constexpr int DEF = default_ncb(DP, sizeof(T)), WV = assign_waves(DP, sizeof(T));
    if constexpr (DEF == 2) {
        if (g.ncb == 1)
            return launch_n<T, DP, 1, WV>(x, B, N, d, blob, ntiles, g, w, labels, min_dist, obj_part, nblk,
                                          scratch, counts, K, hist, s);
    }
    return launch_n<T, DP, DEF, WV>(x, B, N, d, blob, ntiles, g, w, labels, min_dist, obj_part, nblk, scratch,
                                    counts, K, hist, s);
}

template <typename T>
static hipError_t launch_dp(int DP, const void* x, int64_t B, int64_t N, int d, const void* blob,
                            int64_t ntiles, const float* w, int32_t* labels, float* min_dist,
                            double* obj_part, int64_t nblk, void* scratch, int32_t* counts, int64_t K,
                            int32_t* hist, hipStream_t s) {
#define KM_LT(DPV) \
    launch_t<T, DPV>(x, B, N, d, blob, ntiles, w, labels, min_dist, obj_part, nblk, scratch, counts, K, hist, s)
    switch (DP) {
        case 16: return KM_LT(16);
        case 32: return KM_LT(32);
        case 64: return KM_LT(64);
        case 96:
            if constexpr (sizeof(T) == 2) return KM_LT(96);
            else return hipErrorInvalidValue;
        case 128: return KM_LT(128);
        case 256: return KM_LT(256);
        case 512:
            if constexpr (sizeof(T) == 2) return KM_LT(512);
            else return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
#undef KM_LT
}

hipError_t launch_assign_mfma(DType xt, const void* x, int64_t B, int64_t N, int d, int DP,
                              const void* blob, int64_t Kp, const float* w, int32_t* labels,
                              float* min_dist, double* obj_part, int64_t nblk, void* scratch, hipStream_t s,
                              int32_t* counts, int64_t K, int32_t* hist) {
    if (B == 0 || N == 0) return hipSuccess;
    const int64_t ntiles = Kp / tile_rows(DP, dtype_bytes(xt));
    if (xt == DType::F32)
        return launch_dp<float>(DP, x, B, N, d, blob, ntiles, w, labels, min_dist, obj_part, nblk, scratch,
                                counts, K, hist, s);
    if (xt == DType::F16)
        return launch_dp<_Float16>(DP, x, B, N, d, blob, ntiles, w, labels, min_dist, obj_part, nblk, scratch,
                                   counts, K, hist, s);
    return launch_dp<bf16_t>(DP, x, B, N, d, blob, ntiles, w, labels, min_dist, obj_part, nblk, scratch, counts,
                             K, hist, s);
}

}  // namespace km
