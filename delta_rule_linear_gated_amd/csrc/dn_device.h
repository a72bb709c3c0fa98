// dn_device.h -- device-side building blocks for the gfx950 kernels of the
// chunkwise gated delta rule: element types, MFMA tile products over LDS,
// global->LDS staging, small wave reductions.
//
// Every dense contraction of the chunk form is written as an "NT" product
//     D[m][n] += sum_k A[m][k] * B[n][k]
// with BOTH operands stored K-contiguous in LDS (A as [m][k], B as [n][k]).
// A 16x16 output tile is computed by one wave64 with
//   bf16 : v_mfma_f32_16x16x32_bf16 (K step 32) or 16x16x16bf16_1k (K step 16)
//   fp32 : v_mfma_f32_16x16x4_f32   (K step 4)
// Lane l supplies A row (l & 15) and B row (l & 15) with the same K slots, so
// the sum over K does not depend on how the instruction orders K within a step.
// The 4 accumulator floats of lane l are D[4*(l>>4) + i][l & 15], i = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dn {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// LDS row padding (elements) that keeps row starts 16-byte aligned and shifts
// consecutive rows across banks.
template <typename T> struct Pad { static constexpr int value = 16 / sizeof(T); };

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }  // RNE

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------
// One K-step of a 16x16 tile.  a/b point at the tile's first row, at column k0.
template <typename T, int KS> struct Mma;

template <> struct Mma<bf16, 32> {
    static constexpr int kStep = 32;
    __device__ __forceinline__ static f32x4 step(const bf16* a, int lda, const bf16* b, int ldb,
                                                 f32x4 acc) {
        const int l = lane_id();
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(a + (l & 15) * lda + 8 * (l >> 4));
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(b + (l & 15) * ldb + 8 * (l >> 4));
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
    }
};

template <> struct Mma<bf16, 16> {
    static constexpr int kStep = 16;
    __device__ __forceinline__ static f32x4 step(const bf16* a, int lda, const bf16* b, int ldb,
                                                 f32x4 acc) {
        const int l = lane_id();
        const i16x4 av = *reinterpret_cast<const i16x4*>(a + (l & 15) * lda + 4 * (l >> 4));
        const i16x4 bv = *reinterpret_cast<const i16x4*>(b + (l & 15) * ldb + 4 * (l >> 4));
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, acc, 0, 0, 0);
    }
};

template <> struct Mma<float, 4> {
    static constexpr int kStep = 4;
    __device__ __forceinline__ static f32x4 step(const float* a, int lda, const float* b, int ldb,
                                                 f32x4 acc) {
        const int l = lane_id();
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a[(l & 15) * lda + (l >> 4)],
                                                    b[(l & 15) * ldb + (l >> 4)], acc, 0, 0, 0);
    }
};

template <typename T, int K> struct MmaFor {
    static constexpr int ks = sizeof(T) == 4 ? 4 : (K % 32 == 0 ? 32 : 16);
    using type = Mma<T, ks>;
};

// acc += A[16 x K] * B[16 x K]^T for one tile (A, B at the tile's first rows).
//
// A chain of 16x16x16 bf16 steps never takes its accumulator from another MFMA
// shape: it starts from zero and is added to `acc` with VALU adds.  With the
// accumulator handed straight from a 16x16x32 bf16 MFMA to a dependent
// 16x16x16 bf16 MFMA the compiler emits the two back to back without wait
// states, and on gfx950 the second one then reads half-updated accumulator
// rows (observed: rows 4*(l>>4) + {0,1} of the tile come out wrong).
template <typename T, int K>
__device__ __forceinline__ f32x4 tile_nt(const T* A, int lda, const T* B, int ldb, f32x4 acc) {
    using M = typename MmaFor<T, K>::type;
    static_assert(K % M::kStep == 0, "K must be a multiple of the MFMA K step");
    if constexpr (sizeof(T) == 2 && M::kStep == 16) {
        f32x4 part = zero4();
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += M::kStep) part = M::step(A + k0, lda, B + k0, ldb, part);
        return acc + part;
    } else {
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += M::kStep) acc = M::step(A + k0, lda, B + k0, ldb, acc);
        return acc;
    }
}

// Static distribution of the 16x16 tiles of an M x N output over the 4 waves:
// wave w owns tiles w, w + 4, w + 8, ... (row-major tile order).
template <int M, int N> struct Tiles {
    static_assert(M % 16 == 0 && N % 16 == 0, "tile dims");
    static constexpr int TM = M / 16, TN = N / 16, NT = TM * TN;
    static constexpr int PER = (NT + kWaves - 1) / kWaves;
    __device__ __forceinline__ static int tile(int j) { return wave_id() + kWaves * j; }
    __device__ __forceinline__ static bool valid(int j) { return tile(j) < NT; }
    __device__ __forceinline__ static int m0(int j) { return (tile(j) / TN) * 16; }
    __device__ __forceinline__ static int n0(int j) { return (tile(j) % TN) * 16; }
    // row / column of accumulator element i of this lane
    __device__ __forceinline__ static int row(int j, int i) { return m0(j) + 4 * (lane_id() >> 4) + i; }
    __device__ __forceinline__ static int col(int j) { return n0(j) + (lane_id() & 15); }
};

// acc[j] += A * B^T over the tiles this wave owns.  A is [M][K] (lda), B [N][K] (ldb).
template <typename T, int M, int N, int K, int NACC>
__device__ __forceinline__ void gemm_nt(f32x4 (&acc)[NACC], const T* A, int lda, const T* B, int ldb) {
    using TL = Tiles<M, N>;
    static_assert(NACC == TL::PER, "accumulator count");
#pragma unroll
    for (int j = 0; j < TL::PER; ++j) {
        if (TL::valid(j)) acc[j] = tile_nt<T, K>(A + TL::m0(j) * lda, lda, B + TL::n0(j) * ldb, ldb, acc[j]);
    }
}

template <int M, int N, int NACC>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[NACC]) {
    static_assert(NACC == Tiles<M, N>::PER, "accumulator count");
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = zero4();
}

// ---------------------------------------------------------------------------
// Global -> LDS staging of a ROWS x COLS row-major tile (global row stride gld),
// rows >= valid_rows are zero.  f(r, c, x) maps each value (as float) before it
// is rounded to T.  TRANS stores lds[c * ldl + r] instead of lds[r * ldl + c].
template <typename T, int ROWS, int COLS, bool TRANS, class F>
__device__ __forceinline__ void stage(T* lds, int ldl, const T* __restrict__ g, long gld,
                                      int valid_rows, F f) {
    constexpr int VW = 16 / sizeof(T);
    static_assert(COLS % VW == 0, "cols");
    constexpr int NV = ROWS * COLS / VW;
    for (int idx = threadIdx.x; idx < NV; idx += kThreads) {
        const int r = idx / (COLS / VW);
        const int c0 = (idx % (COLS / VW)) * VW;
        T vals[VW];
        if (r < valid_rows) {
            const uint4 raw = *reinterpret_cast<const uint4*>(g + r * gld + c0);
            const T* src = reinterpret_cast<const T*>(&raw);
#pragma unroll
            for (int e = 0; e < VW; ++e) vals[e] = from_f<T>(f(r, c0 + e, to_f(src[e])));
        } else {
#pragma unroll
            for (int e = 0; e < VW; ++e) vals[e] = from_f<T>(0.f);
        }
        if (!TRANS) {
            *reinterpret_cast<uint4*>(lds + r * ldl + c0) = *reinterpret_cast<const uint4*>(vals);
        } else {
#pragma unroll
            for (int e = 0; e < VW; ++e) lds[(c0 + e) * ldl + r] = vals[e];
        }
    }
}

struct Identity {
    __device__ __forceinline__ float operator()(int, int, float x) const { return x; }
};

// Plain copy of a ROWS x COLS tile of T (no mapping), natural or transposed.
template <typename T, int ROWS, int COLS, bool TRANS>
__device__ __forceinline__ void stage_copy(T* lds, int ldl, const T* __restrict__ g, long gld,
                                           int valid_rows) {
    stage<T, ROWS, COLS, TRANS>(lds, ldl, g, gld, valid_rows, Identity());
}

// Sum over the 16 lanes that share (lane >> 4): the lanes holding one output row.
__device__ __forceinline__ float row16_sum(float x) {
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    return x;
}

__device__ __forceinline__ float fexp(float x) { return __expf(x); }

}  // namespace dn
