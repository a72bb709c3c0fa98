// dn_device.h -- device-side building blocks for the gfx950 kernels of the
// chunkwise gated delta rule: element types, MFMA tile products over LDS,
// global->LDS staging, small wave reductions.
//
// Every dense contraction of the chunk form is written as a product
//     D[m][n] += sum_k A[m][k] * B[n][k]
// with each operand stored in LDS either K-contiguous (A as [m][k], B as
// [n][k]) or transposed (A as [k][m], B as [k][n]); a transposed bf16 operand
// is read with ds_read_b64_tr_b16, which hands each lane 4 consecutive K values
// of one row out of 4 rows x 16 columns read by its group of 16 lanes.
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

constexpr int kWaves = 8;
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

// Four consecutive elements of T as one vector (see st4 / ld4 below).
template <typename T> struct Vec4;
template <> struct Vec4<float> { typedef f32x4 type; };
template <> struct Vec4<bf16> { typedef __attribute__((ext_vector_type(4))) __bf16 type; };

// ---------------------------------------------------------------------------
// One K-step of a 16x16 tile: load() fetches this lane's fragment of a tile
// whose first row is at p (row stride ld, at column k0 already), op() is the
// MFMA.  step() = both.
template <typename T, int KS> struct Mma;

// ds_read_b64_tr_b16 at p: within each group of 16 lanes, output lane j gets
// element j % 4 of the 8-byte pieces read by lanes 4k + j / 4 (k = 0..3).  With
// lane i of a group reading row r0 + i / 4, columns c0 + 4 (i % 4) .. + 3 of a
// row-major array, lane j receives column c0 + j of rows r0 .. r0 + 3.
__device__ __forceinline__ i16x4 tr16_b64(const bf16* p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

template <> struct Mma<bf16, 32> {
    static constexpr int kStep = 32;
    typedef bf16x8 Frag;
    __device__ __forceinline__ static Frag load(const bf16* p, int ld) {
        const int l = lane_id();
        return *reinterpret_cast<const bf16x8*>(p + (l & 15) * ld + 8 * (l >> 4));
    }
    // The same fragment from a transposed operand: p at row k0, column m0 of a
    // [k][m] array.  Lane l gets column m0 + (l & 15), rows k0 + 8 (l >> 4) + 0..7.
    __device__ __forceinline__ static Frag load_t(const bf16* p, int ld) {
        const int l = lane_id(), i = l & 15;
        const bf16* a = p + (8 * (l >> 4) + (i >> 2)) * ld + 4 * (i & 3);
        const i16x4 lo = tr16_b64(a), hi = tr16_b64(a + 4 * ld);
        const i16x4 v[2] = {lo, hi};
        return *reinterpret_cast<const bf16x8*>(v);
    }
    __device__ __forceinline__ static f32x4 op(Frag a, Frag b, f32x4 acc) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
    __device__ __forceinline__ static f32x4 step(const bf16* a, int lda, const bf16* b, int ldb, f32x4 acc) {
        return op(load(a, lda), load(b, ldb), acc);
    }
};

template <> struct Mma<bf16, 16> {
    static constexpr int kStep = 16;
    typedef i16x4 Frag;
    __device__ __forceinline__ static Frag load(const bf16* p, int ld) {
        const int l = lane_id();
        return *reinterpret_cast<const i16x4*>(p + (l & 15) * ld + 4 * (l >> 4));
    }
    // transposed operand ([k][m], p at row k0, column m0): rows k0 + 4 (l >> 4) + 0..3
    __device__ __forceinline__ static Frag load_t(const bf16* p, int ld) {
        const int l = lane_id(), i = l & 15;
        return tr16_b64(p + (4 * (l >> 4) + (i >> 2)) * ld + 4 * (i & 3));
    }
    __device__ __forceinline__ static f32x4 op(Frag a, Frag b, f32x4 acc) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
    }
    __device__ __forceinline__ static f32x4 step(const bf16* a, int lda, const bf16* b, int ldb, f32x4 acc) {
        return op(load(a, lda), load(b, ldb), acc);
    }
};

template <> struct Mma<float, 4> {
    static constexpr int kStep = 4;
    typedef float Frag;
    __device__ __forceinline__ static Frag load(const float* p, int ld) {
        const int l = lane_id();
        return p[(l & 15) * ld + (l >> 4)];
    }
    // transposed operand ([k][m], p at row k0, column m0)
    __device__ __forceinline__ static Frag load_t(const float* p, int ld) {
        const int l = lane_id();
        return p[(l >> 4) * ld + (l & 15)];
    }
    __device__ __forceinline__ static f32x4 op(Frag a, Frag b, f32x4 acc) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
    __device__ __forceinline__ static f32x4 step(const float* a, int lda, const float* b, int ldb, f32x4 acc) {
        return op(load(a, lda), load(b, ldb), acc);
    }
};

template <typename T, int K> struct MmaFor {
    static constexpr int ks = sizeof(T) == 4 ? 4 : (K % 32 == 0 ? 32 : 16);
    using type = Mma<T, ks>;
};

// The elements of an MFMA operand fragment as floats, for operands that are
// scaled per element in registers before the product: for Mma<T, KS> lane l
// holds NE = KS / 4 consecutive K values of row (l & 15), starting NE * (l >> 4)
// into the K step (the layout Mma::load reads from a K-contiguous tile).
template <typename T, int KS> struct FragF {
    static constexpr int NE = KS / 4;
    float x[NE];
    // p at the tile's first row and the K step's first column, row stride ld
    __device__ __forceinline__ static int off(int ld) { return (lane_id() & 15) * ld + NE * (lane_id() >> 4); }
    __device__ __forceinline__ void load(const T* p, int ld) {
        const T* q = p + off(ld);
        if constexpr (sizeof(T) == 2 && NE == 8) {
            const bf16x8 v = *reinterpret_cast<const bf16x8*>(q);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
        } else if constexpr (sizeof(T) == 2 && NE == 4) {
            const typename Vec4<bf16>::type v = *reinterpret_cast<const typename Vec4<bf16>::type*>(q);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (float)v[e];
        } else {
            static_assert(sizeof(T) == 4 && NE == 1, "fragment shape");
            x[0] = to_f(q[0]);
        }
    }
    // the same positions of an fp32 array (row stride ld floats, 16-byte aligned rows for NE >= 4)
    __device__ __forceinline__ static void load_f(const float* p, int ld, float (&y)[NE]) {
        const float* q = p + off(ld);
#pragma unroll
        for (int v = 0; v < NE; v += 4) {
            if constexpr (NE >= 4) {
                const f32x4 w = *reinterpret_cast<const f32x4*>(q + v);
                y[v] = w[0];
                y[v + 1] = w[1];
                y[v + 2] = w[2];
                y[v + 3] = w[3];
            }
        }
        if constexpr (NE < 4) y[0] = q[0];
    }
    __device__ __forceinline__ typename Mma<T, KS>::Frag pack() const {
        if constexpr (sizeof(T) == 2 && NE == 8) {
            return bf16x8{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3],
                          (bf16)x[4], (bf16)x[5], (bf16)x[6], (bf16)x[7]};
        } else if constexpr (sizeof(T) == 2 && NE == 4) {
            const typename Vec4<bf16>::type v = {(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
            return __builtin_bit_cast(i16x4, v);
        } else {
            return x[0];
        }
    }
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

// Static distribution of the 16x16 tiles of an M x N output over the waves.
// The waves form a WM x WN grid; each owns an RM x RN block of tiles, so one
// K step loads RM A-fragments and RN B-fragments for RM*RN MFMAs.  Outputs of
// fewer tiles than waves give one tile to each of the first waves.
template <int M, int N> struct Tiles {
    static_assert(M % 16 == 0 && N % 16 == 0, "tile dims");
    static constexpr int TM = M / 16, TN = N / 16, NT = TM * TN;
    static constexpr int pick_wm() {
        if (NT < kWaves) return TM;
        int best = 0, cost = 1 << 30;
        for (int wm = 1; wm <= kWaves; wm *= 2) {
            const int wn = kWaves / wm;
            if (TM % wm || TN % wn) continue;
            const int c = TM / wm + TN / wn;
            if (c < cost) { cost = c; best = wm; }
        }
        return best;
    }
    static constexpr int WM = pick_wm();
    static constexpr int WN = NT < kWaves ? TN : kWaves / WM;
    static constexpr int RM = TM / WM, RN = TN / WN;
    static constexpr int PER = RM * RN;
    static_assert(WM > 0 && WM * WN <= kWaves && RM * WM == TM && RN * WN == TN, "tile grid");
    __device__ __forceinline__ static bool active() { return wave_id() < WM * WN; }
    // the wave's column group (0..WN-1; its RN tiles share rows) and row group (0..WM-1)
    __device__ __forceinline__ static int cg() { return wave_id() % WN; }
    __device__ __forceinline__ static int rg() { return wave_id() / WN; }
    __device__ __forceinline__ static bool valid(int) { return active(); }
    __device__ __forceinline__ static int m0(int j) { return ((wave_id() / WN) * RM + j / RN) * 16; }
    __device__ __forceinline__ static int n0(int j) { return ((wave_id() % WN) * RN + j % RN) * 16; }
    // row / column of accumulator element i of this lane
    __device__ __forceinline__ static int row(int j, int i) { return m0(j) + 4 * (lane_id() >> 4) + i; }
    __device__ __forceinline__ static int col(int j) { return n0(j) + (lane_id() & 15); }
};

// acc[j] += A * B^T over the tiles this wave owns.  A is [M][K] (lda), B [N][K] (ldb).
template <typename T, int M, int N, int K, int NACC>
__device__ __forceinline__ void gemm_nt(f32x4 (&acc)[NACC], const T* A, int lda, const T* B, int ldb) {
    using TL = Tiles<M, N>;
    using MM = typename MmaFor<T, K>::type;
    static_assert(NACC == TL::PER, "accumulator count");
    if (!TL::active()) return;
    const T* a0 = A + TL::m0(0) * lda;
    const T* b0 = B + TL::n0(0) * ldb;
    if constexpr (sizeof(T) == 2 && MM::kStep == 16) {
        // see tile_nt: 16x16x16 chains never inherit another shape's accumulator
#pragma unroll
        for (int j = 0; j < NACC; ++j)
            acc[j] = tile_nt<T, K>(A + TL::m0(j) * lda, lda, B + TL::n0(j) * ldb, ldb, acc[j]);
    } else {
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += MM::kStep) {
            typename MM::Frag fa[TL::RM], fb[TL::RN];
#pragma unroll
            for (int im = 0; im < TL::RM; ++im) fa[im] = MM::load(a0 + im * 16 * lda + k0, lda);
#pragma unroll
            for (int in = 0; in < TL::RN; ++in) fb[in] = MM::load(b0 + in * 16 * ldb + k0, ldb);
#pragma unroll
            for (int im = 0; im < TL::RM; ++im)
#pragma unroll
                for (int in = 0; in < TL::RN; ++in)
                    acc[im * TL::RN + in] = MM::op(fa[im], fb[in], acc[im * TL::RN + in]);
        }
    }
}

// acc[j] += A * B^T over the tiles this wave owns, with A stored [M][K] (TA =
// false) or [K][M] (TA = true) and B stored [N][K] (TB = false) or [K][N] (TB =
// true).  gemm<..., false, false> is gemm_nt.
template <typename T, int M, int N, int K, bool TA, bool TB, int NACC>
__device__ __forceinline__ void gemm(f32x4 (&acc)[NACC], const T* A, int lda, const T* B, int ldb) {
    using TL = Tiles<M, N>;
    using MM = typename MmaFor<T, K>::type;
    static_assert(NACC == TL::PER, "accumulator count");
    static_assert(K % MM::kStep == 0, "K must be a multiple of the MFMA K step");
    if (!TL::active()) return;
    auto fa = [&](int im, int k0) {
        const int m = TL::m0(0) + im * 16;
        return TA ? MM::load_t(A + k0 * lda + m, lda) : MM::load(A + m * lda + k0, lda);
    };
    auto fb = [&](int in, int k0) {
        const int n = TL::n0(0) + in * 16;
        return TB ? MM::load_t(B + k0 * ldb + n, ldb) : MM::load(B + n * ldb + k0, ldb);
    };
    if constexpr (sizeof(T) == 2 && MM::kStep == 16) {
        // 16x16x16 chains never inherit another shape's accumulator (see tile_nt)
#pragma unroll
        for (int im = 0; im < TL::RM; ++im)
#pragma unroll
            for (int in = 0; in < TL::RN; ++in) {
                f32x4 part = zero4();
#pragma unroll
                for (int k0 = 0; k0 < K; k0 += MM::kStep) part = MM::op(fa(im, k0), fb(in, k0), part);
                acc[im * TL::RN + in] = acc[im * TL::RN + in] + part;
            }
    } else {
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += MM::kStep) {
            typename MM::Frag a[TL::RM], b[TL::RN];
#pragma unroll
            for (int im = 0; im < TL::RM; ++im) a[im] = fa(im, k0);
#pragma unroll
            for (int in = 0; in < TL::RN; ++in) b[in] = fb(in, k0);
#pragma unroll
            for (int im = 0; im < TL::RM; ++im)
#pragma unroll
                for (int in = 0; in < TL::RN; ++in)
                    acc[im * TL::RN + in] = MM::op(a[im], b[in], acc[im * TL::RN + in]);
        }
    }
}

// Two products with the same A: acc1 += A * B1^T, acc2 += A * B2^T (layouts as in
// gemm), each A fragment read once for both.
template <typename T, int M, int N, int K, bool TA, bool TB, int NACC>
__device__ __forceinline__ void gemm2(f32x4 (&acc1)[NACC], f32x4 (&acc2)[NACC], const T* A, int lda, const T* B1,
                                      const T* B2, int ldb) {
    using TL = Tiles<M, N>;
    using MM = typename MmaFor<T, K>::type;
    static_assert(NACC == TL::PER, "accumulator count");
    if constexpr (sizeof(T) == 2 && MM::kStep == 16) {
        gemm<T, M, N, K, TA, TB>(acc1, A, lda, B1, ldb);
        gemm<T, M, N, K, TA, TB>(acc2, A, lda, B2, ldb);
    } else {
        if (!TL::active()) return;
        auto fa = [&](int im, int k0) {
            const int m = TL::m0(0) + im * 16;
            return TA ? MM::load_t(A + k0 * lda + m, lda) : MM::load(A + m * lda + k0, lda);
        };
        auto fb = [&](const T* B, int in, int k0) {
            const int n = TL::n0(0) + in * 16;
            return TB ? MM::load_t(B + k0 * ldb + n, ldb) : MM::load(B + n * ldb + k0, ldb);
        };
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += MM::kStep) {
            typename MM::Frag a[TL::RM], b1[TL::RN], b2[TL::RN];
#pragma unroll
            for (int im = 0; im < TL::RM; ++im) a[im] = fa(im, k0);
#pragma unroll
            for (int in = 0; in < TL::RN; ++in) {
                b1[in] = fb(B1, in, k0);
                b2[in] = fb(B2, in, k0);
            }
#pragma unroll
            for (int im = 0; im < TL::RM; ++im)
#pragma unroll
                for (int in = 0; in < TL::RN; ++in) {
                    acc1[im * TL::RN + in] = MM::op(a[im], b1[in], acc1[im * TL::RN + in]);
                    acc2[im * TL::RN + in] = MM::op(a[im], b2[in], acc2[im * TL::RN + in]);
                }
        }
    }
}

template <int M, int N, int NACC>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[NACC]) {
    static_assert(NACC == Tiles<M, N>::PER, "accumulator count");
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = zero4();
}

// Four consecutive elements p[0..3] (16-byte aligned for fp32, 8-byte for bf16):
// one vector store / load.  An accumulator tile gives each lane 4 consecutive
// rows of one column, so these move a lane's 4 values of a tile whose LDS (or
// global) layout is transposed with respect to the tile.

template <typename T> __device__ __forceinline__ void st4(T* p, float a, float b, float c, float d) {
    typename Vec4<T>::type v = {from_f<T>(a), from_f<T>(b), from_f<T>(c), from_f<T>(d)};
    *reinterpret_cast<typename Vec4<T>::type*>(p) = v;
}
template <typename T> __device__ __forceinline__ void st4(T* p, f32x4 x) { st4<T>(p, x[0], x[1], x[2], x[3]); }
template <typename T> __device__ __forceinline__ f32x4 ld4(const T* p) {
    const typename Vec4<T>::type v = *reinterpret_cast<const typename Vec4<T>::type*>(p);
    return f32x4{to_f(v[0]), to_f(v[1]), to_f(v[2]), to_f(v[3])};
}

// ---------------------------------------------------------------------------
// Global -> LDS staging of a ROWS x COLS row-major tile (global row stride gld),
// rows >= valid_rows are zero.  f(r, c, x) maps each value (as float) before it
// is rounded to T.  TRANS stores lds[c * ldl + r] instead of lds[r * ldl + c]
// (through stage_t below).
template <typename T, int ROWS, int COLS, class F>
__device__ __forceinline__ void stage_t(T* lds, int ldl, const T* __restrict__ g, long gld, int valid_rows,
                                        F f);

template <typename T, int ROWS, int COLS, bool TRANS, class F>
__device__ __forceinline__ void stage(T* lds, int ldl, const T* __restrict__ g, long gld,
                                      int valid_rows, F f) {
    if constexpr (TRANS) {
        stage_t<T, ROWS, COLS>(lds, ldl, g, gld, valid_rows, f);
        return;
    }
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
        *reinterpret_cast<uint4*>(lds + r * ldl + c0) = *reinterpret_cast<const uint4*>(vals);
    }
}

// Transposing staging: lds[c * ldl + r] = f(r, c, g[r * gld + c]) for a
// ROWS x COLS row-major global tile.  Each thread moves one VW x VW block
// (VW = 16 bytes of elements): VW 16-byte row loads, a register transpose, VW
// 16-byte LDS stores.  Lanes walk the row blocks first, so one load instruction
// reads whole 128-byte row segments and one store instruction writes
// consecutive 16-byte pieces of an LDS row.  Rows >= valid_rows read as zero.
template <typename T, int ROWS, int COLS, class F>
__device__ __forceinline__ void stage_t(T* lds, int ldl, const T* __restrict__ g, long gld, int valid_rows,
                                        F f) {
    constexpr int VW = 16 / sizeof(T);
    static_assert(ROWS % VW == 0 && COLS % VW == 0, "block");
    constexpr int BR = ROWS / VW, BC = COLS / VW, NB = BR * BC;
    for (int b = threadIdx.x; b < NB; b += kThreads) {
        const int r0 = (b % BR) * VW, c0 = (b / BR) * VW;
        T v[VW][VW];
#pragma unroll
        for (int i = 0; i < VW; ++i) {
            if (r0 + i < valid_rows) {
                const uint4 raw = *reinterpret_cast<const uint4*>(g + (long)(r0 + i) * gld + c0);
                const T* src = reinterpret_cast<const T*>(&raw);
#pragma unroll
                for (int e = 0; e < VW; ++e) v[i][e] = src[e];
            } else {
#pragma unroll
                for (int e = 0; e < VW; ++e) v[i][e] = from_f<T>(0.f);
            }
        }
#pragma unroll
        for (int e = 0; e < VW; ++e) {
            T out[VW];
#pragma unroll
            for (int i = 0; i < VW; ++i) out[i] = from_f<T>(f(r0 + i, c0 + e, to_f(v[i][e])));
            *reinterpret_cast<uint4*>(lds + (c0 + e) * ldl + r0) = *reinterpret_cast<const uint4*>(out);
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
    if constexpr (TRANS)
        stage_t<T, ROWS, COLS>(lds, ldl, g, gld, valid_rows, Identity());
    else
        stage<T, ROWS, COLS, false>(lds, ldl, g, gld, valid_rows, Identity());
}

// ---------------------------------------------------------------------------
// Register-staged tiles: load() issues every global load of a tile at once, a
// later store*() maps, rounds and writes it to LDS.  Issuing the loads of the
// next chunk before computing the current one hides their latency.
//
// Loads are branch-free: addresses are clamped into the tile (rows >= valid
// read row valid - 1, surplus threads re-read the last vector) and the zeroing
// of rows >= valid happens at store time.  A load under a branch makes the
// compiler wait for it at the end of the branch, which serialises the tile.
__device__ __forceinline__ uint4 zero_u4() { return make_uint4(0u, 0u, 0u, 0u); }

// A loaded register passed through an empty asm: no use of it can be scheduled
// above this point.  Applied where a prefetched tile is consumed; otherwise the
// compiler may start reformatting the next chunk's tile right after its load
// (in the previous iteration), which makes the wave wait for the load there.
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
__device__ __forceinline__ uint4 pin(const uint4& v) {
    u32x4 x = {v.x, v.y, v.z, v.w};
    asm volatile("" : "+v"(x));
    return make_uint4(x[0], x[1], x[2], x[3]);
}

// RegN: row-major thread mapping (16-byte vectors, consecutive lanes along a
// row), for natural-layout stores.  Loads are issued in program order (a
// scheduling barrier after each): a prefetch before a loop and the one inside
// it then issue identically, and the wait counts merged at the loop head stay
// precise instead of waiting for every outstanding load and store.
template <typename T, int ROWS, int COLS> struct RegN {
    static constexpr int VW = 16 / sizeof(T), VPR = COLS / VW, NV = ROWS * VPR;
    static constexpr int PER = (NV + kThreads - 1) / kThreads;
    static_assert(COLS % VW == 0, "cols");
    uint4 r[PER];
    int valid_ = ROWS;
    __device__ __forceinline__ static int idx_of(int i) {
        const int idx = threadIdx.x + i * kThreads;
        return idx < NV ? idx : NV - 1;
    }
    // rows >= valid store as zero
    __device__ __forceinline__ void load(const T* __restrict__ g, long gld, int valid) {
        valid_ = valid;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = idx_of(i);
            const int row = idx / VPR, c0 = (idx % VPR) * VW;
            r[i] = *reinterpret_cast<const uint4*>(g + (row < valid ? row : valid - 1) * gld + c0);
            __builtin_amdgcn_sched_barrier(0);   // fixed issue order (see the note above)
        }
    }
    // rows >= valid store as row valid - 1 (for cumulative quantities)
    __device__ __forceinline__ void load_clamped(const T* __restrict__ g, long gld, int valid) {
        load(g, gld, valid);
        valid_ = ROWS;
    }
    // Two-phase: every output vector is formed (f may read LDS) before any is
    // written, so f's LDS reads are not ordered behind this tile's LDS writes.
    template <class F> __device__ __forceinline__ void store(T* lds, int ldl, F f) const {
        uint4 outv[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = idx_of(i);
            const int row = idx / VPR, c0 = (idx % VPR) * VW;
            const uint4 ri = pin(r[i]);
            const T* src = reinterpret_cast<const T*>(&ri);
            T* out = reinterpret_cast<T*>(&outv[i]);
#pragma unroll
            for (int e = 0; e < VW; ++e) {
                const float y = f(row, c0 + e, to_f(src[e]));   // unconditional: no branch around f's LDS reads
                out[e] = from_f<T>(row < valid_ ? y : 0.f);
            }
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = threadIdx.x + i * kThreads;
            if (idx >= NV) continue;
            const int row = idx / VPR, c0 = (idx % VPR) * VW;
            *reinterpret_cast<uint4*>(lds + row * ldl + c0) = outv[i];
        }
    }
    __device__ __forceinline__ void store(T* lds, int ldl) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = threadIdx.x + i * kThreads;
            if (idx >= NV) continue;
            const int row = idx / VPR, c0 = (idx % VPR) * VW;
            *reinterpret_cast<uint4*>(lds + row * ldl + c0) = row < valid_ ? pin(r[i]) : zero_u4();
        }
    }
    // Every vector times a factor of its own, s[i] (rows >= valid as zero).
    __device__ __forceinline__ void store_scaled(T* lds, int ldl, const float (&s)[PER]) const {
        uint4 outv[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = idx_of(i);
            const int row = idx / VPR;
            const uint4 ri = pin(r[i]);
            const T* src = reinterpret_cast<const T*>(&ri);
            T* out = reinterpret_cast<T*>(&outv[i]);
#pragma unroll
            for (int e = 0; e < VW; ++e) out[e] = from_f<T>(row < valid_ ? to_f(src[e]) * s[i] : 0.f);
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = threadIdx.x + i * kThreads;
            if (idx >= NV) continue;
            const int row = idx / VPR, c0 = (idx % VPR) * VW;
            *reinterpret_cast<uint4*>(lds + row * ldl + c0) = outv[i];
        }
    }
    // Two tiles from this one in one two-phase pass: f(row, col, a, y) fills y[0]
    // for l0 and y[1] for l1, so a factor both share is computed once.
    template <class F>
    __device__ __forceinline__ void store2(T* l0, T* l1, int ldl, F f) const {
        uint4 o[2][PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = idx_of(i);
            const int row = idx / VPR, c0 = (idx % VPR) * VW;
            const uint4 ra = pin(r[i]);
            const T* sa = reinterpret_cast<const T*>(&ra);
            T* d0 = reinterpret_cast<T*>(&o[0][i]);
            T* d1 = reinterpret_cast<T*>(&o[1][i]);
#pragma unroll
            for (int e = 0; e < VW; ++e) {
                float y[2];
                f(row, c0 + e, to_f(sa[e]), y);   // unconditional (see store)
                const bool ok = row < valid_;
                d0[e] = from_f<T>(ok ? y[0] : 0.f);
                d1[e] = from_f<T>(ok ? y[1] : 0.f);
            }
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = threadIdx.x + i * kThreads;
            if (idx >= NV) continue;
            const int row = idx / VPR, c0 = (idx % VPR) * VW;
            *reinterpret_cast<uint4*>(l0 + row * ldl + c0) = o[0][i];
            *reinterpret_cast<uint4*>(l1 + row * ldl + c0) = o[1][i];
        }
    }
    // Two tiles from this one whose factors come from per-element registers of
    // the caller: f(i, e, a, y) gets the vector index i (0 .. PER-1) and the
    // element e (0 .. VW-1) of the value a and fills y[0] for l0, y[1] for l1.
    template <class F>
    __device__ __forceinline__ void store2i(T* l0, T* l1, int ldl, F f) const {
        uint4 o[2][PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = idx_of(i);
            const int row = idx / VPR;
            const uint4 ra = pin(r[i]);
            const T* sa = reinterpret_cast<const T*>(&ra);
            T* d0 = reinterpret_cast<T*>(&o[0][i]);
            T* d1 = reinterpret_cast<T*>(&o[1][i]);
#pragma unroll
            for (int e = 0; e < VW; ++e) {
                float y[2];
                f(i, e, to_f(sa[e]), y);
                const bool ok = row < valid_;
                d0[e] = from_f<T>(ok ? y[0] : 0.f);
                d1[e] = from_f<T>(ok ? y[1] : 0.f);
            }
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = threadIdx.x + i * kThreads;
            if (idx >= NV) continue;
            const int row = idx / VPR, c0 = (idx % VPR) * VW;
            *reinterpret_cast<uint4*>(l0 + row * ldl + c0) = o[0][i];
            *reinterpret_cast<uint4*>(l1 + row * ldl + c0) = o[1][i];
        }
    }
    // Three tiles from this one (a) and another of the same shape (b), factors
    // from per-element registers of the caller: f(i, e, a, b, y) fills y[0..2]
    // for l0, l1, l2 (i, e as in store2i).
    template <class F>
    __device__ __forceinline__ void store3i(const RegN& b, T* l0, T* l1, T* l2, int ldl, F f) const {
        uint4 o[3][PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = idx_of(i);
            const int row = idx / VPR;
            const uint4 ra = pin(r[i]), rb = pin(b.r[i]);
            const T* sa = reinterpret_cast<const T*>(&ra);
            const T* sb = reinterpret_cast<const T*>(&rb);
            T* d0 = reinterpret_cast<T*>(&o[0][i]);
            T* d1 = reinterpret_cast<T*>(&o[1][i]);
            T* d2 = reinterpret_cast<T*>(&o[2][i]);
#pragma unroll
            for (int e = 0; e < VW; ++e) {
                float y[3];
                f(i, e, to_f(sa[e]), to_f(sb[e]), y);
                const bool ok = row < valid_;
                d0[e] = from_f<T>(ok ? y[0] : 0.f);
                d1[e] = from_f<T>(ok ? y[1] : 0.f);
                d2[e] = from_f<T>(ok ? y[2] : 0.f);
            }
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = threadIdx.x + i * kThreads;
            if (idx >= NV) continue;
            const int row = idx / VPR, c0 = (idx % VPR) * VW;
            *reinterpret_cast<uint4*>(l0 + row * ldl + c0) = o[0][i];
            *reinterpret_cast<uint4*>(l1 + row * ldl + c0) = o[1][i];
            *reinterpret_cast<uint4*>(l2 + row * ldl + c0) = o[2][i];
        }
    }
    // As store2i / store3i, into register tiles of the same shape instead of LDS
    // (rows >= valid as zero; the outputs then store as they are).
    template <class F> __device__ __forceinline__ void form2i(RegN& o0, RegN& o1, F f) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int row = idx_of(i) / VPR;
            const uint4 ra = pin(r[i]);
            const T* sa = reinterpret_cast<const T*>(&ra);
            T* d0 = reinterpret_cast<T*>(&o0.r[i]);
            T* d1 = reinterpret_cast<T*>(&o1.r[i]);
#pragma unroll
            for (int e = 0; e < VW; ++e) {
                float y[2];
                f(i, e, to_f(sa[e]), y);
                const bool ok = row < valid_;
                d0[e] = from_f<T>(ok ? y[0] : 0.f);
                d1[e] = from_f<T>(ok ? y[1] : 0.f);
            }
        }
        o0.valid_ = o1.valid_ = ROWS;
    }
    template <class F> __device__ __forceinline__ void form3i(const RegN& b, RegN& o0, RegN& o1, RegN& o2, F f) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int row = idx_of(i) / VPR;
            const uint4 ra = pin(r[i]), rb = pin(b.r[i]);
            const T* sa = reinterpret_cast<const T*>(&ra);
            const T* sb = reinterpret_cast<const T*>(&rb);
            T* d0 = reinterpret_cast<T*>(&o0.r[i]);
            T* d1 = reinterpret_cast<T*>(&o1.r[i]);
            T* d2 = reinterpret_cast<T*>(&o2.r[i]);
#pragma unroll
            for (int e = 0; e < VW; ++e) {
                float y[3];
                f(i, e, to_f(sa[e]), to_f(sb[e]), y);
                const bool ok = row < valid_;
                d0[e] = from_f<T>(ok ? y[0] : 0.f);
                d1[e] = from_f<T>(ok ? y[1] : 0.f);
                d2[e] = from_f<T>(ok ? y[2] : 0.f);
            }
        }
        o0.valid_ = o1.valid_ = o2.valid_ = ROWS;
    }
    // Three tiles from this one (a) and another of the same shape (b) in one
    // two-phase pass: f(row, col, a, b, y) fills y[0..2] for tiles l0, l1, l2, so
    // a factor the three share (a per-element gate) is computed once.
    template <class F>
    __device__ __forceinline__ void store3(const RegN& b, T* l0, T* l1, T* l2, int ldl, F f) const {
        uint4 o[3][PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = idx_of(i);
            const int row = idx / VPR, c0 = (idx % VPR) * VW;
            const uint4 ra = pin(r[i]), rb = pin(b.r[i]);
            const T* sa = reinterpret_cast<const T*>(&ra);
            const T* sb = reinterpret_cast<const T*>(&rb);
            T* d0 = reinterpret_cast<T*>(&o[0][i]);
            T* d1 = reinterpret_cast<T*>(&o[1][i]);
            T* d2 = reinterpret_cast<T*>(&o[2][i]);
#pragma unroll
            for (int e = 0; e < VW; ++e) {
                float y[3];
                f(row, c0 + e, to_f(sa[e]), to_f(sb[e]), y);   // unconditional (see store)
                const bool ok = row < valid_;
                d0[e] = from_f<T>(ok ? y[0] : 0.f);
                d1[e] = from_f<T>(ok ? y[1] : 0.f);
                d2[e] = from_f<T>(ok ? y[2] : 0.f);
            }
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = threadIdx.x + i * kThreads;
            if (idx >= NV) continue;
            const int row = idx / VPR, c0 = (idx % VPR) * VW;
            *reinterpret_cast<uint4*>(l0 + row * ldl + c0) = o[0][i];
            *reinterpret_cast<uint4*>(l1 + row * ldl + c0) = o[1][i];
            *reinterpret_cast<uint4*>(l2 + row * ldl + c0) = o[2][i];
        }
    }
};

// RegB: BRW x VW blocks per thread (lanes walk row blocks first), for
// transposed stores (register transpose) and, when the same data is also
// needed untransposed, natural stores from the same registers.  Global loads
// are 16-byte row pieces; a transposed store writes BRW elements (BRW x
// sizeof(T) bytes) of an LDS row.  BRW is the tallest block (VW, VW/2 or VW/4
// rows) that still gives every thread a block, so the tile is spread over the
// workgroup instead of piling 8 x 16 bytes on a few threads.
template <int BYTES> struct VecOf;
template <> struct VecOf<16> { typedef uint4 type; };
template <> struct VecOf<8> { typedef uint2 type; };
template <> struct VecOf<4> { typedef uint32_t type; };

template <typename T, int ROWS, int COLS> struct RegB {
    static constexpr int VW = 16 / sizeof(T);
    static constexpr int pick_brw() {
        int b = VW;
        while (b > 1 && b * sizeof(T) > 4 && (ROWS / b) * (COLS / VW) < kThreads && ROWS % (b / 2) == 0) b /= 2;
        return b;
    }
    static constexpr int BRW = pick_brw();
    static constexpr int BR = ROWS / BRW, BC = COLS / VW, NB = BR * BC;
    static constexpr int PER = (NB + kThreads - 1) / kThreads;
    static_assert(ROWS % BRW == 0 && COLS % VW == 0, "block");
    typedef typename VecOf<BRW * sizeof(T)>::type TV;   // one transposed-row piece
    uint4 r[PER][BRW];
    int valid_ = ROWS;
    __device__ __forceinline__ static int blk(int i) {
        const int b = threadIdx.x + i * kThreads;
        return b < NB ? b : NB - 1;
    }
    __device__ __forceinline__ void load(const T* __restrict__ g, long gld, int valid) {
        valid_ = valid;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int b = blk(i);
            const int r0 = (b % BR) * BRW, c0 = (b / BR) * VW;
#pragma unroll
            for (int e = 0; e < BRW; ++e) {
                const int row = r0 + e < valid ? r0 + e : valid - 1;
                r[i][e] = *reinterpret_cast<const uint4*>(g + row * gld + c0);
                __builtin_amdgcn_sched_barrier(0);   // fixed issue order (see RegN)
            }
        }
    }
    // Blocks this thread owns (threads past the last block hold a duplicate).
    __device__ __forceinline__ static bool owns(int i) { return threadIdx.x + i * kThreads < NB; }
    __device__ __forceinline__ static int col0(int i) { return (blk(i) / BR) * VW; }
    __device__ __forceinline__ static int rowblk(int i) { return blk(i) % BR; }
    // acc[i][k] += sum over the block's rows r of this[r][c] * o[r][c], c = col0(i) + k,
    // for two tiles loaded with the same shape (so the same thread mapping).
    // Every row counts: for tiles loaded with valid = ROWS.
    __device__ __forceinline__ void dot_rows(const RegB& o, float (&acc)[PER][VW]) const {
#pragma unroll
        for (int i = 0; i < PER; ++i)
#pragma unroll
            for (int e = 0; e < BRW; ++e) {
                const uint4 a = pin(r[i][e]), b = pin(o.r[i][e]);
                const T* x = reinterpret_cast<const T*>(&a);
                const T* y = reinterpret_cast<const T*>(&b);
#pragma unroll
                for (int k = 0; k < VW; ++k) acc[i][k] += to_f(x[k]) * to_f(y[k]);
            }
    }
    // lds[c * ldl + r] = f(r, c, x).  Two-phase like RegN::store.
    template <class F> __device__ __forceinline__ void store_t(T* lds, int ldl, F f) const {
        TV outv[PER][VW];
        uint4 rr[PER][BRW];
#pragma unroll
        for (int i = 0; i < PER; ++i)
#pragma unroll
            for (int k = 0; k < BRW; ++k) rr[i][k] = pin(r[i][k]);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int b = blk(i);
            const int r0 = (b % BR) * BRW, c0 = (b / BR) * VW;
#pragma unroll
            for (int e = 0; e < VW; ++e) {
                T* out = reinterpret_cast<T*>(&outv[i][e]);
#pragma unroll
                for (int k = 0; k < BRW; ++k) {
                    const float y = f(r0 + k, c0 + e, to_f(reinterpret_cast<const T*>(&rr[i][k])[e]));
                    out[k] = from_f<T>(r0 + k < valid_ ? y : 0.f);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int b = threadIdx.x + i * kThreads;
            if (b >= NB) continue;
            const int r0 = (b % BR) * BRW, c0 = (b / BR) * VW;
#pragma unroll
            for (int e = 0; e < VW; ++e) *reinterpret_cast<TV*>(lds + (c0 + e) * ldl + r0) = outv[i][e];
        }
    }
    // lds[r * ldl + c] = f(r, c, x).  Two-phase like RegN::store.
    template <class F> __device__ __forceinline__ void store_n(T* lds, int ldl, F f) const {
        uint4 outv[PER][BRW];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int b = blk(i);
            const int r0 = (b % BR) * BRW, c0 = (b / BR) * VW;
#pragma unroll
            for (int e = 0; e < BRW; ++e) {
                const uint4 ri = pin(r[i][e]);
                const T* src = reinterpret_cast<const T*>(&ri);
                T* out = reinterpret_cast<T*>(&outv[i][e]);
#pragma unroll
                for (int k = 0; k < VW; ++k) {
                    const float y = f(r0 + e, c0 + k, to_f(src[k]));
                    out[k] = from_f<T>(r0 + e < valid_ ? y : 0.f);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int b = threadIdx.x + i * kThreads;
            if (b >= NB) continue;
            const int r0 = (b % BR) * BRW, c0 = (b / BR) * VW;
#pragma unroll
            for (int e = 0; e < BRW; ++e) *reinterpret_cast<uint4*>(lds + (r0 + e) * ldl + c0) = outv[i][e];
        }
    }
};

// Coalesced write-back of a ROWS x COLS tile held in LDS (row stride ldl) to
// global memory (row stride gld), 16 bytes per thread and store; rows >=
// valid_rows are not written.
template <typename T, int ROWS, int COLS>
__device__ __forceinline__ void lds_to_global(T* __restrict__ g, long gld, const T* lds, int ldl, int valid_rows) {
    constexpr int VW = 16 / sizeof(T), VPR = COLS / VW, NV = ROWS * VPR;
    static_assert(COLS % VW == 0, "cols");
#pragma unroll
    for (int i = 0; i < (NV + kThreads - 1) / kThreads; ++i) {
        const int idx = threadIdx.x + i * kThreads;
        const int row = idx / VPR, c0 = (idx % VPR) * VW;
        if (idx < NV && row < valid_rows)
            *reinterpret_cast<uint4*>(g + row * gld + c0) = *reinterpret_cast<const uint4*>(lds + row * ldl + c0);
    }
}

// Workgroup -> (head, d_v block) for the sequential kernels (1-D grid of
// nblk * BH workgroups).  Workgroups are handed to the 8 XCDs round-robin by
// id, and each XCD has its own L2; the d_v blocks of one head read the same
// q / k / T / P tiles, so they are given ids that are equal mod 8 (same XCD,
// shared L2).  Falls back to the plain order when BH is not a multiple of 8.
constexpr int kXcds = 8;
__device__ __forceinline__ void head_and_block(int nblk, int BH, int& bh, int& blk, int id = blockIdx.x) {
    if (BH % kXcds == 0) {
        const int x = id % kXcds, k = id / kXcds;
        bh = (k / nblk) * kXcds + x;
        blk = k % nblk;
    } else {
        bh = id / nblk;
        blk = id % nblk;
    }
}

// Sum of x over the lanes l, l ^ 16, l ^ 32, l ^ 48 (one column of the four
// lane groups), in every lane.  v_permlane16_swap (v_permlane32_swap) given x
// twice returns, in each lane, its own x and that of lane l ^ 16 (l ^ 32): the
// partner's value is the first result in the upper half of each pair of lane
// groups, the second in the lower half.  VALU only; a __shfl_xor is an LDS round
// trip.
__device__ __forceinline__ float sum_lane_groups(float x) {
    const int l = lane_id();
    unsigned u = __builtin_bit_cast(unsigned, x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x += __builtin_bit_cast(float, (l & 16) ? a[0] : a[1]);
    u = __builtin_bit_cast(unsigned, x);
    const auto b = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return x + __builtin_bit_cast(float, (l & 32) ? b[0] : b[1]);
}

// x as seen from another lane of the same row of 16 lanes, by a DPP control:
// quad_perm [1,0,3,2] = 0xB1 (lane ^ 1), quad_perm [2,3,0,1] = 0x4E (lane ^ 2),
// row_half_mirror = 0x141 (lane i of 8 <- 7 - i), row_mirror = 0x140 (i of 16 <- 15 - i).
template <int CTRL> __device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes that share (lane >> 4): the lanes holding one output
// row of an MFMA tile.  Butterfly over lane ^ 1, lane ^ 2, then the other
// quad of the 8 and the other 8 of the 16 (every lane of a quad / an 8 holds
// the same partial by then); DPP moves, no LDS traffic.  Every lane of the
// wave must be active.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f<0xB1>(x);
    x += dpp_f<0x4E>(x);
    x += dpp_f<0x141>(x);
    x += dpp_f<0x140>(x);
    return x;
}

// Sum over aligned groups of N consecutive lanes (N = 1, 2, 4, 8, 16 or 32), every
// lane of a group getting the total (the DPP steps of row16_sum, then for 32 the
// partner row's sum by v_permlane16_swap, as in sum_lane_groups).
template <int N> __device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32, "group");
    if (N >= 2) x += dpp_f<0xB1>(x);
    if (N >= 4) x += dpp_f<0x4E>(x);
    if (N >= 8) x += dpp_f<0x141>(x);
    if (N >= 16) x += dpp_f<0x140>(x);
    if (N >= 32) {
        const unsigned u = __builtin_bit_cast(unsigned, x);
        const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        x += __builtin_bit_cast(float, (lane_id() & 16) ? a[0] : a[1]);
    }
    return x;
}

__device__ __forceinline__ float fexp(float x) { return __expf(x); }

}  // namespace dn
