// dn_phase.hip -- chunkwise form of the phase-controlled gate, forward and
// reverse (SFDA summary, "Kernarchitektur" and "Der konstruktive
// Chunk-WY-Theorem", read with real q, k, v and a complex state S = S_re + i S_im):
//
//     S_t = S_{t-1} diag(exp(l_t)) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = Re(S_t q_t)
//
// with l_t = g_t + i theta_t per key channel (g shared by the channels for a
// scalar gate, zero without one).  Within a chunk of C steps, with gam the
// in-chunk cumulative sum of l, E = exp(gam), L the chunk's last row and S0 the
// state entering it, the chunk-WY form holds as for the real gates, in complex
// arithmetic (every transpose a plain one: k is real):
//     G_ts = sum_c k_tc k_sc exp(gam_tc - gam_sc)      H_ts = sum_c q_tc k_sc exp(gam_tc - gam_sc)
//     A = strictly-lower(diag(beta) G),  T = (I + A)^{-1},  P = lower(H)
//     X = (K E) S0^T,  R = diag(beta) (V - X),  U = T R
//     O = Re((Q E) S0^T + P U),   S1 = S0 diag(E_L) + U^T (K exp(gam_L - gam))
// The pair factors exp(gam_t - gam_s) of G and H are formed per pair and
// channel (the forward as exponentials of differences, the per-chunk backward as
// running products of the per-step factors), so none exceeds 1 in magnitude for
// g <= 0, at any decay.
//
// The reverse pass takes each chunk back with complex cotangents
// Zb = dL/dRe Z + i dL/dIm Z: for Z = X Y^T, Xb = Zb conj(Y) and Yb = Zb^T conj(X);
// the triangular system is one transposed solve, lambda = T^H Ub (no adjoint of
// the inverse: the ReWY abstract's residual system, conjugated here); a real
// input x entering as x w gets Re(conj(w) Zb); gam's cotangent flows through
// each exp as Eb conj(E), and dg, dtheta are the real and imaginary parts of
// its reverse cumulative sum.
//
// Four kernels, complex fp32; every product of tiles runs on the fp32 matrix
// cores as real 16x16x4 products of the real and imaginary parts, the
// exponentials and the per-element pair terms on the vector ALUs:
//   phase_prep       grid (chunk, head), every chunk at once: gam, the pairwise
//                    G and H, T by forward substitution; T, P, G per chunk out.
//   phase_fwd_state  grid (head, block of 16 state rows), chunks in order: the
//                    state recurrence, O, the chunk-entry states.
//   phase_bwd_state  grid (head, block of 16 rows), chunks last to first: Ub,
//                    lambda = T^H Ub, dv and the state cotangent; lambda and the
//                    cotangent leaving each chunk out.
//   phase_bwd_chunk  grid (chunk, head), every chunk at once: X and U again, the
//                    row sums and pair cotangents, dq, dk, dbeta, dg, dtheta.
// Row v of S1 depends only on row v of S0 (and row v of dS0 only on row v of
// dS1), so the sequential kernels split the state into blocks of 16 rows, which
// stay in LDS from chunk to chunk.
#include <hip/hip_runtime.h>

#include "dn.h"
#include "dn_device.h"
#include "dn_internal.h"

namespace dn {

namespace {

constexpr int kPT = 256;           // threads per workgroup
constexpr int kC = 16;             // chunk length
constexpr int kBV = 16;            // state rows per workgroup of the sequential kernels
constexpr int kCC = kC * kC;
constexpr int kMats = 6 * kCC;     // per chunk: T re, T im, P re, P im, G re, G im

struct cf {
    float r, i;
};
__device__ __forceinline__ cf cmul(cf a, cf b) { return {a.r * b.r - a.i * b.i, a.r * b.i + a.i * b.r}; }
__device__ __forceinline__ cf cmulc(cf a, cf b) { return {a.r * b.r + a.i * b.i, a.i * b.r - a.r * b.i}; }   // a conj(b)
__device__ __forceinline__ cf cadd(cf a, cf b) { return {a.r + b.r, a.i + b.i}; }
__device__ __forceinline__ cf csub(cf a, cf b) { return {a.r - b.r, a.i - b.i}; }
__device__ __forceinline__ cf cscale(cf a, float s) { return {a.r * s, a.i * s}; }
// exp(re + i im): the angle is reduced to a fraction of a turn in [-1/2, 1/2]
// (its error is that of im / 2 pi in fp32, about 1e-7 of a turn per turn of im),
// then v_sin / v_cos, which take turns.
__device__ __forceinline__ cf cexp_(float re, float im) {
    const float m = __expf(re);
    const float y = im * 0.15915494309189535f;
    const float fr = y - __builtin_rintf(y);
    return {m * __builtin_amdgcn_cosf(fr), m * __builtin_amdgcn_sinf(fr)};
}

// ---------------------------------------------------------------------------
// A chunk's K, Q and log gate l = g + i theta in registers: thread (channel
// c = tid % D, row group tid / D) holds NR consecutive rows, so the in-chunk
// cumulative sum is a prefix over its own rows plus the totals of the earlier
// row groups.  Rows at or past `valid` read row 0 (branch-free loads) and count
// as zero, gate included: they leave the state unchanged.  NTH threads.
template <typename TI, int GATE, int D, int NTH = kPT> struct ChunkIn {
    static constexpr int RG = NTH / D, NR = kC / RG;
    static_assert(RG * NR == kC, "rows");
    float k[NR], q[NR], lr[NR], li[NR];
    static __device__ __forceinline__ int chan() { return threadIdx.x % D; }
    static __device__ __forceinline__ int grp() { return threadIdx.x / D; }
    static __device__ __forceinline__ int row(int r) { return grp() * NR + r; }
    __device__ __forceinline__ void load(const Params& p, long row0, int valid) {
        // the chunk's rows from uniform bases, per-lane 32-bit offsets
        const TI* __restrict__ kp = static_cast<const TI*>(p.k) + row0 * D;
        const TI* __restrict__ qp = static_cast<const TI*>(p.q) + row0 * D;
        const float* __restrict__ thp = p.theta + row0 * D;
        const float* __restrict__ gp = p.g + (GATE == kGateVector ? row0 * D : row0);
        const int c = chan();
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int t = row(r);
            const bool ok = t < valid;
            const int rr = ok ? t : 0, e = rr * D + c;
            const float kk = to_f(kp[e]), qq = to_f(qp[e]), th = thp[e];
            float g = 0.f;
            if (GATE == kGateScalar) g = gp[rr];
            if (GATE == kGateVector) g = gp[e];
            k[r] = ok ? kk : 0.f;
            q[r] = ok ? qq : 0.f;
            lr[r] = ok ? g : 0.f;
            li[r] = ok ? th : 0.f;
        }
    }
    // Inclusive prefix over the thread's rows, in place; the totals to tr / ti.
    __device__ __forceinline__ void prefix(float (*tr)[D], float (*ti)[D]) {
#pragma unroll
        for (int r = 1; r < NR; ++r) {
            lr[r] += lr[r - 1];
            li[r] += li[r - 1];
        }
        tr[grp()][chan()] = lr[NR - 1];
        ti[grp()][chan()] = li[NR - 1];
    }
    // After a barrier: the earlier groups' totals are added (lr, li become gam);
    // returns gam at the chunk's last row, summed in the same order as the last
    // row's own value (the rows past `valid` add zeros), so exp(gam_L - gam_L) = 1.
    __device__ __forceinline__ cf finish(const float (*tr)[D], const float (*ti)[D]) {
        const int c = chan(), g0 = grp();
        float orr = 0.f, oi = 0.f, ar = 0.f, ai = 0.f;
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            const float xr = tr[g][c], xi = ti[g][c];
            if (g < g0) {
                orr += xr;
                oi += xi;
            }
            ar += xr;
            ai += xi;
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            lr[r] += orr;
            li[r] += oi;
        }
        return {ar, ai};
    }
};

// ---------------------------------------------------------------------------
// phase_prep: gam, G, P and T of one chunk; out: the chunk's record of mats.
template <int D> struct PrepLds {
    float K[kC][D + 1], Q[kC][D + 1], gr[kC][D + 1], gi[kC][D + 1];   // rows of D + 1: the pair
    float tr[kPT / D][D], ti[kPT / D][D];                              // loop reads a column of 16 rows
    float Ar[kC][kC + 1], Ai[kC][kC + 1];
    float beta[kC];
};

template <typename TI, int GATE, int D>
__global__ __launch_bounds__(kPT) void phase_prep_kernel(Params p, float* __restrict__ mats) {
    using CI = ChunkIn<TI, GATE, D>;
    __shared__ PrepLds<D> s;
    const int tid = threadIdx.x, n = blockIdx.x, bh = blockIdx.y;
    const int t0 = n * kC, valid = min(kC, p.T - t0);
    const long row0 = (long)bh * p.T + t0;
    CI in;
    in.load(p, row0, valid);
    const float bt = p.beta[row0 + min(tid % kC, valid - 1)];
    in.prefix(s.tr, s.ti);
    if (tid < kC) s.beta[tid] = tid < valid ? bt : 0.f;
    __syncthreads();
    in.finish(s.tr, s.ti);
    {
        const int c = CI::chan();
#pragma unroll
        for (int r = 0; r < CI::NR; ++r) {
            const int t = CI::row(r);
            s.K[t][c] = in.k[r];
            s.Q[t][c] = in.q[r];
            s.gr[t][c] = in.lr[r];
            s.gi[t][c] = in.li[r];
        }
    }
    __syncthreads();
    float* __restrict__ m = mats + ((long)bh * p.NT + n) * kMats;
    {   // pair (t, u), u <= t, one per thread
        const int t = tid / kC, u = tid % kC;
        cf Gs = {0.f, 0.f}, Hs = {0.f, 0.f};
        if (u <= t) {
#pragma unroll 4
            for (int c = 0; c < D; ++c) {
                const cf f = cexp_(s.gr[t][c] - s.gr[u][c], s.gi[t][c] - s.gi[u][c]);
                const float ku = s.K[u][c];
                Gs = cadd(Gs, cscale(f, s.K[t][c] * ku));
                Hs = cadd(Hs, cscale(f, s.Q[t][c] * ku));
            }
        }
        const float b = s.beta[t];
        s.Ar[t][u] = u < t ? b * Gs.r : 0.f;
        s.Ai[t][u] = u < t ? b * Gs.i : 0.f;
        m[2 * kCC + tid] = Hs.r;   // P (zero above the diagonal)
        m[3 * kCC + tid] = Hs.i;
        m[4 * kCC + tid] = Gs.r;
        m[5 * kCC + tid] = Gs.i;
    }
    __syncthreads();
    if (tid < kC) {   // T = (I + A)^{-1}: column u by forward substitution
        const int u = tid;
        cf x[kC];
#pragma unroll
        for (int i = 0; i < kC; ++i) x[i] = {i == u ? 1.f : 0.f, 0.f};
#pragma unroll
        for (int i = 1; i < kC; ++i) {
            cf acc = x[i];
#pragma unroll
            for (int j = 0; j < i; ++j) acc = csub(acc, cmul({s.Ar[i][j], s.Ai[i][j]}, x[j]));
            x[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < kC; ++i) {
            m[i * kC + u] = x[i].r;
            m[kCC + i * kC + u] = x[i].i;
        }
    }
}

// ---------------------------------------------------------------------------
// Register staging of the sequential kernels: the chunk's K, Q, gate, one
// 16-column block of a [T][D] tile (V forward, dO backward), T and P, beta.
template <typename TI, int GATE, int D> struct SeqIn {
    ChunkIn<TI, GATE, D> in;
    float blk;    // element (tid / 16, tid % 16) of the block
    float m[4];   // element tid of T re, T im, P re, P im
    float bt;     // beta of step tid % 16
    __device__ __forceinline__ void load(const Params& p, const void* tile, const float* __restrict__ mats, int bh,
                                         int col0, int n) {
        const int tid = threadIdx.x, t0 = n * kC, valid = min(kC, p.T - t0);
        const long row0 = (long)bh * p.T + t0;
        in.load(p, row0, valid);
        const int t = tid / kBV, v = tid % kBV;
        const TI* __restrict__ tp = static_cast<const TI*>(tile) + row0 * D + col0;
        const float x = to_f(tp[min(t, valid - 1) * D + v]);
        blk = t < valid ? x : 0.f;
        const float* mc = mats + ((long)bh * p.NT + n) * kMats;
#pragma unroll
        for (int j = 0; j < 4; ++j) m[j] = mc[j * kCC + tid];
        const int s = tid % kC;
        const float b = (p.beta + row0)[min(s, valid - 1)];
        bt = s < valid ? b : 0.f;
    }
};

// LDS of the sequential kernels (matrix-core form).  Tiles padded by 4 floats per row
// (the fragment reads of 16 rows x 4 columns and 4 rows x 16 columns spread over
// the banks; the 16-wide ones by 1 at d = 128, where the whole fits two workgroups
// per CU); the state block lives here between chunks.  The small per-chunk arrays
// come first, so ds_read immediates from one address reach them.
template <int D> struct SeqLdsM {
    static constexpr int LD = D + 4, LB = kBV + (D >= 128 ? 1 : 4), LC = kC + (D >= 128 ? 1 : 4);
    float B[kC][LB];                  // V (forward) or dO (backward) block [t][v]
    float Tr[kC][LC], Ti[kC][LC], Pr[kC][LC], Pi[kC][LC];
    float beta[kC];
    union {
        struct {
            float r[kC][LB], i[kC][LB];   // R [t][v] (backward: Ub), from the first product on
        } R;
        struct {
            float r[kPT / D][D], i[kPT / D][D];   // the gate's prefix totals, until the tiles are formed
        } tot;
    } u;
    float Ur[kC][LB], Ui[kC][LB];     // U [t][v] (backward: lambda)
    float Os[kC][LB];                 // O (backward: dv) block, for the write-back
    float elr[D], eli[D];             // E at the last row
    float Sr[kBV][LD], Si[kBV][LD];   // the state block [v][c]
    float kgr[kC][LD], kgi[kC][LD];   // K E
    float qgr[kC][LD], qgi[kC][LD];   // Q E
    float kdr[kC][LD], kdi[kC][LD];   // K exp(gam_L - gam)
};

__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// Fragment of a 16 x K operand for K step j: row l % 16, column 4 j + l / 16 of a
// [16][K] tile (T = false) or of the transposed [K][16] one (T = true), row stride L.
template <int L, bool T> __device__ __forceinline__ float frag(const float* p, int j) {
    const int l = threadIdx.x & 63, li = l & 15, k = 4 * j + (l >> 4);
    return T ? p[k * L + li] : p[li * L + k];
}

// acc + s1 sum_k A1[m][k] B1[n][k] + s2 sum_k A2[m][k] B2[n][k] for one 16 x 16 tile,
// K a multiple of 4 (operands at the tile's first row; LA / LB row strides; TA / TB:
// stored transposed).  Fully unrolled, operands chosen before the loop, so the fragment
// reads of up to 16 K steps are issued ahead of their products.
template <int K, int LA, int LB, bool TA, bool TB>
__device__ __forceinline__ f32x4 mma_pair(f32x4 acc, const float* A1, const float* B1, float s1, const float* A2,
                                          const float* B2, float s2) {
    constexpr int KB = K / 4 < 16 ? K / 4 : 16;
    static_assert(K % 4 == 0 && (K / 4) % KB == 0, "K");
#pragma unroll
    for (int j0 = 0; j0 < K / 4; j0 += KB) {
        float a1[KB], b1[KB], a2[KB], b2[KB];
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            a1[j] = frag<LA, TA>(A1, j0 + j);
            a2[j] = frag<LA, TA>(A2, j0 + j);
            b1[j] = frag<LB, TB>(B1, j0 + j);
            b2[j] = frag<LB, TB>(B2, j0 + j);
        }
#pragma unroll
        for (int j = 0; j < KB; ++j) acc = mma4(s2 * a2[j], b2[j], mma4(s1 * a1[j], b1[j], acc));
    }
    return acc;
}

// As mma_pair for two operands stored [16][K] (neither transposed), with the K
// slots dealt so that a lane's slots are consecutive: lane group l / 16 takes
// k = (l / 16) K / 4 + j at step j (the sum does not depend on which step takes
// which k), so each lane reads its part of a row with 16-byte LDS loads (rows and
// operands 16-byte aligned: LA, LB multiples of 4).
template <int K, int LA, int LB>
__device__ __forceinline__ f32x4 mma_pair_rows(f32x4 acc, const float* A1, const float* B1, float s1,
                                               const float* A2, const float* B2, float s2) {
    constexpr int NS = K / 4, KB = NS < 16 ? NS : 16;
    static_assert(NS % 4 == 0 && NS % KB == 0 && LA % 4 == 0 && LB % 4 == 0, "16-byte rows");
    const int l = threadIdx.x & 63, li = l & 15, k0 = (l >> 4) * NS;
#pragma unroll
    for (int j0 = 0; j0 < NS; j0 += KB) {
        f32x4 a1[KB / 4], b1[KB / 4], a2[KB / 4], b2[KB / 4];
#pragma unroll
        for (int q = 0; q < KB / 4; ++q) {
            a1[q] = *reinterpret_cast<const f32x4*>(A1 + li * LA + k0 + j0 + 4 * q);
            a2[q] = *reinterpret_cast<const f32x4*>(A2 + li * LA + k0 + j0 + 4 * q);
            b1[q] = *reinterpret_cast<const f32x4*>(B1 + li * LB + k0 + j0 + 4 * q);
            b2[q] = *reinterpret_cast<const f32x4*>(B2 + li * LB + k0 + j0 + 4 * q);
        }
#pragma unroll
        for (int j = 0; j < KB; ++j)
            acc = mma4(s2 * a2[j / 4][j % 4], b2[j / 4][j % 4], mma4(s1 * a1[j / 4][j % 4], b1[j / 4][j % 4], acc));
    }
    return acc;
}

// acc + s1 sum_k A1[m][k] B1[n][k] (as mma_pair, one product).
template <int K, int LA, int LB, bool TA, bool TB>
__device__ __forceinline__ f32x4 mma_one(f32x4 acc, const float* A1, const float* B1, float s1) {
    constexpr int KB = K / 4 < 16 ? K / 4 : 16;
    static_assert(K % 4 == 0 && (K / 4) % KB == 0, "K");
#pragma unroll
    for (int j0 = 0; j0 < K / 4; j0 += KB) {
        float a1[KB], b1[KB];
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            a1[j] = frag<LA, TA>(A1, j0 + j);
            b1[j] = frag<LB, TB>(B1, j0 + j);
        }
#pragma unroll
        for (int j = 0; j < KB; ++j) acc = mma4(s1 * a1[j], b1[j], acc);
    }
    return acc;
}

// Commit of the staged registers (phase A of a chunk): the gate's partial sums,
// the block tile, T, P, beta.
template <typename TI, int GATE, int D, class LDS>
__device__ __forceinline__ void seq_commit(SeqIn<TI, GATE, D>& x, LDS& s) {
    const int tid = threadIdx.x;
    x.in.prefix(s.u.tot.r, s.u.tot.i);
    s.B[tid / kBV][tid % kBV] = x.blk;
    const int t = tid / kC, u = tid % kC;
    s.Tr[t][u] = x.m[0];
    s.Ti[t][u] = x.m[1];
    s.Pr[t][u] = x.m[2];
    s.Pi[t][u] = x.m[3];
    if (tid < kC) s.beta[tid] = x.bt;
}

// Phase B: gam, then the gated tiles and E_L from the thread's own rows.
template <typename TI, int GATE, int D, class LDS>
__device__ __forceinline__ void seq_tiles(SeqIn<TI, GATE, D>& x, LDS& s) {
    using CI = ChunkIn<TI, GATE, D>;
    const cf gl = x.in.finish(s.u.tot.r, s.u.tot.i);
    const int c = CI::chan();
#pragma unroll
    for (int r = 0; r < CI::NR; ++r) {
        const int t = CI::row(r);
        const cf E = cexp_(x.in.lr[r], x.in.li[r]);
        const cf Ed = cexp_(gl.r - x.in.lr[r], gl.i - x.in.li[r]);
        const float kk = x.in.k[r], qq = x.in.q[r];
        s.kgr[t][c] = kk * E.r;
        s.kgi[t][c] = kk * E.i;
        s.qgr[t][c] = qq * E.r;
        s.qgi[t][c] = qq * E.i;
        s.kdr[t][c] = kk * Ed.r;
        s.kdi[t][c] = kk * Ed.i;
    }
    if (CI::grp() == 0) {
        const cf EL = cexp_(gl.r, gl.i);
        s.elr[c] = EL.r;
        s.eli[c] = EL.i;
    }
}

// ---------------------------------------------------------------------------
// phase_fwd_state: one workgroup per (head, block of 16 state rows), on the fp32
// matrix cores.  The state block S [16][D] stays in LDS; per chunk
//     X = (K E) S^T,  Yr = Re((Q E) S^T)       (16 x 16, over the D channels)
//     R = beta (V - X),  U = T R,  O = Yr + Re(P U)
//     S1 = S diag(E_L) + U^T (K exp(gam_L - gam))
// each a sum of real 16x16x4 products (fragments as in the per-chunk backward).
// states (if not NULL): the complex state entering each chunk, [BH][NT][2][D][D].
template <typename TI, int GATE, int D>
__global__ __launch_bounds__(kPT) void phase_fwd_state_kernel(Params p, const float* __restrict__ mats,
                                                              float* __restrict__ states) {
    constexpr int NB = D / kBV, NTL = D / 16, NW = kPT / 64;
    __shared__ __align__(16) SeqLdsM<D> s;
    int bh, blk;
    head_and_block(NB, p.BH, bh, blk);
    const int tid = threadIdx.x, v0 = blk * kBV;
    const int lane = tid & 63, wave = tid >> 6, li = lane & 15, lk = lane >> 4;
    for (int idx = tid; idx < kBV * D; idx += kPT) {
        const int v = idx / D, c = idx % D;
        const long e = ((long)bh * D + v0 + v) * D + c;
        s.Sr[v][c] = p.h0 ? p.h0[e] : 0.f;
        s.Si[v][c] = p.h0_im ? p.h0_im[e] : 0.f;
    }
    TI* __restrict__ out = static_cast<TI*>(p.o);
    SeqIn<TI, GATE, D> x;
    x.load(p, p.v, mats, bh, v0, 0);
    for (int n = 0; n < p.NT; ++n) {
        const int valid = min(kC, p.T - n * kC);
        const long row0 = (long)bh * p.T + n * kC;
        seq_commit(x, s);
        __syncthreads();   // (also orders the state block written at the end of the last chunk)
        seq_tiles(x, s);
        x.load(p, p.v, mats, bh, v0, n + 1 < p.NT ? n + 1 : n);   // the next chunk, during this one
        if (states) {   // the state entering this chunk
            float* st = states + ((long)bh * p.NT + n) * 2 * D * D;
            for (int idx = tid; idx < kBV * D; idx += kPT) {
                const int v = idx / D, c = idx % D;
                st[(long)(v0 + v) * D + c] = s.Sr[v][c];
                st[(long)D * D + (long)(v0 + v) * D + c] = s.Si[v][c];
            }
        }
        __syncthreads();
        // X and Yr: items Xr, Xi, Yr; R = beta (V - X) from the X items
        f32x4 yr = zero4();
        for (int it = wave; it < 3; it += NW) {
            // Xr, Yr = Ar Sr^T - Ai Si^T; Xi = Ar Si^T + Ai Sr^T
            constexpr int LD = SeqLdsM<D>::LD;
            const float* ar = it < 2 ? &s.kgr[0][0] : &s.qgr[0][0];
            const float* ai = it < 2 ? &s.kgi[0][0] : &s.qgi[0][0];
            const float* b1 = it == 1 ? &s.Si[0][0] : &s.Sr[0][0];
            const float* b2 = it == 1 ? &s.Sr[0][0] : &s.Si[0][0];
            const f32x4 acc = mma_pair_rows<D, LD, LD>(zero4(), ar, b1, 1.f, ai, b2, it == 1 ? 1.f : -1.f);
            // acc[i] = (t = 4 lk + i, v = li)
            if (it == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 4 * lk + i;
                    s.u.R.r[t][li] = s.beta[t] * (s.B[t][li] - acc[i]);
                }
            } else if (it == 1) {
#pragma unroll
                for (int i = 0; i < 4; ++i) s.u.R.i[4 * lk + i][li] = -s.beta[4 * lk + i] * acc[i];
            } else {
                yr = acc;
            }
        }
        __syncthreads();
        // U = T R: items Ur, Ui
        for (int it = wave; it < 2; it += NW) {
            // Ur = Tr Rr - Ti Ri, Ui = Tr Ri + Ti Rr (R stored [w][v])
            constexpr int LC = SeqLdsM<D>::LC, LBv = SeqLdsM<D>::LB;
            const float* b1 = it ? &s.u.R.i[0][0] : &s.u.R.r[0][0];
            const float* b2 = it ? &s.u.R.r[0][0] : &s.u.R.i[0][0];
            const f32x4 acc = mma_pair<kC, LC, LBv, false, true>(zero4(), &s.Tr[0][0], b1, 1.f, &s.Ti[0][0], b2,
                                                                  it ? 1.f : -1.f);
            float(*uo)[SeqLdsM<D>::LB] = it ? s.Ui : s.Ur;
#pragma unroll
            for (int i = 0; i < 4; ++i) uo[4 * lk + i][li] = acc[i];
        }
        __syncthreads();
        // O = Yr + Pr Ur - Pi Ui (the wave that holds Yr)
        if (wave == 2 % NW) {
            constexpr int LC = SeqLdsM<D>::LC, LBv = SeqLdsM<D>::LB;
            const f32x4 acc =
                mma_pair<kC, LC, LBv, false, true>(yr, &s.Pr[0][0], &s.Ur[0][0], 1.f, &s.Pi[0][0], &s.Ui[0][0], -1.f);
#pragma unroll
            for (int i = 0; i < 4; ++i) s.Os[4 * lk + i][li] = acc[i];
        }
        // S1 = S diag(E_L) + U^T Kd: items (column tile of c, real or imaginary part),
        // held until every item has read S
        constexpr int NI = (2 * NTL + NW - 1) / NW;
        f32x4 s1[NI];
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int it = wave + j * NW;
            s1[j] = zero4();
            if (it >= 2 * NTL) continue;
            const int c = (it >> 1) * 16 + li;
            const float er = s.elr[c], ei = s.eli[c];
            f32x4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float sr = s.Sr[4 * lk + i][c], si = s.Si[4 * lk + i][c];
                acc[i] = (it & 1) ? sr * ei + si * er : sr * er - si * ei;
            }
            // + Ur Kdr - Ui Kdi (re), + Ur Kdi + Ui Kdr (im); A = U^T [v][t], B = Kd [t][c]
            constexpr int LD = SeqLdsM<D>::LD, LBv = SeqLdsM<D>::LB;
            const int n0 = (it >> 1) * 16;
            const float* b1 = (it & 1) ? &s.kdi[0][n0] : &s.kdr[0][n0];
            const float* b2 = (it & 1) ? &s.kdr[0][n0] : &s.kdi[0][n0];
            s1[j] = mma_pair<kC, LBv, LD, true, true>(acc, &s.Ur[0][0], b1, 1.f, &s.Ui[0][0], b2, (it & 1) ? 1.f : -1.f);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int it = wave + j * NW;
            if (it >= 2 * NTL) continue;
            float(*so)[SeqLdsM<D>::LD] = (it & 1) ? s.Si : s.Sr;
#pragma unroll
            for (int i = 0; i < 4; ++i) so[4 * lk + i][(it >> 1) * 16 + li] = s1[j][i];
        }
        if (out) {   // (none when the backward recomputes the states)
            const int t = tid / kBV, vv = tid % kBV;
            if (t < valid) out[(row0 + t) * D + v0 + vv] = from_f<TI>(s.Os[t][vv]);
        }
    }
    __syncthreads();
    for (int idx = tid; idx < kBV * D; idx += kPT) {
        const int v = idx / D, c = idx % D;
        const long e = ((long)bh * D + v0 + v) * D + c;
        if (p.hT) p.hT[e] = s.Sr[v][c];
        if (p.hT_im) p.hT_im[e] = s.Si[v][c];
    }
}

// ---------------------------------------------------------------------------
// phase_bwd_state: one workgroup per (head, block of 16 rows of the state
// cotangent), chunks last to first, on the fp32 matrix cores (the block dS [16][D]
// in LDS).  Per chunk, with dS1 the cotangent leaving it:
//     Ub = conj(Kd) dS1^T + P^H dO,   lambda = T^H Ub,   dv = Re(diag(beta) lambda)
//     dS0 = dS1 diag(conj(E_L)) + dO^T conj(Q E) - (diag(beta) lambda)^T conj(K E)
// Out per chunk: lambda [BH][NT][2][D][C] (row v, then step) and dS1
// [BH][NT][2][D][D], which the per-chunk backward reads.
template <typename TI, int GATE, int D>
__global__ __launch_bounds__(kPT) void phase_bwd_state_kernel(Params p, const float* __restrict__ mats,
                                                              float* __restrict__ lam, float* __restrict__ dS1) {
    constexpr int NB = D / kBV, NTL = D / 16, NW = kPT / 64;
    __shared__ __align__(16) SeqLdsM<D> s;   // Sr / Si: dS; Rr / Ri: Ub; Ur / Ui: lambda
    int bh, blk;
    head_and_block(NB, p.BH, bh, blk);
    const int tid = threadIdx.x, v0 = blk * kBV;
    const int lane = tid & 63, wave = tid >> 6, li = lane & 15, lk = lane >> 4;
    for (int idx = tid; idx < kBV * D; idx += kPT) {
        const int v = idx / D, c = idx % D;
        const long e = ((long)bh * D + v0 + v) * D + c;
        s.Sr[v][c] = p.dhT ? p.dhT[e] : 0.f;
        s.Si[v][c] = p.dhT_im ? p.dhT_im[e] : 0.f;
    }
    TI* __restrict__ dvp = static_cast<TI*>(p.dv);
    SeqIn<TI, GATE, D> x;
    x.load(p, p.dout, mats, bh, v0, p.NT - 1);
    for (int n = p.NT - 1; n >= 0; --n) {
        const int valid = min(kC, p.T - n * kC);
        const long row0 = (long)bh * p.T + n * kC;
        const long chunk = (long)bh * p.NT + n;
        seq_commit(x, s);   // B: the dO block
        __syncthreads();
        seq_tiles(x, s);
        x.load(p, p.dout, mats, bh, v0, n > 0 ? n - 1 : n);   // the previous chunk, during this one
        {   // the cotangent leaving this chunk
            float* d1 = dS1 + chunk * 2 * D * D;
            for (int idx = tid; idx < kBV * D; idx += kPT) {
                const int v = idx / D, c = idx % D;
                d1[(long)(v0 + v) * D + c] = s.Sr[v][c];
                d1[(long)D * D + (long)(v0 + v) * D + c] = s.Si[v][c];
            }
        }
        __syncthreads();
        // Ub = conj(Kd) dS^T + P^H dO: items Ub re, Ub im
        for (int it = wave; it < 2; it += NW) {
            // Kdr dSr + Kdi dSi + Pr^T dO (re), Kdr dSi - Kdi dSr - Pi^T dO (im)
            constexpr int LD = SeqLdsM<D>::LD, LC = SeqLdsM<D>::LC, LBv = SeqLdsM<D>::LB;
            const float* b1 = it ? &s.Si[0][0] : &s.Sr[0][0];
            const float* b2 = it ? &s.Sr[0][0] : &s.Si[0][0];
            f32x4 acc = mma_pair_rows<D, LD, LD>(zero4(), &s.kdr[0][0], b1, 1.f, &s.kdi[0][0], b2, it ? -1.f : 1.f);
            acc = mma_one<kC, LC, LBv, true, true>(acc, it ? &s.Pi[0][0] : &s.Pr[0][0], &s.B[0][0], it ? -1.f : 1.f);
            float(*uo)[SeqLdsM<D>::LB] = it ? s.u.R.i : s.u.R.r;
#pragma unroll
            for (int i = 0; i < 4; ++i) uo[4 * lk + i][li] = acc[i];
        }
        __syncthreads();
        // lambda = T^H Ub: items re, im; dv = beta Re(lambda); lambda out
        for (int it = wave; it < 2; it += NW) {
            // Tr Ubr + Ti Ubi (re), Tr Ubi - Ti Ubr (im); A = conj(T)^T, B = Ub [w][v]
            constexpr int LC = SeqLdsM<D>::LC, LBv = SeqLdsM<D>::LB;
            const float* b1 = it ? &s.u.R.i[0][0] : &s.u.R.r[0][0];
            const float* b2 = it ? &s.u.R.r[0][0] : &s.u.R.i[0][0];
            const f32x4 acc = mma_pair<kC, LC, LBv, true, true>(zero4(), &s.Tr[0][0], b1, 1.f, &s.Ti[0][0], b2,
                                                                 it ? -1.f : 1.f);
            float(*lo)[SeqLdsM<D>::LB] = it ? s.Ui : s.Ur;   // beta lambda, for dS0
#pragma unroll
            for (int i = 0; i < 4; ++i) lo[4 * lk + i][li] = s.beta[4 * lk + i] * acc[i];
            // lambda [v][t]: this lane's 4 steps of row v are consecutive
            float* lp = lam + (chunk * 2 * D + v0 + li) * kC + 4 * lk + (it ? (long)D * kC : 0);
            *reinterpret_cast<f32x4*>(lp) = acc;
            if (!it) {
#pragma unroll
                for (int i = 0; i < 4; ++i) s.Os[4 * lk + i][li] = s.beta[4 * lk + i] * acc[i];
            }
        }
        __syncthreads();
        // dS0 = dS diag(conj(E_L)) + dO^T conj(Q E) - (beta lambda)^T conj(K E): items
        // (column tile of c, real or imaginary part), held until every item has read dS
        constexpr int NI = (2 * NTL + NW - 1) / NW;
        f32x4 s1[NI];
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int it = wave + j * NW;
            s1[j] = zero4();
            if (it >= 2 * NTL) continue;
            const int c = (it >> 1) * 16 + li;
            const float er = s.elr[c], ei = s.eli[c];
            f32x4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float sr = s.Sr[4 * lk + i][c], si = s.Si[4 * lk + i][c];
                acc[i] = (it & 1) ? si * er - sr * ei : sr * er + si * ei;
            }
            // + dO QEr - (blr KEr + bli KEi) (re), - dO QEi - (bli KEr - blr KEi) (im);
            // A = dO^T, (beta lambda)^T [v][t]; B = QE, KE [t][c]
            constexpr int LD = SeqLdsM<D>::LD, LBv = SeqLdsM<D>::LB;
            const int n0 = (it >> 1) * 16;
            const bool im = it & 1;
            acc = mma_one<kC, LBv, LD, true, true>(acc, &s.B[0][0], im ? &s.qgi[0][n0] : &s.qgr[0][n0], im ? -1.f : 1.f);
            s1[j] = mma_pair<kC, LBv, LD, true, true>(acc, im ? &s.Ui[0][0] : &s.Ur[0][0], &s.kgr[0][n0], -1.f,
                                                       im ? &s.Ur[0][0] : &s.Ui[0][0], &s.kgi[0][n0], im ? 1.f : -1.f);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int it = wave + j * NW;
            if (it >= 2 * NTL) continue;
            float(*so)[SeqLdsM<D>::LD] = (it & 1) ? s.Si : s.Sr;
#pragma unroll
            for (int i = 0; i < 4; ++i) so[4 * lk + i][(it >> 1) * 16 + li] = s1[j][i];
        }
        {
            const int t = tid / kBV, vv = tid % kBV;
            if (t < valid) dvp[(row0 + t) * D + v0 + vv] = from_f<TI>(s.Os[t][vv]);
        }
    }
    __syncthreads();
    for (int idx = tid; idx < kBV * D; idx += kPT) {
        const int v = idx / D, c = idx % D;
        const long e = ((long)bh * D + v0 + v) * D + c;
        if (p.dh0) p.dh0[e] = s.Sr[v][c];
        if (p.dh0_im) p.dh0_im[e] = s.Si[v][c];
    }
}

// ---------------------------------------------------------------------------
// phase_bwd_chunk: one workgroup per (chunk, head), from the chunk's entry state
// S0, the cotangent dS1 leaving it, lambda and the forward's T and G:
//     X = (K E) S0^T,  U = T diag(beta) (V - X)
//     Kgb = -lambda conj(S0),  Qgb = dO conj(S0),  Kdb_tc = sum_w dS1_wc conj(U_tw)
//     Ab = -strictly-lower(lambda U^H)      Pb = lower(dO U^H)
//     dbeta = Re rowsum(conj(lambda) (V - X)) + Re rowsum(conj(Ab) G)
// and K, Q, gam get the cotangents of the scaled tiles and of the pairwise G, H.
// Each term is either a block of 16 columns of X and U (from 16 rows of S0) or a
// sum over the state rows, so S0, dS1, lambda and the dO / V columns go through
// LDS one block of 16 state rows at a time (the next block in registers during
// the current one) and the sums stay in matrix-core accumulators across blocks:
// the LDS does not grow with D^2 (two workgroups per CU at d = 64; d = 128 fits).
template <int D, int NTH> struct ChunkBwdLds {
    static constexpr int NQ = D / 16 < 4 ? D / 16 : 4;   // channel parts of X
    // row strides: S0 is read with its rows as the output index (X) and as the
    // reduction index (Kgb, Qgb), dS1 only as the reduction index
    static constexpr int L0 = D + 4, L1 = D + 16, LT = kC + 1;
    // (the arrays of the block loop and of the pair loop first: within the first
    // 64 KB, a ds_read reaches them by its immediate offset from one address)
    union {
        struct {
            float S0r[kBV][L0], S0i[kBV][L0];   // the block's rows w of S0, [w][c]
            float S1r[kBV][L1], S1i[kBV][L1];   // and of dS1
            float Lr[kBV][LT], Li[kBV][LT];     // lambda [w][t]
            float dO[kC][LT], V[kC][LT];        // the block's columns of dO and V, [t][w]
            float Xp[2 * NQ][kC][LT];           // X by channel part (re, im) [t][v]
            float Ur[kC][LT], Ui[kC][LT];       // U [t][v]
        } blk;
        float sums[6][kC][D + 1];   // after the last block: -Kgb, Qgb, Kdb (re, im) [t][c]
    } u2;
    float Tr[kC][LT], Ti[kC][LT];
    float beta[kC];
    float K[kC][D + 1], Q[kC][D + 1];
    float gr[kC][D + 1], gi[kC][D + 1];     // gam
    float Gbr[kC][LT], Gbi[kC][LT];         // cotangent of G (beta Ab)
    float Hbr[kC][LT], Hbi[kC][LT];         // cotangent of H (Pb)
    float kgr[kC][D + 1], kgi[kC][D + 1];   // K E, then the per-step factors exp(gam_t - gam_{t-1})
    float Gr[kC][LT], Gi[kC][LT];
    float dbA[kC][LT];                      // Re(conj(Ab) G) per pair
    union {
        struct {
            float tr[NTH / D][D], ti[NTH / D][D];   // the gate's prefix totals
        } pre;
        struct {
            float red[2 * (NTH / D)][D];   // per-channel partials of the Kd terms of gam_L
            float glp[2 * (NTH / 64)][D];  // per-wave partials of sum_w dS1 conj(S0)
        } post;
    } u1;
};

// Threads of phase_bwd_chunk: 512 (two waves per SIMD) where every phase has work
// for them (d >= 32).
template <int D> constexpr int bwd_chunk_threads() { return D >= 32 ? 512 : 256; }

// Waves per SIMD that the registers must allow: at d = 64 the LDS holds two
// workgroups of 512 threads per CU, four waves per SIMD.
template <int D> constexpr int bwd_chunk_waves() { return D == 64 ? 4 : 1; }

template <typename TI, int GATE, int D>
__global__ __launch_bounds__(bwd_chunk_threads<D>()) __attribute__((amdgpu_waves_per_eu(bwd_chunk_waves<D>())))
void phase_bwd_chunk_kernel(
    Params p, const float* __restrict__ states, const float* __restrict__ mats, const float* __restrict__ lam,
    const float* __restrict__ dS1) {
    constexpr int NTH = bwd_chunk_threads<D>();
    using CI = ChunkIn<TI, GATE, D, NTH>;
    using LDS = ChunkBwdLds<D, NTH>;
    constexpr int NQ = LDS::NQ, KQ = D / NQ, L0 = LDS::L0, L1 = LDS::L1, LT = LDS::LT;
    constexpr int NW = NTH / 64, NTL = D / 16, NBLK = D / kBV;
    constexpr int VEC = kBV * D / NTH, NX = 2 * kCC / NTH;   // per thread and block: state floats, others
    static_assert(VEC >= 1 && VEC * NTH == kBV * D && NX * NTH == 2 * kCC && NTL <= NW, "block loads");
    constexpr int KDI = (2 * NTL + NW - 1) / NW;             // Kdb items per wave
    constexpr int AB_W = 2 % NW, PB_W = 3 % NW;              // the waves of Ab and Pb
    __shared__ __align__(16) LDS b;
    auto& bk = b.u2.blk;
    const int tid = threadIdx.x, n = blockIdx.x, bh = blockIdx.y;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), li = lane & 15, lk = lane >> 4;
    const int t0 = n * kC, valid = min(kC, p.T - t0), L = valid - 1;
    const long row0 = (long)bh * p.T + t0, chunk = (long)bh * p.NT + n;
    const TI* __restrict__ dout = static_cast<const TI*>(p.dout);
    const TI* __restrict__ vin = static_cast<const TI*>(p.v);
    TI* __restrict__ dq = static_cast<TI*>(p.dq);
    TI* __restrict__ dk = static_cast<TI*>(p.dk);

    // The block in registers: VEC consecutive floats of each state array from
    // element tid VEC of the block's 16 x D (row ew, channels ec ..), and NX
    // elements of lambda (re, then im: [w][t]) and of the dO and V columns ([t][w]).
    const float* __restrict__ st0 = states + chunk * 2 * D * D;
    const float* __restrict__ st1 = dS1 + chunk * 2 * D * D;
    const float* __restrict__ lm = lam + chunk * 2 * D * kC;
    const int ew = tid * VEC / D, ec = tid * VEC % D;
    float s0r[VEC], s0i[VEC], s1r[VEC], s1i[VEC], lx[NX], ox[NX];
    auto fetch = [&](int j) {
        const long o = (long)j * kBV * D + tid * VEC;
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            s0r[v] = st0[o + v];
            s0i[v] = st0[(long)D * D + o + v];
            s1r[v] = st1[o + v];
            s1i[v] = st1[(long)D * D + o + v];
        }
#pragma unroll
        for (int x = 0; x < NX; ++x) {
            const int idx = tid + NTH * x, e = idx % kCC, t = e / kBV, w = e % kBV;
            const bool second = idx >= kCC;   // lambda im and V, else lambda re and dO
            lx[x] = lm[(second ? (long)D * kC : 0) + j * kCC + e];
            const bool ok = t < valid;
            const float y = to_f((second ? vin : dout)[(row0 + (ok ? t : 0)) * D + j * kBV + w]);
            ox[x] = ok ? y : 0.f;
        }
    };
    float glr[VEC], gli[VEC];   // sum_w dS1_wc conj(S0_wc) for the thread's channels
#pragma unroll
    for (int v = 0; v < VEC; ++v) glr[v] = gli[v] = 0.f;
    auto commit = [&]() {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            bk.S0r[ew][ec + v] = s0r[v];
            bk.S0i[ew][ec + v] = s0i[v];
            bk.S1r[ew][ec + v] = s1r[v];
            bk.S1i[ew][ec + v] = s1i[v];
            glr[v] += s1r[v] * s0r[v] + s1i[v] * s0i[v];
            gli[v] += s1i[v] * s0r[v] - s1r[v] * s0i[v];
        }
#pragma unroll
        for (int x = 0; x < NX; ++x) {
            const int idx = tid + NTH * x, e = idx % kCC, r = e / kBV, c = e % kBV;
            if (idx < kCC) {
                bk.Lr[r][c] = lx[x];
                bk.dO[r][c] = ox[x];
            } else {
                bk.Li[r][c] = lx[x];
                bk.V[r][c] = ox[x];
            }
        }
    };
    fetch(0);

    // (a) the chunk's K, Q, gam, K E, T, G, beta into LDS
    CI in;
    in.load(p, row0, valid);
    {
        const float* mc = mats + chunk * kMats;
        if (tid < kCC) {
            const int t = tid / kC, u = tid % kC;
            b.Tr[t][u] = mc[tid];
            b.Ti[t][u] = mc[kCC + tid];
            b.Gr[t][u] = mc[4 * kCC + tid];
            b.Gi[t][u] = mc[5 * kCC + tid];
        }
        const float bt = p.beta[row0 + min(tid % kC, valid - 1)];
        if (tid < kC) b.beta[tid] = tid < valid ? bt : 0.f;
    }
    in.prefix(b.u1.pre.tr, b.u1.pre.ti);
    __syncthreads();
    in.finish(b.u1.pre.tr, b.u1.pre.ti);
    {
        const int c = CI::chan();
#pragma unroll
        for (int r = 0; r < CI::NR; ++r) {
            const int t = CI::row(r);
            b.K[t][c] = in.k[r];
            b.Q[t][c] = in.q[r];
            b.gr[t][c] = in.lr[r];
            b.gi[t][c] = in.li[r];
            const cf E = cexp_(in.lr[r], in.li[r]);
            b.kgr[t][c] = in.k[r] * E.r;
            b.kgi[t][c] = in.k[r] * E.i;
        }
    }

    // Every product below runs on the fp32 matrix cores: a complex product is two
    // or four real 16x16x4 MFMA products into one accumulator per real output
    // (signs folded into the A fragment).  Fragments: lane l supplies A row l % 16
    // and B row l % 16 at K slot l / 16; accumulator element i of lane l is
    // output (4 (l / 16) + i, l % 16) of the 16 x 16 tile.
    f32x4 kq[4] = {zero4(), zero4(), zero4(), zero4()};   // wave < NTL: -Kgb re, im, Qgb re, im of tile `wave`
    f32x4 kd[KDI];                                        // Kdb items wave + NW jj: (column tile, re / im)
#pragma unroll
    for (int jj = 0; jj < KDI; ++jj) kd[jj] = zero4();
    f32x4 ap[2] = {zero4(), zero4()};   // -Ab re, im (wave AB_W) or Pb re, im (wave PB_W)
    float db[4] = {0.f, 0.f, 0.f, 0.f};  // wave 0: dbeta partials of steps 4 jj + lk, column li
    for (int j = 0; j < NBLK; ++j) {
        commit();
        __syncthreads();   // (the first time also orders the chunk's tiles of (a))
        if (j + 1 < NBLK) fetch(j + 1);
        // (1) the block's terms of Kgb and Qgb for column tile `wave` (sharing the S0
        //     fragments): -Kgb_r += lr S0r + li S0i, -Kgb_i += li S0r - lr S0i,
        //     Qgb_r += dO S0r, Qgb_i -= dO S0i (A = lambda [w][t] transposed, dO [t][w];
        //     B = S0 [w][c] transposed); then the channel parts of X (items NTL ..)
        if (wave < NTL) {
            const int n0 = wave * 16;
            float lr[4], lq[4], o[4], sr[4], si[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                lr[jj] = frag<LT, true>(&bk.Lr[0][0], jj);
                lq[jj] = frag<LT, true>(&bk.Li[0][0], jj);
                o[jj] = frag<LT, false>(&bk.dO[0][0], jj);
                sr[jj] = frag<L0, true>(&bk.S0r[0][n0], jj);
                si[jj] = frag<L0, true>(&bk.S0i[0][n0], jj);
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                kq[0] = mma4(lq[jj], si[jj], mma4(lr[jj], sr[jj], kq[0]));
                kq[1] = mma4(-lr[jj], si[jj], mma4(lq[jj], sr[jj], kq[1]));
                kq[2] = mma4(o[jj], sr[jj], kq[2]);
                kq[3] = mma4(-o[jj], si[jj], kq[3]);
            }
        }
        for (int x = (wave + NW - NTL % NW) % NW; x < 2 * NQ; x += NW) {
            // channels c0 .. c0 + KQ: Xr = KEr S0r^T - KEi S0i^T, Xi = KEr S0i^T + KEi S0r^T
            const int c0 = (x >> 1) * KQ;
            const bool im = x & 1;
            const f32x4 acc = mma_pair<KQ, D + 1, L0, false, false>(
                zero4(), &b.kgr[0][c0], im ? &bk.S0i[0][c0] : &bk.S0r[0][c0], 1.f, &b.kgi[0][c0],
                im ? &bk.S0r[0][c0] : &bk.S0i[0][c0], im ? 1.f : -1.f);
#pragma unroll
            for (int i = 0; i < 4; ++i) bk.Xp[x][4 * lk + i][li] = acc[i];
        }
        __syncthreads();
        // (2) U = T R with R = diag(beta) (V - X), X the sum of its parts (waves 0, 1:
        //     re, im; each forms the R fragments it needs); wave 0 adds the block's
        //     Re(conj(lambda) (V - X)) to the dbeta partials
        if (wave < 2) {
            const bool im = wave == 1;
            float rr[4], ri[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int s = 4 * jj + lk;
                float xr = 0.f, xi = 0.f;
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    xr += bk.Xp[2 * q][s][li];
                    xi += bk.Xp[2 * q + 1][s][li];
                }
                const float a = bk.V[s][li] - xr, bt = b.beta[s];
                rr[jj] = bt * a;
                ri[jj] = -bt * xi;
                if (!im) db[jj] += bk.Lr[li][s] * a - bk.Li[li][s] * xi;
            }
            // Ur = Tr Rr - Ti Ri, Ui = Tr Ri + Ti Rr (A = T [t][s]; B = R at (s, v) = (4 jj + lk, li))
            f32x4 acc = zero4();
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float a1 = frag<LT, false>(&b.Tr[0][0], jj), a2 = frag<LT, false>(&b.Ti[0][0], jj);
                acc = mma4(a1, im ? ri[jj] : rr[jj], acc);
                acc = mma4(im ? a2 : -a2, im ? rr[jj] : ri[jj], acc);
            }
            float(*uo)[LT] = im ? bk.Ui : bk.Ur;
#pragma unroll
            for (int i = 0; i < 4; ++i) uo[4 * lk + i][li] = acc[i];
        }
        __syncthreads();
        // (3) the block's terms of Kdb (items: column tile, re / im), -Ab and Pb
#pragma unroll
        for (int jj = 0; jj < KDI; ++jj) {
            const int it = wave + jj * NW;
            if (it < 2 * NTL) {
                // Kdb_r += Ur S1r + Ui S1i, Kdb_i += Ur S1i - Ui S1r (A = U [t][w]; B = dS1 [w][c] transposed)
                const int n0 = (it >> 1) * 16;
                const bool im = it & 1;
                kd[jj] = mma_pair<kBV, LT, L1, false, true>(kd[jj], &bk.Ur[0][0],
                                                            im ? &bk.S1i[0][n0] : &bk.S1r[0][n0], 1.f, &bk.Ui[0][0],
                                                            im ? &bk.S1r[0][n0] : &bk.S1i[0][n0], im ? -1.f : 1.f);
            }
        }
        if (wave == AB_W) {
            // -Ab_r += lr Ur + li Ui, -Ab_i += li Ur - lr Ui (A = lambda transposed; B = U [u][w])
            ap[0] = mma_pair<kBV, LT, LT, true, false>(ap[0], &bk.Lr[0][0], &bk.Ur[0][0], 1.f, &bk.Li[0][0],
                                                       &bk.Ui[0][0], 1.f);
            ap[1] = mma_pair<kBV, LT, LT, true, false>(ap[1], &bk.Li[0][0], &bk.Ur[0][0], 1.f, &bk.Lr[0][0],
                                                       &bk.Ui[0][0], -1.f);
        }
        if (wave == PB_W) {
            // Pb_r += dO Ur, Pb_i -= dO Ui (A = dO [t][w]; B = U [u][w])
            ap[0] = mma_one<kBV, LT, LT, false, false>(ap[0], &bk.dO[0][0], &bk.Ur[0][0], 1.f);
            ap[1] = mma_one<kBV, LT, LT, false, false>(ap[1], &bk.dO[0][0], &bk.Ui[0][0], -1.f);
        }
        __syncthreads();   // the block is consumed
    }
    // The sums to LDS over the blocks' space; Gb, Hb, Re(conj(Ab) G); the gl partials
    float(*Kgr)[D + 1] = b.u2.sums[0], (*Kgi)[D + 1] = b.u2.sums[1], (*Qgr)[D + 1] = b.u2.sums[2];
    float(*Qgi)[D + 1] = b.u2.sums[3], (*Kdr)[D + 1] = b.u2.sums[4], (*Kdi)[D + 1] = b.u2.sums[5];
    if (wave < NTL) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 4 * lk + i, c = wave * 16 + li;
            Kgr[t][c] = -kq[0][i];
            Kgi[t][c] = -kq[1][i];
            Qgr[t][c] = kq[2][i];
            Qgi[t][c] = kq[3][i];
        }
    }
#pragma unroll
    for (int jj = 0; jj < KDI; ++jj) {
        const int it = wave + jj * NW;
        if (it < 2 * NTL) {
            float(*ko)[D + 1] = (it & 1) ? Kdi : Kdr;
#pragma unroll
            for (int i = 0; i < 4; ++i) ko[4 * lk + i][(it >> 1) * 16 + li] = kd[jj][i];
        }
    }
    if (wave == AB_W) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 4 * lk + i, u = li;
            const float abr = u < t ? -ap[0][i] : 0.f, abi = u < t ? -ap[1][i] : 0.f;
            b.Gbr[t][u] = b.beta[t] * abr;
            b.Gbi[t][u] = b.beta[t] * abi;
            b.dbA[t][u] = abr * b.Gr[t][u] + abi * b.Gi[t][u];   // Re(conj(Ab) G)
        }
    }
    if (wave == PB_W) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 4 * lk + i, u = li;
            b.Hbr[t][u] = u <= t ? ap[0][i] : 0.f;
            b.Hbi[t][u] = u <= t ? ap[1][i] : 0.f;
        }
    }
    constexpr int TS = NTH / D;                  // threads sharing a channel in (d)
    constexpr int NRD = TS < kC ? kC / TS : 1;   // their rows t = tid / D + TS r
    {   // per-step factors exp(gam_t - gam_{t-1}) over K E (dead), for the pair factors of (d)
        const int c = tid % D, tg = tid / D;
#pragma unroll
        for (int r = 0; r < NRD; ++r) {
            const int t = tg + TS * r;
            if (t >= kC) break;
            const cf e = cexp_(b.gr[t][c] - (t ? b.gr[t - 1][c] : 0.f), b.gi[t][c] - (t ? b.gi[t - 1][c] : 0.f));
            b.kgr[t][c] = e.r;
            b.kgi[t][c] = e.i;
        }
    }
    {   // lanes D / VEC apart hold the same channels: the wave's total, then one partial per wave
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
#pragma unroll
            for (int off = D / VEC; off < 64; off *= 2) {
                glr[v] += __shfl_xor(glr[v], off);
                gli[v] += __shfl_xor(gli[v], off);
            }
        }
        if (lane < D / VEC) {
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                b.u1.post.glp[2 * wave][ec + v] = glr[v];
                b.u1.post.glp[2 * wave + 1][ec + v] = gli[v];
            }
        }
    }
    __syncthreads();
    // dbeta_t = Re sum_v conj(lambda_tv) (V - X)_tv + sum_u Re(conj(Ab_tu) G_tu): the
    // partials of wave 0, summed over the 16 lanes of a DPP row
    if (wave == 0) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int s = 4 * jj + lk;
            const float x = group_sum<16>(db[jj] + (li < s ? b.dbA[s][li] : 0.f));
            if (li == 0 && s < valid) p.dbeta[row0 + s] = x;
        }
    }
    // (d) elements (t, c): the scaled tiles' cotangents, the pairwise G / H terms; dq, dk;
    //     gam's cotangent, stored over the element's own Kgb (read first).  The pair
    //     factors exp(gam_t - gam_u) are running products of the per-step factors
    //     from the diagonal outwards (t as the row: u = t, t - 1, .., 0; as the
    //     column: u = t, .., C - 1), so none exceeds 1 in magnitude for g <= 0.  Each
    //     pair is formed by both of its elements: accumulating the column terms once
    //     per pair through LDS atomics instead measured 1.9x slower.
    {
        const int c = tid % D;
        const int tg = D >= 64 ? __builtin_amdgcn_readfirstlane(tid / D) : tid / D;   // one per wave at D >= 64
        cf kdsum = {0.f, 0.f};
#pragma unroll
        for (int r = 0; r < NRD; ++r) {
            const int t = tg + TS * r;
            if (t >= kC) break;
            const cf Kgb = cscale({Kgr[t][c], Kgi[t][c]}, b.beta[t]), Qgb = {Qgr[t][c], Qgi[t][c]};
            const cf Kdb = {Kdr[t][c], Kdi[t][c]};
            const cf E = cexp_(b.gr[t][c], b.gi[t][c]);
            const cf Ed = cexp_(b.gr[L][c] - b.gr[t][c], b.gi[L][c] - b.gi[t][c]);
            const float kt = b.K[t][c], qt = b.Q[t][c];
            // Re(conj(w) Zb) for the real inputs, Zb conj(Z) for gam
            float dkv = Kgb.r * E.r + Kgb.i * E.i + Kdb.r * Ed.r + Kdb.i * Ed.i;
            float dqv = Qgb.r * E.r + Qgb.i * E.i;
            cf gb = cadd(cmulc(Kgb, cscale(E, kt)), cmulc(Qgb, cscale(E, qt)));
            const cf kdc = cmulc(Kdb, cscale(Ed, kt));
            gb = csub(gb, kdc);
            kdsum = cadd(kdsum, kdc);
            // t as the row: G_tu, H_tu (dG_tu / dk_tc = f k_u)
            cf f = {1.f, 0.f};
            for (int u = t; u >= 0; --u) {
                if (u < t) f = cmul(f, {b.kgr[u + 1][c], b.kgi[u + 1][c]});
                const cf Gb = {b.Gbr[t][u], b.Gbi[t][u]}, Hb = {b.Hbr[t][u], b.Hbi[t][u]};
                const cf wg = cscale(f, b.K[u][c]);
                dkv += Gb.r * wg.r + Gb.i * wg.i;
                dqv += Hb.r * wg.r + Hb.i * wg.i;
                gb = cadd(gb, cmulc(cadd(cscale(Gb, kt), cscale(Hb, qt)), wg));
            }
            // t as the column: G_ut, H_ut
            f = {1.f, 0.f};
            for (int u = t; u < kC; ++u) {
                if (u > t) f = cmul({b.kgr[u][c], b.kgi[u][c]}, f);
                const cf Gb = {b.Gbr[u][t], b.Gbi[u][t]}, Hb = {b.Hbr[u][t], b.Hbi[u][t]};
                const float ku = b.K[u][c], qu = b.Q[u][c];
                dkv += ku * (Gb.r * f.r + Gb.i * f.i) + qu * (Hb.r * f.r + Hb.i * f.i);
                gb = csub(gb, cscale(cmulc(cadd(cscale(Gb, ku), cscale(Hb, qu)), f), kt));
            }
            if (t < valid) {
                dq[(row0 + t) * D + c] = from_f<TI>(dqv);
                dk[(row0 + t) * D + c] = from_f<TI>(dkv);
            }
            Kgr[t][c] = gb.r;
            Kgi[t][c] = gb.i;
        }
        b.u1.post.red[2 * tg][c] = kdsum.r;
        b.u1.post.red[2 * tg + 1][c] = kdsum.i;
    }
    __syncthreads();
    // (e) per channel: gam_L's cotangent (the state's decay and the Kd terms), then the
    //     reverse cumulative sum; dtheta, dg (the scalar gate sums its channels per row,
    //     from the real parts kept over Qgb, which only (d) read)
    float(*dgs)[D + 1] = Qgr;
    if (tid < D) {
        const int c = tid;
        cf acc = {0.f, 0.f};
        for (int g2 = 0; g2 < NW; ++g2) acc = cadd(acc, {b.u1.post.glp[2 * g2][c], b.u1.post.glp[2 * g2 + 1][c]});
        const cf gl = cmulc(acc, cexp_(b.gr[L][c], b.gi[L][c]));   // sum_w dS1 conj(S0 E_L)
        float lr = gl.r, li = gl.i;
        for (int g2 = 0; g2 < TS; ++g2) {
            lr += b.u1.post.red[2 * g2][c];
            li += b.u1.post.red[2 * g2 + 1][c];
        }
        float ar = 0.f, ai = 0.f;
        for (int t = L; t >= 0; --t) {
            ar += Kgr[t][c] + (t == L ? lr : 0.f);
            ai += Kgi[t][c] + (t == L ? li : 0.f);
            p.dtheta[(row0 + t) * D + c] = ai;
            if (GATE == kGateVector) p.dg[(row0 + t) * D + c] = ar;
            dgs[t][c] = ar;
        }
    }
    if (GATE == kGateScalar) {
        __syncthreads();
        if (tid < valid) {
            float acc = 0.f;
            for (int c = 0; c < D; ++c) acc += dgs[tid][c];
            p.dg[row0 + tid] = acc;
        }
    }
}

// ---------------------------------------------------------------------------
template <typename TI, int GATE, int D>
hipError_t phase_launch_d(const Params& p, const PhaseBufs& f, bool backward, hipStream_t stream) {
    const dim3 chunks(p.NT, p.BH), seq(p.BH * (D / kBV)), block(kPT);
    if (!backward) {
        prof_begin(stream, "phase_prep");
        hipLaunchKernelGGL((phase_prep_kernel<TI, GATE, D>), chunks, block, 0, stream, p, f.mats);
        prof_end(stream);
        prof_begin(stream, "phase_fwd_state");
        hipLaunchKernelGGL((phase_fwd_state_kernel<TI, GATE, D>), seq, block, 0, stream, p, f.mats, f.states);
        prof_end(stream);
    } else {
        prof_begin(stream, "phase_bwd_state");
        hipLaunchKernelGGL((phase_bwd_state_kernel<TI, GATE, D>), seq, block, 0, stream, p, f.mats, f.lam, f.dS1);
        prof_end(stream);
        prof_begin(stream, "phase_bwd_chunk");
        hipLaunchKernelGGL((phase_bwd_chunk_kernel<TI, GATE, D>), chunks, dim3(bwd_chunk_threads<D>()), 0, stream, p,
                           f.states, f.mats, f.lam, f.dS1);
        prof_end(stream);
    }
    return hipGetLastError();
}

template <typename TI, int GATE>
hipError_t phase_launch_g(const Params& p, const PhaseBufs& f, bool backward, hipStream_t stream) {
    switch (p.DKr) {
        case 16: return phase_launch_d<TI, GATE, 16>(p, f, backward, stream);
        case 32: return phase_launch_d<TI, GATE, 32>(p, f, backward, stream);
        case 64: return phase_launch_d<TI, GATE, 64>(p, f, backward, stream);
        case 128: return phase_launch_d<TI, GATE, 128>(p, f, backward, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename TI>
hipError_t phase_launch_t(const Problem& pr, const Params& p, const PhaseBufs& f, bool backward, hipStream_t stream) {
    switch (pr.gate) {
        case kGateNone: return phase_launch_g<TI, kGateNone>(p, f, backward, stream);
        case kGateScalar: return phase_launch_g<TI, kGateScalar>(p, f, backward, stream);
        case kGateVector: return phase_launch_g<TI, kGateVector>(p, f, backward, stream);
        default: return hipErrorInvalidValue;
    }
}

__global__ void phase_copy_kernel(const float* __restrict__ src, float* __restrict__ dst, long n) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}
hipError_t phase_copy(const float* src, float* dst, long n, hipStream_t stream) {
    if (!dst || n == 0) return hipSuccess;
    hipLaunchKernelGGL(phase_copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, src, dst, n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_phase(const Problem& pr, const Params& p, const PhaseBufs& f, bool backward, hipStream_t stream) {
    if (pr.B * pr.H == 0) return hipSuccess;
    if (pr.T == 0) {   // no steps: the state (or its cotangent) passes through
        const long n = (long)pr.B * pr.H * pr.dv * pr.dk;
        hipError_t e = backward ? phase_copy(p.dhT, p.dh0, n, stream) : phase_copy(p.h0, p.hT, n, stream);
        if (e != hipSuccess) return e;
        return backward ? phase_copy(p.dhT_im, p.dh0_im, n, stream) : phase_copy(p.h0_im, p.hT_im, n, stream);
    }
    return pr.bf16 ? phase_launch_t<bf16>(pr, p, f, backward, stream)
                   : phase_launch_t<float>(pr, p, f, backward, stream);
}

}  // namespace dn
