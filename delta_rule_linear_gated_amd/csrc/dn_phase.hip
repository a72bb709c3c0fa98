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
// channel, so none exceeds 1 in magnitude for g <= 0, at any decay.
//
// The reverse pass takes each chunk back with complex cotangents
// Zb = dL/dRe Z + i dL/dIm Z: for Z = X Y^T, Xb = Zb conj(Y) and Yb = Zb^T conj(X);
// the triangular system is one transposed solve, lambda = T^H Ub (no adjoint of
// the inverse: the ReWY abstract's residual system, conjugated here); a real
// input x entering as x w gets Re(conj(w) Zb); gam's cotangent flows through
// each exp as Eb conj(E), and dg, dtheta are the real and imaginary parts of
// its reverse cumulative sum.
//
// Four kernels, all fp32 on the vector ALUs:
//   phase_prep       grid (chunk, head), every chunk at once: gam, the pairwise
//                    G and H, T by forward substitution; T, P, G per chunk out.
//   phase_fwd_state  grid (head, block of 16 state rows), chunks in order: the
//                    state recurrence, O, the chunk-entry states.
//   phase_bwd_state  grid (head, block of 16 rows), chunks last to first: Ub,
//                    lambda = T^H Ub, dv and the state cotangent; lambda and the
//                    cotangent leaving each chunk out.
//   phase_bwd_chunk  grid (chunk, head), every chunk at once: X and U again, the
//                    pair cotangents, dq, dk, dbeta, dg, dtheta.
// Row v of S1 depends only on row v of S0 (and row v of dS0 only on row v of
// dS1), so the sequential kernels split the state into blocks of 16 rows.  There
// a row belongs to 16 consecutive lanes (one DPP row), each lane D / 16
// consecutive key channels, and lane j also holds step j of the row's per-step
// values: sums over the key channels are 16-lane DPP sums.
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
        const TI* __restrict__ kp = static_cast<const TI*>(p.k);
        const TI* __restrict__ qp = static_cast<const TI*>(p.q);
        const int c = chan();
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int t = row(r);
            const bool ok = t < valid;
            const long rr = row0 + (ok ? t : 0);
            const long e = rr * D + c;
            const float kk = to_f(kp[e]), qq = to_f(qp[e]), th = p.theta[e];
            float g = 0.f;
            if (GATE == kGateScalar) g = p.g[rr];
            if (GATE == kGateVector) g = p.g[e];
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

// Per-step complex values of W state rows, [C][W + 1] (column v for row v).
template <int W> struct Rows {
    float r[kC][W + 1], i[kC][W + 1];
    __device__ __forceinline__ cf get(int t, int v) const { return {r[t][v], i[t][v]}; }
    __device__ __forceinline__ void set(int t, int v, cf x) {
        r[t][v] = x.r;
        i[t][v] = x.i;
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
        const float x = to_f(static_cast<const TI*>(tile)[(row0 + min(t, valid - 1)) * D + col0 + v]);
        blk = t < valid ? x : 0.f;
        const float* mc = mats + ((long)bh * p.NT + n) * kMats;
#pragma unroll
        for (int j = 0; j < 4; ++j) m[j] = mc[j * kCC + tid];
        const int s = tid % kC;
        const float b = p.beta[row0 + min(s, valid - 1)];
        bt = s < valid ? b : 0.f;
    }
};

// LDS of the sequential kernels (matrix-core form).  Tiles padded by 4 floats per row
// (the fragment reads of 16 rows x 4 columns and 4 rows x 16 columns spread over
// the banks); the state block lives here between chunks.
template <int D> struct SeqLdsM {
    static constexpr int LD = D + 4, LB = kBV + 4, LC = kC + 4;
    float kgr[kC][LD], kgi[kC][LD];   // K E
    float qgr[kC][LD], qgi[kC][LD];   // Q E
    float kdr[kC][LD], kdi[kC][LD];   // K exp(gam_L - gam)
    float elr[D], eli[D];             // E at the last row
    float tr[kPT / D][D], ti[kPT / D][D];
    float Sr[kBV][LD], Si[kBV][LD];   // the state block [v][c]
    float B[kC][LB];                  // V (forward) or dO (backward) block [t][v]
    float Tr[kC][LC], Ti[kC][LC], Pr[kC][LC], Pi[kC][LC];
    float beta[kC];
    float Rr[kC][LB], Ri[kC][LB];     // R [t][v] (backward: Ub)
    float Ur[kC][LB], Ui[kC][LB];     // U [t][v] (backward: lambda)
    float Os[kC][LB];                 // O (backward: dv) block, for the write-back
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
// reads are issued ahead of the products.
template <int K, int LA, int LB, bool TA, bool TB>
__device__ __forceinline__ f32x4 mma_pair(f32x4 acc, const float* A1, const float* B1, float s1, const float* A2,
                                          const float* B2, float s2) {
    float a1[K / 4], b1[K / 4], a2[K / 4], b2[K / 4];
#pragma unroll
    for (int j = 0; j < K / 4; ++j) {
        a1[j] = frag<LA, TA>(A1, j);
        a2[j] = frag<LA, TA>(A2, j);
        b1[j] = frag<LB, TB>(B1, j);
        b2[j] = frag<LB, TB>(B2, j);
    }
#pragma unroll
    for (int j = 0; j < K / 4; ++j) acc = mma4(s2 * a2[j], b2[j], mma4(s1 * a1[j], b1[j], acc));
    return acc;
}

// acc + s1 sum_k A1[m][k] B1[n][k] (as mma_pair, one product).
template <int K, int LA, int LB, bool TA, bool TB>
__device__ __forceinline__ f32x4 mma_one(f32x4 acc, const float* A1, const float* B1, float s1) {
    float a1[K / 4], b1[K / 4];
#pragma unroll
    for (int j = 0; j < K / 4; ++j) {
        a1[j] = frag<LA, TA>(A1, j);
        b1[j] = frag<LB, TB>(B1, j);
    }
#pragma unroll
    for (int j = 0; j < K / 4; ++j) acc = mma4(s1 * a1[j], b1[j], acc);
    return acc;
}

// Commit of the staged registers (phase A of a chunk): the gate's partial sums,
// the block tile, T, P, beta.
template <typename TI, int GATE, int D, class LDS>
__device__ __forceinline__ void seq_commit(SeqIn<TI, GATE, D>& x, LDS& s) {
    const int tid = threadIdx.x;
    x.in.prefix(s.tr, s.ti);
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
    const cf gl = x.in.finish(s.tr, s.ti);
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
            const f32x4 acc = mma_pair<D, LD, LD, false, false>(zero4(), ar, b1, 1.f, ai, b2, it == 1 ? 1.f : -1.f);
            // acc[i] = (t = 4 lk + i, v = li)
            if (it == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 4 * lk + i;
                    s.Rr[t][li] = s.beta[t] * (s.B[t][li] - acc[i]);
                }
            } else if (it == 1) {
#pragma unroll
                for (int i = 0; i < 4; ++i) s.Ri[4 * lk + i][li] = -s.beta[4 * lk + i] * acc[i];
            } else {
                yr = acc;
            }
        }
        __syncthreads();
        // U = T R: items Ur, Ui
        for (int it = wave; it < 2; it += NW) {
            // Ur = Tr Rr - Ti Ri, Ui = Tr Ri + Ti Rr (R stored [w][v])
            constexpr int LC = SeqLdsM<D>::LC, LBv = SeqLdsM<D>::LB;
            const float* b1 = it ? &s.Ri[0][0] : &s.Rr[0][0];
            const float* b2 = it ? &s.Rr[0][0] : &s.Ri[0][0];
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
        {
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
            f32x4 acc = mma_pair<D, LD, LD, false, false>(zero4(), &s.kdr[0][0], b1, 1.f, &s.kdi[0][0], b2,
                                                          it ? -1.f : 1.f);
            acc = mma_one<kC, LC, LBv, true, true>(acc, it ? &s.Pi[0][0] : &s.Pr[0][0], &s.B[0][0], it ? -1.f : 1.f);
            float(*uo)[SeqLdsM<D>::LB] = it ? s.Ri : s.Rr;
#pragma unroll
            for (int i = 0; i < 4; ++i) uo[4 * lk + i][li] = acc[i];
        }
        __syncthreads();
        // lambda = T^H Ub: items re, im; dv = beta Re(lambda); lambda out
        for (int it = wave; it < 2; it += NW) {
            // Tr Ubr + Ti Ubi (re), Tr Ubi - Ti Ubr (im); A = conj(T)^T, B = Ub [w][v]
            constexpr int LC = SeqLdsM<D>::LC, LBv = SeqLdsM<D>::LB;
            const float* b1 = it ? &s.Ri[0][0] : &s.Rr[0][0];
            const float* b2 = it ? &s.Rr[0][0] : &s.Ri[0][0];
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
// S0, the cotangent dS1 leaving it, lambda and the forward's T, P, G:
//     X = (K E) S0^T,  U = T diag(beta) (V - X)
//     Ab = -strictly-lower(lambda U^H)      Pb = lower(dO U^H)
//     dbeta = Re rowsum(conj(lambda) (V - X)) + Re rowsum(conj(Ab) G)
// and K, Q, gam get the cotangents of the scaled tiles and of the pairwise G, H.
template <int D, int NTH> struct ChunkBwdLds {
    float K[kC][D + 1], Q[kC][D + 1], V[kC][D + 1];
    float gr[kC][D + 1], gi[kC][D + 1];     // gam
    float kgr[kC][D + 1], kgi[kC][D + 1];   // K E, then the cotangent of gam
    float Gr[kC][kC + 1], Gi[kC][kC + 1], Tr[kC][kC + 1], Ti[kC][kC + 1], Pr[kC][kC + 1], Pi[kC][kC + 1];
    float beta[kC];
    float tr[NTH / D][D], ti[NTH / D][D];
    // the state entering the chunk (S0 re, im) and the cotangent of the state leaving
    // it (dS1 re, im), D rows each; after the products of (c), the six [C][D] sums
    float SS[4 * D > 6 * kC ? 4 * D : 6 * kC][D + 1];
    float dO[kC][D + 1];
    Rows<D> U, LB, X;                     // U; lambda; X
    float Gbr[kC][kC + 1], Gbi[kC][kC + 1];   // cotangent of G (beta Ab)
    float Hbr[kC][kC + 1], Hbi[kC][kC + 1];   // cotangent of H (Pb)
    float dbA[kC][kC + 1];                    // Re(conj(Ab) G) per pair
    float red[2 * (NTH / D)][D];              // per-channel partial sums over rows
    float glp[2 * (NTH / D)][D];              // partials of sum_w dS1 conj(S0) per channel
};

// Threads of phase_bwd_chunk: 512 (two waves per SIMD) where every phase has work
// for them (d >= 32).
template <int D> constexpr int bwd_chunk_threads() { return D >= 32 ? 512 : 256; }

template <typename TI, int GATE, int D>
__global__ __launch_bounds__(bwd_chunk_threads<D>()) void phase_bwd_chunk_kernel(
    Params p, const float* __restrict__ states, const float* __restrict__ mats, const float* __restrict__ lam,
    const float* __restrict__ dS1) {
    constexpr int NTH = bwd_chunk_threads<D>();
    using CI = ChunkIn<TI, GATE, D, NTH>;
    constexpr int PG = NTH / D <= D ? NTH / D : D, NC = D / PG;   // lanes per state row in (b)
    __shared__ ChunkBwdLds<D, NTH> b;
    float(*S0r)[D + 1] = b.SS, (*S0i)[D + 1] = b.SS + D, (*S1r)[D + 1] = b.SS + 2 * D, (*S1i)[D + 1] = b.SS + 3 * D;
    const int tid = threadIdx.x, n = blockIdx.x, bh = blockIdx.y;
    const int t0 = n * kC, valid = min(kC, p.T - t0), L = valid - 1;
    const long row0 = (long)bh * p.T + t0, chunk = (long)bh * p.NT + n;
    const TI* __restrict__ dout = static_cast<const TI*>(p.dout);
    const TI* __restrict__ vin = static_cast<const TI*>(p.v);
    TI* __restrict__ dq = static_cast<TI*>(p.dq);
    TI* __restrict__ dk = static_cast<TI*>(p.dk);
    // (a) the chunk's data into LDS
    CI in;
    in.load(p, row0, valid);
    {
        const float* st = states + chunk * 2 * D * D;
        const float* d1 = dS1 + chunk * 2 * D * D;
        for (int idx = tid; idx < D * D; idx += NTH) {
            const int r = idx / D, c = idx % D;
            S0r[r][c] = st[idx];
            S0i[r][c] = st[(long)D * D + idx];
            S1r[r][c] = d1[idx];
            S1i[r][c] = d1[(long)D * D + idx];
        }
        const float* lm = lam + chunk * 2 * D * kC;
        for (int idx = tid; idx < D * kC; idx += NTH) {
            const int vv = idx / kC, t = idx % kC;
            b.LB.r[t][vv] = lm[idx];
            b.LB.i[t][vv] = lm[(long)D * kC + idx];
        }
        for (int idx = tid; idx < kC * D; idx += NTH) {
            const int t = idx / D, c = idx % D;
            const bool ok = t < valid;
            const long e = (row0 + (ok ? t : 0)) * D + c;
            const float o = to_f(dout[e]), vv = to_f(vin[e]);
            b.dO[t][c] = ok ? o : 0.f;
            b.V[t][c] = ok ? vv : 0.f;
        }
        const float* mc = mats + chunk * kMats;
        if (tid < kCC) {
            const int t = tid / kC, u = tid % kC;
            b.Tr[t][u] = mc[tid];
            b.Ti[t][u] = mc[kCC + tid];
            b.Pr[t][u] = mc[2 * kCC + tid];
            b.Pi[t][u] = mc[3 * kCC + tid];
            b.Gr[t][u] = mc[4 * kCC + tid];
            b.Gi[t][u] = mc[5 * kCC + tid];
        }
        const float bt = p.beta[row0 + min(tid % kC, valid - 1)];
        if (tid < kC) b.beta[tid] = tid < valid ? bt : 0.f;
    }
    in.prefix(b.tr, b.ti);
    __syncthreads();
    in.finish(b.tr, b.ti);
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
    __syncthreads();
    // Every product below runs on the fp32 matrix cores: a complex product is two
    // or four real 16x16x4 MFMA products into one accumulator per real output
    // (signs folded into the A fragment).  Fragments: lane l supplies A row l % 16
    // and B row l % 16 at K slot l / 16; accumulator element i of lane l is
    // output (4 (l / 16) + i, l % 16) of the 16 x 16 tile.  Work items go to the
    // waves round-robin.
    const int lane = tid & 63, wave = tid >> 6, li = lane & 15, lk = lane >> 4;
    constexpr int NW = NTH / 64, NTL = D / 16;   // waves; 16-wide column tiles of a D-wide output
    auto mma = [](float a, float bb, f32x4 acc) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, acc, 0, 0, 0); };
    // (b) X = (K E) S0^T (kept for dbeta), then R = beta (V - X) over K E (dead once X
    //     is formed) and U = T R; items (column tile of v, real or imaginary part)
    for (int it = wave; it < 2 * NTL; it += NW) {
        // Xr = KEr S0r^T - KEi S0i^T, Xi = KEr S0i^T + KEi S0r^T
        const int n0 = (it >> 1) * 16;
        const float* b1 = (it & 1) ? &S0i[n0][0] : &S0r[n0][0];
        const float* b2 = (it & 1) ? &S0r[n0][0] : &S0i[n0][0];
        const f32x4 acc = mma_pair<D, D + 1, D + 1, false, false>(zero4(), &b.kgr[0][0], b1, 1.f, &b.kgi[0][0], b2,
                                                                  (it & 1) ? 1.f : -1.f);
        float(*xo)[D + 1] = (it & 1) ? b.X.i : b.X.r;
#pragma unroll
        for (int i = 0; i < 4; ++i) xo[4 * lk + i][n0 + li] = acc[i];
    }
    __syncthreads();
    for (int idx = tid; idx < kC * D; idx += NTH) {
        const int t = idx / D, v = idx % D;
        b.kgr[t][v] = b.beta[t] * (b.V[t][v] - b.X.r[t][v]);
        b.kgi[t][v] = -b.beta[t] * b.X.i[t][v];
    }
    __syncthreads();
    for (int it = wave; it < 2 * NTL; it += NW) {
        // Ur = Tr Rr - Ti Ri, Ui = Tr Ri + Ti Rr (R stored [w][v] over K E)
        const int n0 = (it >> 1) * 16;
        const float* b1 = (it & 1) ? &b.kgi[0][n0] : &b.kgr[0][n0];
        const float* b2 = (it & 1) ? &b.kgr[0][n0] : &b.kgi[0][n0];
        const f32x4 acc = mma_pair<kC, kC + 1, D + 1, false, true>(zero4(), &b.Tr[0][0], b1, 1.f, &b.Ti[0][0], b2,
                                                                   (it & 1) ? 1.f : -1.f);
        float(*uo)[D + 1] = (it & 1) ? b.U.i : b.U.r;
#pragma unroll
        for (int i = 0; i < 4; ++i) uo[4 * lk + i][n0 + li] = acc[i];
    }
    __syncthreads();
    // (c) the three sums over the rows v per element (t, c), the pair products, and per
    //     channel the state-decay term of gam_L:
    //       Kgb = -sum_w lambda_tw conj(S0_wc)    Qgb = sum_w dO_tw conj(S0_wc)
    //       Kdb = sum_w dS1_wc conj(U_tw)
    //       Ab = -lambda U^H (strictly lower)      Pb = dO U^H (lower)
    //       gl_c = sum_w dS1_wc conj(S0_wc E_L,c)
    //     Items: Kgb and Qgb per column tile (waves 0 .. NTL - 1), Kdb per column tile
    //     (the next NTL), Ab and Pb (one 16 x 16 tile each, on waves after those or
    //     shared).  Kgb / Qgb / Kdb stay in registers until every wave has read S0 and
    //     dS1, then go to LDS over them.
    f32x4 res[4] = {zero4(), zero4(), zero4(), zero4()};
    const int item = wave < 2 * NTL ? wave : -1;
    if (item >= 0 && item < NTL) {
        const int n0 = item * 16;
        // -Kgb_r = lr S0r + li S0i, -Kgb_i = li S0r - lr S0i, Qgb_r = dO S0r, Qgb_i = -dO S0i
        // (A = lambda, dO [t][w]; B = S0 [w][c]); fragments of 4 K steps read ahead
#pragma unroll
        for (int j0 = 0; j0 < D / 4; j0 += 4) {
            float lr[4], lq[4], o[4], sr[4], si[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                lr[j] = frag<D + 1, false>(&b.LB.r[0][0], j0 + j);
                lq[j] = frag<D + 1, false>(&b.LB.i[0][0], j0 + j);
                o[j] = frag<D + 1, false>(&b.dO[0][0], j0 + j);
                sr[j] = frag<D + 1, true>(&S0r[0][n0], j0 + j);
                si[j] = frag<D + 1, true>(&S0i[0][n0], j0 + j);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                res[0] = mma(lq[j], si[j], mma(lr[j], sr[j], res[0]));
                res[1] = mma(-lr[j], si[j], mma(lq[j], sr[j], res[1]));
                res[2] = mma(o[j], sr[j], res[2]);
                res[3] = mma(-o[j], si[j], res[3]);
            }
        }
    } else if (item >= NTL) {
        const int n0 = (item - NTL) * 16;
        // Kdb_r = Ur S1r + Ui S1i, Kdb_i = Ur S1i - Ui S1r (A = U [t][w], B = dS1 [w][c])
        res[0] = mma_pair<D, D + 1, D + 1, false, true>(res[0], &b.U.r[0][0], &S1r[0][n0], 1.f, &b.U.i[0][0],
                                                        &S1i[0][n0], 1.f);
        res[1] = mma_pair<D, D + 1, D + 1, false, true>(res[1], &b.U.r[0][0], &S1i[0][n0], 1.f, &b.U.i[0][0],
                                                        &S1r[0][n0], -1.f);
    }
    constexpr int AB_WAVE = 2 * NTL < NW ? 2 * NTL : NTL, PB_WAVE = 2 * NTL + 1 < NW ? 2 * NTL + 1 : NTL + 1;
    if (wave == AB_WAVE) {
        // -Ab_r = lr Ur + li Ui, -Ab_i = li Ur - lr Ui (A = lambda [t][w], B = U [u][w])
        const f32x4 ar = mma_pair<D, D + 1, D + 1, false, false>(zero4(), &b.LB.r[0][0], &b.U.r[0][0], 1.f,
                                                                 &b.LB.i[0][0], &b.U.i[0][0], 1.f);
        const f32x4 ai = mma_pair<D, D + 1, D + 1, false, false>(zero4(), &b.LB.i[0][0], &b.U.r[0][0], 1.f,
                                                                 &b.LB.r[0][0], &b.U.i[0][0], -1.f);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 4 * lk + i, u = li;
            const float abr = u < t ? -ar[i] : 0.f, abi = u < t ? -ai[i] : 0.f;
            b.Gbr[t][u] = b.beta[t] * abr;
            b.Gbi[t][u] = b.beta[t] * abi;
            b.dbA[t][u] = abr * b.Gr[t][u] + abi * b.Gi[t][u];   // Re(conj(Ab) G)
        }
    }
    if (wave == PB_WAVE) {
        // Pb_r = dO Ur, Pb_i = -dO Ui (A = dO [t][w], B = U [u][w])
        const f32x4 pr = mma_one<D, D + 1, D + 1, false, false>(zero4(), &b.dO[0][0], &b.U.r[0][0], 1.f);
        const f32x4 pi = mma_one<D, D + 1, D + 1, false, false>(zero4(), &b.dO[0][0], &b.U.i[0][0], -1.f);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 4 * lk + i, u = li;
            b.Hbr[t][u] = u <= t ? pr[i] : 0.f;
            b.Hbi[t][u] = u <= t ? pi[i] : 0.f;
        }
    }
    {   // gl: channel c, rows w of this thread's part (partials over the parts in (e))
        constexpr int NP = NTH / D, WP = D / NP > 0 ? D / NP : 1;
        const int c = tid % D, part = tid / D;
        cf acc = {0.f, 0.f};
        if (part * WP < D) {
#pragma unroll 4
            for (int w = part * WP; w < part * WP + WP; ++w)
                acc = cadd(acc, cmulc({S1r[w][c], S1i[w][c]}, {S0r[w][c], S0i[w][c]}));
        }
        b.glp[2 * part][c] = acc.r;
        b.glp[2 * part + 1][c] = acc.i;
    }
    __syncthreads();
    // S0 and dS1 are dead: the sums go over them, [t][c] each
    float(*Kgr)[D + 1] = b.SS, (*Kgi)[D + 1] = b.SS + kC, (*Qgr)[D + 1] = b.SS + 2 * kC;
    float(*Qgi)[D + 1] = b.SS + 3 * kC, (*Kdr)[D + 1] = b.SS + 4 * kC, (*Kdi)[D + 1] = b.SS + 5 * kC;

    if (item >= 0 && item < NTL) {
        const int n0 = item * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 4 * lk + i, c = n0 + li;
            Kgr[t][c] = -res[0][i];
            Kgi[t][c] = -res[1][i];
            Qgr[t][c] = res[2][i];
            Qgi[t][c] = res[3][i];
        }
    } else if (item >= NTL) {
        const int n0 = (item - NTL) * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            Kdr[4 * lk + i][n0 + li] = res[0][i];
            Kdi[4 * lk + i][n0 + li] = res[1][i];
        }
    }
    __syncthreads();
    // (d) elements (t, c): the scaled tiles' cotangents, the pairwise G / H terms; dq, dk;
    //     gam's cotangent, stored over K E (R since (b); dead).  Each pair's factor is
    //     formed by both of its elements (as row and as column): accumulating the column
    //     terms once per pair through LDS atomics instead measured 1.9x slower.
    constexpr int TS = NTH / D;                         // threads sharing a channel
    constexpr int NRD = TS < kC ? kC / TS : 1;          // their rows t = tid / D + TS r
    {
        const int c = tid % D, tg = tid / D;
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
            // pairs with t as the row (u <= t) and as the column (u >= t)
#pragma unroll 4
            for (int u = 0; u < kC; ++u) {
                const int r2 = u <= t ? t : u, cl = u <= t ? u : t;   // the pair (row, column)
                const cf f = cexp_(b.gr[r2][c] - b.gr[cl][c], b.gi[r2][c] - b.gi[cl][c]);
                const cf Gb = {b.Gbr[r2][cl], b.Gbi[r2][cl]}, Hb = {b.Hbr[r2][cl], b.Hbi[r2][cl]};
                if (u <= t) {   // t is the row: G_tu, H_tu
                    const float ku = b.K[u][c];
                    const cf wg = cscale(f, ku);   // dG_tu / dk_tc
                    dkv += Gb.r * wg.r + Gb.i * wg.i;
                    dqv += Hb.r * wg.r + Hb.i * wg.i;
                    gb = cadd(gb, cadd(cmulc(Gb, cscale(f, kt * ku)), cmulc(Hb, cscale(f, qt * ku))));
                }
                if (u >= t) {   // t is the column: G_ut, H_ut
                    const cf wg = cscale(f, b.K[u][c]), wh = cscale(f, b.Q[u][c]);
                    dkv += Gb.r * wg.r + Gb.i * wg.i + Hb.r * wh.r + Hb.i * wh.i;
                    gb = csub(gb, cadd(cmulc(Gb, cscale(f, b.K[u][c] * kt)), cmulc(Hb, cscale(f, b.Q[u][c] * kt))));
                }
            }
            if (t < valid) {
                dq[(row0 + t) * D + c] = from_f<TI>(dqv);
                dk[(row0 + t) * D + c] = from_f<TI>(dkv);
            }
            b.kgr[t][c] = gb.r;
            b.kgi[t][c] = gb.i;
        }
        b.red[2 * tg][c] = kdsum.r;
        b.red[2 * tg + 1][c] = kdsum.i;
    }
    __syncthreads();
    // (e) per channel: gam_L's cotangent (the state's decay and the Kd terms), then the
    //     reverse cumulative sum; dtheta, dg (the scalar gate sums its channels per row,
    //     from the real parts kept over U, which nothing reads any more)
    float (*dgs)[D + 1] = b.U.r;
    if (tid < D) {
        const int c = tid;
        cf acc = {0.f, 0.f};
        for (int g2 = 0; g2 < NTH / D; ++g2) acc = cadd(acc, {b.glp[2 * g2][c], b.glp[2 * g2 + 1][c]});
        const cf gl = cmulc(acc, cexp_(b.gr[L][c], b.gi[L][c]));   // sum_w dS1 conj(S0 E_L)
        float lr = gl.r, li = gl.i;
        for (int g2 = 0; g2 < TS; ++g2) {
            lr += b.red[2 * g2][c];
            li += b.red[2 * g2 + 1][c];
        }
        float ar = 0.f, ai = 0.f;
        for (int t = L; t >= 0; --t) {
            ar += b.kgr[t][c] + (t == L ? lr : 0.f);
            ai += b.kgi[t][c] + (t == L ? li : 0.f);
            p.dtheta[(row0 + t) * D + c] = ai;
            if (GATE == kGateVector) p.dg[(row0 + t) * D + c] = ar;
            dgs[t][c] = ar;
        }
    }
    // dbeta_t = Re sum_v conj(lambda_tv) (V - X)_tv + sum_u Re(conj(Ab_tu) G_tu): step t
    // by the 16 lanes of one DPP row of the last 256 threads
    if (tid >= NTH - kCC) {
        const int t = (tid - (NTH - kCC)) / 16, j = tid % 16;
        float acc = j < t ? b.dbA[t][j] : 0.f;
        for (int w = j; w < D; w += 16)
            acc += b.LB.r[t][w] * (b.V[t][w] - b.X.r[t][w]) - b.LB.i[t][w] * b.X.i[t][w];
        acc = group_sum<16>(acc);
        if (j == 0 && t < valid) p.dbeta[row0 + t] = acc;
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
