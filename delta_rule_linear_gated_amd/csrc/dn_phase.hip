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
// One workgroup per head walks the chunks in order (forward) or in reverse.
// The state (and its cotangent) lives in registers: a group of PG = 256 / D
// consecutive lanes owns one state row v, each lane NC = D / PG consecutive key
// channels of it; sums over the key channels are lane-group sums.  All
// arithmetic is fp32 on the vector ALUs.
#include <hip/hip_runtime.h>

#include "dn.h"
#include "dn_device.h"
#include "dn_internal.h"

namespace dn {

namespace {

constexpr int kPT = 256;   // threads per workgroup

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

// LDS of the parts both passes share: the chunk's rows and per-chunk matrices.
template <int D, int C> struct PhaseTiles {
    float K[C][D], Q[C][D], V[C][D];
    float gr[C][D], gi[C][D];          // cumulative log gate (re, im)
    float kgr[C][D], kgi[C][D];        // K E
    float qgr[C][D], qgi[C][D];        // Q E
    float kdr[C][D], kdi[C][D];        // K exp(gam_L - gam)
    float Gr[C][C + 1], Gi[C][C + 1];  // G (without beta)
    float Tr[C][C + 1], Ti[C][C + 1];  // A, then T = (I + A)^{-1}
    float Pr[C][C + 1], Pi[C][C + 1];  // P
    float beta[C];
};

// Load the chunk's rows, form gam, the scaled tiles, G, P and T.  Rows past
// `valid` are zero (their gate too), which leaves the state unchanged.  Begins
// writing LDS at once (the caller's previous barrier ordered it after the last
// reads) and ends with a barrier.
template <typename TI, int GATE, int D, int C>
__device__ void chunk_setup(const Params& p, PhaseTiles<D, C>& s, long row0, int valid) {
    const int tid = threadIdx.x;
    const TI* __restrict__ k = static_cast<const TI*>(p.k);
    const TI* __restrict__ q = static_cast<const TI*>(p.q);
    const TI* __restrict__ v = static_cast<const TI*>(p.v);
    for (int idx = tid; idx < C * D; idx += kPT) {
        const int t = idx / D, c = idx % D;
        const bool ok = t < valid;
        const long e = (row0 + (ok ? t : 0)) * D + c;
        s.K[t][c] = ok ? to_f(k[e]) : 0.f;
        s.Q[t][c] = ok ? to_f(q[e]) : 0.f;
        s.V[t][c] = ok ? to_f(v[e]) : 0.f;
        float g = 0.f;
        if (GATE == kGateScalar) g = p.g[row0 + (ok ? t : 0)];
        if (GATE == kGateVector) g = p.g[e];
        s.gr[t][c] = ok ? g : 0.f;
        s.gi[t][c] = ok ? p.theta[e] : 0.f;
    }
    if (tid < C) s.beta[tid] = tid < valid ? p.beta[row0 + tid] : 0.f;
    __syncthreads();
    if (tid < D) {   // in-chunk cumulative sum, one channel per thread
        float ar = 0.f, ai = 0.f;
        for (int t = 0; t < C; ++t) {
            ar += s.gr[t][tid];
            ai += s.gi[t][tid];
            s.gr[t][tid] = ar;
            s.gi[t][tid] = ai;
        }
    }
    __syncthreads();
    const int L = valid - 1;
    for (int idx = tid; idx < C * D; idx += kPT) {
        const int t = idx / D, c = idx % D;
        const cf E = cexp_(s.gr[t][c], s.gi[t][c]);
        const cf Ed = cexp_(s.gr[L][c] - s.gr[t][c], s.gi[L][c] - s.gi[t][c]);
        const float kk = s.K[t][c], qq = s.Q[t][c];
        s.kgr[t][c] = kk * E.r;
        s.kgi[t][c] = kk * E.i;
        s.qgr[t][c] = qq * E.r;
        s.qgi[t][c] = qq * E.i;
        s.kdr[t][c] = kk * Ed.r;
        s.kdi[t][c] = kk * Ed.i;
    }
    // pairwise Gram products (u <= t), each factor exp(gam_t - gam_u) formed per channel
    for (int pr = tid; pr < C * C; pr += kPT) {
        const int t = pr / C, u = pr % C;
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
        s.Gr[t][u] = Gs.r;
        s.Gi[t][u] = Gs.i;
        const float b = s.beta[t];
        s.Tr[t][u] = u < t ? b * Gs.r : 0.f;   // A
        s.Ti[t][u] = u < t ? b * Gs.i : 0.f;
        s.Pr[t][u] = Hs.r;                     // P (zero above the diagonal)
        s.Pi[t][u] = Hs.i;
    }
    __syncthreads();
    // T = (I + A)^{-1}: column u by forward substitution, one thread per column,
    // every column formed from A before any is written back over it
    cf x[C];
    if (tid < C) {
        const int u = tid;
#pragma unroll
        for (int i = 0; i < C; ++i) x[i] = {i == u ? 1.f : 0.f, 0.f};
#pragma unroll
        for (int i = 1; i < C; ++i) {
            cf acc = x[i];
#pragma unroll
            for (int j = 0; j < i; ++j) acc = csub(acc, cmul({s.Tr[i][j], s.Ti[i][j]}, x[j]));
            x[i] = acc;
        }
    }
    __syncthreads();
    if (tid < C) {
#pragma unroll
        for (int i = 0; i < C; ++i) {
            s.Tr[i][tid] = x[i].r;
            s.Ti[i][tid] = x[i].i;
        }
    }
    __syncthreads();
}

// Sum of x over the PG consecutive lanes of a state row's group.
template <int PG> __device__ __forceinline__ float row_sum(float x) { return group_sum<PG>(x); }

// ---------------------------------------------------------------------------
// Per-row complex vectors over the chunk's steps, [C][D + 1] (column v for row v
// of the state).  A row's lanes are one lane group of one wave: what one lane
// stores there the others read back in program order, with no barrier.
template <int D, int C> struct RowVecs {
    float r[C][D + 1], i[C][D + 1];
    __device__ __forceinline__ cf get(int t, int v) const { return {r[t][v], i[t][v]}; }
    __device__ __forceinline__ void set(int t, int v, cf x) {
        r[t][v] = x.r;
        i[t][v] = x.i;
    }
};

// The row's sums over the key channels of (A_t . S_row) for every step t, A one
// or two [C][D] complex tiles given by pointers; lane 0 of the group stores them.
template <int D, int C, int PG, int NC>
__device__ __forceinline__ void row_products(const float (*ar)[D], const float (*ai)[D], const float* sr, const float* si,
                                             int v, int c0, bool conj_a, RowVecs<D, C>& out) {
#pragma unroll 1
    for (int t = 0; t < C; ++t) {
        cf x = {0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const cf A = {ar[t][c0 + c], conj_a ? -ai[t][c0 + c] : ai[t][c0 + c]};
            x = cadd(x, cmul(A, {sr[c], si[c]}));
        }
        x = {row_sum<PG>(x.r), row_sum<PG>(x.i)};
        if (threadIdx.x % PG == 0) out.set(t, v, x);
    }
}

// ---------------------------------------------------------------------------
// Forward: one workgroup per head.  states (if not NULL): the complex state
// entering each chunk, [BH][NT][2][D][D] fp32 (real part, then imaginary).
template <typename TI, int GATE, int D, int C>
__global__ __launch_bounds__(kPT) void phase_fwd_kernel(Params p, float* states) {
    constexpr int PG = kPT / D, NC = D / PG;
    __shared__ PhaseTiles<D, C> s;
    __shared__ RowVecs<D, C> X, Y, U;
    __shared__ float Os[C][D];
    const int tid = threadIdx.x, v = tid / PG, j = tid % PG, c0 = j * NC;
    const int bh = blockIdx.x;
    float sr[NC], si[NC];   // S[v][c0 .. c0 + NC)
    {
        const long o0 = ((long)bh * D + v) * D + c0;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            sr[c] = p.h0 ? p.h0[o0 + c] : 0.f;
            si[c] = p.h0_im ? p.h0_im[o0 + c] : 0.f;
        }
    }
    TI* __restrict__ out = static_cast<TI*>(p.o);
    for (int n = 0; n < p.NT; ++n) {
        const int t0 = n * C, valid = min(C, p.T - t0), L = valid - 1;
        const long row0 = (long)bh * p.T + t0;
        chunk_setup<TI, GATE, D, C>(p, s, row0, valid);
        if (states) {
            float* st = states + (((long)bh * p.NT + n) * 2 * D + v) * D + c0;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                st[c] = sr[c];
                st[(long)D * D + c] = si[c];
            }
        }
        // X_t = (K E)_t . S_v and Y_t = (Q E)_t . S_v
        row_products<D, C, PG, NC>(s.kgr, s.kgi, sr, si, v, c0, false, X);
        row_products<D, C, PG, NC>(s.qgr, s.qgi, sr, si, v, c0, false, Y);
        // U = T R with R = beta (V - X): the row's lanes take every PG-th step
        for (int t = j; t < C; t += PG) {
            cf u = {0.f, 0.f};
            for (int w = 0; w <= t; ++w)
                u = cadd(u, cmul({s.Tr[t][w], s.Ti[t][w]}, cscale(csub({s.V[w][v], 0.f}, X.get(w, v)), s.beta[w])));
            U.set(t, v, u);
        }
        // O = Re(Y + P U)
        for (int t = j; t < C; t += PG) {
            cf o = Y.get(t, v);
            for (int w = 0; w <= t; ++w) o = cadd(o, cmul({s.Pr[t][w], s.Pi[t][w]}, U.get(w, v)));
            Os[t][v] = o.r;
        }
        // S1 = S0 diag(E_L) + U^T (K exp(gam_L - gam)), step by step over the lane's channels
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const cf S = cmul({sr[c], si[c]}, cexp_(s.gr[L][c0 + c], s.gi[L][c0 + c]));
            sr[c] = S.r;
            si[c] = S.i;
        }
#pragma unroll 1
        for (int t = 0; t < C; ++t) {
            const cf u = U.get(t, v);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const cf x = cmul(u, {s.kdr[t][c0 + c], s.kdi[t][c0 + c]});
                sr[c] += x.r;
                si[c] += x.i;
            }
        }
        __syncthreads();
        for (int idx = tid; idx < C * D; idx += kPT) {
            const int t = idx / D, c = idx % D;
            if (t < valid) out[(row0 + t) * D + c] = from_f<TI>(Os[t][c]);
        }
        __syncthreads();
    }
    const long o0 = ((long)bh * D + v) * D + c0;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if (p.hT) p.hT[o0 + c] = sr[c];
        if (p.hT_im) p.hT_im[o0 + c] = si[c];
    }
}

// ---------------------------------------------------------------------------
// Reverse: one workgroup per head, chunks last to first, from the states the
// forward saved.  Per chunk, with the cotangents dO (real) and dS1 (complex):
//     Ub = conj(Kd) dS1^T + P^H dO          lambda = T^H Ub
//     Ab = -strictly-lower(lambda U^H)      Pb = lower(dO U^H)
//     dv = Re(diag(beta) lambda)            dbeta = Re rowsum(conj(lambda) (V - X)) + Re rowsum(conj(Ab) G)
//     dS0 = dS1 diag(conj(E_L)) + dO^T conj(Q E) - (diag(beta) lambda)^T conj(K E)
// and K, Q, gam get the cotangents of the scaled tiles and of the pairwise G, H.
template <int D, int C> struct PhaseBwdLds {
    float S0r[D][D + 1], S0i[D][D + 1];   // state entering the chunk
    float S1r[D][D + 1], S1i[D][D + 1];   // cotangent of the state leaving it
    float dO[C][D];
    RowVecs<D, C> U, LB, X;               // U; Ub, then lambda over it; X
    float Gbr[C][C + 1], Gbi[C][C + 1];   // cotangent of G (beta Ab)
    float Hbr[C][C + 1], Hbi[C][C + 1];   // cotangent of H (Pb)
    float dbA[C][C + 1];                  // Re(conj(Ab) G) per pair
    float red[2 * (kPT / D)][D];          // per-channel partial sums over rows
    float glr[D], gli[D];                 // cotangent of gam_L from the state's decay
};

template <typename TI, int GATE, int D, int C>
__global__ __launch_bounds__(kPT) void phase_bwd_kernel(Params p, const float* states) {
    constexpr int PG = kPT / D, NC = D / PG;
    __shared__ PhaseTiles<D, C> s;
    __shared__ PhaseBwdLds<D, C> b;
    const int tid = threadIdx.x, v = tid / PG, c0 = (tid % PG) * NC;
    const int bh = blockIdx.x;
    float br[NC], bi[NC];   // dS[v][c0 .. c0 + NC), the running state cotangent
    {
        const long o0 = ((long)bh * D + v) * D + c0;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            br[c] = p.dhT ? p.dhT[o0 + c] : 0.f;
            bi[c] = p.dhT_im ? p.dhT_im[o0 + c] : 0.f;
        }
    }
    const TI* __restrict__ dout = static_cast<const TI*>(p.dout);
    TI* __restrict__ dq = static_cast<TI*>(p.dq);
    TI* __restrict__ dk = static_cast<TI*>(p.dk);
    TI* __restrict__ dvv = static_cast<TI*>(p.dv);
    for (int n = p.NT - 1; n >= 0; --n) {
        const int t0 = n * C, valid = min(C, p.T - t0), L = valid - 1;
        const long row0 = (long)bh * p.T + t0;
        // (a) the chunk's state and the cotangent leaving it into LDS, dO rows
        {
            const float* st = states + ((long)bh * p.NT + n) * 2 * D * D;
            for (int idx = tid; idx < D * D; idx += kPT) {
                const int r = idx / D, c = idx % D;
                b.S0r[r][c] = st[idx];
                b.S0i[r][c] = st[(long)D * D + idx];
            }
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                b.S1r[v][c0 + c] = br[c];
                b.S1i[v][c0 + c] = bi[c];
            }
            for (int idx = tid; idx < C * D; idx += kPT) {
                const int t = idx / D, c = idx % D;
                b.dO[t][c] = t < valid ? to_f(dout[(row0 + t) * D + c]) : 0.f;
            }
        }
        chunk_setup<TI, GATE, D, C>(p, s, row0, valid);   // (its barriers order the stores above)
        // (b) the row's X, U, Ub, lambda; dv; the new state cotangent dS0 (the row's lanes
        //     take every PG-th step of the triangular products)
        {
            const int j = tid % PG;
            float sr[NC], si[NC];
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                sr[c] = b.S0r[v][c0 + c];
                si[c] = b.S0i[v][c0 + c];
            }
            row_products<D, C, PG, NC>(s.kgr, s.kgi, sr, si, v, c0, false, b.X);   // X = (K E) S0^T
            row_products<D, C, PG, NC>(s.kdr, s.kdi, br, bi, v, c0, true, b.LB);   // conj(Kd) dS1^T
            for (int t = j; t < C; t += PG) {
                cf u = {0.f, 0.f};
                for (int w = 0; w <= t; ++w)
                    u = cadd(u, cmul({s.Tr[t][w], s.Ti[t][w]}, cscale(csub({s.V[w][v], 0.f}, b.X.get(w, v)), s.beta[w])));
                b.U.set(t, v, u);
                // + P^H dO:  Ub_t += sum_{w >= t} conj(P_wt) dO_wv
                cf acc = b.LB.get(t, v);
                for (int w = t; w < C; ++w) acc = cadd(acc, cscale({s.Pr[w][t], -s.Pi[w][t]}, b.dO[w][v]));
                b.LB.set(t, v, acc);
            }
            // lambda = T^H Ub, in place: lambda_t = sum_{w >= t} conj(T_wt) Ub_w.  Round r of the
            // loop writes steps [r PG, (r + 1) PG) after all of its reads, and later rounds read
            // only steps beyond those
            for (int t = j; t < C; t += PG) {
                cf acc = {0.f, 0.f};
                for (int w = t; w < C; ++w) acc = cadd(acc, cmul({s.Tr[w][t], -s.Ti[w][t]}, b.LB.get(w, v)));
                b.LB.set(t, v, acc);
                if (t < valid) dvv[(row0 + t) * D + v] = from_f<TI>(s.beta[t] * acc.r);
            }
            // dS0 = dS1 diag(conj(E_L)) + dO^T conj(Q E) - (diag(beta) lambda)^T conj(K E), step by
            // step over the lane's channels
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const cf x = cmulc({br[c], bi[c]}, cexp_(s.gr[L][c0 + c], s.gi[L][c0 + c]));
                br[c] = x.r;
                bi[c] = x.i;
            }
#pragma unroll 1
            for (int t = 0; t < C; ++t) {
                const float o = b.dO[t][v];
                const cf l = cscale(b.LB.get(t, v), s.beta[t]);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int cc = c0 + c;
                    const cf x = csub(cscale({s.qgr[t][cc], -s.qgi[t][cc]}, o), cmulc(l, {s.kgr[t][cc], s.kgi[t][cc]}));
                    br[c] += x.r;
                    bi[c] += x.i;
                }
            }
        }
        __syncthreads();
        // (c) pairs: Ab = -lambda U^H (strictly lower), Pb = dO U^H (lower); per channel the
        //     cotangent of gam_L through the state's decay, sum_v dS1 conj(S0 E_L)
        for (int pr = tid; pr < C * C; pr += kPT) {
            const int t = pr / C, u = pr % C;
            cf ab = {0.f, 0.f}, pb = {0.f, 0.f};
            if (u <= t) {
                #pragma unroll 4
                for (int w = 0; w < D; ++w) {
                    const cf Uc = b.U.get(u, w);
                    ab = csub(ab, cmulc(b.LB.get(t, w), Uc));
                    pb = cadd(pb, cmulc({b.dO[t][w], 0.f}, Uc));
                }
            }
            if (u == t) ab = {0.f, 0.f};
            b.Gbr[t][u] = s.beta[t] * ab.r;
            b.Gbi[t][u] = s.beta[t] * ab.i;
            b.Hbr[t][u] = pb.r;
            b.Hbi[t][u] = pb.i;
            b.dbA[t][u] = ab.r * s.Gr[t][u] + ab.i * s.Gi[t][u];   // Re(conj(Ab) G)
        }
        if (tid < D) {
            const int c = tid;
            cf acc = {0.f, 0.f};
            #pragma unroll 4
            for (int w = 0; w < D; ++w) acc = cadd(acc, cmulc({b.S1r[w][c], b.S1i[w][c]}, {b.S0r[w][c], b.S0i[w][c]}));
            const cf EL = cexp_(s.gr[L][c], s.gi[L][c]);
            const cf gl = cmulc(acc, EL);
            b.glr[c] = gl.r;
            b.gli[c] = gl.i;
        }
        __syncthreads();
        // (d) elements (t, c): the scaled tiles' cotangents from sums over the rows v, the
        //     pairwise G / H terms; dq, dk; gam's cotangent, stored over (K E) at the same
        //     element (each element of K E is read only by the thread that replaces it)
        constexpr int TS = kPT / D;   // threads sharing a channel (rows t = tid / D + TS j)
        {
            const int c = tid % D, tg = tid / D;
            cf kdsum = {0.f, 0.f};
            for (int t = tg; t < C; t += TS) {
                cf Kgb = {0.f, 0.f}, Qgb = {0.f, 0.f}, Kdb = {0.f, 0.f};
                #pragma unroll 4
                for (int w = 0; w < D; ++w) {
                    const cf S = {b.S0r[w][c], b.S0i[w][c]};
                    Kgb = csub(Kgb, cmulc(b.LB.get(t, w), S));
                    Qgb = cadd(Qgb, cmulc({b.dO[t][w], 0.f}, S));
                    Kdb = cadd(Kdb, cmulc({b.S1r[w][c], b.S1i[w][c]}, b.U.get(t, w)));
                }
                Kgb = cscale(Kgb, s.beta[t]);
                const cf E = cexp_(s.gr[t][c], s.gi[t][c]);
                const cf Ed = cexp_(s.gr[L][c] - s.gr[t][c], s.gi[L][c] - s.gi[t][c]);
                const float kt = s.K[t][c], qt = s.Q[t][c];
                // Re(conj(w) Zb) for the real inputs, Zb conj(Z) for gam
                float dkv = Kgb.r * E.r + Kgb.i * E.i + Kdb.r * Ed.r + Kdb.i * Ed.i;
                float dqv = Qgb.r * E.r + Qgb.i * E.i;
                cf gb = cadd(cmulc(Kgb, {s.kgr[t][c], s.kgi[t][c]}), cmulc(Qgb, {s.qgr[t][c], s.qgi[t][c]}));
                const cf kdc = cmulc(Kdb, {s.kdr[t][c], s.kdi[t][c]});
                gb = csub(gb, kdc);
                kdsum = cadd(kdsum, kdc);
                // pairs with t as the row (u <= t) and as the column (w >= t)
                #pragma unroll 4
                for (int u = 0; u < C; ++u) {
                    const int r = u <= t ? t : u, cl = u <= t ? u : t;   // the pair (row, column)
                    const cf f = cexp_(s.gr[r][c] - s.gr[cl][c], s.gi[r][c] - s.gi[cl][c]);
                    const cf Gb = {b.Gbr[r][cl], b.Gbi[r][cl]}, Hb = {b.Hbr[r][cl], b.Hbi[r][cl]};
                    if (u <= t) {   // t is the row: G_tu, H_tu
                        const float ku = s.K[u][c];
                        const cf wg = cscale(f, ku);       // dG_tu / dk_tc
                        dkv += Gb.r * wg.r + Gb.i * wg.i;
                        dqv += Hb.r * wg.r + Hb.i * wg.i;
                        gb = cadd(gb, cadd(cmulc(Gb, cscale(f, kt * ku)), cmulc(Hb, cscale(f, qt * ku))));
                    }
                    if (u >= t) {   // t is the column: G_ut, H_ut
                        const cf wg = cscale(f, s.K[u][c]), wh = cscale(f, s.Q[u][c]);
                        dkv += Gb.r * wg.r + Gb.i * wg.i + Hb.r * wh.r + Hb.i * wh.i;
                        gb = csub(gb, cadd(cmulc(Gb, cscale(f, s.K[u][c] * kt)), cmulc(Hb, cscale(f, s.Q[u][c] * kt))));
                    }
                }
                if (t < valid) {
                    dq[(row0 + t) * D + c] = from_f<TI>(dqv);
                    dk[(row0 + t) * D + c] = from_f<TI>(dkv);
                }
                s.kgr[t][c] = gb.r;
                s.kgi[t][c] = gb.i;
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
            float lr = b.glr[c], li = b.gli[c];
            for (int g2 = 0; g2 < TS; ++g2) {
                lr += b.red[2 * g2][c];
                li += b.red[2 * g2 + 1][c];
            }
            float ar = 0.f, ai = 0.f;
            for (int t = L; t >= 0; --t) {
                ar += s.kgr[t][c] + (t == L ? lr : 0.f);
                ai += s.kgi[t][c] + (t == L ? li : 0.f);
                p.dtheta[(row0 + t) * D + c] = ai;
                if (GATE == kGateVector) p.dg[(row0 + t) * D + c] = ar;
                dgs[t][c] = ar;
            }
        }
        // dbeta_t = Re sum_v conj(lambda_tv) (V - X)_tv + sum_u Re(conj(Ab_tu) G_tu)
        if (tid >= kPT - C) {
            const int t = tid - (kPT - C);
            if (t < valid) {
                float acc = 0.f;
                #pragma unroll 4
                for (int w = 0; w < D; ++w)
                    acc += b.LB.r[t][w] * (s.V[t][w] - b.X.r[t][w]) - b.LB.i[t][w] * b.X.i[t][w];
                for (int u = 0; u < t; ++u) acc += b.dbA[t][u];
                p.dbeta[row0 + t] = acc;
            }
        }
        __syncthreads();
        if (GATE == kGateScalar && tid < valid) {
            float acc = 0.f;
            for (int c = 0; c < D; ++c) acc += dgs[tid][c];
            p.dg[row0 + tid] = acc;
        }
        __syncthreads();
    }
    const long o0 = ((long)bh * D + v) * D + c0;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if (p.dh0) p.dh0[o0 + c] = br[c];
        if (p.dh0_im) p.dh0_im[o0 + c] = bi[c];
    }
}

template <typename TI, int GATE, int D>
hipError_t phase_launch_d(const Params& p, float* states, bool backward, hipStream_t stream) {
    constexpr int C = 16;
    const dim3 grid(p.BH), block(kPT);
    if (backward) {
        prof_begin(stream, "phase_bwd");
        hipLaunchKernelGGL((phase_bwd_kernel<TI, GATE, D, C>), grid, block, 0, stream, p, states);
    } else {
        prof_begin(stream, "phase_fwd");
        hipLaunchKernelGGL((phase_fwd_kernel<TI, GATE, D, C>), grid, block, 0, stream, p, states);
    }
    prof_end(stream);
    return hipGetLastError();
}

template <typename TI, int GATE>
hipError_t phase_launch_g(const Params& p, float* states, bool backward, hipStream_t stream) {
    switch (p.DKr) {
        case 16: return phase_launch_d<TI, GATE, 16>(p, states, backward, stream);
        case 32: return phase_launch_d<TI, GATE, 32>(p, states, backward, stream);
        case 64: return phase_launch_d<TI, GATE, 64>(p, states, backward, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename TI>
hipError_t phase_launch_t(const Problem& pr, const Params& p, float* states, bool backward, hipStream_t stream) {
    switch (pr.gate) {
        case kGateNone: return phase_launch_g<TI, kGateNone>(p, states, backward, stream);
        case kGateScalar: return phase_launch_g<TI, kGateScalar>(p, states, backward, stream);
        case kGateVector: return phase_launch_g<TI, kGateVector>(p, states, backward, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

namespace {
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

hipError_t launch_phase(const Problem& pr, const Params& p, float* states, bool backward, hipStream_t stream) {
    if (pr.B * pr.H == 0) return hipSuccess;
    if (pr.T == 0) {   // no steps: the state (or its cotangent) passes through
        const long n = (long)pr.B * pr.H * pr.dv * pr.dk;
        hipError_t e = backward ? phase_copy(p.dhT, p.dh0, n, stream) : phase_copy(p.h0, p.hT, n, stream);
        if (e != hipSuccess) return e;
        return backward ? phase_copy(p.dhT_im, p.dh0_im, n, stream) : phase_copy(p.h0_im, p.hT_im, n, stream);
    }
    return pr.bf16 ? phase_launch_t<bf16>(pr, p, states, backward, stream)
                   : phase_launch_t<float>(pr, p, states, backward, stream);
}

}  // namespace dn
