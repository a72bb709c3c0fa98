// dn_fwd_kernels.h -- forward-pass kernels of the chunkwise gated delta rule.
//
// Per head the state S (d_v x d_k) evolves as
//     S_t = S_{t-1} Diag(e^{g_t}) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t
// (ReWY abstract: DeltaNet / GDN / KDA; SFDA summary "Kernarchitektur",
// transposed, zero phase).  The sequence is cut into chunks of C steps.  Inside
// a chunk, with gam the in-chunk cumulative log-decay, Gam = e^gam and S0 the
// state entering the chunk (SFDA summary, "Der konstruktive Chunk-WY-Theorem":
// the chunk's transition product is the decay product minus a rank <= C
// correction with a triangular core; "Zentrale Beitraege": exact affine chunk
// transfer):
//     A   = strictly-lower( diag(beta) (K Gam)(K / Gam)^T )     pairwise decays e^{gam_t - gam_s}
//     P   = lower( (Q Gam)(K / Gam)^T )
//     T   = (I + A)^{-1}                                         (forward substitution)
//     U   = T diag(beta) (V - (K Gam) S0^T)                      the chunk's corrected writes
//     O   = (Q Gam) S0^T + P U
//     S1  = S0 Diag(Gam_C) + U^T (K Gam_C / Gam)
// prep_kernel builds gam, T and P for every chunk in parallel; fwd_state_kernel
// walks the chunks of one head (one d_v block of it) in order, keeping S in
// MFMA accumulators, and writes O as it goes.
//
// Gates: kGateNone (DeltaNet), kGateScalar (GDN: pairwise decays applied as
// e^{gam_t - gam_s} on the C x C scores, never above 1 for g <= 0), kGateVector
// (KDA: per-channel decays, factored through a per-chunk centre gam_C / 2 so
// that K e^{gam - centre} and K e^{centre - gam} stay within e^{+-|gam_C|/2} --
// the centred contraction of the ReWY abstract).
#pragma once

#include <type_traits>

#include "dn_device.h"
#include "dn_internal.h"

namespace dn {

template <int GATE, int DK> struct GateLayout {
    static constexpr int GW = GATE == kGateVector ? DK : 1;  // gam values per step
};

// ---------------------------------------------------------------------------
// prep_kernel: grid (NT, BH), one chunk per workgroup.  TRANS_OUT stores T^T
// and P^T instead of T and P (the layout the reverse pass reads).
template <typename TI, int GATE, int C, int DK, bool TRANS_OUT>
__global__ __launch_bounds__(kThreads) void prep_kernel(Params p) {
    constexpr int LDK = DK + Pad<TI>::value;
    constexpr int LDA = C + 4;
    constexpr int GW = GateLayout<GATE, DK>::GW;
    constexpr bool VEC = GATE == kGateVector;
    __shared__ float gam_s[C * GW];
    __shared__ float beta_s[C];
    __shared__ __align__(16) TI Kp[C * LDK];               // K, or K e^{gam - centre}
    __shared__ __align__(16) TI Km[VEC ? C * LDK : 16];    // K e^{centre - gam} (vector gate)
    __shared__ __align__(16) TI Qp[C * LDK];               // Q, or Q e^{gam - centre}
    __shared__ __align__(16) float A_s[C * LDA];

    const int n = blockIdx.x, bh = blockIdx.y;
    const int t0 = n * C;
    const int valid = min(C, p.T - t0);
    const long row0 = (long)bh * p.T + t0;
    const TI* __restrict__ q = static_cast<const TI*>(p.q) + row0 * DK;
    const TI* __restrict__ k = static_cast<const TI*>(p.k) + row0 * DK;
    const float* __restrict__ beta = p.beta + row0;

    // -- cumulative log-decay within the chunk
    if (GATE == kGateScalar) {
        if (wave_id() == 0) {
            const int t = lane_id();
            float x = (t < valid) ? p.g[row0 + t] : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off);
                if (t >= off) x += y;
            }
            if (t < C) {
                gam_s[t] = x;
                if (t < valid) p.gam[row0 + t] = x;
            }
        }
    } else if (GATE == kGateVector) {
        for (int c = threadIdx.x; c < DK; c += kThreads) {
            float acc = 0.f;
            for (int t = 0; t < C; ++t) {
                if (t < valid) acc += p.g[(row0 + t) * DK + c];
                gam_s[t * DK + c] = acc;
                if (t < valid) p.gam[(row0 + t) * DK + c] = acc;
            }
        }
    }
    for (int t = threadIdx.x; t < C; t += kThreads) beta_s[t] = t < valid ? beta[t] : 0.f;
    __syncthreads();

    // -- stage K and Q (centred per-channel factors for the vector gate)
    if (VEC) {
        const float* gl = gam_s + (valid - 1) * DK;  // gam_C
        stage<TI, C, DK, false>(Kp, LDK, k, DK, valid, [&](int r, int c, float x) {
            return x * fexp(gam_s[r * DK + c] - 0.5f * gl[c]);
        });
        stage<TI, C, DK, false>(Km, LDK, k, DK, valid, [&](int r, int c, float x) {
            return x * fexp(0.5f * gl[c] - gam_s[r * DK + c]);
        });
        stage<TI, C, DK, false>(Qp, LDK, q, DK, valid, [&](int r, int c, float x) {
            return x * fexp(gam_s[r * DK + c] - 0.5f * gl[c]);
        });
    } else {
        stage_copy<TI, C, DK, false>(Kp, LDK, k, DK, valid);
        stage_copy<TI, C, DK, false>(Qp, LDK, q, DK, valid);
    }
    __syncthreads();

    // -- gated Gram matrices: A (strict lower, scaled by beta_t) and P (lower)
    const TI* KmP = VEC ? Km : Kp;
    TI* __restrict__ Pout = static_cast<TI*>(p.Pm) + ((long)bh * p.NT + n) * C * C;
    {
        using TL = Tiles<C, C>;
        f32x4 acc[TL::PER];
        f32x4 accp[TL::PER];
#pragma unroll
        for (int j = 0; j < TL::PER; ++j) {
            acc[j] = zero4();
            accp[j] = zero4();
            if (!TL::valid(j) || TL::n0(j) > TL::m0(j)) continue;   // strictly upper tiles are zero
            acc[j] = tile_nt<TI, DK>(Kp + TL::m0(j) * LDK, LDK, KmP + TL::n0(j) * LDK, LDK, acc[j]);
            accp[j] = tile_nt<TI, DK>(Qp + TL::m0(j) * LDK, LDK, KmP + TL::n0(j) * LDK, LDK, accp[j]);
        }
        // gate factors and masks (LDS reads only), then the stores
        if (TL::active()) {
#pragma unroll
            for (int j = 0; j < TL::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = TL::row(j, i), s = TL::col(j);
                    const float e = (GATE == kGateScalar && s <= t) ? fexp(gam_s[t] - gam_s[s]) : 1.f;
                    acc[j][i] = s < t ? beta_s[t] * acc[j][i] * e : 0.f;
                    accp[j][i] = s <= t ? accp[j][i] * e : 0.f;
                }
#pragma unroll
            for (int j = 0; j < TL::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = TL::row(j, i), s = TL::col(j);
                    A_s[t * LDA + s] = acc[j][i];
                    if (TRANS_OUT)
                        Pout[s * C + t] = from_f<TI>(accp[j][i]);
                    else
                        Pout[t * C + s] = from_f<TI>(accp[j][i]);
                }
        }
    }
    __syncthreads();

    // -- T = (I + A)^{-1}: column c of T solves (I + A) x = e_c by forward
    //    substitution; lane c of wave 0 owns column c, A rows are LDS broadcasts.
    if (wave_id() == 0) {
        const int c = lane_id();
        float x[C];
#pragma unroll
        for (int i = 0; i < C; ++i) {
            float acc = (i == c) ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < i; ++j) acc -= A_s[i * LDA + j] * x[j];
            x[i] = acc;
        }
        if (c < C) {
            TI* __restrict__ Tout = static_cast<TI*>(p.Tm) + ((long)bh * p.NT + n) * C * C;
            if (TRANS_OUT) {
#pragma unroll
                for (int i = 0; i < C; ++i) Tout[c * C + i] = from_f<TI>(x[i]);
            } else {
#pragma unroll
                for (int i = 0; i < C; ++i) Tout[i * C + c] = from_f<TI>(x[i]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Per-chunk gate data held in registers between prefetch and commit, and the
// decay factors it leaves in LDS:
//   scalar gate: rowf[t] = e^{gam_t}, rowf[C + t] = e^{gam_C - gam_t}, gam_s[t]
//   vector gate: gam_s[t][c] (factors computed per element from it)
template <int GATE, int C, int DK> struct GateRegs {
    static constexpr bool VEC = GATE == kGateVector;
    RegN<float, VEC ? C : 4, VEC ? DK : 4> gv;   // vector gate: the chunk's gam rows
    float gs = 0.f, gC = 0.f, b = 0.f;          // scalar gate: gam_t, gam_C; beta_t (thread t < C)
    int valid_ = C;
    // branch-free: row indices are clamped into the chunk, masking happens in commit()
    __device__ __forceinline__ void load(const float* __restrict__ gam, const float* __restrict__ beta,
                                         int valid) {
        valid_ = valid;
        const int t = threadIdx.x;
        const int tt = t < valid ? t : valid - 1;
        b = beta[tt];
        if (GATE == kGateScalar) {
            gs = gam[tt];
            gC = gam[valid - 1];
        }
        if (VEC) gv.load_clamped(gam, DK, valid);
    }
    __device__ __forceinline__ void commit(float* rowf, float* gam_s, float* beta_s) const {
        const int t = threadIdx.x;
        if (t < C) beta_s[t] = t < valid_ ? b : 0.f;
        if (GATE == kGateScalar && t < C) {
            rowf[t] = fexp(gs);
            rowf[C + t] = fexp(gC - gs);
            gam_s[t] = gs;
        }
        if (VEC) gv.store(gam_s, DK);
    }
};

// Decay factors read back from LDS after GateRegs::commit.
template <int GATE, int C, int DK> struct GateLds {
    const float* rowf;
    const float* gam_s;
    int last;                  // valid - 1
    const float* gl = nullptr; // vector gate: a copy of row `last` of gam_s, if gam_s is reused
    // e^{gam[t][c]}
    __device__ __forceinline__ float G(int t, int c) const {
        if (GATE == kGateNone) return 1.f;
        if (GATE == kGateScalar) return rowf[t];
        return fexp(gam_s[t * DK + c]);
    }
    // e^{gam_C[c] - gam[t][c]}
    __device__ __forceinline__ float Gd(int t, int c) const {
        if (GATE == kGateNone) return 1.f;
        if (GATE == kGateScalar) return rowf[C + t];
        return fexp(gam_s[last * DK + c] - gam_s[t * DK + c]);
    }
    // e^{gam_C[c]}
    __device__ __forceinline__ float GC(int c) const {
        if (GATE == kGateNone) return 1.f;
        if (GATE == kGateScalar) return rowf[last];
        return fexp(gl ? gl[c] : gam_s[last * DK + c]);
    }
};

// ---------------------------------------------------------------------------
// fwd_state_kernel: grid (DV / BV, BH).  Walks the chunks of one head in order
// for one block of BV state rows (rows of S are independent: each row only
// mixes with itself through the key dimension).  The global tiles of chunk
// n + 1 are loaded into registers while chunk n is computed.
//   SAVE    : write the state entering each chunk (I/O type) to p.states
//   OUTPUT  : write O and hT.  Off for the recompute pass of the backward, where
//             the workspace holds T^T (and P is not needed).
template <typename TI, int GATE, int C, int DK, int BV, bool SAVE, bool OUTPUT>
__global__ __launch_bounds__(kThreads) void fwd_state_kernel(Params p) {
    constexpr int PAD = Pad<TI>::value;
    constexpr int LDK = DK + PAD;
    constexpr int LDC = C + PAD;
    constexpr int LDV = BV + PAD;
    constexpr int GW = GateLayout<GATE, DK>::GW;
    __shared__ float gam_s[GATE == kGateVector ? C * DK : C];
    __shared__ float rowf[2 * C];
    __shared__ float beta_s[C];
    __shared__ __align__(16) TI Ss[BV * LDK];    // S0 (operand copy) [v][c]
    __shared__ __align__(16) TI Qg[C * LDK];     // Q Gam            [t][c]
    __shared__ __align__(16) TI Kg[C * LDK];     // K Gam            [t][c]
    __shared__ __align__(16) TI KdT[DK * LDC];   // (K Gam_C / Gam)^T [c][t]
    __shared__ __align__(16) TI Vb[C * LDV];     // V block          [t][v]
    __shared__ __align__(16) TI Tl[C * LDC];     // T                [t][s]
    __shared__ __align__(16) TI Pl[C * LDC];     // P                [t][s]
    // R^T [v][t]; after (d) it holds the chunk's O [t][v] until the next iteration writes it back
    constexpr int RT_ELEMS = BV * LDC > C * LDV ? BV * LDC : C * LDV;
    __shared__ __align__(16) TI RT[RT_ELEMS];
    __shared__ __align__(16) TI UT[BV * LDC];    // U^T              [v][t]

    const int DVr = p.DVr;
    const int bh = blockIdx.y;
    const int v0 = blockIdx.x * BV;
    using TS = Tiles<BV, DK>;
    f32x4 S[TS::PER];
#pragma unroll
    for (int j = 0; j < TS::PER; ++j) {
        S[j] = zero4();
        if (p.h0 && TS::active()) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[j][i] = p.h0[((long)bh * DVr + v0 + TS::row(j, i)) * DK + TS::col(j)];
        }
    }

    // registers of the next chunk
    RegN<TI, C, DK> rq;
    RegB<TI, C, DK> rk;
    RegN<TI, C, BV> rv;
    std::conditional_t<OUTPUT, RegN<TI, C, C>, RegB<TI, C, C>> rT;
    RegN<TI, OUTPUT ? C : 16, OUTPUT ? C : 16> rP;
    GateRegs<GATE, C, DK> rg;
    auto prefetch = [&](int n) {
        const int t0 = n * C;
        const int valid = min(C, p.T - t0);
        const long row0 = (long)bh * p.T + t0;
        const long cc = ((long)bh * p.NT + n) * C * C;
        rg.load(p.gam + row0 * GW, p.beta + row0, valid);
        rq.load(static_cast<const TI*>(p.q) + row0 * DK, DK, valid);
        rk.load(static_cast<const TI*>(p.k) + row0 * DK, DK, valid);
        rv.load(static_cast<const TI*>(p.v) + row0 * DVr + v0, DVr, valid);
        rT.load(static_cast<const TI*>(p.Tm) + cc, C, C);
        if constexpr (OUTPUT) rP.load(static_cast<const TI*>(p.Pm) + cc, C, C);
    };
    prefetch(0);

    for (int n = 0; n < p.NT; ++n) {
        const int t0 = n * C;
        const int valid = min(C, p.T - t0);
        const long row0 = (long)bh * p.T + t0;
        // write back the previous chunk's O (a full chunk of work after it was formed,
        // so the stores never sit just ahead of a wait on this chunk's loads)
        if (OUTPUT && n > 0)
            lds_to_global<TI, C, BV>(static_cast<TI*>(p.o) + (row0 - C) * DVr + v0, DVr, RT, LDV, C);
        // (a) state operand (saved from LDS below)
        if (TS::active()) {
#pragma unroll
            for (int j = 0; j < TS::PER; ++j) {
#pragma unroll
                for (int i = 0; i < 4; ++i) Ss[TS::row(j, i) * LDK + TS::col(j)] = from_f<TI>(S[j][i]);
            }
        }
        // (b) commit this chunk's tiles to LDS
        rg.commit(rowf, gam_s, beta_s);
        __syncthreads();
        const GateLds<GATE, C, DK> gf{rowf, gam_s, valid - 1};
        if (GATE == kGateNone) {
            rq.store(Qg, LDK);
            rk.store_n(Kg, LDK, Identity());
            rk.store_t(KdT, LDC, Identity());
        } else {
            rq.store(Qg, LDK, [&](int r, int c, float x) { return x * gf.G(r, c); });
            rk.store_n(Kg, LDK, [&](int r, int c, float x) { return x * gf.G(r, c); });
            rk.store_t(KdT, LDC, [&](int r, int c, float x) { return x * gf.Gd(r, c); });
        }
        rv.store(Vb, LDV);
        if constexpr (OUTPUT) {
            rT.store(Tl, LDC);
            rP.store(Pl, LDC);
        } else {
            rT.store_t(Tl, LDC, Identity());
        }
        __syncthreads();
        if (n + 1 < p.NT) prefetch(n + 1);
        if (SAVE)
            lds_to_global<TI, BV, DK>(static_cast<TI*>(p.states) + (((long)bh * p.NT + n) * DVr + v0) * DK, DK, Ss,
                                      LDK, BV);

        // (c) X = (K Gam) S0^T ;  R = diag(beta) (V - X)  -> R^T
        using TX = Tiles<C, BV>;
        {
            f32x4 X[TX::PER];
            zero_acc<C, BV>(X);
            gemm_nt<TI, C, BV, DK>(X, Kg, LDK, Ss, LDK);
            if (TX::active()) {
                // all LDS reads, then all LDS writes (see RegN::store)
                float rv_[TX::PER][4];
#pragma unroll
                for (int j = 0; j < TX::PER; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = TX::row(j, i), c = TX::col(j);
                        rv_[j][i] = beta_s[t] * (to_f(Vb[t * LDV + c]) - X[j][i]);
                    }
#pragma unroll
                for (int j = 0; j < TX::PER; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) RT[TX::col(j) * LDC + TX::row(j, i)] = from_f<TI>(rv_[j][i]);
            }
        }
        __syncthreads();
        // (d) U = T R  -> U^T
        {
            f32x4 U[TX::PER];
            zero_acc<C, BV>(U);
            gemm_nt<TI, C, BV, C>(U, Tl, LDC, RT, LDC);
            if (TX::active()) {
#pragma unroll
                for (int j = 0; j < TX::PER; ++j) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) UT[TX::col(j) * LDC + TX::row(j, i)] = from_f<TI>(U[j][i]);
                }
            }
        }
        __syncthreads();
        // (e) O = (Q Gam) S0^T + P U   (into RT, dead since (d); written back next iteration)
        if (OUTPUT) {
            f32x4 O[TX::PER];
            zero_acc<C, BV>(O);
            gemm_nt<TI, C, BV, DK>(O, Qg, LDK, Ss, LDK);
            gemm_nt<TI, C, BV, C>(O, Pl, LDC, UT, LDC);
            if (TX::active()) {
#pragma unroll
                for (int j = 0; j < TX::PER; ++j) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) RT[TX::row(j, i) * LDV + TX::col(j)] = from_f<TI>(O[j][i]);
                }
            }
        }
        // (f) S1 = S0 Diag(Gam_C) + U^T (K Gam_C / Gam)
        if (GATE != kGateNone && TS::active()) {
#pragma unroll
            for (int j = 0; j < TS::PER; ++j) {
                const float f = gf.GC(TS::col(j));
#pragma unroll
                for (int i = 0; i < 4; ++i) S[j][i] *= f;
            }
        }
        gemm_nt<TI, BV, DK, C>(S, UT, LDC, KdT, LDC);
        __syncthreads();
    }
    if (OUTPUT && p.NT > 0) {
        const int t0 = (p.NT - 1) * C;
        lds_to_global<TI, C, BV>(static_cast<TI*>(p.o) + ((long)bh * p.T + t0) * DVr + v0, DVr, RT, LDV,
                                 min(C, p.T - t0));
    }
    if (OUTPUT && p.hT && TS::active()) {
#pragma unroll
        for (int j = 0; j < TS::PER; ++j) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                p.hT[((long)bh * DVr + v0 + TS::row(j, i)) * DK + TS::col(j)] = S[j][i];
        }
    }
}

}  // namespace dn
