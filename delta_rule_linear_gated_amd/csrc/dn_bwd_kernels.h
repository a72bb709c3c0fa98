// dn_bwd_kernels.h -- backward-pass kernels (reduced ReWY form).
//
// Cotangents: dO for the outputs and dS1 for the state leaving a chunk
// (dhT for the last chunk).  Differentiating the chunk form of
// dn_fwd_kernels.h line by line, with the triangular system (I + A) U = R
// differentiated as one residual system (ReWY abstract) -- a single transposed
// solve, no adjoint of the explicit inverse T:
//     dU     = P^T dO + Kd dS1^T                     Kd = K Gam_C / Gam
//     lambda = (I + A)^{-T} dU = T^T dU
//     dS0    = dS1 Diag(Gam_C) + dO^T (Q Gam) - (diag(beta) lambda)^T (K Gam)
//     dV     = diag(beta) lambda
//     dA     = -strictly-lower(lambda U^T)           dP = lower(dO U^T)
//     dbeta  = rowsum(lambda (V - (K Gam) S0^T)) + [A term]
// bwd_state_kernel carries dS backwards through the chunks (sequential in
// chunks, parallel over d_v blocks) and leaves lambda and dS1 per chunk;
// bwd_chunk_kernel then finishes every chunk independently:
//   * U is recomputed from the saved S0;
//   * the A and P adjoints reach K and Q through key-gradient products
//     (dA~ K, dA~^T K, dP~ K, dP~^T Q), and the gate gradient of the scalar gate
//     is read off those same products (sum_c k (dA~ K) etc.) instead of
//     re-forming the K K^T / Q K^T Gram matrices (the scalar-gate reduction of
//     the ReWY abstract);
//   * for the vector gate the same products run on the centred factors
//     K e^{gam - c}, K e^{c - gam}, Q e^{gam - c} (centred contraction), and the
//     per-channel gate gradient is elementwise;
//   * dg is the reverse cumulative sum of d gam inside the chunk.
#pragma once

#include "dn_device.h"
#include "dn_fwd_kernels.h"
#include "dn_internal.h"

namespace dn {

// ---------------------------------------------------------------------------
// bwd_state_kernel: grid (DV / BV, BH), chunks walked from last to first; the
// global tiles of chunk n - 1 are loaded into registers while chunk n is
// computed.  The workspace holds T^T and P^T here (prep_kernel<..., true>).
template <typename TI, int GATE, int C, int DK, int BV>
__global__ __launch_bounds__(kThreads) void bwd_state_kernel(Params p) {
    constexpr int PAD = Pad<TI>::value;
    constexpr int LDK = DK + PAD;
    constexpr int LDC = C + PAD;
    constexpr int GW = GateLayout<GATE, DK>::GW;
    __shared__ float gam_s[GATE == kGateVector ? C * DK : 4];
    __shared__ float rowf[2 * C];
    __shared__ float beta_s[C];
    __shared__ __align__(16) TI dSs[BV * LDK];   // dS1 operand     [v][c]
    __shared__ __align__(16) TI Kd[C * LDK];     // K Gam_C / Gam   [t][c]
    __shared__ __align__(16) TI PT[C * LDC];     // P^T             [t][s]
    __shared__ __align__(16) TI TT[C * LDC];     // T^T             [t][s]
    __shared__ __align__(16) TI dOT[BV * LDC];   // dO^T block      [v][t]
    __shared__ __align__(16) TI QgT[DK * LDC];   // (Q Gam)^T       [c][t]
    __shared__ __align__(16) TI KgT[DK * LDC];   // (K Gam)^T       [c][t]
    __shared__ __align__(16) TI dUT[BV * LDC];   // dU^T            [v][t]
    __shared__ __align__(16) TI bLT[BV * LDC];   // -(beta lambda)^T [v][t]

    const int DVr = p.DVr;
    const int bh = blockIdx.y;
    const int v0 = blockIdx.x * BV;
    using TS = Tiles<BV, DK>;
    f32x4 dS[TS::PER];
#pragma unroll
    for (int j = 0; j < TS::PER; ++j) {
        dS[j] = zero4();
        if (p.dhT && TS::active()) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dS[j][i] = p.dhT[((long)bh * DVr + v0 + TS::row(j, i)) * DK + TS::col(j)];
        }
    }

    RegB<TI, C, DK> rq, rk;
    RegB<TI, C, BV> rdo;
    RegN<TI, C, C> rPT, rTT;
    GateRegs<GATE, C, DK> rg;
    auto prefetch = [&](int n) {
        const int t0 = n * C;
        const int valid = min(C, p.T - t0);
        const long row0 = (long)bh * p.T + t0;
        const long cc = ((long)bh * p.NT + n) * C * C;
        rg.load(p.gam + row0 * GW, p.beta + row0, valid);
        rq.load(static_cast<const TI*>(p.q) + row0 * DK, DK, valid);
        rk.load(static_cast<const TI*>(p.k) + row0 * DK, DK, valid);
        rdo.load(static_cast<const TI*>(p.dout) + row0 * DVr + v0, DVr, valid);
        rPT.load(static_cast<const TI*>(p.Pm) + cc, C, C);
        rTT.load(static_cast<const TI*>(p.Tm) + cc, C, C);
    };
    prefetch(p.NT - 1);

    for (int n = p.NT - 1; n >= 0; --n) {
        const int t0 = n * C;
        const int valid = min(C, p.T - t0);
        const long row0 = (long)bh * p.T + t0;
        // (a) dS1 of this chunk: operand copy and workspace copy
        TI* __restrict__ dsv = static_cast<TI*>(p.dS1) + (((long)bh * p.NT + n) * DVr + v0) * DK;
        if (TS::active()) {
#pragma unroll
            for (int j = 0; j < TS::PER; ++j) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = TS::row(j, i), c = TS::col(j);
                    const TI x = from_f<TI>(dS[j][i]);
                    dSs[r * LDK + c] = x;
                    dsv[r * DK + c] = x;
                }
            }
        }
        // (b) commit this chunk's tiles
        rg.commit(rowf, gam_s, beta_s);
        __syncthreads();
        const GateLds<GATE, C, DK> gf{rowf, gam_s, valid - 1};
        if (GATE == kGateNone) {
            rk.store_n(Kd, LDK, Identity());
            rq.store_t(QgT, LDC, Identity());
            rk.store_t(KgT, LDC, Identity());
        } else {
            rk.store_n(Kd, LDK, [&](int r, int c, float x) { return x * gf.Gd(r, c); });
            rq.store_t(QgT, LDC, [&](int r, int c, float x) { return x * gf.G(r, c); });
            rk.store_t(KgT, LDC, [&](int r, int c, float x) { return x * gf.G(r, c); });
        }
        rdo.store_t(dOT, LDC, Identity());
        rPT.store(PT, LDC);
        rTT.store(TT, LDC);
        __syncthreads();
        if (n > 0) prefetch(n - 1);

        using TX = Tiles<C, BV>;
        // (c) dU = P^T dO + Kd dS1^T  -> dU^T
        {
            f32x4 dU[TX::PER];
            zero_acc<C, BV>(dU);
            gemm_nt<TI, C, BV, C>(dU, PT, LDC, dOT, LDC);
            gemm_nt<TI, C, BV, DK>(dU, Kd, LDK, dSs, LDK);
            if (TX::active()) {
#pragma unroll
                for (int j = 0; j < TX::PER; ++j) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) dUT[TX::col(j) * LDC + TX::row(j, i)] = from_f<TI>(dU[j][i]);
                }
            }
        }
        __syncthreads();
        // (d) lambda = T^T dU ; dv = beta lambda ; keep -(beta lambda)^T
        {
            f32x4 L[TX::PER];
            zero_acc<C, BV>(L);
            gemm_nt<TI, C, BV, C>(L, TT, LDC, dUT, LDC);
            TI* __restrict__ lam = static_cast<TI*>(p.lam) + ((long)bh * p.NT + n) * C * DVr + v0;
            TI* __restrict__ dv = static_cast<TI*>(p.dv) + row0 * DVr + v0;
            if (TX::active()) {
#pragma unroll
                for (int j = 0; j < TX::PER; ++j) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = TX::row(j, i), c = TX::col(j);
                        const float l = L[j][i];
                        const float bl = beta_s[t] * l;
                        lam[(long)t * DVr + c] = from_f<TI>(l);
                        if (t < valid) dv[(long)t * DVr + c] = from_f<TI>(bl);
                        bLT[c * LDC + t] = from_f<TI>(-bl);
                    }
                }
            }
        }
        __syncthreads();
        // (e) dS0 = dS1 Diag(Gam_C) + dO^T (Q Gam) - (beta lambda)^T (K Gam)
        if (GATE != kGateNone && TS::active()) {
#pragma unroll
            for (int j = 0; j < TS::PER; ++j) {
                const float f = gf.GC(TS::col(j));
#pragma unroll
                for (int i = 0; i < 4; ++i) dS[j][i] *= f;
            }
        }
        gemm_nt<TI, BV, DK, C>(dS, dOT, LDC, QgT, LDC);
        gemm_nt<TI, BV, DK, C>(dS, bLT, LDC, KgT, LDC);
        __syncthreads();
    }
    if (p.dh0 && TS::active()) {
#pragma unroll
        for (int j = 0; j < TS::PER; ++j) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                p.dh0[((long)bh * DVr + v0 + TS::row(j, i)) * DK + TS::col(j)] = dS[j][i];
        }
    }
}

// ---------------------------------------------------------------------------
// bwd_chunk_kernel: grid (NT, BH); every chunk finished independently.
// D = d_k = d_v.  LDS is carved by phase (see the offsets below).
template <typename TI, int GATE, int C, int D>
struct BwdChunkSmem {
    static constexpr int PAD = Pad<TI>::value;
    static constexpr int LD = D + PAD;   // rows of D elements
    static constexpr int LC = C + PAD;   // rows of C elements
    static constexpr int GW = GateLayout<GATE, D>::GW;
    static constexpr size_t E = sizeof(TI);
    static constexpr size_t al(size_t x) { return (x + 255) & ~size_t(255); }
    static constexpr size_t CxD = al(C * LD * E);    // [C][D] tile
    static constexpr size_t DxD = al(D * LD * E);    // [D][D] tile
    static constexpr size_t DxC = al(D * LC * E);    // [D][C] tile
    static constexpr size_t CxC = al(C * LC * E);    // [C][C] tile
    // persistent
    static constexpr size_t LAM = 0;                 // lambda  [t][v]   phases A, D, B
    static constexpr size_t UB = LAM + CxD;          // U       [t][v]   phases A, D, B
    static constexpr size_t DOB = UB + CxD;          // dO      [t][v]   phases D, B (T in phase A)
    static constexpr size_t BIG = DOB + CxD;
    // phase A
    static constexpr size_t A_KG = BIG;              // K Gam   [t][c]
    static constexpr size_t A_S0 = A_KG + CxD;       // S0      [v][c]
    static constexpr size_t A_RT = A_S0 + DxD;       // R^T     [v][t]
    static constexpr size_t A_END = A_RT + DxC;
    static constexpr size_t A_T = DOB;               // T       [t][s]
    // phase D
    static constexpr size_t D_S0T = BIG;             // S0^T    [c][v]
    static constexpr size_t D_DS1T = D_S0T + DxD;    // dS1^T   [c][v]
    static constexpr size_t D_END = D_DS1T + DxD;
    // phase B/C
    static constexpr size_t B_DA = BIG;              // dA~     [t][s]
    static constexpr size_t B_DAT = B_DA + CxC;      // dA~^T beta  [s][t]
    static constexpr size_t B_DP = B_DAT + CxC;      // dP~     [t][s]
    static constexpr size_t B_DPT = B_DP + CxC;      // dP~^T   [s][t]
    static constexpr size_t C_KRT = 0;               // (K or K e^{c-gam})^T  [c][s]   (over LAM/UB)
    static constexpr size_t C_KLT = C_KRT + DxC;     // (K e^{gam-c})^T        [c][t]   (vector only)
    static constexpr size_t C_QLT = B_DPT + CxC;     // (Q or Q e^{gam-c})^T  [c][t]
    static constexpr size_t C_END = C_QLT + DxC;
    // small fp32 arrays
    static constexpr size_t F_END0 = A_END > D_END ? A_END : D_END;
    static constexpr size_t F_END1 = F_END0 > C_END ? F_END0 : C_END;
    static constexpr size_t GAM = al(F_END1);                        // gam  [C][GW]
    static constexpr size_t BETA = GAM + al(C * GW * 4);             // beta [C]
    static constexpr size_t RED_R = BETA + al(C * 4);                // row partials [D/16][C]
    static constexpr int SPLIT = kThreads / D > 0 ? kThreads / D : 1;
    static constexpr int REDC_ROWS = (C / 16) > SPLIT ? (C / 16) : SPLIT;
    static constexpr size_t RED_C = RED_R + al((D / 16) * C * 4);    // column partials [C/16][D]
    static constexpr size_t LASTS = RED_C + al(REDC_ROWS * D * 4);   // sum_v S0 dS1 per channel [D]
    static constexpr size_t DBR = LASTS + al(D * 4);                 // dbeta partial [C]
    static constexpr size_t ROWF = DBR + al(C * 4);                  // scalar gate row factors [2][C]
    static constexpr size_t TOTAL = ROWF + al(2 * C * 4);
    // d gam of the vector gate [C][D] fp32, written once every phase-C tile is dead
    static constexpr size_t DGB = BIG;
    static_assert(GATE != kGateVector || DGB + C * D * 4 <= TOTAL, "d gam buffer");
    static_assert(C_KLT + DxC <= BIG || GATE != kGateVector, "K+ tile must fit below BIG");
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

template <typename TI, int GATE, int C, int D>
__global__ __launch_bounds__(kThreads) void bwd_chunk_kernel(Params p) {
    using L = BwdChunkSmem<TI, GATE, C, D>;
    constexpr int LD = L::LD, LC = L::LC, GW = L::GW;
    constexpr bool VEC = GATE == kGateVector;
    constexpr bool SCA = GATE == kGateScalar;
    __shared__ __align__(16) char smem[L::TOTAL];
    TI* lamb = reinterpret_cast<TI*>(smem + L::LAM);
    TI* Ub = reinterpret_cast<TI*>(smem + L::UB);
    TI* dOb = reinterpret_cast<TI*>(smem + L::DOB);
    float* gam_s = reinterpret_cast<float*>(smem + L::GAM);
    float* beta_s = reinterpret_cast<float*>(smem + L::BETA);
    float* red_r = reinterpret_cast<float*>(smem + L::RED_R);
    float* red_c = reinterpret_cast<float*>(smem + L::RED_C);
    float* lastS = reinterpret_cast<float*>(smem + L::LASTS);
    float* dbr = reinterpret_cast<float*>(smem + L::DBR);
    float* rowf = reinterpret_cast<float*>(smem + L::ROWF);   // scalar gate: e^{gam_t}, e^{gam_C - gam_t}
    float* dgb = reinterpret_cast<float*>(smem + L::DGB);

    const int n = blockIdx.x, bh = blockIdx.y;
    const int t0 = n * C;
    const int valid = min(C, p.T - t0);
    const long row0 = (long)bh * p.T + t0;
    const long chunk = (long)bh * p.NT + n;
    const TI* __restrict__ q = static_cast<const TI*>(p.q) + row0 * D;
    const TI* __restrict__ k = static_cast<const TI*>(p.k) + row0 * D;
    const TI* __restrict__ v = static_cast<const TI*>(p.v) + row0 * D;
    const TI* __restrict__ dO = static_cast<const TI*>(p.dout) + row0 * D;
    const TI* __restrict__ S0g = static_cast<const TI*>(p.states) + chunk * D * D;
    const TI* __restrict__ dS1g = static_cast<const TI*>(p.dS1) + chunk * D * D;
    const TI* __restrict__ lamg = static_cast<const TI*>(p.lam) + chunk * C * D;

    using TO = Tiles<C, D>;   // every C x D output of this kernel uses this tile map
    using TCC = Tiles<C, C>;

    // ---------------- prologue: gate, beta, row factors, sum_v S0 dS1, k at this lane's elements
    load_gam_beta<GATE, C, D>(gam_s, beta_s, p.gam + row0 * GW, p.beta + row0, valid);
    {
        // sum over v of S0[v][c] dS1[v][c] (gradient of S0 Diag(Gam_C) with respect to gam_C)
        constexpr int SPLIT = kThreads / D > 0 ? kThreads / D : 1;
        float* part = red_c;  // [SPLIT][D] scratch, consumed below before red_c is used again
        for (int idx = threadIdx.x; idx < D * SPLIT; idx += kThreads) {
            const int c = idx % D, h = idx / D;
            float acc = 0.f;
            for (int vv = h; vv < D; vv += SPLIT) acc += to_f(S0g[(long)vv * D + c]) * to_f(dS1g[(long)vv * D + c]);
            part[h * D + c] = acc;
        }
        __syncthreads();
        for (int c = threadIdx.x; c < D; c += kThreads) {
            float acc = 0.f;
            for (int h = 0; h < SPLIT; ++h) acc += part[h * D + c];
            lastS[c] = acc;
        }
    }
    if (SCA) {
        for (int t = threadIdx.x; t < C; t += kThreads) {
            const float gl0 = gam_s[valid - 1];
            rowf[t] = fexp(gam_s[t]);
            rowf[C + t] = fexp(gl0 - gam_s[t]);
        }
    }
    float kv[TO::PER][4];
#pragma unroll
    for (int j = 0; j < TO::PER; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = TO::row(j, i);
            kv[j][i] = (TO::active() && t < valid) ? to_f(k[(long)t * D + TO::col(j)]) : 0.f;
        }
    __syncthreads();
    const float* gl = gam_s + (valid - 1) * GW;
    // per-element decay factors: Gm = e^{gam}, Gd = e^{gam_C - gam}; vector gate also
    // fp = e^{gam - centre}, fm = e^{centre - gam} with centre = gam_C / 2
    auto Gm = [&](int t, int c) -> float {
        if (GATE == kGateNone) return 1.f;
        return SCA ? rowf[t] : fexp(gam_s[t * D + c]);
    };
    auto Gd = [&](int t, int c) -> float {
        if (GATE == kGateNone) return 1.f;
        return SCA ? rowf[C + t] : fexp(gl[c] - gam_s[t * D + c]);
    };

    // ---------------- phase A: X = (K Gam) S0^T, R = beta (V - X), U = T R, dbeta_R
    {
        TI* Kg = reinterpret_cast<TI*>(smem + L::A_KG);
        TI* S0 = reinterpret_cast<TI*>(smem + L::A_S0);
        TI* RT = reinterpret_cast<TI*>(smem + L::A_RT);
        TI* Tl = reinterpret_cast<TI*>(smem + L::A_T);
        if (VEC)
            stage<TI, C, D, false>(Kg, LD, k, D, valid, [&](int r, int c, float x) { return x * fexp(gam_s[r * D + c]); });
        else
            stage_copy<TI, C, D, false>(Kg, LD, k, D, valid);   // scalar: Gam_t applied to X's rows
        stage_copy<TI, D, D, false>(S0, LD, S0g, D, D);
        stage_copy<TI, C, D, false>(lamb, LD, lamg, D, C);
        stage_copy<TI, C, C, true>(Tl, LC, static_cast<const TI*>(p.Tm) + chunk * C * C, C, C);  // ws holds T^T
        __syncthreads();
        f32x4 X[TO::PER];
        zero_acc<C, D>(X);
        gemm_nt<TI, C, D, D>(X, Kg, LD, S0, LD);
        if (TO::active()) {
#pragma unroll
            for (int j = 0; j < TO::PER; ++j) {
                float part[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = TO::row(j, i), c = TO::col(j);
                    const float vv = t < valid ? to_f(v[(long)t * D + c]) : 0.f;
                    const float xr = vv - (SCA ? rowf[t] : 1.f) * X[j][i];
                    part[i] = to_f(lamb[t * LD + c]) * xr;
                    RT[c * LC + t] = from_f<TI>(beta_s[t] * xr);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float s = row16_sum(part[i]);
                    if ((lane_id() & 15) == 0) red_r[(TO::n0(j) / 16) * C + TO::row(j, i)] = s;
                }
            }
        }
        __syncthreads();
        for (int t = threadIdx.x; t < C; t += kThreads) {
            float s = 0.f;
            for (int b = 0; b < D / 16; ++b) s += red_r[b * C + t];
            dbr[t] = s;
        }
        f32x4 U[TO::PER];
        zero_acc<C, D>(U);
        gemm_nt<TI, C, D, C>(U, Tl, LC, RT, LC);
        __syncthreads();  // T (over dO) and RT dead after this point
        if (TO::active()) {
#pragma unroll
            for (int j = 0; j < TO::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) Ub[TO::row(j, i) * LD + TO::col(j)] = from_f<TI>(U[j][i]);
        }
    }

    // ---------------- phase D: dO S0, lambda S0, U dS1 (contractions over d_v)
    // dq accumulates dL/dq, dk dL/dk, dkp the part of dL/dk reached through
    // factors e^{+gam} (K Gam, K e^{gam - centre}); the rest of dk came through
    // e^{-gam} factors, so d gam = q.dq + k.(2 dkp - dk) + the gam_C terms.
    f32x4 dq[TO::PER], dk[TO::PER], dkp[TO::PER];
    zero_acc<C, D>(dq);
    zero_acc<C, D>(dk);
    zero_acc<C, D>(dkp);
    {
        TI* S0T = reinterpret_cast<TI*>(smem + L::D_S0T);
        TI* dS1T = reinterpret_cast<TI*>(smem + L::D_DS1T);
        stage_copy<TI, D, D, true>(S0T, LD, S0g, D, D);
        stage_copy<TI, D, D, true>(dS1T, LD, dS1g, D, D);
        stage_copy<TI, C, D, false>(dOb, LD, dO, D, valid);
        __syncthreads();
        f32x4 tmp[TO::PER];
        zero_acc<C, D>(tmp);
        gemm_nt<TI, C, D, D>(tmp, dOb, LD, S0T, LD);
        if (TO::active()) {
#pragma unroll
            for (int j = 0; j < TO::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) dq[j][i] = tmp[j][i] * Gm(TO::row(j, i), TO::col(j));
        }
        zero_acc<C, D>(tmp);
        gemm_nt<TI, C, D, D>(tmp, lamb, LD, S0T, LD);
        if (TO::active()) {
#pragma unroll
            for (int j = 0; j < TO::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = TO::row(j, i);
                    const float x = -beta_s[t] * tmp[j][i] * Gm(t, TO::col(j));
                    dk[j][i] = x;
                    dkp[j][i] = x;
                }
        }
        zero_acc<C, D>(tmp);
        gemm_nt<TI, C, D, D>(tmp, Ub, LD, dS1T, LD);
        if (TO::active()) {
#pragma unroll
            for (int j = 0; j < TO::PER; ++j) {
                float colp = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x = tmp[j][i] * Gd(TO::row(j, i), TO::col(j));
                    dk[j][i] += x;
                    colp += kv[j][i] * x;   // Kd * dKd, summed over rows for the gam_C term
                }
                colp += __shfl_xor(colp, 16);
                colp += __shfl_xor(colp, 32);
                if (lane_id() < 16) red_c[(TO::m0(j) / 16) * D + TO::col(j)] = colp;
            }
        }
        __syncthreads();  // S0T / dS1T dead
    }

    // ---------------- phase B: dA~ and dP~ from lambda U^T and dO U^T
    {
        TI* dA = reinterpret_cast<TI*>(smem + L::B_DA);
        TI* dAT = reinterpret_cast<TI*>(smem + L::B_DAT);
        TI* dP = reinterpret_cast<TI*>(smem + L::B_DP);
        TI* dPT = reinterpret_cast<TI*>(smem + L::B_DPT);
        f32x4 acc[TCC::PER];
        if (TCC::active()) {
#pragma unroll
            for (int j = 0; j < TCC::PER; ++j) {
                const bool upper = TCC::n0(j) > TCC::m0(j);
                acc[j] = zero4();
                if (!upper) acc[j] = tile_nt<TI, D>(lamb + TCC::m0(j) * LD, LD, Ub + TCC::n0(j) * LD, LD, acc[j]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = TCC::row(j, i), s = TCC::col(j);
                    float a = 0.f;
                    if (s < t) {
                        a = -acc[j][i];  // dA = -lambda U^T
                        if (SCA) a *= fexp(gam_s[t] - gam_s[s]);
                    }
                    dA[t * LC + s] = from_f<TI>(a);
                    dAT[s * LC + t] = from_f<TI>(beta_s[t] * a);
                }
            }
#pragma unroll
            for (int j = 0; j < TCC::PER; ++j) {
                const bool upper = TCC::n0(j) > TCC::m0(j);
                acc[j] = zero4();
                if (!upper) acc[j] = tile_nt<TI, D>(dOb + TCC::m0(j) * LD, LD, Ub + TCC::n0(j) * LD, LD, acc[j]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = TCC::row(j, i), s = TCC::col(j);
                    float a = 0.f;
                    if (s <= t) {
                        a = acc[j][i];
                        if (SCA) a *= fexp(gam_s[t] - gam_s[s]);
                    }
                    dP[t * LC + s] = from_f<TI>(a);
                    dPT[s * LC + t] = from_f<TI>(a);
                }
            }
        }
        __syncthreads();  // lambda, U, dO dead
    }

    // ---------------- phase C: key-gradient products
    {
        const TI* dA = reinterpret_cast<const TI*>(smem + L::B_DA);
        const TI* dAT = reinterpret_cast<const TI*>(smem + L::B_DAT);
        const TI* dP = reinterpret_cast<const TI*>(smem + L::B_DP);
        const TI* dPT = reinterpret_cast<const TI*>(smem + L::B_DPT);
        TI* KrT = reinterpret_cast<TI*>(smem + L::C_KRT);
        TI* KlT = VEC ? reinterpret_cast<TI*>(smem + L::C_KLT) : KrT;
        TI* QlT = reinterpret_cast<TI*>(smem + L::C_QLT);
        if (VEC) {
            stage_t<TI, C, D>(KrT, LC, k, D, valid,
                              [&](int r, int c, float x) { return x * fexp(0.5f * gl[c] - gam_s[r * D + c]); });
            stage_t<TI, C, D>(KlT, LC, k, D, valid,
                              [&](int r, int c, float x) { return x * fexp(gam_s[r * D + c] - 0.5f * gl[c]); });
            stage_t<TI, C, D>(QlT, LC, q, D, valid,
                              [&](int r, int c, float x) { return x * fexp(gam_s[r * D + c] - 0.5f * gl[c]); });
        } else {
            stage_copy<TI, C, D, true>(KrT, LC, k, D, valid);
            stage_copy<TI, C, D, true>(QlT, LC, q, D, valid);
        }
        __syncthreads();
        auto fpl = [&](int t, int c) -> float { return VEC ? fexp(gam_s[t * D + c] - 0.5f * gl[c]) : 1.f; };
        float dbA[TO::PER][4];
        f32x4 tmp[TO::PER];
        // Y = dA~ Kr :  dK+ = beta Y, dbeta_A = sum_c K+ Y
        zero_acc<C, D>(tmp);
        gemm_nt<TI, C, D, C>(tmp, dA, LC, KrT, LC);
        if (TO::active()) {
#pragma unroll
            for (int j = 0; j < TO::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = TO::row(j, i);
                    const float fp = fpl(t, TO::col(j));
                    const float y = tmp[j][i];
                    dbA[j][i] = kv[j][i] * fp * y;
                    const float x = beta_s[t] * y * fp;
                    dk[j][i] += x;
                    dkp[j][i] += x;
                }
        }
        // Z = (beta dA~)^T Kl and W = dP~^T Ql : both reach k through e^{-gam}
        zero_acc<C, D>(tmp);
        gemm_nt<TI, C, D, C>(tmp, dAT, LC, KlT, LC);
        gemm_nt<TI, C, D, C>(tmp, dPT, LC, QlT, LC);
        if (TO::active()) {
#pragma unroll
            for (int j = 0; j < TO::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float fm = VEC ? 1.f / fpl(TO::row(j, i), TO::col(j)) : 1.f;
                    dk[j][i] += tmp[j][i] * fm;
                }
        }
        // dQ+ = dP~ Kr
        zero_acc<C, D>(tmp);
        gemm_nt<TI, C, D, C>(tmp, dP, LC, KrT, LC);
        if (TO::active()) {
#pragma unroll
            for (int j = 0; j < TO::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) dq[j][i] += tmp[j][i] * fpl(TO::row(j, i), TO::col(j));
        }

        // -------- finish: dq, dk, dbeta, dg
        TI* __restrict__ dqo = static_cast<TI*>(p.dq) + row0 * D;
        TI* __restrict__ dko = static_cast<TI*>(p.dk) + row0 * D;
        float dgm[TO::PER][4];
        if (TO::active()) {
#pragma unroll
            for (int j = 0; j < TO::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = TO::row(j, i), c = TO::col(j);
                    float qq = 0.f;
                    if (t < valid) {
                        dqo[(long)t * D + c] = from_f<TI>(dq[j][i]);
                        dko[(long)t * D + c] = from_f<TI>(dk[j][i]);
                        if (GATE != kGateNone) qq = to_f(q[(long)t * D + c]);
                    }
                    dgm[j][i] = qq * dq[j][i] + kv[j][i] * (2.f * dkp[j][i] - dk[j][i]);
                }
            // dbeta = dbeta_R + rowsum(K+ Y)
#pragma unroll
            for (int j = 0; j < TO::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float s = row16_sum(dbA[j][i]);
                    if ((lane_id() & 15) == 0) red_r[(TO::n0(j) / 16) * C + TO::row(j, i)] = s;
                }
        }
        __syncthreads();
        for (int t = threadIdx.x; t < valid; t += kThreads) {
            float s = dbr[t];
            for (int b = 0; b < D / 16; ++b) s += red_r[b * C + t];
            p.dbeta[row0 + t] = s;
        }
        if (GATE == kGateNone) return;
        __syncthreads();
        // d gam: elementwise terms + the gam_C terms on the last valid row
        if (VEC) {
            if (TO::active()) {
#pragma unroll
                for (int j = 0; j < TO::PER; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) dgb[TO::row(j, i) * D + TO::col(j)] = dgm[j][i];
            }
            __syncthreads();
            for (int c = threadIdx.x; c < D; c += kThreads) {
                float last = fexp(gl[c]) * lastS[c];
                for (int b = 0; b < C / 16; ++b) last += red_c[b * D + c];
                float acc = 0.f;
                for (int t = valid - 1; t >= 0; --t) {
                    acc += dgb[t * D + c] + (t == valid - 1 ? last : 0.f);
                    p.dg[(row0 + t) * D + c] = acc;
                }
            }
        } else {
            if (TO::active()) {
#pragma unroll
                for (int j = 0; j < TO::PER; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float s = row16_sum(dgm[j][i]);
                        if ((lane_id() & 15) == 0) red_r[(TO::n0(j) / 16) * C + TO::row(j, i)] = s;
                    }
            }
            __syncthreads();
            if (wave_id() == 0) {
                // last-row total: sum_c (Gam_C lastS[c] + column partials of Kd dKd)
                float part = 0.f;
                for (int c = lane_id(); c < D; c += 64) {
                    float x = fexp(gl[0]) * lastS[c];
                    for (int b = 0; b < C / 16; ++b) x += red_c[b * D + c];
                    part += x;
                }
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
                const int t = lane_id();
                float x = 0.f;
                if (t < valid) {
                    for (int b = 0; b < D / 16; ++b) x += red_r[b * C + t];
                    if (t == valid - 1) x += part;
                }
                // reverse inclusive scan over t: dg_t = sum_{s >= t} x_s
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float y = __shfl_down(x, off);
                    if (t + off < 64) x += y;
                }
                if (t < valid) p.dg[row0 + t] = x;
            }
        }
    }
}

}  // namespace dn
