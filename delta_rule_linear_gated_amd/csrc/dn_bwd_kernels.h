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
// computed.  T and P (row-major) are transposed on their way into LDS.
template <typename TI, int GATE, int C, int DK, int BV>
__global__ __launch_bounds__(kThreads) void bwd_state_kernel(Params p) {
    constexpr int PAD = Pad<TI>::value;
    constexpr int LDK = DK + PAD;
    constexpr int LDC = C + PAD;
    constexpr int LDV = BV + PAD;
    constexpr int GW = GateLayout<GATE, DK>::GW;
    constexpr bool VEC = GATE == kGateVector;
    __shared__ float gam_s[VEC ? C * DK : C];
    __shared__ float rowf[2 * C];
    __shared__ __align__(16) float beta_s[C];
    __shared__ __align__(16) TI dSs[BV * LDK];   // dS1 operand     [v][c]
    __shared__ __align__(16) TI Kd[C * LDK];     // K Gam_C / Gam   [t][c]
    __shared__ __align__(16) TI PT[C * LDC];     // P^T             [t][s]
    __shared__ __align__(16) TI TT[C * LDC];     // T^T             [t][s]
    __shared__ __align__(16) TI dOT[BV * LDC];   // dO^T block      [v][t]
    __shared__ __align__(16) TI QgT[DK * LDC];   // (Q Gam)^T       [c][t]
    __shared__ __align__(16) TI KgT[DK * LDC];   // (K Gam)^T       [c][t]
    __shared__ __align__(16) TI dUT[BV * LDC];   // dU^T            [v][t]
    __shared__ __align__(16) TI bLT[BV * LDC];   // -(beta lambda)^T [v][t]
    // lambda / dv write-back tiles [C][LDV]: Kd and P^T are dead once dU is formed
    constexpr bool DB_IN_PT = C >= BV;
    __shared__ __align__(16) TI DbSep[DB_IN_PT ? 8 : C * LDV];
    TI* Lb = Kd;
    TI* Db = DB_IN_PT ? PT : DbSep;

    const int DVr = p.DVr;
    int bh, vblk;
    head_and_block(DVr / BV, p.BH, bh, vblk);
    const int v0 = vblk * BV;
    // dS held transposed, dS^T [c][v] tiles (4 consecutive keys of one row v per lane)
    using TS = Tiles<DK, BV>;
    f32x4 dS[TS::PER];
#pragma unroll
    for (int j = 0; j < TS::PER; ++j) {
        dS[j] = zero4();
        if (p.dhT && TS::active()) dS[j] = ld4<float>(p.dhT + ((long)bh * DVr + v0 + TS::col(j)) * DK + TS::row(j, 0));
    }

    RegB<TI, C, DK> rq, rk;
    RegB<TI, C, BV> rdo;
    RegB<TI, C, C> rP, rT;
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
        rP.load(static_cast<const TI*>(p.Pm) + cc, C, C);
        rT.load(static_cast<const TI*>(p.Tm) + cc, C, C);
    };
    prefetch(p.NT - 1);

    for (int n = p.NT - 1; n >= 0; --n) {
        const int t0 = n * C;
        const int valid = min(C, p.T - t0);
        // write back lambda and dv of the chunk done last iteration (a full chunk of
        // work after they were formed); the sync keeps commit() off their tiles
        if (n + 1 < p.NT) {
            const long rp = (long)bh * p.T + (n + 1) * C;
            lds_to_global<TI, C, BV>(static_cast<TI*>(p.lam) + ((long)bh * p.NT + n + 1) * C * DVr + v0, DVr, Lb,
                                     LDV, C);
            lds_to_global<TI, C, BV>(static_cast<TI*>(p.dv) + rp * DVr + v0, DVr, Db, LDV, min(C, p.T - (n + 1) * C));
            __syncthreads();
        }
        // (a) dS1 of this chunk: operand copy (written to the workspace from LDS below)
        if (TS::active()) {
#pragma unroll
            for (int j = 0; j < TS::PER; ++j) st4<TI>(dSs + TS::col(j) * LDK + TS::row(j, 0), dS[j]);
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
        rP.store_t(PT, LDC, Identity());
        rT.store_t(TT, LDC, Identity());
        __syncthreads();
        if (n > 0) prefetch(n - 1);
        lds_to_global<TI, BV, DK>(static_cast<TI*>(p.dS1) + (((long)bh * p.NT + n) * DVr + v0) * DK, DK, dSs, LDK,
                                  BV);

        using TX = Tiles<C, BV>;
        // (c) dU = P^T dO + Kd dS1^T  -> dU^T
        {
            f32x4 dU[TX::PER];
            zero_acc<C, BV>(dU);
            gemm_nt<TI, C, BV, C>(dU, PT, LDC, dOT, LDC);
            gemm_nt<TI, C, BV, DK>(dU, Kd, LDK, dSs, LDK);
            if (TX::active()) {
#pragma unroll
                for (int j = 0; j < TX::PER; ++j) st4<TI>(dUT + TX::col(j) * LDC + TX::row(j, 0), dU[j]);
            }
        }
        __syncthreads();
        // (d) lambda^T = dU^T T ; dv = beta lambda ; keep -(beta lambda)^T.  lambda^T
        //     tiles give a lane 4 consecutive v of one row t of lambda and dv
        {
            using TL = Tiles<BV, C>;
            f32x4 L[TL::PER];
            zero_acc<BV, C>(L);
            gemm_nt<TI, BV, C, C>(L, dUT, LDC, TT, LDC);
            if (TL::active()) {
                float bt[TL::PER];   // LDS reads first, then the writes
#pragma unroll
                for (int j = 0; j < TL::PER; ++j) bt[j] = beta_s[TL::col(j)];
#pragma unroll
                for (int j = 0; j < TL::PER; ++j) {
                    const int t = TL::col(j), c = TL::row(j, 0);
                    const f32x4 bl = bt[j] * L[j];
                    st4<TI>(Lb + t * LDV + c, L[j]);
                    st4<TI>(Db + t * LDV + c, bl);
#pragma unroll
                    for (int i = 0; i < 4; ++i) bLT[(c + i) * LDC + t] = from_f<TI>(-bl[i]);
                }
            }
        }
        __syncthreads();
        // (e) dS0^T = Diag(Gam_C) dS1^T + (Q Gam)^T dO - (K Gam)^T (beta lambda)
        if (GATE != kGateNone && TS::active()) {
#pragma unroll
            for (int j = 0; j < TS::PER; ++j) {
#pragma unroll
                for (int i = 0; i < 4; ++i) dS[j][i] *= gf.GC(TS::row(j, i));
            }
        }
        gemm_nt<TI, DK, BV, C>(dS, QgT, LDC, dOT, LDC);
        gemm_nt<TI, DK, BV, C>(dS, KgT, LDC, bLT, LDC);
        __syncthreads();
    }
    if (p.NT > 0) {   // lambda and dv of chunk 0
        lds_to_global<TI, C, BV>(static_cast<TI*>(p.lam) + (long)bh * p.NT * C * DVr + v0, DVr, Lb, LDV, C);
        lds_to_global<TI, C, BV>(static_cast<TI*>(p.dv) + (long)bh * p.T * DVr + v0, DVr, Db, LDV, min(C, p.T));
    }
    if (p.dh0 && TS::active()) {
#pragma unroll
        for (int j = 0; j < TS::PER; ++j)
            st4<float>(p.dh0 + ((long)bh * DVr + v0 + TS::col(j)) * DK + TS::row(j, 0), dS[j]);
    }
}

// ---------------------------------------------------------------------------
// bwd_chunk_kernel: grid (NT, BH); every chunk finished independently.
// D = d_k = d_v.  The d_v dimension is streamed in blocks of VB columns: the
// block's S0 rows, dS1 rows, lambda, dO and V columns are loaded into registers
// one block ahead and committed to LDS while the previous block computes
//     X_b = (K Gam) S0_b^T,  R_b = beta (V_b - X_b),  U_b = T R_b
//     dQg += dO_b S0_b,  dKg += lambda_b S0_b,  dKd += U_b dS1_b
//     dA  += lambda_b U_b^T,  dP += dO_b U_b^T
// after which the key-gradient products (phase C) finish dq, dk, dbeta, dg.
template <typename TI, int GATE, int C, int D>
struct BwdChunkSmem {
    static constexpr int PAD = Pad<TI>::value;
    static constexpr int VB = D >= 32 ? 32 : D;   // d_v block
    static constexpr int NVB = D / VB;
    static constexpr int LD = D + PAD;            // rows of D elements
    static constexpr int LC = C + PAD;            // rows of C elements
    static constexpr int LVB = VB + PAD;          // rows of VB elements
    static constexpr int GW = GateLayout<GATE, D>::GW;
    static constexpr size_t E = sizeof(TI);
    static constexpr size_t al(size_t x) { return (x + 255) & ~size_t(255); }
    // persistent through the d_v loop
    static constexpr size_t KG = 0;                                  // K (or K Gam)   [C][LD]
    static constexpr size_t TL = KG + al(C * LD * E);                // T              [C][LC]
    static constexpr size_t LOOP = TL + al(C * LC * E);
    // d_v loop, one block
    static constexpr size_t S0B = LOOP;                              // S0 rows        [VB][LD]
    static constexpr size_t S0BT = S0B + al(VB * LD * E);            // S0 block^T     [D][LVB]
    static constexpr size_t DS1T = S0BT + al(D * LVB * E);           // dS1 block^T    [D][LVB]
    static constexpr size_t LAMB = DS1T + al(D * LVB * E);           // lambda block   [C][LVB]
    static constexpr size_t DOB = LAMB + al(C * LVB * E);            // dO block       [C][LVB]
    static constexpr size_t VBL = DOB + al(C * LVB * E);             // V block        [C][LVB]
    static constexpr size_t RTB = VBL + al(C * LVB * E);             // R block^T      [VB][LC]
    static constexpr size_t UB = RTB + al(VB * LC * E);              // U block        [C][LVB]
    static constexpr size_t LOOP_END = UB + al(C * LVB * E);
    // phase C (aliases everything above once the loop is done)
    static constexpr size_t DA = 0;                                  // dA~            [C][LC]
    static constexpr size_t DAT = DA + al(C * LC * E);               // beta dA~^T     [C][LC]
    static constexpr size_t DP = DAT + al(C * LC * E);               // dP~            [C][LC]
    static constexpr size_t DPT = DP + al(C * LC * E);               // dP~^T          [C][LC]
    static constexpr size_t KRT = DPT + al(C * LC * E);              // (K or K e^{c-gam})^T [D][LC]
    static constexpr size_t QLT = KRT + al(D * LC * E);              // (Q or Q e^{gam-c})^T [D][LC]
    static constexpr size_t KLT = QLT + al(D * LC * E);              // (K e^{gam-c})^T (vector) [D][LC]
    static constexpr size_t C_END = GATE == kGateVector ? KLT + al(D * LC * E) : KLT;
    static constexpr size_t BIG_END = LOOP_END > C_END ? LOOP_END : C_END;
    // small fp32 arrays
    static constexpr size_t GAM = al(BIG_END);                                    // gam [C][D] or [C]
    static constexpr size_t ROWF = GAM + al(GATE == kGateVector ? C * D * 4 : C * 4);  // [2][C] (scalar)
    static constexpr size_t BETA = ROWF + al(2 * C * 4);                          // [C]
    static constexpr size_t RED_R = BETA + al(C * 4);                             // [D/16][C] row partials
    static constexpr size_t RED_C = RED_R + al((D / 16) * C * 4);                 // [C/16][D] column partials
    static constexpr size_t LASTS = RED_C + al((C / 16) * D * 4);                 // [D]
    static constexpr size_t DBR = LASTS + al(D * 4);                              // [C]
    static constexpr size_t TOTAL = DBR + al(C * 4);
    // dq / dk write-back tiles [C][LD] each at offset 0; d gam of the vector gate
    // [C][D] fp32 after them, written once every phase-C tile is dead
    static constexpr size_t DGB = al(2 * C * LD * E);
    static_assert(GATE != kGateVector || DGB + C * D * 4 <= BIG_END, "d gam buffer");
    // per-thread partials of sum_v S0 dS1 [row blocks of the S0 register tile][D] fp32,
    // at offset 0 right after the d_v loop
    using RS = RegB<TI, VB, D>;
    static_assert(RS::BR * D * 4 <= BIG_END, "S0 dS1 partials");
    static_assert(2 * C * LD * E <= BIG_END, "write-back tiles");
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

template <typename TI, int GATE, int C, int D>
__global__ __launch_bounds__(kThreads) void bwd_chunk_kernel(Params p) {
    using L = BwdChunkSmem<TI, GATE, C, D>;
    constexpr int LD = L::LD, LC = L::LC, LVB = L::LVB, GW = L::GW;
    constexpr int VB = L::VB, NVB = L::NVB;
    constexpr bool VEC = GATE == kGateVector;
    constexpr bool SCA = GATE == kGateScalar;
    __shared__ __align__(16) char smem[L::TOTAL];
    TI* KG = reinterpret_cast<TI*>(smem + L::KG);
    TI* TLs = reinterpret_cast<TI*>(smem + L::TL);
    TI* S0B = reinterpret_cast<TI*>(smem + L::S0B);
    TI* S0BT = reinterpret_cast<TI*>(smem + L::S0BT);
    TI* DS1T = reinterpret_cast<TI*>(smem + L::DS1T);
    TI* LAMB = reinterpret_cast<TI*>(smem + L::LAMB);
    TI* DOB = reinterpret_cast<TI*>(smem + L::DOB);
    TI* VBL = reinterpret_cast<TI*>(smem + L::VBL);
    TI* RTB = reinterpret_cast<TI*>(smem + L::RTB);
    TI* UB = reinterpret_cast<TI*>(smem + L::UB);
    float* gam_s = reinterpret_cast<float*>(smem + L::GAM);
    float* rowf = reinterpret_cast<float*>(smem + L::ROWF);
    float* beta_s = reinterpret_cast<float*>(smem + L::BETA);
    float* red_r = reinterpret_cast<float*>(smem + L::RED_R);
    float* red_c = reinterpret_cast<float*>(smem + L::RED_C);
    float* lastS = reinterpret_cast<float*>(smem + L::LASTS);
    float* dbr = reinterpret_cast<float*>(smem + L::DBR);
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

    using TO = Tiles<C, D>;    // C x D outputs: dq, dk
    using TCC = Tiles<C, C>;   // dA, dP
    using TX = Tiles<C, VB>;   // X_b, U_b

    // ---------------- prologue: gate, K, T, the first d_v block, k at this lane's elements
    GateRegs<GATE, C, D> rg;
    rg.load(p.gam + row0 * GW, p.beta + row0, valid);
    RegN<TI, C, D> rK;
    rK.load(k, D, valid);
    RegN<TI, C, C> rT;
    rT.load(static_cast<const TI*>(p.Tm) + chunk * C * C, C, C);
    RegB<TI, VB, D> rS0, rdS1;
    RegN<TI, C, VB> rlam, rdo, rv;
    auto load_block = [&](int b) {
        const int v0 = b * VB;
        rS0.load(S0g + (long)v0 * D, D, VB);
        rdS1.load(dS1g + (long)v0 * D, D, VB);
        rlam.load(lamg + v0, D, C);
        rdo.load(dO + v0, D, valid);
        rv.load(v + v0, D, valid);
    };
    load_block(0);
    // sum_v S0[v][c] dS1[v][c] over this thread's rows of every block
    float ls[L::RS::PER][L::RS::VW] = {};
    rg.commit(rowf, gam_s, beta_s);
    __syncthreads();
    const GateLds<GATE, C, D> gf{rowf, gam_s, valid - 1};
    if (VEC)
        rK.store(KG, LD, [&](int r, int c, float x) { return x * gf.G(r, c); });
    else
        rK.store(KG, LD);   // scalar: Gam_t is applied to X's rows
    rT.store(TLs, LC);
    auto commit_block = [&]() {
        rS0.dot_rows(rdS1, ls);
        rS0.store_n(S0B, LD, Identity());
        rS0.store_t(S0BT, LVB, Identity());
        rdS1.store_t(DS1T, LVB, Identity());
        rlam.store(LAMB, LVB);
        rdo.store(DOB, LVB);
        rv.store(VBL, LVB);
    };
    commit_block();
    __syncthreads();

    // ---------------- d_v loop
    f32x4 dq[TO::PER], dkp[TO::PER], dkm[TO::PER], dA[TCC::PER], dP[TCC::PER];
    zero_acc<C, D>(dq);
    zero_acc<C, D>(dkp);
    zero_acc<C, D>(dkm);
    zero_acc<C, C>(dA);
    zero_acc<C, C>(dP);
    float dbr_part[TX::PER][4] = {};
#pragma unroll 1
    for (int b = 0; b < NVB; ++b) {
        if (b + 1 < NVB) load_block(b + 1);
        // X_b = (K Gam) S0_b^T and the two S0 contractions
        f32x4 X[TX::PER];
        zero_acc<C, VB>(X);
        gemm_nt<TI, C, VB, D>(X, KG, LD, S0B, LD);
        gemm_nt<TI, C, D, VB>(dq, DOB, LVB, S0BT, LVB);
        gemm_nt<TI, C, D, VB>(dkp, LAMB, LVB, S0BT, LVB);
        if (TX::active()) {
            float rb[TX::PER][4];   // LDS reads first, then the writes
#pragma unroll
            for (int j = 0; j < TX::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = TX::row(j, i), c = TX::col(j);
                    const float xr = to_f(VBL[t * LVB + c]) - (SCA ? rowf[t] : 1.f) * X[j][i];
                    dbr_part[j][i] += to_f(LAMB[t * LVB + c]) * xr;
                    rb[j][i] = beta_s[t] * xr;
                }
#pragma unroll
            for (int j = 0; j < TX::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) RTB[TX::col(j) * LC + TX::row(j, i)] = from_f<TI>(rb[j][i]);
        }
        __syncthreads();
        // U_b = T R_b
        {
            f32x4 U[TX::PER];
            zero_acc<C, VB>(U);
            gemm_nt<TI, C, VB, C>(U, TLs, LC, RTB, LC);
            if (TX::active()) {
#pragma unroll
                for (int j = 0; j < TX::PER; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) UB[TX::row(j, i) * LVB + TX::col(j)] = from_f<TI>(U[j][i]);
            }
        }
        __syncthreads();
        gemm_nt<TI, C, D, VB>(dkm, UB, LVB, DS1T, LVB);
        gemm_nt<TI, C, C, VB>(dA, LAMB, LVB, UB, LVB);
        gemm_nt<TI, C, C, VB>(dP, DOB, LVB, UB, LVB);
        __syncthreads();
        if (b + 1 < NVB) {
            commit_block();
            __syncthreads();
        }
    }

    // q and k for the key-gradient products (loads in flight during the epilogues below)
    RegB<TI, C, D> rq, rk;
    rq.load(q, D, valid);
    rk.load(k, D, valid);

    // ---------------- dbeta_R, sum_v S0 dS1, and the d_v-contraction epilogues
    float* lsred = reinterpret_cast<float*>(smem);   // d_v-loop tiles are dead
    if (TX::active()) {
#pragma unroll
        for (int im = 0; im < TX::RM; ++im)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float s = 0.f;
#pragma unroll
                for (int in = 0; in < TX::RN; ++in) s += dbr_part[im * TX::RN + in][i];
                s = row16_sum(s);
                if ((lane_id() & 15) == 0) red_r[TX::cg() * C + TX::row(im * TX::RN, i)] = s;
            }
    }
#pragma unroll
    for (int i = 0; i < L::RS::PER; ++i) {
        if (L::RS::owns(i)) {
#pragma unroll
            for (int k = 0; k < L::RS::VW; ++k) lsred[L::RS::rowblk(i) * D + L::RS::col0(i) + k] = ls[i][k];
        }
    }
    __syncthreads();   // row and column partials complete
    for (int t = threadIdx.x; t < C; t += kThreads) {
        float s = 0.f;
        for (int b = 0; b < TX::WN; ++b) s += red_r[b * C + t];
        dbr[t] = s;
    }
    for (int c = threadIdx.x; c < D; c += kThreads) {
        float s = 0.f;
        for (int h = 0; h < L::RS::BR; ++h) s += lsred[h * D + c];
        lastS[c] = s;
    }
    __syncthreads();   // red_r and the partials are reused below
    // dq = Gam dQg ; dk+ = -beta Gam dKg ; dk- = Gd dKd
    if (TO::active()) {
#pragma unroll
        for (int j = 0; j < TO::PER; ++j) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = TO::row(j, i), c = TO::col(j);
                const float G = gf.G(t, c);
                dq[j][i] *= G;
                dkp[j][i] *= -beta_s[t] * G;
                dkm[j][i] *= gf.Gd(t, c);
            }
        }
    }

    // ---------------- phase B: dA~ and dP~ into LDS
    {
        TI* DAs = reinterpret_cast<TI*>(smem + L::DA);
        TI* DATs = reinterpret_cast<TI*>(smem + L::DAT);
        TI* DPs = reinterpret_cast<TI*>(smem + L::DP);
        TI* DPTs = reinterpret_cast<TI*>(smem + L::DPT);
        if (TCC::active()) {
            float bt[TCC::PER][4];   // LDS reads first, then the writes
#pragma unroll
            for (int j = 0; j < TCC::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = TCC::row(j, i), s2 = TCC::col(j);
                    const float e = (SCA && s2 <= t) ? fexp(gam_s[t] - gam_s[s2]) : 1.f;
                    dP[j][i] = s2 <= t ? dP[j][i] * e : 0.f;
                    dA[j][i] = s2 < t ? -dA[j][i] * e : 0.f;   // dA = -lambda U^T
                    bt[j][i] = beta_s[t];
                }
#pragma unroll
            for (int j = 0; j < TCC::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = TCC::row(j, i), s2 = TCC::col(j);
                    DAs[t * LC + s2] = from_f<TI>(dA[j][i]);
                    DATs[s2 * LC + t] = from_f<TI>(bt[j][i] * dA[j][i]);
                    DPs[t * LC + s2] = from_f<TI>(dP[j][i]);
                    DPTs[s2 * LC + t] = from_f<TI>(dP[j][i]);
                }
        }
    }

    // ---------------- phase C: key-gradient products
    {
        const TI* DAs = reinterpret_cast<const TI*>(smem + L::DA);
        const TI* DATs = reinterpret_cast<const TI*>(smem + L::DAT);
        const TI* DPs = reinterpret_cast<const TI*>(smem + L::DP);
        const TI* DPTs = reinterpret_cast<const TI*>(smem + L::DPT);
        TI* KrT = reinterpret_cast<TI*>(smem + L::KRT);
        TI* QlT = reinterpret_cast<TI*>(smem + L::QLT);
        TI* KlT = VEC ? reinterpret_cast<TI*>(smem + L::KLT) : KrT;
        const float* gl = gam_s + (valid - 1) * GW;
        // fp = e^{gam - centre} (vector gate; 1 otherwise), centre = gam_C / 2
        auto fpl = [&](int t, int c) -> float { return VEC ? fexp(gam_s[t * D + c] - 0.5f * gl[c]) : 1.f; };
        if (VEC) {
            rk.store_t(KrT, LC, [&](int r, int c, float x) { return x / fpl(r, c); });
            rk.store_t(KlT, LC, [&](int r, int c, float x) { return x * fpl(r, c); });
            rq.store_t(QlT, LC, [&](int r, int c, float x) { return x * fpl(r, c); });
        } else {
            rk.store_t(KrT, LC, Identity());
            rq.store_t(QlT, LC, Identity());
        }
        __syncthreads();
        // k and q at this lane's elements, read back from the staged tiles; the
        // gam_C column sums of Kd dKd (dk- holds only the Kd path so far)
        float kv[TO::PER][4], qv[TO::PER][4];
        if (TO::active()) {
#pragma unroll
            for (int j = 0; j < TO::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = TO::row(j, i), c = TO::col(j);
                    const float fp = fpl(t, c);
                    kv[j][i] = to_f(KrT[c * LC + t]) * fp;
                    qv[j][i] = to_f(QlT[c * LC + t]) / fp;
                }
#pragma unroll
            for (int in = 0; in < TO::RN; ++in) {
                float colp = 0.f;
#pragma unroll
                for (int im = 0; im < TO::RM; ++im)
#pragma unroll
                    for (int i = 0; i < 4; ++i) colp += kv[im * TO::RN + in][i] * dkm[im * TO::RN + in][i];
                colp += __shfl_xor(colp, 16);
                colp += __shfl_xor(colp, 32);
                if (lane_id() < 16) red_c[TO::rg() * D + TO::col(in)] = colp;
            }
        }
        float dbA[TO::PER][4];
        f32x4 tmp[TO::PER];
        // Y = dA~ Kr :  dK+ = beta Y, dbeta_A = sum_c K+ Y
        zero_acc<C, D>(tmp);
        gemm_nt<TI, C, D, C>(tmp, DAs, LC, KrT, LC);
        if (TO::active()) {
#pragma unroll
            for (int j = 0; j < TO::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = TO::row(j, i);
                    const float fp = fpl(t, TO::col(j));
                    const float y = tmp[j][i];
                    dbA[j][i] = kv[j][i] * fp * y;
                    dkp[j][i] += beta_s[t] * y * fp;
                }
        }
        // Z = (beta dA~)^T Kl and W = dP~^T Ql : both reach k through e^{-gam}
        zero_acc<C, D>(tmp);
        gemm_nt<TI, C, D, C>(tmp, DATs, LC, KlT, LC);
        gemm_nt<TI, C, D, C>(tmp, DPTs, LC, QlT, LC);
        if (TO::active()) {
#pragma unroll
            for (int j = 0; j < TO::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) dkm[j][i] += tmp[j][i] / fpl(TO::row(j, i), TO::col(j));
        }
        // dQ+ = dP~ Kr
        zero_acc<C, D>(tmp);
        gemm_nt<TI, C, D, C>(tmp, DPs, LC, KrT, LC);
        if (TO::active()) {
#pragma unroll
            for (int j = 0; j < TO::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) dq[j][i] += tmp[j][i] * fpl(TO::row(j, i), TO::col(j));
        }

        // -------- finish: dq, dk = dk+ + dk-, dbeta, d gam = q.dq + k.(dk+ - dk-)
        float dgm[TO::PER][4];
        __syncthreads();   // phase-C tiles dead: dq / dk go through LDS for coalesced stores
        TI* dqs = reinterpret_cast<TI*>(smem + L::DA);
        TI* dks = dqs + C * LD;
        if (TO::active()) {
#pragma unroll
            for (int j = 0; j < TO::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = TO::row(j, i), c = TO::col(j);
                    dqs[t * LD + c] = from_f<TI>(dq[j][i]);
                    dks[t * LD + c] = from_f<TI>(dkp[j][i] + dkm[j][i]);
                    dgm[j][i] = qv[j][i] * dq[j][i] + kv[j][i] * (dkp[j][i] - dkm[j][i]);
                }
            // dbeta = dbeta_R + rowsum(K+ Y)
#pragma unroll
            for (int im = 0; im < TO::RM; ++im)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float s2 = 0.f;
#pragma unroll
                    for (int in = 0; in < TO::RN; ++in) s2 += dbA[im * TO::RN + in][i];
                    s2 = row16_sum(s2);
                    if ((lane_id() & 15) == 0) red_r[TO::cg() * C + TO::row(im * TO::RN, i)] = s2;
                }
        }
        __syncthreads();
        lds_to_global<TI, C, D>(static_cast<TI*>(p.dq) + row0 * D, D, dqs, LD, valid);
        lds_to_global<TI, C, D>(static_cast<TI*>(p.dk) + row0 * D, D, dks, LD, valid);
        for (int t = threadIdx.x; t < valid; t += kThreads) {
            float s2 = dbr[t];
            for (int b = 0; b < TO::WN; ++b) s2 += red_r[b * C + t];
            p.dbeta[row0 + t] = s2;
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
                for (int b = 0; b < TO::WM; ++b) last += red_c[b * D + c];
                float acc = 0.f;
                for (int t = valid - 1; t >= 0; --t) {
                    acc += dgb[t * D + c] + (t == valid - 1 ? last : 0.f);
                    p.dg[(row0 + t) * D + c] = acc;
                }
            }
        } else {
            if (TO::active()) {
#pragma unroll
                for (int im = 0; im < TO::RM; ++im)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float s2 = 0.f;
#pragma unroll
                        for (int in = 0; in < TO::RN; ++in) s2 += dgm[im * TO::RN + in][i];
                        s2 = row16_sum(s2);
                        if ((lane_id() & 15) == 0) red_r[TO::cg() * C + TO::row(im * TO::RN, i)] = s2;
                    }
            }
            __syncthreads();
            if (wave_id() == 0) {
                // last-row total: sum_c (Gam_C lastS[c] + column partials of Kd dKd)
                float part = 0.f;
                for (int c = lane_id(); c < D; c += 64) {
                    float x = gf.GC(c) * lastS[c];
                    for (int b = 0; b < TO::WM; ++b) x += red_c[b * D + c];
                    part += x;
                }
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
                const int t = lane_id();
                float x = 0.f;
                if (t < valid) {
                    for (int b = 0; b < TO::WN; ++b) x += red_r[b * C + t];
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
