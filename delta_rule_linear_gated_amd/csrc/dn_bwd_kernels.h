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
//   * for the vector gate the same products run block by block over 16-step
//     blocks of the contraction, on keys and queries scaled relative to the gate
//     at a block boundary and with each block's partial rescaled (the centred
//     contraction, centred per 16-row block: vec_key_products), and the
//     per-channel gate gradient is elementwise;
//   * dg is the reverse cumulative sum of d gam inside the chunk.
#pragma once

#include "dn_device.h"
#include "dn_fwd_kernels.h"
#include "dn_internal.h"

namespace dn {

// ---------------------------------------------------------------------------
// bwd_state_kernel: grid (rows / BV) * nseg * BH, the chunks of one segment
// walked from last to first; the global tiles of chunk n - 1 are loaded into
// registers while chunk n is computed.  Every tile is kept in its natural
// layout (T and P as saved, row major); operands contracted over their leading
// index are read with the transposing LDS load.
//   SUMMARY: segment summary of the chunk-parallel scan, the mirror image of the
//            forward's: dS through the segment from zero (the last segment from
//            dhT), plus DK rows that start as the identity and see dO = 0 and end
//            as the transpose of the segment's transition matrix
//            (dS_start = dS_end P_s^T + dS_start|zero end); end states to
//            p.seg_end, nothing else written.
// Otherwise, with segments, a segment starts from the dS the combine left in
// p.seg_start (the last from dhT) and writes lambda, dv and dS1 of its chunks.
// LDS arrays of the backward state pass (see FwdStateArrays).
template <typename TI, int GATE, int C, int DK, int BV> struct BwdStateArrays {
    static constexpr int PAD = Pad<TI>::value, LDK = DK + PAD, LDC = C + PAD, LDV = BV + PAD;
    static constexpr bool VEC = GATE == kGateVector, SCA = GATE == kGateScalar;
    float gam_s[C];
    __align__(16) float egc[VEC ? DK : 4];   // e^{gam_C} per channel (vector gate)
    __align__(16) float rowf[2 * C];
    __align__(16) float beta_s[C];
    __align__(16) TI dSs[BV * LDK];   // dS1 operand     [v][c]
    __align__(16) TI Kd[C * LDK];     // K (vector gate: K Gam_C / Gam)  [t][c]
    __align__(16) TI Kn[VEC ? C * LDK : 8];   // -K Gam (vector gate)    [t][c]
    __align__(16) TI Qg[C * LDK];     // Q (vector gate: Q Gam)          [t][c]
    __align__(16) TI Pl[C * LDC];     // P               [s][t]
    __align__(16) TI Tl[C * LDC];     // T               [s][t]
    __align__(16) TI dOb[C * LDV];    // dO block        [t][v]
    __align__(16) TI dOg[SCA ? C * LDV : 8];  // dO Gam (scalar gate)    [t][v]
    __align__(16) TI dUT[BV * LDC];   // dU^T            [v][t]
    // lambda and dv = beta lambda [t][v], written back a chunk later; without a
    // vector gate the dS update takes -beta lambda (Gam) from Dn, else dv itself
    __align__(16) TI Lb[C * LDV];
    __align__(16) TI Db[C * LDV];
    __align__(16) TI Dn[VEC ? 8 : C * LDV];
};

// The pass for workgroup `wg` of its grid (LDS arrays as restrict pointers, as
// for fwd_state_body).
template <typename TI, int GATE, int C, int DK, int BV, bool SUMMARY>
__device__ __forceinline__ void bwd_state_body(const Params& p, int wg, float* __restrict__ gam_s,
                                               float* __restrict__ egc, float* __restrict__ rowf,
                                               float* __restrict__ beta_s, TI* __restrict__ dSs,
                                               TI* __restrict__ Kd, TI* __restrict__ Kn, TI* __restrict__ Qg,
                                               TI* __restrict__ Pl, TI* __restrict__ Tl, TI* __restrict__ dOb,
                                               TI* __restrict__ dOg, TI* __restrict__ dUT, TI* __restrict__ Lb,
                                               TI* __restrict__ Db, TI* __restrict__ Dn) {
    constexpr int PAD = Pad<TI>::value;
    constexpr int LDK = DK + PAD;
    constexpr int LDC = C + PAD;
    constexpr int LDV = BV + PAD;
    constexpr int GW = GateLayout<GATE, DK>::GW;
    constexpr bool VEC = GATE == kGateVector;
    constexpr bool SCA = GATE == kGateScalar;
    // A scalar gate is a row scaling: Q and K stay unscaled (K staged once) and the
    // decays go to the C x BV operands -- e^{gam_C - gam_t} to the K dS1^T part of
    // dU, e^{gam_t} to copies of dO and of -beta lambda for the dS update.  The
    // vector gate scales Q and K per element, from gate values held in registers
    // in the layout of the K / Q register tiles (VecGate).

    const int DVr = p.DVr;
    const int rows = DVr + (SUMMARY ? DK : 0);
    const int nblk = rows / BV;
    int bh, sb;
    head_and_block(nblk * p.nseg, p.BH, bh, sb, wg);
    const int seg = sb / nblk, vblk = sb - seg * nblk;
    const int v0 = vblk * BV;
    const bool trans = SUMMARY && v0 >= DVr;   // rows of the transposed transition
    if (trans && (seg == 0 || seg == p.nseg - 1)) return;
    const int n0 = seg * p.seg_len, n1 = min(p.NT, n0 + p.seg_len);
    const bool last = seg == p.nseg - 1;
    // dS held transposed, dS^T [c][v] tiles (4 consecutive keys of one row v per lane)
    using TS = Tiles<DK, BV>;
    f32x4 dS[TS::PER];
    const float* init = last ? (trans ? nullptr : (p.dhT ? p.dhT + (long)bh * DVr * DK : nullptr))
                             : (SUMMARY ? nullptr : p.seg_start + ((long)bh * p.nseg + seg) * DVr * DK);
#pragma unroll
    for (int j = 0; j < TS::PER; ++j) {
        dS[j] = zero4();
        if (init && TS::active()) dS[j] = ld4<float>(init + (long)(v0 + TS::col(j)) * DK + TS::row(j, 0));
        if (trans && TS::active()) {
#pragma unroll
            for (int i = 0; i < 4; ++i) dS[j][i] = TS::row(j, i) == v0 - DVr + TS::col(j) ? 1.f : 0.f;
        }
    }
    const int vcol = trans ? 0 : v0;   // (transition rows load a valid dO block and zero it)

    RegN<TI, C, DK> rq, rk;
    using RDO = RegN<TI, C, BV>;
    RDO rdo;
    RegN<TI, C, C> rP, rT;
    GateRegs<GATE, C, DK, false> rg;
    VecGate<TI, C, DK> vg;   // vector gate
    // scalar gate: gam of the rows of this thread's dO vectors (dO e^{gam} is formed
    // from registers, so the commit needs no barrier between the gate and the tiles)
    float gdo[SCA ? RDO::PER : 1];
    // Vector gate: the chunk's gated tiles K e^{gam_C - gam}, -K e^{gam}, Q e^{gam}
    // and e^{gam_C}, formed in registers at the end of the previous iteration from
    // K, Q and the gate loaded one chunk before that (as in the forward state pass).
    using VG = VecGate<TI, C, DK>;
    RegN<TI, C, VEC ? DK : 8> pkd, pkn, pqg;
    float pec[VEC ? VG::VW : 1];
    auto prefetch_kq = [&](int n) {   // vector gate: K, Q and the gate of chunk n
        if constexpr (VEC) {
            const int t0 = n * C;
            const int valid = min(C, p.T - t0);
            const long row0 = (long)bh * p.T + t0;
            vg.load(p.gam + row0 * GW, valid);
            __builtin_amdgcn_sched_barrier(0);
            rq.load(static_cast<const TI*>(p.q) + row0 * DK, DK, valid);
            rk.load(static_cast<const TI*>(p.k) + row0 * DK, DK, valid);
        }
    };
    auto form = [&]() {   // vector gate: the tiles of the chunk in rq / rk / vg
        if constexpr (VEC) {
            rk.form3i(rq, pkd, pkn, pqg, [&](int i, int e, float k, float q, float* y) {
                const float ge = vg.g[i][e];
                const float f = fexp(ge);
                y[0] = k * fexp(vg.gc[e] - ge);
                y[1] = -k * f;
                y[2] = q * f;
            });
#pragma unroll
            for (int e = 0; e < VG::VW; ++e) pec[e] = fexp(vg.gc[e]);
        }
    };
    auto prefetch = [&](int n) {   // the rest of chunk n (everything without a vector gate)
        const int t0 = n * C;
        const int valid = min(C, p.T - t0);
        const long row0 = (long)bh * p.T + t0;
        const long cc = ((long)bh * p.NT + n) * C * C;
        rg.load(p.gam + row0 * GW, p.beta + row0, valid);
        if constexpr (SCA) {
#pragma unroll
            for (int i = 0; i < RDO::PER; ++i) gdo[i] = p.gam[row0 + min(RDO::idx_of(i) / RDO::VPR, valid - 1)];
        }
        __builtin_amdgcn_sched_barrier(0);   // gate first, then the tiles, in order (see RegN)
        if constexpr (!VEC) {
            rq.load(static_cast<const TI*>(p.q) + row0 * DK, DK, valid);
            rk.load(static_cast<const TI*>(p.k) + row0 * DK, DK, valid);
        }
        rdo.load(static_cast<const TI*>(p.dout) + row0 * DVr + vcol, DVr, valid);
        if (trans) rdo.valid_ = 0;   // stores as zero
        rP.load(static_cast<const TI*>(p.Pm) + cc, C, C);
        rT.load(static_cast<const TI*>(p.Tm) + cc, C, C);
    };
    prefetch_kq(n1 - 1);
    prefetch(n1 - 1);
    form();
    prefetch_kq(n1 - 2 >= n0 ? n1 - 2 : n0);

    using TX = Tiles<C, BV>;    // dU  [t][v]
    using TL = Tiles<BV, C>;    // lambda^T [v][t]
    for (int n = n1 - 1; n >= n0; --n) {
        const int t0 = n * C;
        const int valid = min(C, p.T - t0);
        // (a) dS1 of this chunk: operand copy (written to the workspace from LDS below)
        if (TS::active()) {
#pragma unroll
            for (int j = 0; j < TS::PER; ++j) st4<TI>(dSs + TS::col(j) * LDK + TS::row(j, 0), dS[j]);
        }
        // (b) commit this chunk's tiles (the barrier ending the previous chunk ordered
        // these writes after its reads; nothing below reads the gate just committed
        // before the next barrier)
        rg.commit(rowf, gam_s, beta_s);
        const GateLds<GATE, C, DK> gf{rowf, gam_s, valid - 1};
        if constexpr (VEC) {   // the tiles formed last iteration (K e^{gam_C - gam}, -K e^{gam}, Q e^{gam})
            if ((int)threadIdx.x < VG::VPR) {
#pragma unroll
                for (int e = 0; e < VG::VW; ++e) egc[VG::col0() + e] = pec[e];
            }
            pkd.store(Kd, LDK);
            pkn.store(Kn, LDK);
            pqg.store(Qg, LDK);
        } else {
            rk.store(Kd, LDK);
            rq.store(Qg, LDK);
        }
        rdo.store(dOb, LDV);
        if constexpr (SCA) {
            float eg[RDO::PER];
#pragma unroll
            for (int i = 0; i < RDO::PER; ++i) eg[i] = fexp(gdo[i]);
            rdo.store_scaled(dOg, LDV, eg);
        }
        rP.store(Pl, LDC);
        rT.store(Tl, LDC);
        // lambda and dv of the chunk done last iteration (in Lb / Db until (d) below)
        if (!SUMMARY && n + 1 < n1) {
            const long rp = (long)bh * p.T + (n + 1) * C;
            lds_to_global<TI, C, BV>(static_cast<TI*>(p.lam) + ((long)bh * p.NT + n + 1) * C * DVr + v0, DVr, Lb,
                                     LDV, C);
            lds_to_global<TI, C, BV>(static_cast<TI*>(p.dv) + rp * DVr + v0, DVr, Db, LDV, min(C, p.T - (n + 1) * C));
        }
        __syncthreads();
        if (!SUMMARY && !VEC)
            lds_to_global<TI, BV, DK>(static_cast<TI*>(p.dS1) + (((long)bh * p.NT + n) * DVr + v0) * DK, DK, dSs,
                                      LDK, BV);
        // the next chunk's loads after the dS1 save and unconditional (see the
        // forward state kernel); with the per-channel gate only once the first
        // product below is issued (its reverse pass 2 % faster, the scalar gate's
        // 3.5 % slower)
        if (!VEC) prefetch(n > n0 ? n - 1 : n0);

        // (c) dU = P^T dO + Kd dS1^T  -> dU^T   (P and dO read as [k][m] / [k][n])
        {
            f32x4 dU[TX::PER];
            zero_acc<C, BV>(dU);
            gemm<TI, C, BV, DK, false, false>(dU, Kd, LDK, dSs, LDK);
            if (VEC) prefetch(n > n0 ? n - 1 : n0);
            if (SCA && TX::active()) {   // rows t of K dS1^T times e^{gam_C - gam_t}
#pragma unroll
                for (int j = 0; j < TX::PER; ++j) dU[j] *= ld4<float>(rowf + C + TX::row(j, 0));
            }
            gemm<TI, C, BV, C, true, true>(dU, Pl, LDC, dOb, LDV);
            if (TX::active()) {
#pragma unroll
                for (int j = 0; j < TX::PER; ++j) st4<TI>(dUT + TX::col(j) * LDC + TX::row(j, 0), dU[j]);
            }
        }
        // the part of the dS update that needs no lambda, here rather than in (e):
        // dS^T <- Diag(Gam_C) dS^T + (Q Gam)^T dO (the dS1 operand is the copy in
        // LDS; overlapping this with dU shortens the chain by 3 %)
        if (GATE != kGateNone && TS::active()) {
#pragma unroll
            for (int j = 0; j < TS::PER; ++j) {
#pragma unroll
                for (int i = 0; i < 4; ++i) dS[j][i] *= VEC ? egc[TS::row(j, i)] : gf.GC(TS::row(j, i));
            }
        }
        gemm<TI, DK, BV, C, true, true>(dS, Qg, LDK, SCA ? dOg : dOb, LDV);
        __syncthreads();
        // the per-channel gate saves dS1 here (dSs is next written at the next
        // chunk's start)
        if (!SUMMARY && VEC)
            lds_to_global<TI, BV, DK>(static_cast<TI*>(p.dS1) + (((long)bh * p.NT + n) * DVr + v0) * DK, DK, dSs,
                                      LDK, BV);
        // (d) lambda^T = dU^T T ; dv = beta lambda.  lambda^T tiles give a lane 4
        //     consecutive v of one row t of lambda and dv
        {
            f32x4 Lm[TL::PER];
            zero_acc<BV, C>(Lm);
            gemm<TI, BV, C, C, false, true>(Lm, dUT, LDC, Tl, LDC);
            if (TL::active()) {
                float bt[TL::PER];   // LDS reads first, then the writes
#pragma unroll
                for (int j = 0; j < TL::PER; ++j) bt[j] = beta_s[TL::col(j)];
#pragma unroll
                for (int j = 0; j < TL::PER; ++j) {
                    const int t = TL::col(j), off = t * LDV + TL::row(j, 0);
                    st4<TI>(Lb + off, Lm[j]);
                    st4<TI>(Db + off, bt[j] * Lm[j]);
                    if (!VEC) st4<TI>(Dn + off, (-(SCA ? rowf[t] : 1.f) * bt[j]) * Lm[j]);
                }
            }
        }
        __syncthreads();
        // (e) dS0^T = Diag(Gam_C) dS1^T + (Q Gam)^T dO - (K Gam)^T (beta lambda),
        //     the first two terms already added in (c)
        gemm<TI, DK, BV, C, true, true>(dS, VEC ? Kn : Kd, LDK, VEC ? Db : Dn, LDV);
        if constexpr (VEC) {   // the previous chunk's tiles, then the inputs of the one before
            form();
            prefetch_kq(n - 2 >= n0 ? n - 2 : n0);
        }
        __syncthreads();
    }
    if (!SUMMARY && n1 > n0) {   // lambda and dv of the segment's first chunk
        lds_to_global<TI, C, BV>(static_cast<TI*>(p.lam) + ((long)bh * p.NT + n0) * C * DVr + v0, DVr, Lb, LDV, C);
        lds_to_global<TI, C, BV>(static_cast<TI*>(p.dv) + ((long)bh * p.T + n0 * C) * DVr + v0, DVr, Db, LDV,
                                 min(C, p.T - n0 * C));
    }
    if (!SUMMARY && seg == 0 && p.dh0 && TS::active()) {
#pragma unroll
        for (int j = 0; j < TS::PER; ++j)
            st4<float>(p.dh0 + ((long)bh * DVr + v0 + TS::col(j)) * DK + TS::row(j, 0), dS[j]);
    }
    if (SUMMARY && TS::active()) {
        float* out = p.seg_end + ((long)bh * p.nseg + seg) * rows * DK;
#pragma unroll
        for (int j = 0; j < TS::PER; ++j) st4<float>(out + (long)(v0 + TS::col(j)) * DK + TS::row(j, 0), dS[j]);
    }
}

template <typename TI, int GATE, int C, int DK, int BV, bool SUMMARY = false>
__global__ __launch_bounds__(kThreads) void bwd_state_kernel(Params p) {
    __shared__ BwdStateArrays<TI, GATE, C, DK, BV> a;
    bwd_state_body<TI, GATE, C, DK, BV, SUMMARY>(p, blockIdx.x, a.gam_s, a.egc, a.rowf, a.beta_s, a.dSs, a.Kd, a.Kn,
                                                 a.Qg, a.Pl, a.Tl, a.dOb, a.dOg, a.dUT, a.Lb, a.Db, a.Dn);
}

// The recomputing backward's forward state pass (chunk states into the
// workspace) and the backward state pass in one launch.  The reverse pass needs
// no chunk state, so the two chains are independent: workgroups [0, nf) walk the
// forward chains, the others the reverse ones, and the two kinds overlay their
// LDS arrays, so that one of each shares a compute unit where LDS and registers
// allow.  Both chains are latency-bound; side by side each hides the other's waits.
template <typename TI, int GATE, int C, int DK, int BV>
__global__ __launch_bounds__(kThreads) void recompute_bwd_state_kernel(Params p, int nf) {
    __shared__ union {
        FwdStateArrays<TI, GATE, C, DK, BV, false> f;
        BwdStateArrays<TI, GATE, C, DK, BV> b;
    } u;
    if ((int)blockIdx.x < nf) {
        auto& a = u.f;
        fwd_state_body<TI, GATE, C, DK, BV, true, false>(p, blockIdx.x, a.gam_s, a.egc, a.rowf, a.beta_s, a.Ss, a.Qg,
                                                         a.Kg, a.Kd, a.Vb, a.Tl, a.Pl, a.Rb, a.Ud);
    } else {
        auto& a = u.b;
        bwd_state_body<TI, GATE, C, DK, BV, false>(p, blockIdx.x - nf, a.gam_s, a.egc, a.rowf, a.beta_s, a.dSs, a.Kd,
                                                   a.Kn, a.Qg, a.Pl, a.Tl, a.dOb, a.dOg, a.dUT, a.Lb, a.Db, a.Dn);
    }
}

// ---------------------------------------------------------------------------
// bwd_chunk_kernel: grid (NT, BH); every chunk finished independently.
// D = d_k = d_v.  The d_v dimension is streamed in blocks of VB columns: the
// block's S0 rows, dS1 rows, lambda, dO, V and U columns (US: U = T R of the
// chunk as the forward saved it) are loaded into registers two blocks ahead and
// committed to LDS while the previous block computes
//     (without US: X_b = (K Gam) S0_b^T,  R_b = beta (V_b - X_b),  U_b = T R_b)
//     dQg += dO_b S0_b,  dKg += lambda_b S0_b,  dKd += U_b dS1_b
//     dA  += lambda_b U_b^T,  dP += dO_b U_b^T
// after which the key-gradient products (phase C) finish dq, dk, dbeta, dg.
// The residual's part of dbeta, sum_v lambda (V - X) with X = (K Gam) S0^T,
// needs no X: sum_v lambda X = sum_c (K Gam) (lambda S0), and lambda S0 is dKg;
// sum_v lambda V is formed from the V and lambda registers at each commit.
// Every LDS tile keeps its natural (global) layout; operands contracted over
// their leading index are read with the transposing LDS load.  The products are
// accumulated transposed where that gives a lane 4 consecutive elements of a
// row of the stored result (dq^T, dk^T, dA^T, dP^T), so results go to LDS with
// one vector store per tile.
template <typename TI, int GATE, int C, int D, bool US>
struct BwdChunkSmem {
    static constexpr int PAD = Pad<TI>::value;
    // d_v block: 32 (16 for fp32 at D = 128, whose tiles are twice the bytes), or 64
    // where LDS has room for two such blocks (WIDE: bf16, no per-channel gate tile,
    // D = 128, C = 64; without US only with R formed in place over V, no R buffer)
    static constexpr bool WIDE = GATE != kGateVector && sizeof(TI) == 2 && D == 128 && C == 64;
    static constexpr bool RINPLACE = !US && WIDE;
    static constexpr int VB = WIDE ? 64 : (D >= 32 ? (sizeof(TI) == 4 && D > 64 ? 16 : 32) : D);
    static constexpr int NVB = D / VB;
    static constexpr int LD = D + PAD;            // rows of D elements
    static constexpr int LC = C + PAD;            // rows of C elements
    static constexpr int LVB = VB + PAD;          // rows of VB elements
    static constexpr int GW = GateLayout<GATE, D>::GW;
    static constexpr bool VEC = GATE == kGateVector;
    static constexpr size_t E = sizeof(TI);
    static constexpr size_t al(size_t x) { return (x + 255) & ~size_t(255); }
    // persistent through the d_v loop (K also through phase C without a vector gate)
    static constexpr size_t KG = 0;                                  // K (or K Gam)   [C][LD]
    static constexpr size_t TL = KG + al(C * LD * E);                // T (without US) [C][LC]
    static constexpr size_t LOOP = TL + (US ? 0 : al(C * LC * E));
    // d_v loop: two buffers of one block's tiles (offsets within a buffer), so the
    // next block is committed while this one computes
    static constexpr size_t S0B = 0;                                 // S0 rows        [VB][LD]
    static constexpr size_t DS1B = S0B + al(VB * LD * E);            // dS1 rows       [VB][LD]
    static constexpr size_t LAMB = DS1B + al(VB * LD * E);           // lambda block   [C][LVB]
    static constexpr size_t DOB = LAMB + al(C * LVB * E);            // dO block       [C][LVB]
    static constexpr size_t UBL = DOB + al(C * LVB * E);             // U block (without US: V, then U) [C][LVB]
    static constexpr size_t BLK = UBL + al(C * LVB * E);
    static constexpr size_t RB = LOOP + 2 * BLK;                     // R block (without US, 32 wide) [C][LVB]
    static constexpr size_t LOOP_END = RB + (US || RINPLACE ? 0 : al(C * LVB * E));
    // phase C (over the d_v-loop tiles)
    static constexpr size_t DA = LOOP;                               // dA~            [C][LC]
    static constexpr size_t DAB = DA + al(C * LC * E);               // beta_t dA~     [C][LC]
    static constexpr size_t DP = DAB + al(C * LC * E);               // dP~            [C][LC]
    static constexpr size_t QL = DP + al(C * LC * E);                // Q (Q e^{gam-c}) [C][LD]
    static constexpr size_t KR = QL + al(C * LD * E);                // K e^{c-gam}    [C][LD] (vector)
    static constexpr size_t KL = KR + al(C * LD * E);                // K e^{gam-c}    [C][LD] (vector)
    static constexpr size_t C_END = VEC ? KL + al(C * LD * E) : KR;
    static constexpr size_t BIG_END = LOOP_END > C_END ? LOOP_END : C_END;
    // small fp32 arrays; the vector gate's gam rows padded (LDGM floats): its
    // per-element factors are read a column of 16 rows at a time
    static constexpr int LDGM = D + 4;
    static constexpr size_t GAM = al(BIG_END);                                    // gam [C][LDGM] or [C]
    static constexpr size_t ROWF = GAM + al(VEC ? C * LDGM * 4 : C * 4);          // [2][C] (scalar)
    static constexpr size_t BETA = ROWF + al(2 * C * 4);                          // [C]
    static constexpr size_t RED_R = BETA + al(C * 4);                             // [D/16][C] row partials (dbeta_A)
    static constexpr size_t RED_G = RED_R + al((D / 16) * C * 4);                 // [D/16][C] row partials (d gam)
    using RV = RegN<TI, C, VB>;   // register tiles of the lambda / dO / U / V blocks
    static constexpr size_t RED_V = RED_G + al((D / 16) * C * 4);                 // [RV::VPR][C] row partials (lambda . V)
    static constexpr size_t RED_C = RED_V + al(RV::VPR * C * 4);                  // [C/16][D] column partials
    static constexpr size_t LASTS = RED_C + al((C / 16) * D * 4);                 // [D]
    static constexpr size_t KCO = LASTS + al(D * 4);                              // [C] Kaczmarz dk coefficients
    static constexpr size_t DIAGP = KCO + al(C * 4);                              // [C] diagonal of dP (vector gate)
    static constexpr size_t TOTAL = DIAGP + al(VEC ? C * 4 : 0);
    // dq / dk write-back tiles [C][LD] each at offset 0; after them the per-thread
    // partials of sum_v S0 dS1 [row blocks of the S0 register tile][LDS_] fp32
    using RS = RegB<TI, VB, D>;
    static constexpr int LDS_ = D + 4;   // rows of the partials (padded: eight lanes store to eight rows)
    static constexpr size_t LSRED = al(2 * C * LD * E);
    static_assert(LSRED + RS::BR * LDS_ * 4 <= BIG_END, "S0 dS1 partials");
    static_assert(2 * C * LD * E <= BIG_END, "write-back tiles");
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// Key-gradient products of the per-channel gate for the wave's tiles of the
// D x C outputs, all transposed ([c][t] / [c][s]):
//     Y^T [c][t] = sum_{s} dA~[t][s] k_sc e^{gam_tc - gam_sc}
//     DQ^T[c][t] = sum_{s} dP~[t][s] k_sc e^{gam_tc - gam_sc}
//     Z^T [c][s] = sum_{t} (beta dA~)[t][s] k_tc e^{gam_tc - gam_sc} + sum_{t} dP~[t][s] q_tc e^{gam_tc - gam_sc}
// (dA~, beta dA~, dP~ stored [t][s] and masked; their rows and columns are
// the chunk's steps).  The contraction is split into 16-step blocks b, with
// rho_b = gam at the last row of block b (rho_{-1} = 0):
//   Y, DQ: Kc = k e^{rho_b - gam} (b = the row's own block) is the operand, and
//          each block's partial is scaled by e^{gam_t - rho_b} on the accumulator;
//   Z:     Kr = k e^{gam - rho_{b-1}}, Qr = q e^{gam - rho_{b-1}} (b = the row's
//          block) are the operands, each block's partial scaled by e^{rho_{b-1} - gam_s}.
// For g <= 0 every factor is at most 1 except on the partial of the output's own
// block, where it grows at most by the decay of 16 steps (the centred
// contraction of the ReWY abstract, centred per 16-row block).
// gam_s: [C][LDG] fp32; Kc, Kr, Qr: [C][ld]; DA, DAB, DP: [C][lc].
// The results go straight into the caller's accumulators: dkp += beta_t Y,
// dq += DQ, dkm += Z, and dbA[j] = sum over the lane's 4 channels of k Y (kraw:
// k at the lane's elements of each tile, as given).
template <typename TI, int C, int D, int LDG, int NACC>
__device__ __forceinline__ void vec_key_products(f32x4 (&dkp)[NACC], f32x4 (&dq)[NACC], f32x4 (&dkm)[NACC],
                                                 float (&dbA)[NACC], const typename Vec4<TI>::type (&kraw)[NACC],
                                                 const float* beta_s, const TI* Kc, const TI* Kr, const TI* Qr,
                                                 int ld, const TI* DA, const TI* DAB, const TI* DP, int lc,
                                                 const float* gam_s) {
    using TO = Tiles<D, C>;
    using MM = typename MmaFor<TI, 16>::type;   // one 16-step block per partial
    static_assert(NACC == TO::PER, "accumulator count");
    constexpr int NB = C / 16, RM = TO::RM, RN = TO::RN;
    if (!TO::active()) return;
    // The RM tiles of one column group share their steps (n0, block ob), so each
    // dA~ / beta dA~ / dP~ fragment is read once for all of them; each tile still
    // sums its blocks in ascending order.
#pragma unroll
    for (int in = 0; in < RN; ++in) {
        const int n0 = TO::n0(in), ob = n0 / 16, t = TO::col(in);   // steps n0.. (block ob); this lane's t
        f32x4 gt[RM], y[RM], dqp[RM], z[RM];
#pragma unroll
        for (int im = 0; im < RM; ++im) {
            gt[im] = ld4<float>(gam_s + t * LDG + TO::row(im * RN + in, 0));   // this lane's 4 channels c..
            y[im] = zero4();
            dqp[im] = zero4();
            z[im] = zero4();
        }
        // Y, DQ: blocks b <= ob
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b > ob) break;
            f32x4 py[RM], pq[RM];
#pragma unroll
            for (int im = 0; im < RM; ++im) {
                py[im] = zero4();
                pq[im] = zero4();
            }
#pragma unroll
            for (int k0 = 0; k0 < 16; k0 += MM::kStep) {
                const auto fda = MM::load(DA + n0 * lc + 16 * b + k0, lc);
                const auto fdp = MM::load(DP + n0 * lc + 16 * b + k0, lc);
#pragma unroll
                for (int im = 0; im < RM; ++im) {
                    const auto fa = MM::load_t(Kc + (16 * b + k0) * ld + TO::m0(im * RN + in), ld);
                    py[im] = MM::op(fa, fda, py[im]);
                    pq[im] = MM::op(fa, fdp, pq[im]);
                }
            }
#pragma unroll
            for (int im = 0; im < RM; ++im) {
                const f32x4 rb = ld4<float>(gam_s + (16 * b + 15) * LDG + TO::row(im * RN + in, 0));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float fct = fexp(gt[im][i] - rb[i]);
                    y[im][i] += fct * py[im][i];
                    dqp[im][i] += fct * pq[im][i];
                }
            }
        }
        // Z: blocks b >= ob (here t is the output's step s)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b < ob) continue;
            f32x4 pz[RM];
#pragma unroll
            for (int im = 0; im < RM; ++im) pz[im] = zero4();
#pragma unroll
            for (int k0 = 0; k0 < 16; k0 += MM::kStep) {
                const auto fab = MM::load_t(DAB + (16 * b + k0) * lc + n0, lc);
                const auto fpt = MM::load_t(DP + (16 * b + k0) * lc + n0, lc);
#pragma unroll
                for (int im = 0; im < RM; ++im) {
                    const int m0 = TO::m0(im * RN + in);
                    pz[im] = MM::op(MM::load_t(Kr + (16 * b + k0) * ld + m0, ld), fab, pz[im]);
                    pz[im] = MM::op(MM::load_t(Qr + (16 * b + k0) * ld + m0, ld), fpt, pz[im]);
                }
            }
#pragma unroll
            for (int im = 0; im < RM; ++im) {
                const f32x4 rp = b > 0 ? ld4<float>(gam_s + (16 * b - 1) * LDG + TO::row(im * RN + in, 0)) : zero4();
#pragma unroll
                for (int i = 0; i < 4; ++i) z[im][i] += fexp(rp[i] - gt[im][i]) * pz[im][i];
            }
        }
#pragma unroll
        for (int im = 0; im < RM; ++im) {
            const int j = im * RN + in;
            const f32x4 kv = f32x4{to_f(kraw[j][0]), to_f(kraw[j][1]), to_f(kraw[j][2]), to_f(kraw[j][3])};
            const f32x4 d4 = kv * y[im];
            dbA[j] = d4[0] + d4[1] + d4[2] + d4[3];
            dkp[j] += beta_s[t] * y[im];
            dq[j] += dqp[im];
            dkm[j] += z[im];
        }
    }
}

template <typename TI, int GATE, int C, int D, bool US>
__global__ __launch_bounds__(kThreads) void bwd_chunk_kernel(Params p) {
    using L = BwdChunkSmem<TI, GATE, C, D, US>;
    constexpr int LD = L::LD, LC = L::LC, LVB = L::LVB, GW = L::GW;
    constexpr int VB = L::VB, NVB = L::NVB;
    constexpr bool VEC = GATE == kGateVector;
    constexpr bool SCA = GATE == kGateScalar;
    __shared__ __align__(16) char smem[L::TOTAL];
    TI* KG = reinterpret_cast<TI*>(smem + L::KG);
    TI* TLs = reinterpret_cast<TI*>(smem + L::TL);
    // tiles of block-buffer i
    auto blk = [&](int i, size_t off) { return reinterpret_cast<TI*>(smem + L::LOOP + i * L::BLK + off); };
    TI* RB = reinterpret_cast<TI*>(smem + L::RB);
    float* gam_s = reinterpret_cast<float*>(smem + L::GAM);
    float* rowf = reinterpret_cast<float*>(smem + L::ROWF);
    float* beta_s = reinterpret_cast<float*>(smem + L::BETA);
    float* red_r = reinterpret_cast<float*>(smem + L::RED_R);
    float* red_g = reinterpret_cast<float*>(smem + L::RED_G);
    float* red_v = reinterpret_cast<float*>(smem + L::RED_V);
    float* red_c = reinterpret_cast<float*>(smem + L::RED_C);
    float* lastS = reinterpret_cast<float*>(smem + L::LASTS);
    float* kco = reinterpret_cast<float*>(smem + L::KCO);
    float* diagp = reinterpret_cast<float*>(smem + L::DIAGP);

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
    const TI* __restrict__ Ug = static_cast<const TI*>(p.Um) + chunk * C * D;

    using TO = Tiles<D, C>;    // dq^T, dk^T         [c][t]
    using TCC = Tiles<C, C>;   // dA^T, dP^T         [s][t]
    using TX = Tiles<VB, C>;   // X_b^T, U_b^T       [v][t]  (without US)

    // ---------------- prologue: gate, K, the first d_v blocks
    // (the Kaczmarz step's 1 / (||k_t||^2 + eps) of step t = thread index, used only
    // by the finish: loaded first, branch-free (beta stands in without the step), so
    // its latency hides behind the whole chunk)
    const float krn_t = (p.kz ? p.krn + row0 : p.beta + row0)[min((int)threadIdx.x, valid - 1)];
    GateRegs<GATE, C, D> rg;
    rg.load(p.gam + row0 * GW, p.beta + row0, valid);
    // K: with two (64-wide) blocks loaded after the gate's barrier and staged after
    // block 0's commit, so that barrier waits for fewer loads
    constexpr bool KLATE = NVB == 2 && !VEC;
    RegN<TI, C, D> rK;
    if (!KLATE) rK.load(k, D, valid);
    RegN<TI, C, C> rT;
    if (!US) rT.load(static_cast<const TI*>(p.Tm) + chunk * C * C, C, C);
    // two register sets: the loads of block b + 2 are issued when block b is
    // committed, so two blocks of loads are in flight during the loop
    using RV = typename L::RV;
    struct BlockRegs {
        RegB<TI, VB, D> S0, dS1;
        RV lam, dO, U, V;
    } rb[2];
    auto load_block = [&](BlockRegs& r, int b) {
        const int v0 = b * VB;
        r.S0.load(S0g + (long)v0 * D, D, VB);
        r.dS1.load(dS1g + (long)v0 * D, D, VB);
        r.lam.load(lamg + v0, D, C);
        if (US) r.U.load(Ug + v0, D, C);
        r.dO.load(dO + v0, D, valid);
        r.V.load(v + v0, D, valid);
    };
    load_block(rb[0], 0);
    // sum_v S0[v][c] dS1[v][c] over this thread's rows of every block
    float ls[L::RS::PER][L::RS::VW] = {};
    rg.commit(rowf, gam_s, beta_s, L::LDGM);
    __syncthreads();
    if (NVB > 2) load_block(rb[1], 1);   // after the gate's barrier: it waits for fewer loads
    if (KLATE) rK.load(k, D, valid);
    const GateLds<GATE, C, D, L::LDGM> gf{rowf, gam_s, valid - 1};
    if (VEC)
        rK.store(KG, LD, [&](int r, int c, float x) { return x * gf.G(r, c); });
    else if (!KLATE)
        rK.store(KG, LD);   // scalar: Gam_t is applied on the C x D results
    if (!US) rT.store(TLs, LC);
    // sum_v lambda V over this thread's vectors of the block tiles (rows past the
    // sequence excluded: V is loaded clamped there)
    float lv[RV::PER] = {};
    auto commit_block = [&](BlockRegs& r, int i) {
        r.S0.dot_rows(r.dS1, ls);
#pragma unroll
        for (int x = 0; x < RV::PER; ++x) {
            const uint4 la = pin(r.lam.r[x]), va = pin(r.V.r[x]);
            const TI* le = reinterpret_cast<const TI*>(&la);
            const TI* ve = reinterpret_cast<const TI*>(&va);
            float s2 = 0.f;
#pragma unroll
            for (int e = 0; e < RV::VW; ++e) s2 += to_f(le[e]) * to_f(ve[e]);
            lv[x] += RV::idx_of(x) / RV::VPR < valid ? s2 : 0.f;
        }
        // the sums are formed here: left to their use at the finish, the compiler
        // sinks the products there and keeps both register tiles alive until then
#pragma unroll
        for (int x = 0; x < L::RS::PER; ++x)
#pragma unroll
            for (int y = 0; y < L::RS::VW; ++y) asm volatile("" : "+v"(ls[x][y]));
        r.S0.store_n(blk(i, L::S0B), LD, Identity());
        r.dS1.store_n(blk(i, L::DS1B), LD, Identity());
        r.lam.store(blk(i, L::LAMB), LVB);
        r.dO.store(blk(i, L::DOB), LVB);
        (US ? r.U : r.V).store(blk(i, L::UBL), LVB);
    };
    commit_block(rb[0], 0);
    if (KLATE) rK.store(KG, LD);
    __syncthreads();
    // with two (64-wide) blocks, block 1's loads only now: they arrive during block
    // 0's products, where issued in the prologue they held its barriers back (with
    // four blocks the prologue's are half the bytes and block 1 is best loaded
    // there); then block 2's into the set just committed
    if (NVB == 2) load_block(rb[1], 1);
    if (NVB > 2) load_block(rb[0], 2);

    // ---------------- d_v loop
    f32x4 dq[TO::PER], dkp[TO::PER], dkm[TO::PER], dA[TCC::PER], dP[TCC::PER];
    zero_acc<D, C>(dq);
    zero_acc<D, C>(dkp);
    zero_acc<D, C>(dkm);
    zero_acc<C, C>(dA);
    zero_acc<C, C>(dP);
    // q (and k for the vector gate) for the key-gradient products, loaded at the
    // start of the last d_v block (whose second register set is free by then; q
    // is not among the cache-warmed tiles, so it comes from far away)
    RegN<TI, C, D> rq, rk;
    // vector gate: k and q at this lane's elements of the output tiles (4 consecutive
    // c of row t), as given and kept packed, loaded with them (rows past the
    // sequence read row valid - 1 and count as zero)
    typedef typename Vec4<TI>::type V4;
    V4 kraw[TO::PER], qraw[TO::PER];
#pragma unroll
    for (int b = 0; b < NVB; ++b) {
        if (b == NVB - 1) {
            rq.load(q, D, valid);
            if (VEC) rk.load(k, D, valid);
            if (VEC && TO::active()) {
#pragma unroll
                for (int j = 0; j < TO::PER; ++j) {
                    const int t = TO::col(j), tt = min(t, valid - 1);
                    kraw[j] = *reinterpret_cast<const V4*>(k + (long)tt * D + TO::row(j, 0));
                    qraw[j] = *reinterpret_cast<const V4*>(q + (long)tt * D + TO::row(j, 0));
                }
            }
        }
        TI* S0B = blk(b & 1, L::S0B);
        TI* DS1B = blk(b & 1, L::DS1B);
        TI* LAMB = blk(b & 1, L::LAMB);
        TI* DOB = blk(b & 1, L::DOB);
        TI* UB = blk(b & 1, L::UBL);
        if constexpr (US) {
            // the two S0 contractions (S0 rows read as [k][m]), then the two over U
            gemm2<TI, D, C, VB, true, false>(dq, dkp, S0B, LD, DOB, LAMB, LVB);
            gemm<TI, D, C, VB, true, false>(dkm, DS1B, LD, UB, LVB);
            gemm2<TI, C, C, VB, false, false>(dA, dP, UB, LVB, LAMB, DOB, LVB);
            // block b + 1 into the other buffer (its last reader, block b - 1, ended at
            // the previous barrier), read after the barrier below; then the loads of
            // block b + 3 into the registers it leaves free
            if (b + 1 < NVB) {
                commit_block(rb[(b + 1) & 1], (b + 1) & 1);
                if (b + 3 < NVB) load_block(rb[(b + 1) & 1], b + 3);
                __syncthreads();
            }
        } else {
            // X_b^T = S0_b (K Gam)^T and the two S0 contractions (S0 rows read as [k][m])
            f32x4 X[TX::PER];
            zero_acc<VB, C>(X);
            gemm<TI, VB, C, D, false, false>(X, S0B, LD, KG, LD);
            gemm2<TI, D, C, VB, true, false>(dq, dkp, S0B, LD, DOB, LAMB, LVB);
            if (TX::active()) {
                f32x4 rr[TX::PER];   // LDS reads first, then the writes
#pragma unroll
                for (int j = 0; j < TX::PER; ++j) {
                    const int t = TX::col(j), c = TX::row(j, 0);
                    rr[j] = beta_s[t] * (ld4<TI>(UB + t * LVB + c) - (SCA ? rowf[t] : 1.f) * X[j]);
                }
#pragma unroll
                for (int j = 0; j < TX::PER; ++j)
                    st4<TI>((L::RINPLACE ? UB : RB) + TX::col(j) * LVB + TX::row(j, 0), rr[j]);
            }
            __syncthreads();
            // block b + 1 into the other buffer (free since block b - 1 ended), read after
            // the two barriers below
            if (b + 1 < NVB) {
                commit_block(rb[(b + 1) & 1], (b + 1) & 1);
                if (b + 3 < NVB) load_block(rb[(b + 1) & 1], b + 3);
            }
            // U_b^T = R_b^T T^T  (R rows read as [k][m]) over the V block
            {
                f32x4 U[TX::PER];
                zero_acc<VB, C>(U);
                gemm<TI, VB, C, C, true, false>(U, L::RINPLACE ? UB : RB, LVB, TLs, LC);
                if (L::RINPLACE) __syncthreads();   // every wave has read R before U overwrites it
                if (TX::active()) {
#pragma unroll
                    for (int j = 0; j < TX::PER; ++j) st4<TI>(UB + TX::col(j) * LVB + TX::row(j, 0), U[j]);
                }
            }
            __syncthreads();
            gemm<TI, D, C, VB, true, false>(dkm, DS1B, LD, UB, LVB);
            gemm2<TI, C, C, VB, false, false>(dA, dP, UB, LVB, LAMB, DOB, LVB);
            // no barrier here: the next writes into this buffer (the commit of block
            // b + 2) and into RB come after the next block's first barrier (with R in
            // place, block b + 1's R goes to the other buffer)
        }
    }


    // sum_v lambda X at row t as sum_c (K Gam)[t][c] dKg[t][c] (over this lane's 4 c;
    // K Gam with the operand values X was formed from), then
    // dq = Gam dQg ; dk+ = -beta Gam dKg ; dk- = Gd dKd   (element c = row, t = col)
    float xdot[TO::PER];
    if (TO::active()) {
#pragma unroll
        for (int j = 0; j < TO::PER; ++j) {
            const int t = TO::col(j);
            const f32x4 kg = ld4<TI>(KG + t * LD + TO::row(j, 0));
            float x = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) x += kg[i] * (VEC ? 1.f : gf.G(t, TO::row(j, i))) * dkp[j][i];
            xdot[j] = x;
        }
#pragma unroll
        for (int j = 0; j < TO::PER; ++j) {
            const int t = TO::col(j);
            const float bt = beta_s[t];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = TO::row(j, i);
                const float G = gf.G(t, c);
                dq[j][i] *= G;
                dkp[j][i] *= -bt * G;
                dkm[j][i] *= gf.Gd(t, c);
            }
        }
    }

    // ---------------- phase B: dA~, beta dA~ and dP~ into LDS (element s = row, t = col)
    __syncthreads();   // the last block's tiles, which phase B overwrites, are dead
    {
        TI* DAs = reinterpret_cast<TI*>(smem + L::DA);
        TI* DABs = reinterpret_cast<TI*>(smem + L::DAB);
        TI* DPs = reinterpret_cast<TI*>(smem + L::DP);
        if (TCC::active()) {
            f32x4 a[TCC::PER], ab[TCC::PER], pp[TCC::PER];   // LDS reads first, then the writes
#pragma unroll
            for (int j = 0; j < TCC::PER; ++j) {
                const int t = TCC::col(j);
                const float bt = beta_s[t];
                const float gt = SCA ? gam_s[t] : 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s2 = TCC::row(j, i);
                    const float e = (SCA && s2 <= t) ? fexp(gt - gam_s[s2]) : 1.f;
                    // the vector gate's key products leave out the diagonal of dP: it is
                    // added in fp32 in phase C (see there)
                    pp[j][i] = (VEC ? s2 < t : s2 <= t) ? dP[j][i] * e : 0.f;
                    if (VEC && s2 == t) diagp[t] = dP[j][i];
                    a[j][i] = s2 < t ? -dA[j][i] * e : 0.f;   // dA = -lambda U^T
                    ab[j][i] = bt * a[j][i];
                }
            }
#pragma unroll
            for (int j = 0; j < TCC::PER; ++j) {
                const int off = TCC::col(j) * LC + TCC::row(j, 0);
                st4<TI>(DAs + off, a[j]);
                st4<TI>(DABs + off, ab[j]);
                st4<TI>(DPs + off, pp[j]);
            }
        }
    }

    // ---------------- phase C: key-gradient products
    {
        const TI* DAs = reinterpret_cast<const TI*>(smem + L::DA);
        const TI* DABs = reinterpret_cast<const TI*>(smem + L::DAB);
        const TI* DPs = reinterpret_cast<const TI*>(smem + L::DP);
        TI* Ql = reinterpret_cast<TI*>(smem + L::QL);
        // K rows: the loop's K tile without a vector gate, else K e^{c - gam} / K e^{gam - c}
        TI* Kr = VEC ? reinterpret_cast<TI*>(smem + L::KR) : KG;
        TI* Kl = VEC ? reinterpret_cast<TI*>(smem + L::KL) : KG;
        const float* gl = gam_s + (valid - 1) * (VEC ? L::LDGM : GW);
        if (VEC) {
            // K e^{rho_b - gam}, K e^{gam - rho_{b-1}}, Q e^{gam - rho_{b-1}} with rho_b the
            // gate at the last row of the row's 16-row block b (see vec_key_products)
            rk.store3(rq, Kr, Kl, Ql, LD, [&](int r, int c, float k, float q, float* y) {
                const int b = r >> 4;
                const float g = gam_s[r * L::LDGM + c];
                const float rb = gam_s[(16 * b + 15) * L::LDGM + c];
                const float rp = b > 0 ? gam_s[(16 * b - 1) * L::LDGM + c] : 0.f;
                const float fr = fexp(g - rp);
                y[0] = k * fexp(rb - g);
                y[1] = k * fr;
                y[2] = q * fr;
            });
        } else {
            rq.store(Ql, LD);
        }
        __syncthreads();
        // Warm the caches for the workgroup that most likely starts next on this
        // XCD: workgroups start in id order and go to the XCDs round-robin, so it
        // is this id plus the number resident at once.  One dword of every
        // 128-byte line of its prologue tiles (K, the first 64 rows of S0 and dS1
        // and columns of lambda, U (or T without US), dO and V -- the first two
        // 32-wide d_v blocks or one 64-wide --, the gate and beta rows; up to 2
        // lines per thread), held in registers and consumed only at the end, so
        // nothing waits for them.
        int warm[2];
        {
            const long ids = (long)gridDim.x * gridDim.y;
            const long nid = min((long)blockIdx.y * gridDim.x + blockIdx.x + p.resident, ids - 1);
            const int nbh = (int)(nid / gridDim.x), nn = (int)(nid - (long)nbh * gridDim.x);
            const int nvalid = min(C, p.T - nn * C);
            const long nrow0 = (long)nbh * p.T + (long)nn * C;
            const long nchunk = (long)nbh * p.NT + nn;
            constexpr int E = sizeof(TI), NB = NVB < 2 ? NVB : (VB >= 64 ? 1 : 2);
            constexpr int LPR = (NB * VB * E + 127) / 128;   // lines per row of the lambda / U / dO / V blocks
            const int nK = (nvalid * D * E + 127) / 128;
            constexpr int nS = (NB * VB * D * E + 127) / 128;
            constexpr int nU = US ? C * LPR : (C * C * E + 127) / 128;   // U by row, or T by line
            const int nG = (nvalid * GW * 4 + 127) / 128, nB = (nvalid * 4 + 127) / 128;   // gate and beta rows
            // contiguous: K, S0, dS1; by row: lambda (C rows), U (C rows; T contiguous
            // without US), dO, V; then gate, beta
            const int b1 = nK, b2 = b1 + nS, b3 = b2 + nS, b4 = b3 + C * LPR, b5 = b4 + nU,
                      b6 = b5 + nvalid * LPR, b7 = b6 + nvalid * LPR, b8 = b7 + (GATE != kGateNone ? nG : 0),
                      nl = b8 + nB;
            const char* kb = reinterpret_cast<const char*>(static_cast<const TI*>(p.k) + nrow0 * D);
            const char* sb = reinterpret_cast<const char*>(static_cast<const TI*>(p.states) + nchunk * D * D);
            const char* db = reinterpret_cast<const char*>(static_cast<const TI*>(p.dS1) + nchunk * D * D);
            const char* lb = reinterpret_cast<const char*>(static_cast<const TI*>(p.lam) + nchunk * C * D);
            const char* ub = US ? reinterpret_cast<const char*>(static_cast<const TI*>(p.Um) + nchunk * C * D)
                                : reinterpret_cast<const char*>(static_cast<const TI*>(p.Tm) + nchunk * C * C);
            const char* ob = reinterpret_cast<const char*>(static_cast<const TI*>(p.dout) + nrow0 * D);
            const char* vb = reinterpret_cast<const char*>(static_cast<const TI*>(p.v) + nrow0 * D);
            const char* gb = reinterpret_cast<const char*>(p.gam + nrow0 * GW);
            const char* bb = reinterpret_cast<const char*>(p.beta + nrow0);
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int i = min((int)threadIdx.x + r * kThreads, nl - 1);
                const int s = i < b3 ? 0 : (i < b4 ? 1 : (i < b5 ? 2 : (i < b6 ? 3 : (i < b7 ? 4 : 5))));
                const int j = i - (s == 1 ? b3 : (s == 2 ? b4 : (s == 3 ? b5 : b6)));
                // row segments by row and line; contiguous segments (K, S0, dS1, gate,
                // beta) by line
                const char* base = s == 1 ? lb : (s == 2 ? ub : (s == 3 ? ob : vb));
                long off = (long)(j / LPR) * D * E + (j % LPR) * 128;
                if (!US && s == 2) off = (long)j * 128;
                if (s == 0) {
                    base = i < b1 ? kb : (i < b2 ? sb : db);
                    off = (long)(i - (i < b1 ? 0 : (i < b2 ? b1 : b2))) * 128;
                }
                if (s == 5) {
                    base = i < b8 ? gb : bb;
                    off = (long)(i - (i < b8 ? b7 : b8)) * 128;
                }
                warm[r] = *reinterpret_cast<const int*>(base + off);
            }
        }
        // k and q at this lane's elements (4 consecutive c of row t), read back from the
        // staged tiles without a vector gate; the gam_C column sums of Kd dKd (dk- holds
        // only the Kd path so far)
        // without a vector gate k and q come from the staged tiles (dead before the
        // finish, so held in registers); with it from the packed loads above
        f32x4 kv_[TO::PER], qv_[TO::PER];
        auto cvt = [](const V4& x) { return f32x4{to_f(x[0]), to_f(x[1]), to_f(x[2]), to_f(x[3])}; };
        auto kv = [&](int j) -> f32x4 {
            if constexpr (VEC) return cvt(kraw[j]); else return kv_[j];
        };
        if (TO::active()) {
#pragma unroll
            for (int j = 0; j < TO::PER; ++j) {
                const int t = TO::col(j), c0 = TO::row(j, 0);
                if constexpr (VEC) {
                    if (t >= valid) {
                        kraw[j] = V4{};
                        qraw[j] = V4{};
                    }
                } else {
                    kv_[j] = ld4<TI>(Kr + t * LD + c0);
                    qv_[j] = ld4<TI>(Ql + t * LD + c0);
                }
            }
            // column sums over t (the 16 lanes of a tile row, the wave's RN tiles) per c
#pragma unroll
            for (int im = 0; im < TO::RM; ++im)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float colp = 0.f;
#pragma unroll
                    for (int in = 0; in < TO::RN; ++in)
                        colp += kv(im * TO::RN + in)[i] * dkm[im * TO::RN + in][i];
                    colp = row16_sum(colp);
                    if ((lane_id() & 15) == 0) red_c[TO::cg() * D + TO::row(im * TO::RN, i)] = colp;
                }
        }
        float dbA[TO::PER];   // sum over this lane's 4 c of k Y at row t = TO::col(j)
        if constexpr (VEC) {
            // Y, dQ+ and Z + W tile by tile, block by block (see vec_key_products)
            vec_key_products<TI, C, D, L::LDGM>(dkp, dq, dkm, dbA, kraw, beta_s, Kr, Kl, Ql, LD, DAs, DABs, DPs, LC,
                                                gam_s);
            // The diagonal of dP (a score with no decay) enters dq as dP_tt k_t and dk- as
            // dP_tt q_t; its two terms of d gam, q (dP_tt k) - k (dP_tt q), cancel exactly.
            // Added here in fp32 from the same k and q, they cancel to rounding, where
            // through the scaled bf16 operands of the products they would not (with strong
            // decay they dominate the small d gam)
            if (TO::active()) {
#pragma unroll
                for (int j = 0; j < TO::PER; ++j) {
                    const float dpt = TO::col(j) < valid ? diagp[TO::col(j)] : 0.f;
                    qv_[j] = cvt(qraw[j]);
                    dq[j] += dpt * kv(j);
                    dkm[j] += dpt * qv_[j];
                }
            }
        } else {
            f32x4 tmp[TO::PER], dqp[TO::PER];
            // Y^T = Kr^T dA~^T :  dK+ = beta Y, dbeta_A = sum_c K Y; and dQ+^T = Kr^T dP~^T
            // from the same Kr fragments
            zero_acc<D, C>(tmp);
            zero_acc<D, C>(dqp);
            gemm2<TI, D, C, C, true, false>(tmp, dqp, Kr, LD, DAs, DPs, LC);
            if (TO::active()) {
#pragma unroll
                for (int j = 0; j < TO::PER; ++j) {
                    const int t = TO::col(j);
                    const f32x4 d4 = kv(j) * tmp[j];
                    dbA[j] = d4[0] + d4[1] + d4[2] + d4[3];
                    dkp[j] += beta_s[t] * tmp[j];
                }
            }
            // Z^T = Kl^T (beta dA~) and W^T = Ql^T dP~ : both reach k through e^{-gam}
            zero_acc<D, C>(tmp);
            gemm<TI, D, C, C, true, true>(tmp, Kl, LD, DABs, LC);
            gemm<TI, D, C, C, true, true>(tmp, Ql, LD, DPs, LC);
            if (TO::active()) {
#pragma unroll
                for (int j = 0; j < TO::PER; ++j) {
                    dkm[j] += tmp[j];
                    dq[j] += dqp[j];
                }
            }
        }

        // -------- finish: dq, dk = dk+ + dk-, dbeta, d gam = q.dq + k.(dk+ - dk-)
        // (Kaczmarz step: dk also gets -2 dbeta_t beta_t k_t / (||k_t||^2 + eps), once
        // dbeta_t is reduced, and dbeta becomes d eta = dbeta / (||k_t||^2 + eps))
        __syncthreads();   // phase-C tiles dead: dq / dk go through LDS for coalesced stores
        TI* dqs = reinterpret_cast<TI*>(smem);
        TI* dks = dqs + C * LD;
        float* lsred = reinterpret_cast<float*>(smem + L::LSRED);
        const bool kz = p.kz != 0;
        f32x4 dgm[TO::PER], dkt[TO::PER];
        if (TO::active()) {
#pragma unroll
            for (int j = 0; j < TO::PER; ++j) {
                const int off = TO::col(j) * LD + TO::row(j, 0);
                dkt[j] = dkp[j] + dkm[j];
                st4<TI>(dqs + off, dq[j]);
                if (!kz) st4<TI>(dks + off, dkt[j]);
                dgm[j] = qv_[j] * dq[j] + kv(j) * (dkp[j] - dkm[j]);
            }
            // row partials over c (4 per lane, 4 lane groups, RM tiles) of K+ Y (dbeta)
            // and, for the scalar gate, of d gam
#pragma unroll
            for (int in = 0; in < TO::RN; ++in) {
                float sb = 0.f, sg = 0.f;
#pragma unroll
                for (int im = 0; im < TO::RM; ++im) {
                    sb += dbA[im * TO::RN + in] - xdot[im * TO::RN + in];
                    const f32x4 x = dgm[im * TO::RN + in];
                    sg += x[0] + x[1] + x[2] + x[3];
                }
                sb = sum_lane_groups(sb);
                if (SCA) sg = sum_lane_groups(sg);
                if (lane_id() < 16) {
                    red_r[TO::rg() * C + TO::col(in)] = sb;
                    if (SCA) red_g[TO::rg() * C + TO::col(in)] = sg;
                }
            }
        }
        // sum_v lambda V: the row partials of the block tiles' owners
#pragma unroll
        for (int x = 0; x < RV::PER; ++x) {
            const int idx = threadIdx.x + x * kThreads;
            if (idx < RV::NV) red_v[(idx % RV::VPR) * C + idx / RV::VPR] = lv[x];
        }
        // per-thread partials of sum_v S0 dS1 (gate terms only)
        if (GATE != kGateNone) {
#pragma unroll
            for (int i = 0; i < L::RS::PER; ++i) {
                if (L::RS::owns(i)) {
#pragma unroll
                    for (int kk = 0; kk < L::RS::VW; kk += 4)
                        st4<float>(lsred + L::RS::rowblk(i) * L::LDS_ + L::RS::col0(i) + kk,
                                   f32x4{ls[i][kk], ls[i][kk + 1], ls[i][kk + 2], ls[i][kk + 3]});
                }
            }
        }
        __syncthreads();
        for (int t = threadIdx.x; t < valid; t += kThreads) {
            float s2 = 0.f;
            for (int b = 0; b < RV::VPR; ++b) s2 += red_v[b * C + t];
            for (int b = 0; b < TO::WM; ++b) s2 += red_r[b * C + t];
            if (kz) {
                const float rn = t == (int)threadIdx.x ? krn_t : p.krn[row0 + t];
                kco[t] = -2.f * s2 * beta_s[t] * rn;
                s2 *= rn;
            }
            p.dbeta[row0 + t] = s2;
        }
        if (kz) {
            __syncthreads();
            if (TO::active()) {
#pragma unroll
                for (int j = 0; j < TO::PER; ++j) {
                    const int t = TO::col(j);
                    st4<TI>(dks + t * LD + TO::row(j, 0), dkt[j] + (t < valid ? kco[t] : 0.f) * kv(j));
                }
            }
            __syncthreads();
        }
        lds_to_global<TI, C, D>(static_cast<TI*>(p.dq) + row0 * D, D, dqs, LD, valid);
        lds_to_global<TI, C, D>(static_cast<TI*>(p.dk) + row0 * D, D, dks, LD, valid);
        if constexpr (GATE != kGateNone) {
            // gam_C terms from sum_v S0 dS1 and the Kd dKd column sums: per channel
            // (vector gate, lastS), or their total over the channels (scalar gate)
            if constexpr (VEC) {
                if (wave_id() < (D + 63) / 64) {
                    const int c = threadIdx.x;
                    if (c < D) {
                        float ssum = 0.f;
                        for (int h = 0; h < L::RS::BR; ++h) ssum += lsred[h * L::LDS_ + c];
                        float cs = 0.f;
                        for (int b = 0; b < TO::WN; ++b) cs += red_c[b * D + c];
                        lastS[c] = fexp(gl[c]) * ssum + cs;   // the whole last-row term of channel c
                    }
                }
                // d gam_t = sum_{s >= t} of the elementwise terms (rows past the sequence
                // count as zero), plus the gam_C term lastS, which enters at the last valid
                // row and so reaches every valid row.  In registers, per 16-step tile: a
                // suffix scan over its 16 lanes (DPP row shifts: lane i adds lane i + n of
                // its row, 0 past the row end) and the tile's total; then the totals of the
                // later tiles, of this wave directly and of the later column groups of
                // waves through LDS (red_g: [WN][D], unused by this gate).
                float* tl = red_g;
                static_assert(TO::WN * D <= (D / 16) * C, "tile totals");
                f32x4 tot[TO::PER];
                if (TO::active()) {
#pragma unroll
                    for (int j = 0; j < TO::PER; ++j) {
                        const bool in_seq = TO::col(j) < valid;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            float x = in_seq ? dgm[j][i] : 0.f;
                            tot[j][i] = row16_sum(x);
                            x += dpp_f<0x101>(x);
                            x += dpp_f<0x102>(x);
                            x += dpp_f<0x104>(x);
                            x += dpp_f<0x108>(x);
                            dgm[j][i] = x;
                        }
                    }
#pragma unroll
                    for (int im = 0; im < TO::RM; ++im) {
                        f32x4 sw = zero4();
#pragma unroll
                        for (int in = 0; in < TO::RN; ++in) sw += tot[im * TO::RN + in];
                        if ((lane_id() & 15) == 0) st4<float>(tl + TO::cg() * D + TO::row(im * TO::RN, 0), sw);
                    }
                }
                __syncthreads();
                if (TO::active()) {
#pragma unroll
                    for (int im = 0; im < TO::RM; ++im) {
                        const int c = TO::row(im * TO::RN, 0);
                        f32x4 off = ld4<float>(lastS + c);
                        for (int g = TO::cg() + 1; g < TO::WN; ++g) off += ld4<float>(tl + g * D + c);
#pragma unroll
                        for (int in = TO::RN - 1; in >= 0; --in) {
                            const int j = im * TO::RN + in, t = TO::col(j);
                            if (t < valid) st4<float>(p.dg + (row0 + t) * D + c, dgm[j] + off);
                            off += tot[j];
                        }
                    }
                }
            } else if (wave_id() == 0) {
                // one wave, no barrier: the gam_C term summed over the channels
                // (e^{gam_C} sum_v S0 dS1 + the Kd dKd column sums), then
                // d gam_t = sum_{s >= t} x_s with that term on the last valid row
                float xc = 0.f;
                for (int c = lane_id(); c < D; c += 64) {
                    float ssum = 0.f;
                    for (int h = 0; h < L::RS::BR; ++h) ssum += lsred[h * L::LDS_ + c];
                    float cs = 0.f;
                    for (int b = 0; b < TO::WN; ++b) cs += red_c[b * D + c];
                    xc += gf.GC(c) * ssum + cs;
                }
                xc = row16_sum(xc);
                const float tot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, xc), 0)) +
                                  __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, xc), 16)) +
                                  __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, xc), 32)) +
                                  __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, xc), 48));
                const int t = lane_id();
                float x = 0.f;
                if (t < valid) {
                    for (int b = 0; b < TO::WM; ++b) x += red_g[b * C + t];
                    if (t == valid - 1) x += tot;
                }
                // reverse inclusive scan over the 64 lanes: within each row of 16
                // lanes by DPP row shifts (lane i adds lane i + n of its row, 0 past
                // the row end), then the totals of the later rows
                x += dpp_f<0x101>(x);
                x += dpp_f<0x102>(x);
                x += dpp_f<0x104>(x);
                x += dpp_f<0x108>(x);
                const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
                const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
                const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
                const int row = t >> 4;
                x += (row < 1 ? r1 : 0.f) + (row < 2 ? r2 : 0.f) + (row < 3 ? r3 : 0.f);
                if (t < valid) p.dg[row0 + t] = x;
            }
        }
        asm volatile("" ::"v"(warm[0]), "v"(warm[1]));   // the warming loads' only use
    }
}

}  // namespace dn
