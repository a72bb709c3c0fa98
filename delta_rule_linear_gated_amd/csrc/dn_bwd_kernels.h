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
template <typename TI, int GATE, int C, int DK, int BV, bool SUMMARY = false>
__global__ __launch_bounds__(kThreads) void bwd_state_kernel(Params p) {
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
    // vector gate scales Q and K per element.
    __shared__ float gam_s[VEC ? C * DK : C];
    __shared__ __align__(16) float rowf[2 * C];
    __shared__ __align__(16) float beta_s[C];
    __shared__ __align__(16) TI dSs[BV * LDK];   // dS1 operand     [v][c]
    __shared__ __align__(16) TI Kd[C * LDK];     // K (vector gate: K Gam_C / Gam)  [t][c]
    __shared__ __align__(16) TI Kn[VEC ? C * LDK : 8];   // -K Gam (vector gate)    [t][c]
    __shared__ __align__(16) TI Qg[C * LDK];     // Q (vector gate: Q Gam)          [t][c]
    __shared__ __align__(16) TI Pl[C * LDC];     // P               [s][t]
    __shared__ __align__(16) TI Tl[C * LDC];     // T               [s][t]
    __shared__ __align__(16) TI dOb[C * LDV];    // dO block        [t][v]
    __shared__ __align__(16) TI dOg[SCA ? C * LDV : 8];  // dO Gam (scalar gate)    [t][v]
    __shared__ __align__(16) TI dUT[BV * LDC];   // dU^T            [v][t]
    // lambda and dv = beta lambda [t][v], written back a chunk later; without a
    // vector gate the dS update takes -beta lambda (Gam) from Dn, else dv itself
    __shared__ __align__(16) TI Lb[C * LDV];
    __shared__ __align__(16) TI Db[C * LDV];
    __shared__ __align__(16) TI Dn[VEC ? 8 : C * LDV];

    const int DVr = p.DVr;
    const int rows = DVr + (SUMMARY ? DK : 0);
    const int nblk = rows / BV;
    int bh, sb;
    head_and_block(nblk * p.nseg, p.BH, bh, sb);
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
    GateRegs<GATE, C, DK> rg;
    // scalar gate: gam of the rows of this thread's dO vectors (dO e^{gam} is formed
    // from registers, so the commit needs no barrier between the gate and the tiles)
    float gdo[SCA ? RDO::PER : 1];
    auto prefetch = [&](int n) {
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
        rq.load(static_cast<const TI*>(p.q) + row0 * DK, DK, valid);
        rk.load(static_cast<const TI*>(p.k) + row0 * DK, DK, valid);
        rdo.load(static_cast<const TI*>(p.dout) + row0 * DVr + vcol, DVr, valid);
        if (trans) rdo.valid_ = 0;   // stores as zero
        rP.load(static_cast<const TI*>(p.Pm) + cc, C, C);
        rT.load(static_cast<const TI*>(p.Tm) + cc, C, C);
    };
    prefetch(n1 - 1);

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
        // these writes after its reads; only the vector gate's scaling below reads the
        // gate just committed)
        rg.commit(rowf, gam_s, beta_s);
        if constexpr (VEC) __syncthreads();
        const GateLds<GATE, C, DK> gf{rowf, gam_s, valid - 1};
        if (VEC) {
            // K e^{gam_C - gam}, -K e^{gam} and Q e^{gam} (one exp for the last two)
            rk.store3(rq, Kd, Kn, Qg, LDK, [&](int r, int c, float k, float q, float* y) {
                const float e = gf.G(r, c);
                y[0] = k * gf.Gd(r, c);
                y[1] = -k * e;
                y[2] = q * e;
            });
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
        if (!SUMMARY)
            lds_to_global<TI, BV, DK>(static_cast<TI*>(p.dS1) + (((long)bh * p.NT + n) * DVr + v0) * DK, DK, dSs,
                                      LDK, BV);
        // the next chunk's loads last and unconditional (see the forward state kernel)
        prefetch(n > n0 ? n - 1 : n0);

        // (c) dU = P^T dO + Kd dS1^T  -> dU^T   (P and dO read as [k][m] / [k][n])
        {
            f32x4 dU[TX::PER];
            zero_acc<C, BV>(dU);
            gemm<TI, C, BV, DK, false, false>(dU, Kd, LDK, dSs, LDK);
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
                for (int i = 0; i < 4; ++i) dS[j][i] *= gf.GC(TS::row(j, i));
            }
        }
        gemm<TI, DK, BV, C, true, true>(dS, Qg, LDK, SCA ? dOg : dOb, LDV);
        __syncthreads();
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

// ---------------------------------------------------------------------------
// bwd_chunk_kernel: grid (NT, BH); every chunk finished independently.
// D = d_k = d_v.  The d_v dimension is streamed in blocks of VB columns: the
// block's S0 rows, dS1 rows, lambda, dO and V columns are loaded into registers
// one block ahead and committed to LDS while the previous block computes
//     X_b = (K Gam) S0_b^T,  R_b = beta (V_b - X_b),  U_b = T R_b
//     dQg += dO_b S0_b,  dKg += lambda_b S0_b,  dKd += U_b dS1_b
//     dA  += lambda_b U_b^T,  dP += dO_b U_b^T
// after which the key-gradient products (phase C) finish dq, dk, dbeta, dg.
// Every LDS tile keeps its natural (global) layout; operands contracted over
// their leading index are read with the transposing LDS load.  The products are
// accumulated transposed where that gives a lane 4 consecutive elements of a
// row of the stored result (X^T, U^T, dq^T, dk^T, dA^T, dP^T), so results go
// to LDS with one vector store per tile.
template <typename TI, int GATE, int C, int D>
struct BwdChunkSmem {
    static constexpr int PAD = Pad<TI>::value;
    static constexpr int VB = D >= 32 ? 32 : D;   // d_v block
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
    static constexpr size_t TL = KG + al(C * LD * E);                // T              [C][LC]
    static constexpr size_t LOOP = TL + al(C * LC * E);
    // d_v loop: two buffers of one block's tiles (offsets within a buffer), so the
    // next block is committed while this one computes
    static constexpr size_t S0B = 0;                                 // S0 rows        [VB][LD]
    static constexpr size_t DS1B = S0B + al(VB * LD * E);            // dS1 rows       [VB][LD]
    static constexpr size_t LAMB = DS1B + al(VB * LD * E);           // lambda block   [C][LVB]
    static constexpr size_t DOB = LAMB + al(C * LVB * E);            // dO block       [C][LVB]
    static constexpr size_t VBL = DOB + al(C * LVB * E);             // V block, then U block [C][LVB]
    static constexpr size_t BLK = VBL + al(C * LVB * E);
    static constexpr size_t RB = LOOP + 2 * BLK;                     // R block        [C][LVB]
    static constexpr size_t LOOP_END = RB + al(C * LVB * E);
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
    static constexpr size_t RED_B = RED_G + al((D / 16) * C * 4);                 // [VB/16][C] row partials (dbeta_R)
    static constexpr size_t RED_C = RED_B + al((VB / 16) * C * 4);                // [C/16][D] column partials
    static constexpr size_t LASTS = RED_C + al((C / 16) * D * 4);                 // [D]
    static constexpr size_t KCO = LASTS + al(D * 4);                              // [C] Kaczmarz dk coefficients
    static constexpr size_t TOTAL = KCO + al(C * 4);
    // dq / dk write-back tiles [C][LD] each at offset 0; d gam of the vector gate
    // [C][LDG] fp32 after them, written once every phase-C tile is dead
    static constexpr size_t DGB = al(2 * C * LD * E);
    static constexpr int LDG = D + 4;   // d gam rows (fp32, padded: its accumulator stores stay conflict-free)
    static_assert(!VEC || DGB + C * LDG * 4 <= BIG_END, "d gam buffer");
    // per-thread partials of sum_v S0 dS1 [row blocks of the S0 register tile][LDS_] fp32,
    // beside the write-back tiles (and d gam)
    using RS = RegB<TI, VB, D>;
    static constexpr int LDS_ = D + 4;   // rows of the partials (padded: eight lanes store to eight rows)
    static constexpr size_t LSRED = VEC ? DGB + al(C * LDG * 4) : DGB;
    static_assert(LSRED + RS::BR * LDS_ * 4 <= BIG_END, "S0 dS1 partials");
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
    // tiles of block-buffer i (V and then U share a slot: V is dead once R is formed)
    auto blk = [&](int i, size_t off) { return reinterpret_cast<TI*>(smem + L::LOOP + i * L::BLK + off); };
    TI* RB = reinterpret_cast<TI*>(smem + L::RB);
    float* gam_s = reinterpret_cast<float*>(smem + L::GAM);
    float* rowf = reinterpret_cast<float*>(smem + L::ROWF);
    float* beta_s = reinterpret_cast<float*>(smem + L::BETA);
    float* red_r = reinterpret_cast<float*>(smem + L::RED_R);
    float* red_g = reinterpret_cast<float*>(smem + L::RED_G);
    float* red_b = reinterpret_cast<float*>(smem + L::RED_B);
    float* red_c = reinterpret_cast<float*>(smem + L::RED_C);
    float* lastS = reinterpret_cast<float*>(smem + L::LASTS);
    float* dgb = reinterpret_cast<float*>(smem + L::DGB);
    float* kco = reinterpret_cast<float*>(smem + L::KCO);

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

    using TO = Tiles<D, C>;    // dq^T, dk^T         [c][t]
    using TCC = Tiles<C, C>;   // dA^T, dP^T         [s][t]
    using TX = Tiles<VB, C>;   // X_b^T, U_b^T       [v][t]

    // ---------------- prologue: gate, K, T, the first d_v block
    GateRegs<GATE, C, D> rg;
    rg.load(p.gam + row0 * GW, p.beta + row0, valid);
    RegN<TI, C, D> rK;
    rK.load(k, D, valid);
    RegN<TI, C, C> rT;
    rT.load(static_cast<const TI*>(p.Tm) + chunk * C * C, C, C);
    // two register sets: the loads of block b + 2 are issued when block b is
    // committed, so two blocks of loads are in flight during the loop
    struct BlockRegs {
        RegB<TI, VB, D> S0, dS1;
        RegN<TI, C, VB> lam, dO, V;
    } rb[2];
    auto load_block = [&](BlockRegs& r, int b) {
        const int v0 = b * VB;
        r.S0.load(S0g + (long)v0 * D, D, VB);
        r.dS1.load(dS1g + (long)v0 * D, D, VB);
        r.lam.load(lamg + v0, D, C);
        r.dO.load(dO + v0, D, valid);
        r.V.load(v + v0, D, valid);
    };
    load_block(rb[0], 0);
    if (NVB > 1) load_block(rb[1], 1);
    // sum_v S0[v][c] dS1[v][c] over this thread's rows of every block
    float ls[L::RS::PER][L::RS::VW] = {};
    rg.commit(rowf, gam_s, beta_s, L::LDGM);
    __syncthreads();
    const GateLds<GATE, C, D, L::LDGM> gf{rowf, gam_s, valid - 1};
    if (VEC)
        rK.store(KG, LD, [&](int r, int c, float x) { return x * gf.G(r, c); });
    else
        rK.store(KG, LD);   // scalar: Gam_t is applied to X's rows
    rT.store(TLs, LC);
    auto commit_block = [&](BlockRegs& r, int i) {
        r.S0.dot_rows(r.dS1, ls);
        r.S0.store_n(blk(i, L::S0B), LD, Identity());
        r.dS1.store_n(blk(i, L::DS1B), LD, Identity());
        r.lam.store(blk(i, L::LAMB), LVB);
        r.dO.store(blk(i, L::DOB), LVB);
        r.V.store(blk(i, L::VBL), LVB);
    };
    commit_block(rb[0], 0);
    __syncthreads();
    if (NVB > 2) load_block(rb[0], 2);

    // ---------------- d_v loop
    f32x4 dq[TO::PER], dkp[TO::PER], dkm[TO::PER], dA[TCC::PER], dP[TCC::PER];
    zero_acc<D, C>(dq);
    zero_acc<D, C>(dkp);
    zero_acc<D, C>(dkm);
    zero_acc<C, C>(dA);
    zero_acc<C, C>(dP);
    float dbr_part[TX::PER] = {};   // sum over this lane's 4 v of lambda (V - X) at row t = TX::col(j)
    // q (and k for the vector gate) for the key-gradient products, loaded at the
    // start of the last d_v block (whose second register set is free by then; q
    // is not among the cache-warmed tiles, so it comes from far away)
    RegN<TI, C, D> rq, rk;
#pragma unroll
    for (int b = 0; b < NVB; ++b) {
        if (b == NVB - 1) {
            rq.load(q, D, valid);
            if (VEC) rk.load(k, D, valid);
        }
        TI* S0B = blk(b & 1, L::S0B);
        TI* DS1B = blk(b & 1, L::DS1B);
        TI* LAMB = blk(b & 1, L::LAMB);
        TI* DOB = blk(b & 1, L::DOB);
        TI* VBL = blk(b & 1, L::VBL);
        TI* UB = VBL;
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
                const f32x4 xr = ld4<TI>(VBL + t * LVB + c) - (SCA ? rowf[t] : 1.f) * X[j];
                const f32x4 lm = ld4<TI>(LAMB + t * LVB + c);
                dbr_part[j] += lm[0] * xr[0] + lm[1] * xr[1] + lm[2] * xr[2] + lm[3] * xr[3];
                rr[j] = beta_s[t] * xr;
            }
#pragma unroll
            for (int j = 0; j < TX::PER; ++j) st4<TI>(RB + TX::col(j) * LVB + TX::row(j, 0), rr[j]);
        }
        __syncthreads();
        // block b + 1 into the other buffer (free since block b - 1 ended), read after
        // the two barriers below
        if (b + 1 < NVB) {
            commit_block(rb[(b + 1) & 1], (b + 1) & 1);
            if (b + 3 < NVB) load_block(rb[(b + 1) & 1], b + 3);
        }
        // U_b^T = R_b^T T^T  (R rows read as [k][m])
        {
            f32x4 U[TX::PER];
            zero_acc<VB, C>(U);
            gemm<TI, VB, C, C, true, false>(U, RB, LVB, TLs, LC);
            if (TX::active()) {
#pragma unroll
                for (int j = 0; j < TX::PER; ++j) st4<TI>(UB + TX::col(j) * LVB + TX::row(j, 0), U[j]);
            }
        }
        __syncthreads();
        gemm<TI, D, C, VB, true, false>(dkm, DS1B, LD, UB, LVB);
        gemm2<TI, C, C, VB, false, false>(dA, dP, UB, LVB, LAMB, DOB, LVB);
        // no barrier here: the next writes into this buffer (the commit of block
        // b + 2) and into RB come after the next block's first barrier
    }


    // dq = Gam dQg ; dk+ = -beta Gam dKg ; dk- = Gd dKd   (element c = row, t = col)
    if (TO::active()) {
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
                    pp[j][i] = s2 <= t ? dP[j][i] * e : 0.f;
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
        // fp = e^{gam - centre} (vector gate; 1 otherwise), centre = gam_C / 2
        auto fpl = [&](int t, int c) -> float { return VEC ? fexp(gam_s[t * L::LDGM + c] - 0.5f * gl[c]) : 1.f; };
        auto fp4 = [&](int t, int c0) -> f32x4 {
            if constexpr (VEC) {
                const f32x4 g4 = ld4<float>(gam_s + t * L::LDGM + c0), c4 = ld4<float>(gl + c0);
                return f32x4{fexp(g4[0] - 0.5f * c4[0]), fexp(g4[1] - 0.5f * c4[1]), fexp(g4[2] - 0.5f * c4[2]),
                             fexp(g4[3] - 0.5f * c4[3])};
            } else {
                return f32x4{1.f, 1.f, 1.f, 1.f};
            }
        };
        if (VEC) {
            // K e^{c - gam}, K e^{gam - c}, Q e^{gam - c}: one exp per element
            rk.store3(rq, Kr, Kl, Ql, LD, [&](int r, int c, float k, float q, float* y) {
                const float e = fpl(r, c);
                y[0] = __fdividef(k, e);
                y[1] = k * e;
                y[2] = q * e;
            });
        } else {
            rq.store(Ql, LD);
        }
        __syncthreads();
        // Warm the caches for the workgroup that most likely starts next on this
        // XCD: workgroups start in id order and go to the XCDs round-robin, so it
        // is this id plus the number resident at once.  One dword of every
        // 128-byte line of its prologue tiles (K, T, the first two d_v blocks of
        // S0, dS1, lambda, dO and V, the gate and beta rows; up to 2 lines per
        // thread), held in registers and consumed only at the end, so nothing
        // waits for them.
        int warm[2];
        {
            const long ids = (long)gridDim.x * gridDim.y;
            const long nid = min((long)blockIdx.y * gridDim.x + blockIdx.x + p.resident, ids - 1);
            const int nbh = (int)(nid / gridDim.x), nn = (int)(nid - (long)nbh * gridDim.x);
            const int nvalid = min(C, p.T - nn * C);
            const long nrow0 = (long)nbh * p.T + (long)nn * C;
            const long nchunk = (long)nbh * p.NT + nn;
            constexpr int E = sizeof(TI), NB = NVB < 2 ? NVB : 2;
            constexpr int LPR = (NB * VB * E + 127) / 128;   // lines per row of the lambda / dO / V blocks
            const int nK = (nvalid * D * E + 127) / 128;
            constexpr int nT = (C * C * E + 127) / 128, nS = (NB * VB * D * E + 127) / 128;
            const int nG = (nvalid * GW * 4 + 127) / 128, nB = (nvalid * 4 + 127) / 128;   // gate and beta rows
            const int b1 = nK, b2 = b1 + nT, b3 = b2 + nS, b4 = b3 + nS, b5 = b4 + C * LPR, b6 = b5 + nvalid * LPR,
                      b7 = b6 + nvalid * LPR, b8 = b7 + (GATE != kGateNone ? nG : 0), nl = b8 + nB;
            const char* kb = reinterpret_cast<const char*>(static_cast<const TI*>(p.k) + nrow0 * D);
            const char* tb = reinterpret_cast<const char*>(static_cast<const TI*>(p.Tm) + nchunk * C * C);
            const char* sb = reinterpret_cast<const char*>(static_cast<const TI*>(p.states) + nchunk * D * D);
            const char* db = reinterpret_cast<const char*>(static_cast<const TI*>(p.dS1) + nchunk * D * D);
            const char* lb = reinterpret_cast<const char*>(static_cast<const TI*>(p.lam) + nchunk * C * D);
            const char* ob = reinterpret_cast<const char*>(static_cast<const TI*>(p.dout) + nrow0 * D);
            const char* vb = reinterpret_cast<const char*>(static_cast<const TI*>(p.v) + nrow0 * D);
            const char* gb = reinterpret_cast<const char*>(p.gam + nrow0 * GW);
            const char* bb = reinterpret_cast<const char*>(p.beta + nrow0);
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int i = min((int)threadIdx.x + r * kThreads, nl - 1);
                const int s = i < b4 ? 0 : (i < b5 ? 1 : (i < b6 ? 2 : (i < b7 ? 3 : 4)));
                const int j = i - (s == 0 ? 0 : (s == 1 ? b4 : (s == 2 ? b5 : b6)));
                // contiguous segments (K, T, S0, dS1, gate, beta) by line; row segments by
                // row and line
                const char* base = s == 1 ? lb : (s == 2 ? ob : vb);
                long off = (long)(j / LPR) * D * E + (j % LPR) * 128;
                if (s == 0) {
                    base = i < b1 ? kb : (i < b2 ? tb : (i < b3 ? sb : db));
                    off = (long)(i - (i < b1 ? 0 : (i < b2 ? b1 : (i < b3 ? b2 : b3)))) * 128;
                }
                if (s == 4) {
                    base = i < b8 ? gb : bb;
                    off = (long)(i - (i < b8 ? b7 : b8)) * 128;
                }
                warm[r] = *reinterpret_cast<const int*>(base + off);
            }
        }
        // k and q at this lane's elements (4 consecutive c of row t), read back from the
        // staged tiles; the gam_C column sums of Kd dKd (dk- holds only the Kd path so far)
        f32x4 kv[TO::PER], qv[TO::PER];
        if (TO::active()) {
#pragma unroll
            for (int j = 0; j < TO::PER; ++j) {
                const int t = TO::col(j), c0 = TO::row(j, 0);
                const f32x4 fp = fp4(t, c0);
                kv[j] = ld4<TI>(Kr + t * LD + c0) * fp;
                qv[j] = ld4<TI>(Ql + t * LD + c0) / fp;
            }
            // column sums over t (the 16 lanes of a tile row, the wave's RN tiles) per c
#pragma unroll
            for (int im = 0; im < TO::RM; ++im)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float colp = 0.f;
#pragma unroll
                    for (int in = 0; in < TO::RN; ++in)
                        colp += kv[im * TO::RN + in][i] * dkm[im * TO::RN + in][i];
                    colp = row16_sum(colp);
                    if ((lane_id() & 15) == 0) red_c[TO::cg() * D + TO::row(im * TO::RN, i)] = colp;
                }
        }
        float dbA[TO::PER];   // sum over this lane's 4 c of K+ Y at row t = TO::col(j)
        f32x4 tmp[TO::PER];
        // Y^T = Kr^T dA~^T :  dK+ = beta Y, dbeta_A = sum_c K+ Y
        zero_acc<D, C>(tmp);
        gemm<TI, D, C, C, true, false>(tmp, Kr, LD, DAs, LC);
        if (TO::active()) {
#pragma unroll
            for (int j = 0; j < TO::PER; ++j) {
                const int t = TO::col(j);
                const f32x4 fp = fp4(t, TO::row(j, 0));
                const f32x4 yf = tmp[j] * fp;
                const f32x4 d4 = kv[j] * yf;
                dbA[j] = d4[0] + d4[1] + d4[2] + d4[3];
                dkp[j] += beta_s[t] * yf;
            }
        }
        // Z^T = Kl^T (beta dA~) and W^T = Ql^T dP~ : both reach k through e^{-gam}
        zero_acc<D, C>(tmp);
        gemm<TI, D, C, C, true, true>(tmp, Kl, LD, DABs, LC);
        gemm<TI, D, C, C, true, true>(tmp, Ql, LD, DPs, LC);
        if (TO::active()) {
#pragma unroll
            for (int j = 0; j < TO::PER; ++j) dkm[j] += tmp[j] / fp4(TO::col(j), TO::row(j, 0));
        }
        // dQ+^T = Kr^T dP~^T
        zero_acc<D, C>(tmp);
        gemm<TI, D, C, C, true, false>(tmp, Kr, LD, DPs, LC);
        if (TO::active()) {
#pragma unroll
            for (int j = 0; j < TO::PER; ++j) dq[j] += tmp[j] * fp4(TO::col(j), TO::row(j, 0));
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
                dgm[j] = qv[j] * dq[j] + kv[j] * (dkp[j] - dkm[j]);
            }
            // row partials over c (4 per lane, 4 lane groups, RM tiles) of K+ Y (dbeta)
            // and, for the scalar gate, of d gam
#pragma unroll
            for (int in = 0; in < TO::RN; ++in) {
                float sb = 0.f, sg = 0.f;
#pragma unroll
                for (int im = 0; im < TO::RM; ++im) {
                    sb += dbA[im * TO::RN + in];
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
        // dbeta_R row partials over v (X^T tiles: 4 v per lane, 4 lane groups)
        if (TX::active()) {
#pragma unroll
            for (int j = 0; j < TX::PER; ++j) {
                const float sr = sum_lane_groups(dbr_part[j]);
                if (lane_id() < 16) red_b[(TX::m0(j) / 16) * C + TX::col(j)] = sr;
            }
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
            for (int b = 0; b < VB / 16; ++b) s2 += red_b[b * C + t];
            for (int b = 0; b < TO::WM; ++b) s2 += red_r[b * C + t];
            if (kz) {
                const float rn = p.krn[row0 + t];
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
                    st4<TI>(dks + t * LD + TO::row(j, 0), dkt[j] + (t < valid ? kco[t] : 0.f) * kv[j]);
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
                // d gam: elementwise terms + the gam_C terms on the last valid row
                if (TO::active()) {
#pragma unroll
                    for (int j = 0; j < TO::PER; ++j) st4<float>(dgb + TO::col(j) * L::LDG + TO::row(j, 0), dgm[j]);
                }
                __syncthreads();
                // d gam_t = sum_{s >= t} per channel, in NSG segments of RSG rows (one
                // thread each: the suffix sums of its rows), then the totals of the
                // later segments (through red_c, dead since lastS was formed)
                constexpr int NSG = kThreads / D < C / 16 ? kThreads / D : C / 16;
                constexpr int RSG = C / NSG;
                static_assert(NSG >= 1 && NSG * D <= kThreads && C % NSG == 0, "segments");
                const int c = threadIdx.x % D, sg = threadIdx.x / D;
                float sfx[RSG];
                if (sg < NSG) {
                    const float last = lastS[c];
                    float acc = 0.f;
#pragma unroll
                    for (int r = RSG - 1; r >= 0; --r) {
                        const int t = sg * RSG + r;
                        acc += t < valid ? dgb[t * L::LDG + c] + (t == valid - 1 ? last : 0.f) : 0.f;
                        sfx[r] = acc;
                    }
                    red_c[sg * D + c] = acc;
                }
                __syncthreads();
                if (sg < NSG) {
                    float off = 0.f;
                    for (int s2 = sg + 1; s2 < NSG; ++s2) off += red_c[s2 * D + c];
#pragma unroll
                    for (int r = 0; r < RSG; ++r) {
                        const int t = sg * RSG + r;
                        if (t < valid) p.dg[(row0 + t) * D + c] = sfx[r] + off;
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
