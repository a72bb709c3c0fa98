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
// (KDA: per-channel decays; the C x C products split each pair's decay at a
// per-channel reference, the gate at the last row of a 16-row block, so that
// no factor exceeds the decay of 16 steps -- the centred contraction of the
// ReWY abstract, centred per 16-row block).
#pragma once

#include <type_traits>

#include "dn_device.h"
#include "dn_internal.h"

namespace dn {

template <int GATE, int DK> struct GateLayout {
    static constexpr int GW = GATE == kGateVector ? DK : 1;  // gam values per step
};

// ---------------------------------------------------------------------------
// 16 x 16 fp32 block product on the matrix cores, row-major operands:
//     acc += A[16][16] * B[16][16]
// (v_mfma_f32_16x16x4_f32: lane l holds A[l & 15][k0 + (l >> 4)] and
// B[k0 + (l >> 4)][l & 15]; the result is D[4 (l >> 4) + i][l & 15].)
__device__ __forceinline__ f32x4 mm16_nn(const float* A, int lda, const float* B, int ldb, f32x4 acc) {
    const int l = lane_id();
#pragma unroll
    for (int k0 = 0; k0 < 16; k0 += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[(l & 15) * lda + k0 + (l >> 4)], B[(k0 + (l >> 4)) * ldb + (l & 15)],
                                                   acc, 0, 0, 0);
    return acc;
}

// T = (I + A)^{-1} for a strictly lower C x C matrix A (fp32 in LDS, row
// stride ld), written to Ts (fp32, row stride ld).  With 16 x 16 blocks:
//   diagonal blocks  T_bb = (I + A_bb)^{-1}: forward substitution, all blocks at
//                    once on wave 0 (lane = block * 16 + column);
//   off-diagonal     T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj, filled by distance
//                    i - j = 1, 2, ...; one wave per block, fp32 MFMA;
//   above the block diagonal T is zero.
// Ysc is per-wave scratch for one 16 x 16 fp32 block.  Ends with a barrier.
template <int C>
__device__ __forceinline__ void unit_lower_inverse(const float* A, float* Ts, int ld, float* Ysc) {
    constexpr int NBK = C / 16;
    // zero the strictly-upper blocks
    for (int idx = threadIdx.x; idx < C * C; idx += kThreads) {
        const int r = idx / C, c = idx % C;
        if ((c >> 4) > (r >> 4)) Ts[r * ld + c] = 0.f;
    }
    if (wave_id() == 0) {
        const int l = lane_id(), b = l >> 4, c = l & 15;
        if (b < NBK) {
            const float* Ab = A + (16 * b) * ld + 16 * b;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = (i == c) ? 1.f : 0.f;
            // right-looking: once x_j is final, remove its contribution from the rows below
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                float a[16];
#pragma unroll
                for (int i = jj + 1; i < 16; ++i) a[i] = Ab[i * ld + jj];
#pragma unroll
                for (int i = jj + 1; i < 16; ++i) x[i] -= a[i] * x[jj];
            }
            float* Tb = Ts + (16 * b) * ld + 16 * b;
#pragma unroll
            for (int i = 0; i < 16; ++i) Tb[i * ld + c] = x[i];
        }
    }
    __syncthreads();
#pragma unroll
    for (int dist = 1; dist < NBK; ++dist) {
        const int jb = wave_id();
        if (jb < NBK - dist) {
            const int ib = jb + dist;
            float* Y = Ysc + wave_id() * 256;
            f32x4 y = zero4();
            for (int kb = jb; kb < ib; ++kb)
                y = mm16_nn(A + (16 * ib) * ld + 16 * kb, ld, Ts + (16 * kb) * ld + 16 * jb, ld, y);
            const int l = lane_id();
#pragma unroll
            for (int i = 0; i < 4; ++i) Y[(4 * (l >> 4) + i) * 16 + (l & 15)] = y[i];
            // (the same wave reads Y back: LDS operations of one wave complete in order)
            f32x4 t = zero4();
            t = mm16_nn(Ts + (16 * ib) * ld + 16 * ib, ld, Y, 16, t);
            float* Tij = Ts + (16 * ib) * ld + 16 * jb;
#pragma unroll
            for (int i = 0; i < 4; ++i) Tij[(4 * (l >> 4) + i) * ld + (l & 15)] = -t[i];
        }
        __syncthreads();
    }
}

// LDS carving of prep_kernel.  R0 holds the staged K / Q tiles until the Gram
// products are done, then the fp32 inverse, its block scratch and the P tile.
template <typename TI, int GATE, int C, int DK> struct PrepSmem {
    static constexpr bool VEC = GATE == kGateVector;
    static constexpr int LDK = DK + Pad<TI>::value;
    static constexpr int LDA = C + 4;                   // fp32 C x C rows
    static constexpr int LC = C + Pad<TI>::value;       // I/O-type C x C rows
    static constexpr int GW = GateLayout<GATE, DK>::GW;
    // vector gate: gam rows padded to DK + 8 floats, so that 16 rows read 16 bytes
    // each at one column hit distinct banks
    static constexpr int LDG = VEC ? DK + 8 : 1;
    static constexpr size_t al(size_t x) { return (x + 255) & ~size_t(255); }
    // K and Q as loaded
    static constexpr size_t KP = 0;
    static constexpr size_t KM = KP + al(C * LDK * sizeof(TI));
    static constexpr size_t QP = KM;
    static constexpr size_t R0_END = KM + al(C * LDK * sizeof(TI));
    static constexpr size_t TS = 0;                     // fp32 [C][LDA]
    static constexpr size_t YSC = TS + al(C * LDA * 4); // fp32 [C/16][256]
    static constexpr size_t PS = YSC + al((C / 16) * 256 * 4);   // TI [C][LC]
    static constexpr size_t R0B_END = PS + al(C * LC * sizeof(TI));
    static constexpr size_t R0 = R0_END > R0B_END ? R0_END : R0B_END;
    static constexpr size_t AS = R0;                    // fp32 [C][LDA]
    // gam [C][GW] fp32 ([C][LDG] for the vector gate, whose gam shares A's
    // space: it is dead once the Gram products are done, before A is written),
    // so that two workgroups fit per CU
    static constexpr size_t GAM = VEC ? AS : AS + al(C * LDA * 4);
    static constexpr size_t GAM_END =
        VEC ? AS + al(C * LDA * 4 > C * LDG * 4 ? C * LDA * 4 : C * LDG * 4) : GAM + al(C * GW * 4);
    static constexpr size_t BETA = GAM_END;
    // vector gate: segment totals of the per-channel cumsum [NSEG][DK] fp32, in
    // the K tiles' space (dead before K is staged)
    static constexpr int NSEG = (kThreads / DK) < C ? (kThreads / DK) : C;
    static constexpr size_t TOT = KP;
    static_assert(!VEC || NSEG * DK * 4 <= R0_END, "cumsum totals");
    static constexpr size_t TOTAL = BETA + al(C * 4);
};

// Gram products of the per-channel gate (KDA) for the wave's tiles of the C x C
// output:
//     acc  (t, s) = sum_c k_tc k_sc e^{gam_tc - gam_sc}
//     accp (t, s) = sum_c q_tc k_sc e^{gam_tc - gam_sc}
// over the lower tiles (row block i >= column block j; the caller masks).  The
// decay of a pair is split at a per-channel reference, rho_j = gam at the last
// row of the column block: the column operand is k_s e^{rho_j - gam_s} and the
// row operands k_t e^{gam_t - rho_j}, q_t e^{gam_t - rho_j}, both formed in
// registers from the loaded tiles.  For g <= 0 both factors are at most 1 below
// the diagonal blocks; on a diagonal block the row factor grows at most by the
// decay of the block's 16 rows (the centred contraction of the ReWY abstract,
// centred per 16-row block instead of per chunk, so its range is set by 16
// steps, not C).  K, Q: [C][ldk] as loaded; gam_s: [C][LDG] fp32.
template <typename TI, int C, int DK, int LDG, int NACC>
__device__ __forceinline__ void vec_gram(f32x4 (&acc)[NACC], f32x4 (&accp)[NACC], const TI* K, const TI* Q,
                                         int ldk, const float* gam_s) {
    using TL = Tiles<C, C>;
    using MM = typename MmaFor<TI, DK>::type;
    using FF = FragF<TI, MM::kStep>;
    constexpr int NE = FF::NE;
    static_assert(TL::RN == 1, "one column block per wave");
    if (!TL::active()) return;
    const int s0 = TL::n0(0);                     // the wave's column block
    const float* rho = gam_s + (s0 + 15) * LDG;   // its last row
#pragma unroll
    for (int k0 = 0; k0 < DK; k0 += MM::kStep) {
        float r[NE], gs[NE];
        FF::load_f(rho + k0, 0, r);   // row rho at this lane's columns
        FF::load_f(gam_s + s0 * LDG + k0, LDG, gs);
        FF b;
        b.load(K + s0 * ldk + k0, ldk);
#pragma unroll
        for (int e = 0; e < NE; ++e) b.x[e] *= fexp(r[e] - gs[e]);
        const typename MM::Frag fb = b.pack();
#pragma unroll
        for (int j = 0; j < NACC; ++j) {
            const int t0 = TL::m0(j);
            if (s0 > t0) continue;   // strictly upper tile: zero
            float gt[NE];
            FF::load_f(gam_s + t0 * LDG + k0, LDG, gt);
            FF a, q;
            a.load(K + t0 * ldk + k0, ldk);
            q.load(Q + t0 * ldk + k0, ldk);
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                const float f = fexp(gt[e] - r[e]);
                a.x[e] *= f;
                q.x[e] *= f;
            }
            acc[j] = MM::op(a.pack(), fb, acc[j]);
            accp[j] = MM::op(q.pack(), fb, accp[j]);
        }
    }
}

// ---------------------------------------------------------------------------
// prep_kernel: grid (NT, BH), one chunk per workgroup: gam, P and T of the
// chunk (T and P row-major; the reverse pass transposes them while staging).
// Waves per SIMD prep_kernel is compiled for: three workgroups per compute unit
// (registers capped at 80) where three fit in LDS, not below d = 64, where the
// cap would spill (C = 64, bf16); with the vector gate two (128) where two fit;
// else the default two waves.
template <typename TI, int GATE, int C, int DK> constexpr int prep_waves() {
    constexpr size_t T = PrepSmem<TI, GATE, C, DK>::TOTAL;
    if (DK >= 64 && 3 * T <= 160 * 1024) return 3 * kWaves / 4;
    if (GATE == kGateVector && 2 * T <= 160 * 1024) return 2 * kWaves / 4;
    return kWaves / 4;
}

template <typename TI, int GATE, int C, int DK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(prep_waves<TI, GATE, C, DK>())))
void prep_kernel(Params p) {
    using L = PrepSmem<TI, GATE, C, DK>;
    constexpr int LDK = L::LDK, LDA = L::LDA, LC = L::LC;
    constexpr bool VEC = L::VEC;
    __shared__ __align__(16) char smem[L::TOTAL];
    TI* Kp = reinterpret_cast<TI*>(smem + L::KP);   // K
    TI* Qp = reinterpret_cast<TI*>(smem + L::QP);   // Q
    float* Ts = reinterpret_cast<float*>(smem + L::TS);
    float* Ysc = reinterpret_cast<float*>(smem + L::YSC);
    TI* Ps = reinterpret_cast<TI*>(smem + L::PS);
    float* A_s = reinterpret_cast<float*>(smem + L::AS);
    float* gam_s = reinterpret_cast<float*>(smem + L::GAM);
    float* beta_s = reinterpret_cast<float*>(smem + L::BETA);

    const int n = blockIdx.x, bh = blockIdx.y;
    const int t0 = n * C;
    const int valid = min(C, p.T - t0);
    const long row0 = (long)bh * p.T + t0;
    const TI* __restrict__ q = static_cast<const TI*>(p.q) + row0 * DK;
    const TI* __restrict__ k = static_cast<const TI*>(p.k) + row0 * DK;
    const float* __restrict__ beta = p.beta + row0;
    // the chunk's gate and beta first (lane t, every wave, branch-free): the scan
    // below waits for them, the K / Q tiles are needed only after it
    const int tl = min(lane_id(), valid - 1);
    const float g_in = GATE == kGateScalar ? p.g[row0 + tl] : 0.f;
    const float b_in = beta[tl];
    // vector gate: the RS rows of one channel this thread's cumsum segment covers
    // (see below), also loaded ahead of the K / Q tiles
    constexpr int RSV = VEC ? C / L::NSEG : 1;
    float gx[RSV];
    if constexpr (VEC) {
        const int c = threadIdx.x % DK, seg = min((int)threadIdx.x / DK, L::NSEG - 1);
#pragma unroll
        for (int r = 0; r < RSV; ++r) gx[r] = p.g[(row0 + min(seg * RSV + r, valid - 1)) * DK + c];
    }
    RegN<TI, C, DK> rq, rk;
    // Kaczmarz step: eta of the rows whose key norms this thread finishes (below);
    // branch-free, from beta (a valid array) when there is no Kaczmarz step
    float eta_in[RegN<TI, C, DK>::PER];
    const float* __restrict__ eta = (p.kz ? p.eta : p.beta) + row0;
#pragma unroll
    for (int i = 0; i < RegN<TI, C, DK>::PER; ++i)
        eta_in[i] = eta[min(RegN<TI, C, DK>::idx_of(i) / RegN<TI, C, DK>::VPR, valid - 1)];
    rq.load(q, DK, valid);
    rk.load(k, DK, valid);

    // -- cumulative log-decay within the chunk
    if (GATE == kGateScalar) {
        if (wave_id() == 0) {
            const int t = lane_id();
            float x = t < valid ? g_in : 0.f;
            // inclusive prefix sum over the 64 lanes: within each row of 16 lanes by
            // DPP row shifts (lane i adds lane i - n of its row, 0 before the row
            // start), then the totals of the earlier rows
            x += dpp_f<0x111>(x);
            x += dpp_f<0x112>(x);
            x += dpp_f<0x114>(x);
            x += dpp_f<0x118>(x);
            const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 15));
            const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 31));
            const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 47));
            const int row = t >> 4;
            x += (row > 0 ? r0 : 0.f) + (row > 1 ? r1 : 0.f) + (row > 2 ? r2 : 0.f);
            if (t < C) {
                gam_s[t] = x;
                if (t < valid) p.gam[row0 + t] = x;
            }
        }
    } else if constexpr (GATE == kGateVector) {
        // per-channel cumsum in two levels: NSEG segments of RS rows per channel, one
        // thread each (its RS rows, loaded above, and a local prefix sum), then the
        // totals of the earlier segments
        constexpr int NSEG = L::NSEG, RS = C / NSEG;
        float* tot = reinterpret_cast<float*>(smem + L::TOT);
        const int c = threadIdx.x % DK, seg = threadIdx.x / DK;
        float x[RS];
        static_assert(RS == RSV, "segment rows");
        if (seg < NSEG) {
#pragma unroll
            for (int r = 0; r < RS; ++r) x[r] = seg * RS + r < valid ? gx[r] : 0.f;
#pragma unroll
            for (int r = 1; r < RS; ++r) x[r] += x[r - 1];
            tot[seg * DK + c] = x[RS - 1];
        }
        __syncthreads();
        if (seg < NSEG) {
            float off = 0.f;
            for (int s2 = 0; s2 < seg; ++s2) off += tot[s2 * DK + c];
#pragma unroll
            for (int r = 0; r < RS; ++r) {
                const int t = seg * RS + r;
                const float y = x[r] + off;
                gam_s[t * L::LDG + c] = y;
                if (t < valid) p.gam[(row0 + t) * DK + c] = y;
            }
        }
    }
    if (p.kz) {
        // Kaczmarz step (KLA abstract): beta_t = eta_t / (||k_t||^2 + eps) from the
        // key rows in registers; a row's vectors sit in one aligned group of VPR lanes
        using RK = RegN<TI, C, DK>;
#pragma unroll
        for (int i = 0; i < RK::PER; ++i) {
            const uint4 ri = rk.r[i];
            const TI* src = reinterpret_cast<const TI*>(&ri);
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < RK::VW; ++e) {
                const float x = to_f(src[e]);
                ss += x * x;
            }
            ss = group_sum<RK::VPR>(ss);
            const int idx = threadIdx.x + i * kThreads, row = idx / RK::VPR;
            if (idx < RK::NV && idx % RK::VPR == 0) {
                const float rn = 1.f / (ss + p.eps);
                const float b = row < valid ? eta_in[i] * rn : 0.f;
                beta_s[row] = b;
                if (row < valid) {
                    p.kb[row0 + row] = b;
                    p.krn[row0 + row] = rn;
                }
            }
        }
    } else {
        if ((int)threadIdx.x < C) beta_s[threadIdx.x] = (int)threadIdx.x < valid ? b_in : 0.f;
    }
    __syncthreads();

    // -- stage K and Q as loaded (the per-channel gate scales the operand
    //    fragments in registers, below)
    rk.store(Kp, LDK);
    rq.store(Qp, LDK);
    __syncthreads();

    // -- gated Gram matrices: A (strict lower, scaled by beta_t) and P (lower)
    {
        using TL = Tiles<C, C>;
        f32x4 acc[TL::PER], accp[TL::PER];
#pragma unroll
        for (int j = 0; j < TL::PER; ++j) {
            acc[j] = zero4();
            accp[j] = zero4();
        }
        if constexpr (!VEC) {
#pragma unroll
            for (int j = 0; j < TL::PER; ++j) {
                if (!TL::valid(j) || TL::n0(j) > TL::m0(j)) continue;   // strictly upper tiles are zero
                acc[j] = tile_nt<TI, DK>(Kp + TL::m0(j) * LDK, LDK, Kp + TL::n0(j) * LDK, LDK, acc[j]);
                accp[j] = tile_nt<TI, DK>(Qp + TL::m0(j) * LDK, LDK, Kp + TL::n0(j) * LDK, LDK, accp[j]);
            }
        } else {
            vec_gram<TI, C, DK, L::LDG>(acc, accp, Kp, Qp, LDK, gam_s);
        }
        // gate factors and masks (LDS reads only)
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
        }
        __syncthreads();   // K / Q tiles dead: R0 becomes the inverse's and P's space
        if (TL::active()) {
#pragma unroll
            for (int j = 0; j < TL::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = TL::row(j, i), s = TL::col(j);
                    A_s[t * LDA + s] = acc[j][i];
                    Ps[t * LC + s] = from_f<TI>(accp[j][i]);
                }
        }
    }
    __syncthreads();
    const long cc = ((long)bh * p.NT + n) * C * C;
    lds_to_global<TI, C, C>(static_cast<TI*>(p.Pm) + cc, C, Ps, LC, C);

    // Per-channel gate: warm the caches for the workgroup that most likely starts
    // next on this XCD (workgroups start in id order and go to the XCDs
    // round-robin: this id plus the number resident at once): one dword of every
    // 128-byte line of its K, Q, gate and beta rows, while this one's inverse
    // runs, consumed only at the end. With a scalar gate or none the three
    // workgroups resident per CU already hide the loads and warming costs time.
    int warm[2] = {0, 0};
    if constexpr (GATE == kGateVector) {
        const long ids = (long)gridDim.x * gridDim.y;
        const long nid = min((long)blockIdx.y * gridDim.x + blockIdx.x + p.resident, ids - 1);
        const int nbh = (int)(nid / gridDim.x), nn = (int)(nid - (long)nbh * gridDim.x);
        const int nvalid = min(C, p.T - nn * C);
        const long nrow0 = (long)nbh * p.T + (long)nn * C;
        constexpr int E = sizeof(TI);
        const int nK = (nvalid * DK * E + 127) / 128, nG = (nvalid * DK * 4 + 127) / 128;
        const int b1 = nK, b2 = b1 + nK, b3 = b2 + nG, nl = b3 + (nvalid * 4 + 127) / 128;
        const char* kb = reinterpret_cast<const char*>(static_cast<const TI*>(p.k) + nrow0 * DK);
        const char* qb = reinterpret_cast<const char*>(static_cast<const TI*>(p.q) + nrow0 * DK);
        const char* gb = reinterpret_cast<const char*>(p.g + nrow0 * DK);
        const char* bb = reinterpret_cast<const char*>((p.kz ? p.eta : p.beta) + nrow0);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int i = min((int)threadIdx.x + r * kThreads, nl - 1);
            const char* base = i < b1 ? kb : (i < b2 ? qb : (i < b3 ? gb : bb));
            const long off = (long)(i - (i < b1 ? 0 : (i < b2 ? b1 : (i < b3 ? b2 : b3)))) * 128;
            warm[r] = *reinterpret_cast<const int*>(base + off);
        }
    }

    // -- T = (I + A)^{-1}
    unit_lower_inverse<C>(A_s, Ts, LDA, Ysc);

    // -- T to global memory, 16 bytes per store
    {
        constexpr int VW = 16 / sizeof(TI), VPR = C / VW, NV = C * VPR;
        TI* __restrict__ Tout = static_cast<TI*>(p.Tm) + cc;
        for (int idx = threadIdx.x; idx < NV; idx += kThreads) {
            const int r = idx / VPR, c0 = (idx % VPR) * VW;
            TI out[VW];
#pragma unroll
            for (int e = 0; e < VW; ++e) out[e] = from_f<TI>(Ts[r * LDA + c0 + e]);
            *reinterpret_cast<uint4*>(Tout + r * C + c0) = *reinterpret_cast<const uint4*>(out);
        }
    }
    asm volatile("" ::"v"(warm[0]), "v"(warm[1]));   // the warming loads' only use
}

// ---------------------------------------------------------------------------
// Per-chunk gate data held in registers between prefetch and commit, and the
// decay factors it leaves in LDS:
//   scalar gate: rowf[t] = e^{gam_t}, rowf[C + t] = e^{gam_C - gam_t}, gam_s[t]
//   vector gate: gam_s[t][c] (factors computed per element from it)
// VT = false leaves the vector gate's tile out (the state kernels hold it in a
// VecGate instead, see below).
template <int GATE, int C, int DK, bool VT = true> struct GateRegs {
    static constexpr bool VEC = GATE == kGateVector && VT;
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
        __builtin_amdgcn_sched_barrier(0);   // fixed issue order (see RegN)
        if (GATE == kGateScalar) {
            gs = gam[tt];
            __builtin_amdgcn_sched_barrier(0);
            gC = gam[valid - 1];
            __builtin_amdgcn_sched_barrier(0);
        }
        if (VEC) gv.load_clamped(gam, DK, valid);
    }
    // ldg: row stride of gam_s (vector gate)
    __device__ __forceinline__ void commit(float* rowf, float* gam_s, float* beta_s, int ldg = DK) const {
        const int t = threadIdx.x;
        if (t < C) beta_s[t] = t < valid_ ? b : 0.f;
        if (GATE == kGateScalar && t < C) {
            rowf[t] = fexp(gs);
            rowf[C + t] = fexp(gC - gs);
            gam_s[t] = gs;
        }
        if (VEC) gv.store(gam_s, ldg);
    }
};

// Per-channel gate of one chunk in registers, laid out like the elements of a
// RegN<TI, C, DK> tile (a K or Q tile): g[i][e] is gam at element e of the
// thread's vector i of that tile (row clamped into the chunk like the tile's
// own loads), gc[e] gam_C at the same columns.  A thread's vectors all start at
// the same column (kThreads is a multiple of the vectors per row), so one set
// of gam_C values serves all of them; for the vectors past the tile's end (not
// stored) the values are in-bounds duplicates.  The scaled tiles are then formed
// straight from registers: no gate tile in LDS, no barrier between the gate and
// the tiles.
template <typename TI, int C, int DK> struct VecGate {
    using RT = RegN<TI, C, DK>;
    static constexpr int VW = RT::VW, VPR = RT::VPR, PER = RT::PER;
    static_assert(VW % 4 == 0 && kThreads % VPR == 0, "gate vectors");
    float g[PER][VW];
    float gc[VW];
    __device__ __forceinline__ static int col0() { return ((int)threadIdx.x % VPR) * VW; }
    __device__ __forceinline__ void load(const float* __restrict__ gam, int valid) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = RT::idx_of(i);
            const int row = min(idx / VPR, valid - 1), c0 = (idx % VPR) * VW;
#pragma unroll
            for (int v = 0; v < VW / 4; ++v) {
                const float4 x = *reinterpret_cast<const float4*>(gam + (long)row * DK + c0 + 4 * v);
                g[i][4 * v] = x.x;
                g[i][4 * v + 1] = x.y;
                g[i][4 * v + 2] = x.z;
                g[i][4 * v + 3] = x.w;
                __builtin_amdgcn_sched_barrier(0);   // fixed issue order (see RegN)
            }
        }
#pragma unroll
        for (int v = 0; v < VW / 4; ++v) {
            const float4 x = *reinterpret_cast<const float4*>(gam + (long)(valid - 1) * DK + col0() + 4 * v);
            gc[4 * v] = x.x;
            gc[4 * v + 1] = x.y;
            gc[4 * v + 2] = x.z;
            gc[4 * v + 3] = x.w;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
};

// Decay factors read back from LDS after GateRegs::commit.
template <int GATE, int C, int DK, int LDG = DK> struct GateLds {   // LDG: row stride of gam_s (vector gate)
    const float* rowf;
    const float* gam_s;
    int last;                  // valid - 1
    const float* gl = nullptr; // vector gate: a copy of row `last` of gam_s, if gam_s is reused
    // e^{gam[t][c]}
    __device__ __forceinline__ float G(int t, int c) const {
        if (GATE == kGateNone) return 1.f;
        if (GATE == kGateScalar) return rowf[t];
        return fexp(gam_s[t * LDG + c]);
    }
    // e^{gam_C[c] - gam[t][c]}
    __device__ __forceinline__ float Gd(int t, int c) const {
        if (GATE == kGateNone) return 1.f;
        if (GATE == kGateScalar) return rowf[C + t];
        return fexp(gam_s[last * LDG + c] - gam_s[t * LDG + c]);
    }
    // e^{gam_C[c]}
    __device__ __forceinline__ float GC(int c) const {
        if (GATE == kGateNone) return 1.f;
        if (GATE == kGateScalar) return rowf[last];
        return fexp(gl ? gl[c] : gam_s[last * LDG + c]);
    }
};

// ---------------------------------------------------------------------------
// fwd_state_kernel: grid (rows / BV) * nseg * BH.  Walks the chunks of one
// segment of one head in order for one block of BV state rows (rows of S are
// independent: each row only mixes with itself through the key dimension).  The
// global tiles of chunk n + 1 are loaded into registers while chunk n is
// computed.
//   SAVE    : write the state entering each chunk (I/O type) to p.states (with
//             OUTPUT also U = T R of each chunk to p.Um)
//   OUTPUT  : write O and hT.  Off for the recompute pass of the backward (P is
//             not needed there).
//   neither : segment summary of the chunk-parallel scan (exact affine chunk
//             transfer, SFDA summary): the segment's rows of S from a zero state
//             (the first segment from h0), plus DK rows that start as the
//             identity and see V = 0, so that they end as the segment's
//             transition matrix P_s (S_end = S_start P_s + S_end|zero start);
//             the end states go to p.seg_end.
// With segments (p.nseg > 1) and SAVE or OUTPUT, a segment starts from the
// boundary state the combine left in p.seg_start (the first from h0).
// Static LDS of fwd_state_kernel (bytes), mirrored from its declarations.
template <typename TI, int GATE, int C, int DK, int BV> constexpr size_t fwd_state_lds() {
    constexpr size_t E = sizeof(TI);
    constexpr int P = Pad<TI>::value, LDK = DK + P, LDC = C + P, LDV = BV + P;
    constexpr int G = GATE == kGateVector ? C + DK : C;   // gam (+ e^{gam_C} per channel)
    constexpr int NK = GATE == kGateVector ? 3 : 2;   // Q, K (+ K Gam_C / Gam); an upper bound without output
    constexpr int NV = GATE == kGateScalar ? 3 : 2;   // V (then U), R (+ U Gam_C / Gam)
    return 4 * (G + 3 * C) + E * (BV * LDK + NK * C * LDK + NV * C * LDV + 2 * C * LDC) + 96;
}

// LDS arrays of the forward state pass.  The kernel declares them one by one;
// a launch that runs another pass in its other workgroups overlays both passes'
// arrays in a union of these structs.
template <typename TI, int GATE, int C, int DK, int BV, bool OUTPUT> struct FwdStateArrays {
    static constexpr int PAD = Pad<TI>::value, LDK = DK + PAD, LDC = C + PAD, LDV = BV + PAD;
    static constexpr bool VEC = GATE == kGateVector, SCA = GATE == kGateScalar;
    float gam_s[C];
    __align__(16) float egc[VEC ? DK : 4];   // e^{gam_C} per channel (vector gate)
    float rowf[2 * C];
    __align__(16) float beta_s[C];
    __align__(16) TI Ss[BV * LDK];    // S0 (operand copy) [v][c]
    __align__(16) TI Qg[OUTPUT ? C * LDK : 8];   // Q (vector gate: Q Gam)  [t][c]
    __align__(16) TI Kg[C * LDK];     // K (vector gate: K Gam)            [t][c]
    __align__(16) TI Kd[VEC ? C * LDK : 8];   // K Gam_C / Gam (vector gate) [t][c]
    __align__(16) TI Vb[C * LDV];     // V block [t][v]; after (c) U [t][v]
    __align__(16) TI Tl[C * LDC];     // T                 [t][s]
    __align__(16) TI Pl[OUTPUT ? C * LDC : 8];   // P (only with the output)  [t][s]
    // R [t][v]; after (d) it holds the chunk's O [t][v] until the next iteration writes it back
    __align__(16) TI Rb[C * LDV];
    __align__(16) TI Ud[SCA ? C * LDV : 8];   // U Gam_C / Gam (scalar gate) [t][v]
};

// The pass for workgroup `wg` of its grid.  Each LDS array arrives as a restrict
// pointer, so after inlining the compiler knows they do not overlap.
template <typename TI, int GATE, int C, int DK, int BV, bool SAVE, bool OUTPUT>
__device__ __forceinline__ void fwd_state_body(const Params& p, int wg, float* __restrict__ gam_s,
                                               float* __restrict__ egc, float* __restrict__ rowf,
                                               float* __restrict__ beta_s, TI* __restrict__ Ss,
                                               TI* __restrict__ Qg, TI* __restrict__ Kg, TI* __restrict__ Kd,
                                               TI* __restrict__ Vb, TI* __restrict__ Tl, TI* __restrict__ Pl,
                                               TI* __restrict__ Rb, TI* __restrict__ Ud) {
    constexpr int PAD = Pad<TI>::value;
    constexpr int LDK = DK + PAD;
    constexpr int LDC = C + PAD;
    constexpr int LDV = BV + PAD;
    constexpr int GW = GateLayout<GATE, DK>::GW;
    constexpr bool VEC = GATE == kGateVector;
    constexpr bool SCA = GATE == kGateScalar;
    // Every tile in its natural layout; operands contracted over their leading
    // index are read with the transposing LDS load.  A scalar gate is a row
    // scaling, so Q and K stay unscaled (staged once) and the decays are applied
    // to the C x BV results instead: e^{gam_t} to X and to the Q S0^T part of O,
    // e^{gam_C - gam_t} to a second copy of U that feeds the state update.  The
    // per-channel vector gate scales Q and K per element, from gate values held
    // in registers in the layout of the K / Q register tiles (VecGate).
    TI* const Ub = Vb;                           // V is dead once R is formed

    constexpr bool SUMMARY = !SAVE && !OUTPUT;
    const int DVr = p.DVr;
    const int rows = DVr + (SUMMARY ? DK : 0);
    const int nblk = rows / BV;
    int bh, sb;
    head_and_block(nblk * p.nseg, p.BH, bh, sb, wg);
    const int seg = sb / nblk, vblk = sb - seg * nblk;
    const int v0 = vblk * BV;
    const bool trans = SUMMARY && v0 >= DVr;   // rows of the transition matrix
    // only the inner segments' transitions enter the combine
    if (trans && (seg == 0 || seg == p.nseg - 1)) return;
    const int n0 = seg * p.seg_len, n1 = min(p.NT, n0 + p.seg_len);
    // the state is held transposed, S^T [c][v] tiles: a lane's 4 values are 4
    // consecutive keys c of one row v of S (one vector store into S0's [v][c] copy)
    using TS = Tiles<DK, BV>;
    f32x4 S[TS::PER];
    const float* init = seg == 0 ? (trans ? nullptr : (p.h0 ? p.h0 + (long)bh * DVr * DK : nullptr))
                                 : (SUMMARY ? nullptr : p.seg_start + ((long)bh * p.nseg + seg) * DVr * DK);
#pragma unroll
    for (int j = 0; j < TS::PER; ++j) {
        S[j] = zero4();
        if (init && TS::active()) S[j] = ld4<float>(init + (long)(v0 + TS::col(j)) * DK + TS::row(j, 0));
        if (trans && TS::active()) {
#pragma unroll
            for (int i = 0; i < 4; ++i) S[j][i] = TS::row(j, i) == v0 - DVr + TS::col(j) ? 1.f : 0.f;
        }
    }
    const int vcol = trans ? 0 : v0;   // (transition rows load a valid V block and zero it)

    // registers of the next chunk
    RegN<TI, C, DK> rq, rk;
    RegN<TI, C, BV> rv;
    RegN<TI, C, C> rT;
    RegN<TI, OUTPUT ? C : 16, OUTPUT ? C : 16> rP;
    GateRegs<GATE, C, DK, false> rg;
    VecGate<TI, C, DK> vg;   // vector gate
    // Vector gate: the chunk's gated tiles K Gam, Q Gam, K Gam_C / Gam and e^{gam_C}
    // are formed in registers at the end of the previous iteration (beside its
    // matrix-core work, the exponentials off the commit's path), from K, Q and the
    // gate loaded one chunk before that; the commit only stores them.
    using VG = VecGate<TI, C, DK>;
    RegN<TI, C, VEC ? DK : 8> pkg, pqg, pkd;
    float pec[VEC ? VG::VW : 1];
    auto prefetch_kq = [&](int n) {   // vector gate: K, Q and the gate of chunk n
        if constexpr (VEC) {
            const int t0 = n * C;
            const int valid = min(C, p.T - t0);
            const long row0 = (long)bh * p.T + t0;
            vg.load(p.gam + row0 * GW, valid);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (OUTPUT) rq.load(static_cast<const TI*>(p.q) + row0 * DK, DK, valid);
            rk.load(static_cast<const TI*>(p.k) + row0 * DK, DK, valid);
        }
    };
    auto form = [&]() {   // vector gate: the tiles of the chunk in rq / rk / vg
        if constexpr (VEC) {
            if constexpr (OUTPUT) {
                rq.form3i(rk, pqg, pkg, pkd, [&](int i, int e, float q, float k, float* y) {
                    const float ge = vg.g[i][e];
                    const float f = fexp(ge);
                    y[0] = q * f;
                    y[1] = k * f;
                    y[2] = k * fexp(vg.gc[e] - ge);
                });
            } else {
                rk.form2i(pkg, pkd, [&](int i, int e, float k, float* y) {
                    const float ge = vg.g[i][e];
                    y[0] = k * fexp(ge);
                    y[1] = k * fexp(vg.gc[e] - ge);
                });
            }
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
        __builtin_amdgcn_sched_barrier(0);   // gate first, then the tiles, in order (see RegN)
        if constexpr (!VEC) {
            if constexpr (OUTPUT) rq.load(static_cast<const TI*>(p.q) + row0 * DK, DK, valid);   // Q only feeds O
            rk.load(static_cast<const TI*>(p.k) + row0 * DK, DK, valid);
        }
        rv.load(static_cast<const TI*>(p.v) + row0 * DVr + vcol, DVr, valid);
        if (trans) rv.valid_ = 0;   // stores as zero
        rT.load(static_cast<const TI*>(p.Tm) + cc, C, C);
        if constexpr (OUTPUT) rP.load(static_cast<const TI*>(p.Pm) + cc, C, C);
    };
    prefetch_kq(n0);
    prefetch(n0);
    form();
    prefetch_kq(n0 + 1 < n1 ? n0 + 1 : n0);

    // X^T, U^T and O^T tiles [v][t]: a lane holds 4 consecutive v of one row t of
    // R, U and O (one vector LDS access each)
    using TX = Tiles<BV, C>;
    for (int n = n0; n < n1; ++n) {
        const int t0 = n * C;
        const int valid = min(C, p.T - t0);
        const long row0 = (long)bh * p.T + t0;
        // (a) state operand (saved from LDS below)
        if (TS::active()) {
#pragma unroll
            for (int j = 0; j < TS::PER; ++j) st4<TI>(Ss + TS::col(j) * LDK + TS::row(j, 0), S[j]);
        }
        // (b) commit this chunk's tiles to LDS (the barrier ending the previous
        // chunk ordered these writes after its reads; nothing below reads the gate
        // just committed before the next barrier)
        rg.commit(rowf, gam_s, beta_s);
        const GateLds<GATE, C, DK> gf{rowf, gam_s, valid - 1};
        if constexpr (VEC) {   // the tiles formed last iteration (Q e^{gam}, K e^{gam}, K e^{gam_C - gam})
            if ((int)threadIdx.x < VG::VPR) {
#pragma unroll
                for (int e = 0; e < VG::VW; ++e) egc[VG::col0() + e] = pec[e];
            }
            if constexpr (OUTPUT) pqg.store(Qg, LDK);
            pkg.store(Kg, LDK);
            pkd.store(Kd, LDK);
        } else {
            if constexpr (OUTPUT) rq.store(Qg, LDK);
            rk.store(Kg, LDK);
        }
        rv.store(Vb, LDV);
        rT.store(Tl, LDC);
        if constexpr (OUTPUT) rP.store(Pl, LDC);
        // the previous chunk's O (in Rb until (c) below overwrites it)
        if (OUTPUT && n > n0)
            lds_to_global<TI, C, BV>(static_cast<TI*>(p.o) + (row0 - C) * DVr + v0, DVr, Rb, LDV, C);
        __syncthreads();
        // the state entering the chunk (Ss is not written again before the next
        // chunk); the per-channel gate's after (d) instead, beside U (its forward
        // pass 1 % faster, the scalar gate's 1 % slower)
        if (SAVE && !VEC)
            lds_to_global<TI, BV, DK>(static_cast<TI*>(p.states) + (((long)bh * p.NT + n) * DVr + v0) * DK, DK, Ss,
                                      LDK, BV);
        // The next chunk's loads come after the stores issued so far and
        // unconditionally (the last chunk reloads itself): the wait counts at the loop
        // head are merged over the first entry (the loads alone) and the back edge,
        // and with the loads behind the stores there they stay close to exact instead
        // of waiting for every outstanding load and store (the saves of U, and with
        // the per-channel gate of the state, come later in the chunk: measured).
        prefetch(n + 1 < n1 ? n + 1 : n);

        // (c) X^T = S0 (K Gam)^T ;  R = diag(beta) (V - X); with the output, the
        //     S0 (Q Gam)^T part of O^T in the same pass over S0's fragments
        f32x4 OT[TX::PER];
        zero_acc<BV, C>(OT);
        {
            f32x4 X[TX::PER];
            zero_acc<BV, C>(X);
            if constexpr (OUTPUT)
                gemm2<TI, BV, C, DK, false, false>(X, OT, Ss, LDK, Kg, Qg, LDK);
            else
                gemm<TI, BV, C, DK, false, false>(X, Ss, LDK, Kg, LDK);
            if (TX::active()) {
                f32x4 r[TX::PER];   // all LDS reads, then all LDS writes (see RegN::store)
#pragma unroll
                for (int j = 0; j < TX::PER; ++j) {
                    const int t = TX::col(j), c = TX::row(j, 0);
                    r[j] = beta_s[t] * (ld4<TI>(Vb + t * LDV + c) - (SCA ? rowf[t] : 1.f) * X[j]);
                }
#pragma unroll
                for (int j = 0; j < TX::PER; ++j) st4<TI>(Rb + TX::col(j) * LDV + TX::row(j, 0), r[j]);
            }
        }
        __syncthreads();
        // (d) U^T = R^T T^T  (R read as [k][m])
        {
            f32x4 U[TX::PER];
            zero_acc<BV, C>(U);
            gemm<TI, BV, C, C, true, false>(U, Rb, LDV, Tl, LDC);
            if (TX::active()) {
#pragma unroll
                for (int j = 0; j < TX::PER; ++j) {
                    const int t = TX::col(j), off = t * LDV + TX::row(j, 0);
                    st4<TI>(Ub + off, U[j]);
                    if (SCA) st4<TI>(Ud + off, rowf[C + t] * U[j]);
                }
            }
        }
        __syncthreads();
        // U of this chunk (all C rows: rows past the sequence are zero), beside the
        // products that read it; saved by the forward proper only (the backward's
        // recomputing pass leaves U to the chunk backward)
        if (SAVE && OUTPUT)
            lds_to_global<TI, C, BV>(static_cast<TI*>(p.Um) + ((long)bh * p.NT + n) * C * DVr + v0, DVr, Ub, LDV, C);
        if (SAVE && VEC)
            lds_to_global<TI, BV, DK>(static_cast<TI*>(p.states) + (((long)bh * p.NT + n) * DVr + v0) * DK, DK, Ss,
                                      LDK, BV);
        // (e) O^T = S0 (Q Gam)^T (from (c)) + U^T P^T   (O into Rb, dead since (d); written back
        //     next iteration)
        if (OUTPUT) {
            if (SCA && TX::active()) {
#pragma unroll
                for (int j = 0; j < TX::PER; ++j) OT[j] *= rowf[TX::col(j)];
            }
            gemm<TI, BV, C, C, true, false>(OT, Ub, LDV, Pl, LDC);
            if (TX::active()) {
#pragma unroll
                for (int j = 0; j < TX::PER; ++j) st4<TI>(Rb + TX::col(j) * LDV + TX::row(j, 0), OT[j]);
            }
        }
        // (f) S1^T = Diag(Gam_C) S0^T + (K Gam_C / Gam)^T U   (both read as [k][m] / [k][n])
        if (GATE != kGateNone && TS::active()) {
#pragma unroll
            for (int j = 0; j < TS::PER; ++j) {
#pragma unroll
                for (int i = 0; i < 4; ++i) S[j][i] *= VEC ? egc[TS::row(j, i)] : gf.GC(TS::row(j, i));
            }
        }
        gemm<TI, DK, BV, C, true, true>(S, VEC ? Kd : Kg, LDK, SCA ? Ud : Ub, LDV);
        if constexpr (VEC) {   // the next chunk's tiles, then the inputs of the one after
            form();
            prefetch_kq(n + 2 < n1 ? n + 2 : n1 - 1);
        }
        __syncthreads();
    }
    if (OUTPUT && n1 > n0) {
        const int t0 = (n1 - 1) * C;
        lds_to_global<TI, C, BV>(static_cast<TI*>(p.o) + ((long)bh * p.T + t0) * DVr + v0, DVr, Rb, LDV,
                                 min(C, p.T - t0));
    }
    if (OUTPUT && p.hT && n1 == p.NT && TS::active()) {
#pragma unroll
        for (int j = 0; j < TS::PER; ++j)
            st4<float>(p.hT + ((long)bh * DVr + v0 + TS::col(j)) * DK + TS::row(j, 0), S[j]);
    }
    if (SUMMARY && TS::active()) {
        float* out = p.seg_end + ((long)bh * p.nseg + seg) * rows * DK;
#pragma unroll
        for (int j = 0; j < TS::PER; ++j) st4<float>(out + (long)(v0 + TS::col(j)) * DK + TS::row(j, 0), S[j]);
    }
}

template <typename TI, int GATE, int C, int DK, int BV, bool SAVE, bool OUTPUT>
__global__ __launch_bounds__(kThreads) void fwd_state_kernel(Params p) {
    __shared__ FwdStateArrays<TI, GATE, C, DK, BV, OUTPUT> a;
    fwd_state_body<TI, GATE, C, DK, BV, SAVE, OUTPUT>(p, blockIdx.x, a.gam_s, a.egc, a.rowf, a.beta_s, a.Ss, a.Qg,
                                                      a.Kg, a.Kd, a.Vb, a.Tl, a.Pl, a.Rb, a.Ud);
}

}  // namespace dn
