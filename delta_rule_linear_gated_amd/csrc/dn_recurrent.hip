// dn_recurrent.hip -- the recurrent (token-by-token) form of the operator: T
// steps of
//     S_t = S_{t-1} Diag(exp(g_t)) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t
// with the fp32 state updated in place (the decode workload; the recurrent form
// of the Fast Weight Attention abstract, the KLA abstract's decode setting).
//
// Phase-controlled gate (SFDA summary, "Kernarchitektur" and its real
// implementation, real inputs): the state is complex, S = A + i B, the gate of
// key channel c is exp(g) exp(i theta), i.e. a 2 x 2 rotation-decay of the pair
// (A[:, c], B[:, c]); the erase with k acts on A and B, the write of v on A, and
// the output is Re(S q) = A q.  theta = 0 with B = 0 is the plain recurrence.
//
// Rows of S are independent (row v only mixes with itself through the keys), so
// a workgroup takes 16 rows of one head: a wave holds 4 rows, 16 lanes per row,
// E = DK / 16 consecutive keys per lane, and both row sums of a step (S k and
// S q) are DPP reductions over the 16 lanes.  The state is read once and written
// once per call; the per-step inputs of step t + 1 are loaded during step t.
#include "dn_device.h"
#include "dn_internal.h"

namespace dn {

namespace {

constexpr int kRecThreads = 256;
constexpr int kRecRows = 16;   // state rows per workgroup: 4 waves x 4 rows

template <typename TI, int GATE, int DK, bool PHASE> struct StepIn {
    static constexpr int E = DK / 16;
    float k[E], q[E], a[GATE == kGateVector ? E : 1], th[PHASE ? E : 1];
    float v = 0.f, beta = 0.f;
    __device__ __forceinline__ void load(const Params& p, long tok, int v_row, int c0) {
        const TI* kp = static_cast<const TI*>(p.k) + tok * DK + c0;
        const TI* qp = static_cast<const TI*>(p.q) + tok * DK + c0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            k[e] = to_f(kp[e]);
            q[e] = to_f(qp[e]);
        }
        v = to_f(static_cast<const TI*>(p.v)[tok * p.DVr + v_row]);
        beta = p.kz ? p.eta[tok] : p.beta[tok];
        if (GATE == kGateScalar) a[0] = p.g[tok];
        if (GATE == kGateVector) {
#pragma unroll
            for (int e = 0; e < E; ++e) a[e] = p.g[tok * DK + c0 + e];
        }
        if (PHASE) {
#pragma unroll
            for (int e = 0; e < E; ++e) th[e] = p.theta[tok * DK + c0 + e];
        }
    }
};

template <typename TI, int GATE, int DK, bool PHASE>
__global__ __launch_bounds__(kRecThreads) void recurrent_kernel(Params p) {
    constexpr int E = DK / 16;
    const int DV = p.DVr;
    const int nblk = DV / kRecRows;
    const int bh = blockIdx.x / nblk, blk = blockIdx.x - (blockIdx.x / nblk) * nblk;
    const int lane = lane_id(), w = wave_id();
    const int j = lane & 15;
    const int v = blk * kRecRows + w * 4 + (lane >> 4);   // this lane's state row
    const int c0 = j * E;                                 // its first key
    float* srow = p.hT + ((long)bh * DV + v) * DK + c0;
    float s[E];
#pragma unroll
    for (int e = 0; e < E; e += 4) {
        if constexpr (E >= 4) {
            const f32x4 x = ld4<float>(srow + e);
            s[e] = x[0], s[e + 1] = x[1], s[e + 2] = x[2], s[e + 3] = x[3];
        }
    }
    if constexpr (E < 4) {
#pragma unroll
        for (int e = 0; e < E; ++e) s[e] = srow[e];
    }
    // imaginary part of the state rows (phase-controlled gate only)
    float* irow = PHASE ? p.hT_im + ((long)bh * DV + v) * DK + c0 : nullptr;
    float sb[PHASE ? E : 1];
    if constexpr (PHASE) {
#pragma unroll
        for (int e = 0; e < E; ++e) sb[e] = irow[e];
    }
    StepIn<TI, GATE, DK, PHASE> cur, nxt;
    const long tok0 = (long)bh * p.T;
    if (p.T > 0) cur.load(p, tok0, v, c0);
    for (int t = 0; t < p.T; ++t) {
        nxt.load(p, tok0 + (t + 1 < p.T ? t + 1 : t), v, c0);   // next step's inputs (in bounds)
        // decay (with the phase: rotation-decay), then the erase / write of the
        // delta rule, then the read-out
        if constexpr (PHASE) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float m = GATE == kGateScalar ? fexp(cur.a[0]) : (GATE == kGateVector ? fexp(cur.a[e]) : 1.f);
                float sn, cs;
                sincosf(cur.th[e], &sn, &cs);
                const float ar = s[e], ai = sb[e];
                s[e] = m * (cs * ar - sn * ai);
                sb[e] = m * (sn * ar + cs * ai);
            }
        } else if (GATE == kGateScalar) {
            const float a = fexp(cur.a[0]);
#pragma unroll
            for (int e = 0; e < E; ++e) s[e] *= a;
        } else if (GATE == kGateVector) {
#pragma unroll
            for (int e = 0; e < E; ++e) s[e] *= fexp(cur.a[e]);
        }
        float pk = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) pk += s[e] * cur.k[e];
        pk = row16_sum(pk);
        float pkb = 0.f;   // imaginary part of S k
        if constexpr (PHASE) {
#pragma unroll
            for (int e = 0; e < E; ++e) pkb += sb[e] * cur.k[e];
            pkb = row16_sum(pkb);
        }
        float beta = cur.beta;
        if (p.kz) {   // Kaczmarz step (KLA abstract): beta_t = eta_t / (||k_t||^2 + eps)
            float kk = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) kk += cur.k[e] * cur.k[e];
            beta /= row16_sum(kk) + p.eps;
        }
        const float u = beta * (cur.v - pk);
        float oq = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            s[e] += u * cur.k[e];
            oq += s[e] * cur.q[e];
        }
        if constexpr (PHASE) {   // the imaginary part is only erased
            const float w = -beta * pkb;
#pragma unroll
            for (int e = 0; e < E; ++e) sb[e] += w * cur.k[e];
        }
        oq = row16_sum(oq);
        if (j == 0) static_cast<TI*>(p.o)[(tok0 + t) * DV + v] = from_f<TI>(oq);
        cur = nxt;
    }
    if constexpr (E >= 4) {
#pragma unroll
        for (int e = 0; e < E; e += 4) st4<float>(srow + e, s[e], s[e + 1], s[e + 2], s[e + 3]);
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) srow[e] = s[e];
    }
    if constexpr (PHASE) {
#pragma unroll
        for (int e = 0; e < E; ++e) irow[e] = sb[e];
    }
}

template <typename TI, int GATE, int DK> hipError_t launch_rec(const Problem& pr, const Params& p, hipStream_t s) {
    const long blocks = (long)pr.B * pr.H * (pr.dv / kRecRows);
    if (p.theta)
        hipLaunchKernelGGL((recurrent_kernel<TI, GATE, DK, true>), dim3((unsigned)blocks), dim3(kRecThreads), 0, s, p);
    else
        hipLaunchKernelGGL((recurrent_kernel<TI, GATE, DK, false>), dim3((unsigned)blocks), dim3(kRecThreads), 0, s, p);
    return hipGetLastError();
}

template <typename TI, int GATE> hipError_t rec_dk(const Problem& pr, const Params& p, hipStream_t s) {
    switch (pr.dk) {
        case 16: return launch_rec<TI, GATE, 16>(pr, p, s);
        case 32: return launch_rec<TI, GATE, 32>(pr, p, s);
        case 64: return launch_rec<TI, GATE, 64>(pr, p, s);
        case 128: return launch_rec<TI, GATE, 128>(pr, p, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename TI> hipError_t rec_gate(const Problem& pr, const Params& p, hipStream_t s) {
    switch (pr.gate) {
        case kGateNone: return rec_dk<TI, kGateNone>(pr, p, s);
        case kGateScalar: return rec_dk<TI, kGateScalar>(pr, p, s);
        case kGateVector: return rec_dk<TI, kGateVector>(pr, p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_recurrent(const Problem& pr, const Params& p, hipStream_t stream) {
    if ((long)pr.B * pr.H * pr.dv == 0 || pr.T == 0) return hipSuccess;
    prof_begin(stream, p.theta ? "recurrent_phase" : "recurrent");
    const hipError_t e = pr.bf16 ? rec_gate<bf16>(pr, p, stream) : rec_gate<float>(pr, p, stream);
    prof_end(stream);
    return e;
}

}  // namespace dn
