// dn_launch.hip -- workspace carving, support table and the launch sequences;
// the kernels themselves are instantiated in the per-variant units.
#include "dn_launch.h"

namespace dn {

namespace {

__global__ void copy_state_kernel(const float* __restrict__ src, float* __restrict__ dst, long n) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

hipError_t copy_state(const float* src, float* dst, long n, hipStream_t stream) {
    if (!dst || n == 0) return hipSuccess;
    const int blocks = (int)((n + 255) / 256);
    hipLaunchKernelGGL(copy_state_kernel, dim3(blocks), dim3(256), 0, stream, src, dst, n);
    return hipGetLastError();
}

// Combine of the chunk-parallel scan (exact affine chunk transfer, SFDA
// summary): the boundary states of the segments, in fp32, from the segment
// summaries E_s (rows < DV of p.seg_end: the pass over segment s from a zero
// state, the first -- forward -- or last -- backward -- segment from h0 / dhT)
// and the transition matrices M_s (rows >= DV: P_s forward, P_s^T backward):
//     c = E_first;  for each later segment s in walking order:
//         seg_start[s] = c;  c = c M_s + E_s
// Forward, seg_start[s] is the state entering segment s; backward, the dS
// leaving it.  One workgroup per 16 rows of one head: c as MFMA accumulator
// tiles, M_s staged in LDS; the next step's M and E rows are in flight in
// registers while a product runs.
template <int DK>
__global__ __launch_bounds__(kThreads) void scan_combine_kernel(Params p, int forward) {
    constexpr int LDM = DK + Pad<float>::value;
    using TO = Tiles<16, DK>;   // the 16 x DK rows of c, as MFMA accumulator tiles
    constexpr int NV4 = DK * DK / 4, PER4 = (NV4 + kThreads - 1) / kThreads;
    __shared__ __align__(16) float Ms[DK * LDM];
    __shared__ __align__(16) float cr[16 * LDM];
    const int DV = p.DVr, G = p.nseg, rows = DV + DK;
    const int nrb = DV / 16;
    const int bh = blockIdx.x / nrb, rb = blockIdx.x - (blockIdx.x / nrb) * nrb;
    const float* E = p.seg_end + (long)bh * G * rows * DK;
    float* out = p.seg_start + (long)bh * G * DV * DK;
    auto seg_at = [&](int s) { return forward ? s : G - 1 - s; };
    // rows rb*16 .. rb*16+15 of segment g's summary, at this lane's accumulator positions
    auto load_rows = [&](int g, f32x4 (&x)[TO::PER]) {
        const float* e = E + ((long)g * rows + rb * 16) * DK;
#pragma unroll
        for (int j = 0; j < TO::PER; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[j][i] = TO::active() ? e[TO::row(j, i) * DK + TO::col(j)] : 0.f;
    };
    // segment g's transition matrix (rows DV .. DV + DK - 1 of its summary) into registers
    // (a plain float array: an array of float4 structs is not kept in registers)
    auto load_m = [&](int g, float (&mr)[PER4 * 4]) {
        const float4* m = reinterpret_cast<const float4*>(E + ((long)g * rows + DV) * DK);
#pragma unroll
        for (int i = 0; i < PER4; ++i) {
            const int idx = threadIdx.x + i * kThreads;
            const float4 x = m[idx < NV4 ? idx : NV4 - 1];
            mr[4 * i] = x.x;
            mr[4 * i + 1] = x.y;
            mr[4 * i + 2] = x.z;
            mr[4 * i + 3] = x.w;
        }
    };
    f32x4 c[TO::PER], er[TO::PER];
    float mr[PER4 * 4];
    load_rows(seg_at(0), c);
    if (G > 2) {   // the first inner step's M and E rows
        load_m(seg_at(1), mr);
        load_rows(seg_at(1), er);
    }
    for (int s = 1; s < G; ++s) {
        const int g = seg_at(s);
        if (TO::active()) {
            float* o = out + ((long)g * DV + rb * 16) * DK;
#pragma unroll
            for (int j = 0; j < TO::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[TO::row(j, i) * DK + TO::col(j)] = c[j][i];
        }
        if (s == G - 1) break;
        __syncthreads();   // the previous product's LDS reads are done
#pragma unroll
        for (int i = 0; i < PER4; ++i) {
            const int idx = threadIdx.x + i * kThreads;
            if (idx < NV4) {
                const int r = idx / (DK / 4), c4 = idx - r * (DK / 4);
                *reinterpret_cast<float4*>(Ms + r * LDM + 4 * c4) =
                    float4{mr[4 * i], mr[4 * i + 1], mr[4 * i + 2], mr[4 * i + 3]};
            }
        }
        if (TO::active()) {
#pragma unroll
            for (int j = 0; j < TO::PER; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) cr[TO::row(j, i) * LDM + TO::col(j)] = c[j][i];
        }
        __syncthreads();
        f32x4 e[TO::PER];
#pragma unroll
        for (int j = 0; j < TO::PER; ++j) e[j] = er[j];
        {   // the next step's M and E rows, in flight during this product (unconditional:
            // the last inner step reloads its own)
            const int gn = seg_at(s + 1 < G - 1 ? s + 1 : s);
            load_m(gn, mr);
            load_rows(gn, er);
        }
        f32x4 acc[TO::PER];
#pragma unroll
        for (int j = 0; j < TO::PER; ++j) acc[j] = zero4();
        gemm<float, 16, DK, DK, false, true>(acc, cr, LDM, Ms, LDM);   // c M_g + E_g (fp32 MFMA)
#pragma unroll
        for (int j = 0; j < TO::PER; ++j) c[j] = acc[j] + e[j];
    }
}

}  // namespace

hipError_t launch_scan_combine(const Params& p, int DK, bool forward, hipStream_t stream) {
    const dim3 grid((unsigned)(p.BH * (p.DVr / 16))), block(kThreads);
    prof_begin(stream, "scan_combine");
    switch (DK) {
        case 16: hipLaunchKernelGGL(scan_combine_kernel<16>, grid, block, 0, stream, p, forward ? 1 : 0); break;
        case 32: hipLaunchKernelGGL(scan_combine_kernel<32>, grid, block, 0, stream, p, forward ? 1 : 0); break;
        case 64: hipLaunchKernelGGL(scan_combine_kernel<64>, grid, block, 0, stream, p, forward ? 1 : 0); break;
        case 128: hipLaunchKernelGGL(scan_combine_kernel<128>, grid, block, 0, stream, p, forward ? 1 : 0); break;
        default: prof_end(stream); return hipErrorInvalidValue;
    }
    prof_end(stream);
    return hipGetLastError();
}

namespace {

const LaunchFn kFwd[2][3] = {{launch_fwd_f32_g0, launch_fwd_f32_g1, launch_fwd_f32_g2},
                             {launch_fwd_bf16_g0, launch_fwd_bf16_g1, launch_fwd_bf16_g2}};
const LaunchFn kBwd[2][3] = {{launch_bwd_f32_g0, launch_bwd_f32_g1, launch_bwd_f32_g2},
                             {launch_bwd_bf16_g0, launch_bwd_bf16_g1, launch_bwd_bf16_g2}};

}  // namespace

bool supported(const Problem& pr) {
    if (pr.dk != pr.dv) return false;
    DN_DISPATCH(fits_rt)
    return false;
}

// The scan pays when the sequential kernels' grid at their narrowest d_v block
// (16 rows) covers less than half of the device's 256 compute units: then each
// chain is cut into about 2 * 256 / grid segments (at most 32, at least 4
// chunks each), so that every unit runs two chains.  Sequences of fewer than 32
// chunks, where the three extra launches per pass cost more than they save, stay
// sequential.  Fixed numbers, not the current device's, so that workspace sizes
// depend on the shape alone.
ScanPlan scan_plan(const Problem& pr) {
    // two workgroups of the narrow-block state kernels fit on a compute unit: aim
    // for two chains per unit
    constexpr long kUnits = 256, kSegFill = 2, kMaxSeg = 32, kMinLen = 4;
    const long NT = pr.T > 0 ? ((long)pr.T + pr.C - 1) / pr.C : 0;
    const long grid = (long)(pr.dv / 16 > 0 ? pr.dv / 16 : 1) * pr.B * pr.H;
    ScanPlan sp{1, (int)NT};
    if (pr.no_scan || NT < 8 * kMinLen || grid <= 0 || 2 * grid >= kUnits) return sp;
    long g = kSegFill * kUnits / grid;
    if (g > kMaxSeg) g = kMaxSeg;
    if (g > NT / kMinLen) g = NT / kMinLen;
    if (g < 2) return sp;
    const long len = (NT + g - 1) / g;
    sp.seg_len = (int)len;
    sp.nseg = (int)((NT + len - 1) / len);
    return sp;
}

namespace {
struct Sizes {
    size_t gam, cc, lam, st, kz, seg_end, seg_start;
};
Sizes sizes(const Problem& pr) {
    const size_t E = pr.bf16 ? 2 : 4;
    const size_t BH = (size_t)pr.B * pr.H;
    const size_t NT = pr.T > 0 ? ((size_t)pr.T + pr.C - 1) / pr.C : 0;
    const size_t gw = pr.gate == kGateVector ? (size_t)pr.dk : 1;
    Sizes z;
    z.gam = al256(pr.gate == kGateNone ? 0 : BH * pr.T * gw * 4);
    z.cc = al256(BH * NT * pr.C * pr.C * E);
    z.lam = al256(BH * NT * pr.C * pr.dv * E);
    z.st = al256(BH * NT * (size_t)pr.dv * pr.dk * E);
    z.kz = pr.kz ? al256(2 * BH * pr.T * 4) : 0;
    const ScanPlan sp = scan_plan(pr);
    const size_t G = sp.nseg > 1 ? (size_t)sp.nseg : 0;
    z.seg_end = al256(BH * G * (size_t)(pr.dv + pr.dk) * pr.dk * 4);
    z.seg_start = al256(BH * G * (size_t)pr.dv * pr.dk * 4);
    return z;
}
}  // namespace

WsLayout ws_layout(const Problem& pr, int pass) {
    const Sizes z = sizes(pr);
    const bool chunk_data = pass != 1;   // forward, or a backward that recomputes
    WsLayout w{};
    size_t off = 0;
    w.gam = off;
    if (chunk_data) off += z.gam;
    w.Tm = off;
    if (chunk_data) off += z.cc;
    w.Pm = off;
    if (chunk_data) off += z.cc;
    w.lam = off;
    if (pass != 0) off += z.lam;
    w.dS1 = off;
    if (pass != 0) off += z.st;
    w.states = off;
    if (pass == 2) off += z.st;
    w.kz = off;
    if (chunk_data) off += z.kz;
    w.seg_end = off;   // scan buffers (every pass; the recomputing backward reuses them)
    off += z.seg_end;
    w.seg_start = off;
    off += z.seg_start;
    w.total = off;
    return w;
}

SavedLayout saved_layout(const Problem& pr) {
    const Sizes z = sizes(pr);
    SavedLayout l{};
    l.states = 0;
    l.Tm = z.st;
    l.Pm = l.Tm + z.cc;
    l.Um = l.Pm + z.cc;
    l.gam = l.Um + z.lam;
    l.kz = l.gam + z.gam;
    l.total = l.kz + z.kz;
    return l;
}

hipError_t launch_forward(const Problem& pr, const Params& p, bool save_states, hipStream_t stream) {
    if (pr.B * pr.H == 0) return hipSuccess;
    if (pr.T == 0) return copy_state(p.h0, p.hT, (long)pr.B * pr.H * pr.dv * pr.dk, stream);
    if (pr.gate < 0 || pr.gate > 2) return hipErrorInvalidValue;
    return kFwd[pr.bf16 ? 1 : 0][pr.gate](pr, p, save_states, stream);
}

hipError_t launch_backward(const Problem& pr, const Params& p, bool have_states, hipStream_t stream) {
    if (pr.B * pr.H == 0) return hipSuccess;
    if (pr.T == 0) return copy_state(p.dhT, p.dh0, (long)pr.B * pr.H * pr.dv * pr.dk, stream);
    if (pr.gate < 0 || pr.gate > 2) return hipErrorInvalidValue;
    return kBwd[pr.bf16 ? 1 : 0][pr.gate](pr, p, have_states, stream);
}

}  // namespace dn
