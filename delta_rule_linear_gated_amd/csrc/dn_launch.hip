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

namespace {
struct Sizes {
    size_t gam, cc, lam, st, kz;
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
    w.total = off;
    return w;
}

SavedLayout saved_layout(const Problem& pr) {
    const Sizes z = sizes(pr);
    SavedLayout l{};
    l.states = 0;
    l.Tm = z.st;
    l.Pm = l.Tm + z.cc;
    l.gam = l.Pm + z.cc;
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
