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

int pick_bv(const Problem& pr) { return pr.dv < 64 ? pr.dv : 64; }

bool supported(const Problem& pr) {
    if (pr.dk != pr.dv) return false;
    DN_DISPATCH(fits_rt)
    return false;
}

WsLayout ws_layout(const Problem& pr, bool backward, bool need_states) {
    WsLayout w{};
    const size_t E = pr.bf16 ? 2 : 4;
    const size_t BH = (size_t)pr.B * pr.H;
    const size_t NT = pr.T > 0 ? ((size_t)pr.T + pr.C - 1) / pr.C : 0;
    const size_t gw = pr.gate == kGateVector ? (size_t)pr.dk : 1;
    size_t off = 0;
    w.gam = off;
    off += al256(pr.gate == kGateNone ? 0 : BH * pr.T * gw * 4);
    w.Tm = off;
    off += al256(BH * NT * pr.C * pr.C * E);
    w.Pm = off;
    off += al256(BH * NT * pr.C * pr.C * E);
    w.lam = off;
    if (backward) off += al256(BH * NT * pr.C * pr.dv * E);
    w.dS1 = off;
    if (backward) off += al256(BH * NT * (size_t)pr.dv * pr.dk * E);
    w.states = off;
    if (need_states) off += al256(BH * NT * (size_t)pr.dv * pr.dk * E);
    w.total = off;
    return w;
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
