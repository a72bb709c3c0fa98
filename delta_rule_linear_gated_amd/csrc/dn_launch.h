// dn_launch.h -- launch templates shared by the per-variant translation units
// (one per pass x I/O type x gate, compiled in parallel).
#pragma once

#include <atomic>

#include "dn_bwd_kernels.h"
#include "dn_fwd_kernels.h"
#include "dn_internal.h"

namespace dn {

typedef hipError_t (*LaunchFn)(const Problem&, const Params&, bool, hipStream_t);

// Entry points defined by dn_{fwd,bwd}_{bf16,f32}_g{0,1,2}.hip.
#define DN_DECLARE_VARIANT(PASS, DT, G) \
    hipError_t launch_##PASS##_##DT##_g##G(const Problem&, const Params&, bool, hipStream_t);
DN_DECLARE_VARIANT(fwd, bf16, 0) DN_DECLARE_VARIANT(fwd, bf16, 1) DN_DECLARE_VARIANT(fwd, bf16, 2)
DN_DECLARE_VARIANT(fwd, f32, 0) DN_DECLARE_VARIANT(fwd, f32, 1) DN_DECLARE_VARIANT(fwd, f32, 2)
DN_DECLARE_VARIANT(bwd, bf16, 0) DN_DECLARE_VARIANT(bwd, bf16, 1) DN_DECLARE_VARIANT(bwd, bf16, 2)
DN_DECLARE_VARIANT(bwd, f32, 0) DN_DECLARE_VARIANT(bwd, f32, 1) DN_DECLARE_VARIANT(bwd, f32, 2)

constexpr size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

// Static LDS of each kernel (bytes), mirrored from the kernels' declarations
// so that configurations that cannot fit are never instantiated.
template <typename TI, int GATE, int C, int DK> constexpr size_t prep_lds() {
    return PrepSmem<TI, GATE, C, DK>::TOTAL;
}
template <typename TI, int GATE, int C, int DK, int BV> constexpr size_t bwd_state_lds() {
    constexpr size_t E = sizeof(TI);
    constexpr int P = Pad<TI>::value, LDK = DK + P, LDC = C + P, LDV = BV + P;
    constexpr int G = GATE == kGateVector ? C + DK : C;   // gam (+ e^{gam_C} per channel)
    constexpr int NK = GATE == kGateVector ? 3 : 2;   // K, Q (+ -K Gam)
    // dO, lambda, dv, then -beta lambda (Gam) without a vector gate, dO Gam with a scalar one
    constexpr int NV = GATE == kGateVector ? 3 : (GATE == kGateScalar ? 5 : 4);
    return 4 * (G + 3 * C) + E * (BV * LDK + NK * C * LDK + 2 * C * LDC + NV * C * LDV + BV * LDC) + 128;
}
constexpr size_t kLdsMax = 160 * 1024;

// bwd_chunk's layout asserts are only meaningful when the configuration fits;
// evaluate its TOTAL lazily through this helper.
// A d_v block BV of the sequential kernels is usable when both fit in LDS.
template <typename TI, int GATE, int C, int D, int BV> constexpr bool state_fits() {
    return BV <= D && fwd_state_lds<TI, GATE, C, D, BV>() <= kLdsMax && bwd_state_lds<TI, GATE, C, D, BV>() <= kLdsMax;
}
template <typename TI, int GATE, int C, int D> struct Fits {
    static constexpr int BVMIN = D < 16 ? D : 16;
    static constexpr bool small = prep_lds<TI, GATE, C, D>() <= kLdsMax && state_fits<TI, GATE, C, D, BVMIN>();
    // fp32 with the per-channel gate cannot hold the chunk backward's tiles at D = 128,
    // nor at D = 64 with C = 64
    static constexpr bool value = small && !(sizeof(TI) == 4 && D > 64 && GATE == kGateVector) &&
                                  !(sizeof(TI) == 4 && D == 64 && GATE == kGateVector && C == 64);
};

// Compute units of the current device (cached per device).
inline int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// Workgroups of kernel K (kThreads threads, static LDS only) resident on one
// compute unit at once. The kernel is a template argument so that each kernel
// keeps a cache of its own: every kernel here has the same function type.
template <auto K> int resident_per_cu() {
    static std::atomic<int> cache{0};
    int v = cache.load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, K, kThreads, 0) != hipSuccess || v <= 0) v = 1;
        cache.store(v, std::memory_order_relaxed);
    }
    return v;
}

// d_v block of the sequential kernels: the widest of 64, 32, 16 (at most D, and
// fitting in LDS) whose grid of (D / BV) * BH workgroups still gives every
// compute unit one; the narrowest when none does (few heads: more, shorter
// chains per chunk).
template <typename TI, int GATE, int C, int D> int state_block(int BH) {
    const int cus = device_cus();
    const bool ok[3] = {state_fits<TI, GATE, C, D, 64>(), state_fits<TI, GATE, C, D, 32>(),
                        state_fits<TI, GATE, C, D, 16>()};
    const int bvs[3] = {64, 32, 16};
    int last = D < 16 ? D : 16;
    for (int i = 0; i < 3; ++i) {
        if (!ok[i]) continue;
        last = bvs[i];
        if ((D / bvs[i]) * BH >= cus) return bvs[i];
    }
    return last;
}

// OUTPUT is a template argument so that the forward and the backward units each
// instantiate only the variants they launch.
// Sequential state kernels: MODE 0 = the pass itself (forward: OUTPUT selects
// O / hT, `save` the chunk states; with segments each segment starts from the
// combine's boundary state), MODE 1 = segment summaries of the scan (DK more
// rows, the transition matrix).  The grid covers every (row block, segment,
// head); the d_v block is chosen for BH * nseg heads' worth of chains.
template <typename TI, int GATE, int C, int D, int BV, bool OUTPUT>
void launch_fwd_state(const Params& p, int BH, bool save, int mode, hipStream_t stream) {
    const int rows = D + (mode ? D : 0);
    const dim3 grid((rows / BV) * BH * p.nseg), block(kThreads);
    if (mode)
        hipLaunchKernelGGL((fwd_state_kernel<TI, GATE, C, D, BV, false, false>), grid, block, 0, stream, p);
    else if (!OUTPUT || save)
        hipLaunchKernelGGL((fwd_state_kernel<TI, GATE, C, D, BV, true, OUTPUT>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((fwd_state_kernel<TI, GATE, C, D, BV, false, true>), grid, block, 0, stream, p);
}

template <typename TI, int GATE, int C, int D, bool OUTPUT>
void fwd_state(const Params& p, int BH, bool save, int mode, hipStream_t stream) {
    const int bv = state_block<TI, GATE, C, D>(BH * p.nseg);
    if constexpr (state_fits<TI, GATE, C, D, 64>())
        if (bv == 64) return launch_fwd_state<TI, GATE, C, D, 64, OUTPUT>(p, BH, save, mode, stream);
    if constexpr (state_fits<TI, GATE, C, D, 32>())
        if (bv == 32) return launch_fwd_state<TI, GATE, C, D, 32, OUTPUT>(p, BH, save, mode, stream);
    if constexpr (state_fits<TI, GATE, C, D, 16>())
        launch_fwd_state<TI, GATE, C, D, 16, OUTPUT>(p, BH, save, mode, stream);
}

template <typename TI, int GATE, int C, int D, int BV>
void launch_bwd_state(const Params& p, int BH, int mode, hipStream_t stream) {
    const int rows = D + (mode ? D : 0);
    const dim3 grid((rows / BV) * BH * p.nseg), block(kThreads);
    if (mode)
        hipLaunchKernelGGL((bwd_state_kernel<TI, GATE, C, D, BV, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((bwd_state_kernel<TI, GATE, C, D, BV, false>), grid, block, 0, stream, p);
}

template <typename TI, int GATE, int C, int D>
void bwd_state(const Params& p, int BH, int mode, hipStream_t stream) {
    const int bv = state_block<TI, GATE, C, D>(BH * p.nseg);
    if constexpr (state_fits<TI, GATE, C, D, 64>())
        if (bv == 64) return launch_bwd_state<TI, GATE, C, D, 64>(p, BH, mode, stream);
    if constexpr (state_fits<TI, GATE, C, D, 32>())
        if (bv == 32) return launch_bwd_state<TI, GATE, C, D, 32>(p, BH, mode, stream);
    if constexpr (state_fits<TI, GATE, C, D, 16>())
        launch_bwd_state<TI, GATE, C, D, 16>(p, BH, mode, stream);
}

// The forward state pass, through the scan when the plan has segments.
template <typename TI, int GATE, int C, int D, bool OUTPUT>
hipError_t fwd_state_pass(const Params& p, int BH, bool save, const char* name, const char* sname, hipStream_t stream) {
    if (p.nseg > 1) {
        prof_begin(stream, sname);
        fwd_state<TI, GATE, C, D, OUTPUT>(p, BH, false, 1, stream);
        prof_end(stream);
        const hipError_t e = launch_scan_combine(p, D, true, stream);
        if (e != hipSuccess) return e;
    }
    prof_begin(stream, name);
    fwd_state<TI, GATE, C, D, OUTPUT>(p, BH, save, 0, stream);
    prof_end(stream);
    return hipSuccess;
}

template <typename TI, int GATE, int C, int D>
hipError_t fwd_impl(const Problem& pr, const Params& p, bool save, hipStream_t stream) {
    if constexpr (!Fits<TI, GATE, C, D>::value) {
        return hipErrorInvalidConfiguration;
    } else {
        const int BH = pr.B * pr.H;
        Params pp = p;   // resident: used by the per-channel gate's cache warming
        pp.resident = device_cus() * resident_per_cu<prep_kernel<TI, GATE, C, D>>();
        prof_begin(stream, "prep");
        hipLaunchKernelGGL((prep_kernel<TI, GATE, C, D>), dim3(p.NT, BH), dim3(kThreads), 0, stream, pp);
        prof_end(stream);
        const hipError_t e = fwd_state_pass<TI, GATE, C, D, true>(p, BH, save, "fwd_state", "fwd_summary", stream);
        return e != hipSuccess ? e : hipGetLastError();
    }
}

// The recomputing backward without segments: its forward state pass and the
// backward state pass in one launch (recompute_bwd_state_kernel), when two of its
// workgroups fit on a compute unit; false (nothing launched) otherwise.
template <typename TI, int GATE, int C, int D, int BV>
bool launch_recompute_bwd_state(const Params& p, int BH, hipStream_t stream) {
    if (resident_per_cu<recompute_bwd_state_kernel<TI, GATE, C, D, BV>>() < 2) return false;
    const int nf = (p.DVr / BV) * BH;
    prof_begin(stream, "fwd_state_recompute+bwd_state");
    hipLaunchKernelGGL((recompute_bwd_state_kernel<TI, GATE, C, D, BV>), dim3(2 * nf), dim3(kThreads), 0, stream, p,
                       nf);
    prof_end(stream);
    return true;
}

template <typename TI, int GATE, int C, int D>
bool recompute_with_bwd_state(const Params& p, int BH, hipStream_t stream) {
    const int bv = state_block<TI, GATE, C, D>(BH);
    if constexpr (state_fits<TI, GATE, C, D, 64>())
        if (bv == 64) return launch_recompute_bwd_state<TI, GATE, C, D, 64>(p, BH, stream);
    if constexpr (state_fits<TI, GATE, C, D, 32>())
        if (bv == 32) return launch_recompute_bwd_state<TI, GATE, C, D, 32>(p, BH, stream);
    if constexpr (state_fits<TI, GATE, C, D, 16>())
        if (bv == 16) return launch_recompute_bwd_state<TI, GATE, C, D, 16>(p, BH, stream);
    return false;
}

template <typename TI, int GATE, int C, int D>
hipError_t bwd_impl(const Problem& pr, const Params& p, bool have_states, hipStream_t stream) {
    if constexpr (!Fits<TI, GATE, C, D>::value) {
        return hipErrorInvalidConfiguration;
    } else {
        const int BH = pr.B * pr.H;
        bool fused = false;   // the recomputed forward state pass and bwd_state in one launch
        if (!have_states) {   // recomputation policy: gam, T, P and the states into the workspace
            Params pp = p;
            pp.resident = device_cus() * resident_per_cu<prep_kernel<TI, GATE, C, D>>();
            prof_begin(stream, "prep_recompute");
            hipLaunchKernelGGL((prep_kernel<TI, GATE, C, D>), dim3(p.NT, BH), dim3(kThreads), 0, stream, pp);
            prof_end(stream);
            fused = p.nseg == 1 && recompute_with_bwd_state<TI, GATE, C, D>(p, BH, stream);
            if (!fused) {
                const hipError_t e = fwd_state_pass<TI, GATE, C, D, false>(p, BH, true, "fwd_state_recompute",
                                                                          "fwd_summary_recompute", stream);
                if (e != hipSuccess) return e;
            }
        }
        if (p.nseg > 1) {   // the reverse scan: segment summaries of dS, then the combine
            prof_begin(stream, "bwd_summary");
            bwd_state<TI, GATE, C, D>(p, BH, 1, stream);
            prof_end(stream);
            const hipError_t e = launch_scan_combine(p, D, false, stream);
            if (e != hipSuccess) return e;
        }
        if (!fused) {
            prof_begin(stream, "bwd_state");
            bwd_state<TI, GATE, C, D>(p, BH, 0, stream);
            prof_end(stream);
        }
        // with saved states the forward also saved U; recomputed, U is formed again here
        Params pc = p;
        prof_begin(stream, "bwd_chunk");
        if (have_states) {
            pc.resident = device_cus() * resident_per_cu<bwd_chunk_kernel<TI, GATE, C, D, true>>();
            hipLaunchKernelGGL((bwd_chunk_kernel<TI, GATE, C, D, true>), dim3(p.NT, BH), dim3(kThreads), 0, stream, pc);
        } else {
            pc.resident = device_cus() * resident_per_cu<bwd_chunk_kernel<TI, GATE, C, D, false>>();
            hipLaunchKernelGGL((bwd_chunk_kernel<TI, GATE, C, D, false>), dim3(p.NT, BH), dim3(kThreads), 0, stream,
                               pc);
        }
        prof_end(stream);
        return hipGetLastError();
    }
}

template <typename TI, int GATE, int C, int D> bool fits_rt() { return Fits<TI, GATE, C, D>::value; }

// Dispatch over (dtype, gate, C, D).  F is a functor template wrapper.
#define DN_DISPATCH_D(TI, GATE, C, FN, ...)                                      \
    switch (pr.dk) {                                                             \
        case 16: return FN<TI, GATE, C, 16>(__VA_ARGS__);                        \
        case 32: return FN<TI, GATE, C, 32>(__VA_ARGS__);                        \
        case 64: return FN<TI, GATE, C, 64>(__VA_ARGS__);                        \
        case 128: return FN<TI, GATE, C, 128>(__VA_ARGS__);                      \
        default: break;                                                          \
    }
#define DN_DISPATCH_C(TI, GATE, FN, ...)                                         \
    switch (pr.C) {                                                              \
        case 16: DN_DISPATCH_D(TI, GATE, 16, FN, __VA_ARGS__) break;             \
        case 32: DN_DISPATCH_D(TI, GATE, 32, FN, __VA_ARGS__) break;             \
        case 64: DN_DISPATCH_D(TI, GATE, 64, FN, __VA_ARGS__) break;             \
        default: break;                                                          \
    }
#define DN_DISPATCH_G(TI, FN, ...)                                               \
    switch (pr.gate) {                                                           \
        case kGateNone: DN_DISPATCH_C(TI, kGateNone, FN, __VA_ARGS__) break;     \
        case kGateScalar: DN_DISPATCH_C(TI, kGateScalar, FN, __VA_ARGS__) break; \
        case kGateVector: DN_DISPATCH_C(TI, kGateVector, FN, __VA_ARGS__) break; \
        default: break;                                                          \
    }
#define DN_DISPATCH(FN, ...)                                                     \
    if (pr.bf16) {                                                               \
        DN_DISPATCH_G(bf16, FN, __VA_ARGS__)                                     \
    } else {                                                                     \
        DN_DISPATCH_G(float, FN, __VA_ARGS__)                                    \
    }


// Defines launch_<PASS>_<DT>_g<G>: dispatch over (C, D) for one I/O type and gate.
#define DN_DEFINE_VARIANT(PASS, DT, TI, G)                                                        \
    hipError_t launch_##PASS##_##DT##_g##G(const Problem& pr, const Params& p, bool flag,         \
                                           hipStream_t stream) {                                  \
        DN_DISPATCH_C(TI, G, PASS##_impl, pr, p, flag, stream)                                    \
        return hipErrorInvalidConfiguration;                                                      \
    }

}  // namespace dn
