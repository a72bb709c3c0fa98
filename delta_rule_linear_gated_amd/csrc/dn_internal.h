// dn_internal.h -- what the C-ABI layer and the kernels share: the problem
// descriptor, the workspace layout and the launch entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dn {

enum Gate { kGateNone = 0, kGateScalar = 1, kGateVector = 2 };

// Everything a launch needs.  Element pointers are device pointers; the
// element type of q/k/v/o/dO/dq/dk/dv/states/T/P/lambda/dS1 is the I/O type
// (fp32 or bf16).  Layouts are row-major:
//   q, k, dq, dk        [BH][T][DK]         v, o, dO, dv        [BH][T][DV]
//   beta, dbeta         [BH][T]   fp32      g, dg  [BH][T] or [BH][T][DK]  fp32
//   h0, hT, dh0, dhT    [BH][DV][DK] fp32   states              [BH][NT][DV][DK]
// per-chunk quantities of the forward, kept in the caller's saved buffer when
// the forward saves (the backward then reads them there) and in the workspace
// otherwise:
//   gam   fp32 in-chunk cumulative log-decay, same layout as g
//   Tm    [BH][NT][C][C]   (I + A)^{-1} of each chunk
//   Pm    [BH][NT][C][C]   causal intra-chunk score matrix of each chunk
//   Um    [BH][NT][C][DV]  U = T R of each chunk, the forward's matrix-core
//                          operand (saved buffer only: written by a forward that
//                          saves states; the chunk backward then reads it instead
//                          of recomputing it)
//   kb    [BH][T] fp32     Kaczmarz step beta_t = eta_t / (||k_t||^2 + eps)
//   krn   [BH][T] fp32     1 / (||k_t||^2 + eps)   (both only with the flag)
// workspace of the backward:
//   lam   [BH][NT][C][DV]  triangular-residual adjoint
//   dS1   [BH][NT][DV][DK] state cotangent leaving each chunk
struct Params {
    int BH, T, NT, DKr, DVr;  // runtime copies (the kernels also get them as template args)
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const float* beta;   // beta_t as the kernels use it (kb with the Kaczmarz flag)
    const float* eta;    // Kaczmarz flag: the caller's eta (read by prep and the recurrent kernel)
    const float* g;
    const float* h0;
    const float* dhT;
    void* o;
    float* hT;
    void* dq;
    void* dk;
    void* dv;
    float* dbeta;
    float* dg;
    float* dh0;
    void* states;  // read by the backward, written by the forward
    float* gam;
    void* Tm;
    void* Pm;
    void* Um;
    void* lam;
    void* dS1;
    float* kb;    // Kaczmarz flag: written by prep, read through `beta` afterwards
    float* krn;
    float eps;
    int kz;       // 1: Kaczmarz step (beta from eta and the keys)
    // chunk-parallel scan of the state passes (nseg == 1: one sequential pass).
    // Segment s covers chunks [s * seg_len, min(NT, (s + 1) * seg_len)).
    //   seg_end   [BH][nseg][DVr + DKr][DKr] fp32: each segment's state pass from a
    //             zero state (rows < DVr) and from the identity with zero V / dO
    //             (rows >= DVr: the segment's transition matrix)
    //   seg_start [BH][nseg][DVr][DKr] fp32: the true state entering each segment
    //             (forward) or leaving it (backward), from the combine
    int nseg, seg_len;
    float* seg_end;
    float* seg_start;
    // workgroups of the chunk backward resident on the device at once (the
    // distance, in workgroup ids, to the one that most likely starts next on
    // the same XCD)
    int resident;
    // phase-controlled gate: theta [BH][T][DK] fp32 and the imaginary parts of the
    // state [BH][DV][DK] fp32 (the real parts are h0 / hT and dh0 / dhT); the
    // backward of the chunkwise form writes dtheta like theta
    const float* theta;
    float* hT_im;
    const float* h0_im;
    const float* dhT_im;
    float* dh0_im;
    float* dtheta;
};

struct Problem {
    int B, H, T, dk, dv, C;
    int bf16;   // 1: bf16 I/O, 0: fp32 I/O
    int gate;   // Gate
    int kz;     // Kaczmarz step flag
    int no_scan;   // force one sequential state pass
};

// Segments of the chunk-parallel state scan for this problem: 1 (a plain
// sequential pass) unless the sequential kernels would leave most compute units
// idle (few heads); then about enough segments to fill the device, each of at
// least two chunks.  seg_len = chunks per segment.
struct ScanPlan {
    int nseg, seg_len;
};
ScanPlan scan_plan(const Problem& pr);

// Workspace carving per pass (0 forward, 1 backward with saved data, 2 backward
// recomputing it).  Offsets in bytes from the workspace base; every region
// starts on a 256-byte boundary; regions a pass does not use have size 0.
struct WsLayout {
    size_t gam, Tm, Pm, lam, dS1, states, kz, seg_end, seg_start, total;
};
WsLayout ws_layout(const Problem& pr, int pass);

// The forward's saved buffer: chunk-entry states, T, P, U, gam, Kaczmarz data
// (kb then krn) (same alignment).
struct SavedLayout {
    size_t states, Tm, Pm, Um, gam, kz, total;
};
SavedLayout saved_layout(const Problem& pr);

// Kernel launch sequences (all enqueue on `stream`, none synchronises).
hipError_t launch_forward(const Problem& pr, const Params& p, bool save_states, hipStream_t stream);
hipError_t launch_backward(const Problem& pr, const Params& p, bool have_states, hipStream_t stream);
// Combine of the chunk-parallel state scan (p.nseg > 1): p.seg_end -> p.seg_start,
// segments walked first to last (forward) or last to first (backward).
hipError_t launch_scan_combine(const Params& p, int DK, bool forward, hipStream_t stream);
// Recurrent form: T steps per head, state p.hT (fp32, in place), outputs p.o.
hipError_t launch_recurrent(const Problem& pr, const Params& p, hipStream_t stream);
// Chunkwise form of the phase-controlled gate (dn_phase.hip), chunks of 16, fp32:
//   states [BH][NT][2][DV][DK]  complex state entering each chunk (forward: written
//                               when not NULL; backward: read)
//   mats   [BH][NT][6][16][16]  T re, T im, P re, P im, G re, G im per chunk (written
//                               by the forward, read by the backward)
//   lam    [BH][NT][2][DV][16]  lambda of each chunk, row v then step (backward scratch)
//   dS1    [BH][NT][2][DV][DK]  state cotangent leaving each chunk (backward scratch)
struct PhaseBufs {
    float* states;
    float* mats;
    float* lam;
    float* dS1;
};
hipError_t launch_phase(const Problem& pr, const Params& p, const PhaseBufs& f, bool backward, hipStream_t stream);
bool supported(const Problem& pr);
// Scratch array of dn_chunk_fwd_noalloc (dn_noalloc.hip): the current device's
// address of it, looked up once per device.
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

// Optional per-kernel timing (dn_profile.cpp); no-ops unless enabled.
void prof_begin(hipStream_t stream, const char* name);
void prof_end(hipStream_t stream);

}  // namespace dn
