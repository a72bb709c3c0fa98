// dn_api.cpp -- the C ABI (include/dn.h): host-side validation, workspace
// carving and dispatch to the kernel launchers.  Pure host code: every check
// runs before the first HIP call, so a bad call enqueues nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <utility>
#include <vector>

#include "dn.h"
#include "dn_internal.h"

namespace {

thread_local char g_err[512] = "";

dn_status fail(dn_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

#define DN_TRY(expr)                      \
    do {                                  \
        const dn_status st_ = (expr);     \
        if (st_ != DN_OK) return st_;     \
    } while (0)

dn_status check_flags(const dn_shape* s) {
    if (s->flags & ~(DN_FLAG_KACZMARZ | DN_FLAG_NO_SCAN)) return fail(DN_ERR_INVALID, "unknown flags 0x%x", s->flags);
    if ((s->flags & DN_FLAG_KACZMARZ) && !(std::isfinite(s->eps) && s->eps >= 0.f))
        return fail(DN_ERR_INVALID, "Kaczmarz eps must be finite and >= 0");
    return DN_OK;
}

struct Dims {
    size_t BH, T, NT, dk, dv, E, gw;
};

dn_status check_shape(const dn_shape* s, dn::Problem* pr, Dims* d) {
    if (!s) return fail(DN_ERR_INVALID, "shape is NULL");
    if (s->B < 0 || s->H < 0 || s->T < 0) return fail(DN_ERR_SHAPE, "B, H, T must be >= 0");
    if (s->dk <= 0 || s->dv <= 0) return fail(DN_ERR_SHAPE, "dk and dv must be > 0");
    if (s->C <= 0) return fail(DN_ERR_SHAPE, "chunk size C must be > 0");
    if (s->dtype != DN_F32 && s->dtype != DN_BF16) return fail(DN_ERR_DTYPE, "unknown dtype %d", s->dtype);
    if (s->gate < DN_GATE_NONE || s->gate > DN_GATE_VECTOR) return fail(DN_ERR_INVALID, "unknown gate %d", s->gate);
    DN_TRY(check_flags(s));
    if ((long long)s->B * s->H > 65535) return fail(DN_ERR_UNSUPPORTED, "B*H must be <= 65535");
    if (s->C != 16 && s->C != 32 && s->C != 64) return fail(DN_ERR_UNSUPPORTED, "C must be 16, 32 or 64");
    if (s->dk != s->dv) return fail(DN_ERR_UNSUPPORTED, "dk must equal dv");
    if (s->dk != 16 && s->dk != 32 && s->dk != 64 && s->dk != 128)
        return fail(DN_ERR_UNSUPPORTED, "dk must be 16, 32, 64 or 128");
    pr->B = s->B;
    pr->H = s->H;
    pr->T = s->T;
    pr->dk = s->dk;
    pr->dv = s->dv;
    pr->C = s->C;
    pr->bf16 = s->dtype == DN_BF16;
    pr->gate = s->gate;
    pr->kz = (s->flags & DN_FLAG_KACZMARZ) ? 1 : 0;
    pr->no_scan = (s->flags & DN_FLAG_NO_SCAN) ? 1 : 0;
    if (!dn::supported(*pr))
        return fail(DN_ERR_UNSUPPORTED, "no kernel for dtype=%s gate=%d C=%d d=%d (LDS budget)",
                    pr->bf16 ? "bf16" : "fp32", s->gate, s->C, s->dk);
    d->BH = (size_t)s->B * s->H;
    d->T = (size_t)s->T;
    d->NT = s->T > 0 ? ((size_t)s->T + s->C - 1) / s->C : 0;
    d->dk = (size_t)s->dk;
    d->dv = (size_t)s->dv;
    d->E = pr->bf16 ? 2 : 4;
    d->gw = s->gate == DN_GATE_VECTOR ? (size_t)s->dk : 1;
    return DN_OK;
}

struct Buf {
    const char* name;
    const void* p;
    size_t bytes;
    bool output;
};

// Required pointers must be non-NULL when non-empty; all must be 16-byte
// aligned; outputs may not overlap anything else.
dn_status check_buffers(const std::vector<Buf>& bufs) {
    for (const Buf& b : bufs) {
        if (b.bytes == 0 || !b.p) continue;
        if (reinterpret_cast<uintptr_t>(b.p) % 16 != 0)
            return fail(DN_ERR_INVALID, "%s is not 16-byte aligned", b.name);
    }
    for (size_t i = 0; i < bufs.size(); ++i) {
        const Buf& a = bufs[i];
        if (!a.p || a.bytes == 0) continue;
        for (size_t j = i + 1; j < bufs.size(); ++j) {
            const Buf& b = bufs[j];
            if (!b.p || b.bytes == 0 || (!a.output && !b.output)) continue;
            const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), a1 = a0 + a.bytes;
            const uintptr_t b0 = reinterpret_cast<uintptr_t>(b.p), b1 = b0 + b.bytes;
            if (a0 < b1 && b0 < a1) return fail(DN_ERR_INVALID, "%s overlaps %s", a.name, b.name);
        }
    }
    return DN_OK;
}

// Kaczmarz flag: the caller's beta argument is eta; prep writes beta_t and
// 1 / (||k_t||^2 + eps) to `region` and every later kernel reads beta there.
void set_kaczmarz(dn::Params* p, char* region, const Dims& d, float eps) {
    p->eta = p->beta;
    p->kb = reinterpret_cast<float*>(region);
    p->krn = p->kb + d.BH * d.T;
    p->beta = p->kb;
    p->eps = eps;
    p->kz = 1;
}

// The scan plan and its buffers (in the workspace; unused when nseg == 1).
void set_scan(dn::Params* p, const dn::Problem& pr, char* ws, const dn::WsLayout& w) {
    const dn::ScanPlan sp = dn::scan_plan(pr);
    p->nseg = sp.nseg;
    p->seg_len = sp.seg_len;
    p->seg_end = reinterpret_cast<float*>(ws + w.seg_end);
    p->seg_start = reinterpret_cast<float*>(ws + w.seg_start);
}

dn_status need(const void* p, size_t bytes, const char* name) {
    if (bytes > 0 && !p) return fail(DN_ERR_INVALID, "%s is NULL", name);
    return DN_OK;
}

}  // namespace

extern "C" {

size_t dn_states_bytes(const dn_shape* shape) {
    dn::Problem pr;
    Dims d;
    if (check_shape(shape, &pr, &d) != DN_OK) return 0;
    return dn::saved_layout(pr).total;
}

dn_status dn_states_layout(const dn_shape* shape, size_t offsets[7]) {
    dn::Problem pr;
    Dims d;
    if (!offsets) return fail(DN_ERR_INVALID, "offsets is NULL");
    DN_TRY(check_shape(shape, &pr, &d));
    const dn::SavedLayout l = dn::saved_layout(pr);
    offsets[0] = l.states;
    offsets[1] = l.Tm;
    offsets[2] = l.Pm;
    offsets[3] = l.Um;
    offsets[4] = l.gam;
    offsets[5] = l.kz;
    offsets[6] = l.total;
    return DN_OK;
}

size_t dn_workspace_bytes(const dn_shape* shape, int pass) {
    dn::Problem pr;
    Dims d;
    if (pass < DN_PASS_FWD || pass > DN_PASS_BWD_RECOMPUTE) return 0;
    if (check_shape(shape, &pr, &d) != DN_OK) return 0;
    return dn::ws_layout(pr, pass).total;
}

dn_status dn_workspace_layout(const dn_shape* shape, int pass, size_t offsets[10]) {
    dn::Problem pr;
    Dims d;
    if (!offsets) return fail(DN_ERR_INVALID, "offsets is NULL");
    if (pass < DN_PASS_FWD || pass > DN_PASS_BWD_RECOMPUTE) return fail(DN_ERR_INVALID, "unknown pass %d", pass);
    DN_TRY(check_shape(shape, &pr, &d));
    const dn::WsLayout w = dn::ws_layout(pr, pass);
    offsets[0] = w.gam;
    offsets[1] = w.Tm;
    offsets[2] = w.Pm;
    offsets[3] = w.lam;
    offsets[4] = w.dS1;
    offsets[5] = w.states;
    offsets[6] = w.kz;
    offsets[7] = w.seg_end;
    offsets[8] = w.seg_start;
    offsets[9] = w.total;
    return DN_OK;
}

dn_status dn_chunk_fwd(const dn_shape* shape, const void* q, const void* k, const void* v,
                       const float* beta, const float* g, const float* h0, void* o, float* hT,
                       void* states, void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = '\0';
    dn::Problem pr;
    Dims d;
    DN_TRY(check_shape(shape, &pr, &d));
    const size_t nk = d.BH * d.T * d.dk * d.E, nv = d.BH * d.T * d.dv * d.E;
    const size_t nb = d.BH * d.T * 4, ng = pr.gate == DN_GATE_NONE ? 0 : d.BH * d.T * d.gw * 4;
    const size_t ns = d.BH * d.dv * d.dk * 4;
    const dn::SavedLayout sl = dn::saved_layout(pr);
    const size_t nst = sl.total;
    if (pr.gate == DN_GATE_NONE && g) return fail(DN_ERR_INVALID, "g must be NULL without a gate");
    DN_TRY(need(q, nk, "q"));
    DN_TRY(need(k, nk, "k"));
    DN_TRY(need(v, nv, "v"));
    DN_TRY(need(beta, nb, "beta"));
    DN_TRY(need(g, ng, "g"));
    DN_TRY(need(o, nv, "o"));
    const dn::WsLayout w = dn::ws_layout(pr, DN_PASS_FWD);
    if (ws_bytes < w.total) return fail(DN_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, w.total);
    DN_TRY(need(ws, w.total, "workspace"));
    DN_TRY(check_buffers({{"q", q, nk, false},
                          {"k", k, nk, false},
                          {"v", v, nv, false},
                          {"beta", beta, nb, false},
                          {"g", g, ng, false},
                          {"h0", h0, ns, false},
                          {"o", o, nv, true},
                          {"hT", hT, ns, true},
                          {"states", states, nst, true},
                          {"workspace", ws, w.total, true}}));
    dn::Params p{};
    p.BH = (int)d.BH;
    p.T = (int)d.T;
    p.NT = (int)d.NT;
    p.DKr = (int)d.dk;
    p.DVr = (int)d.dv;
    p.q = q;
    p.k = k;
    p.v = v;
    p.beta = beta;
    p.g = g;
    p.h0 = h0;
    p.o = o;
    p.hT = hT;
    p.states = states;
    // gam, T and P go with the saved states when there are any (the backward reads
    // them there), else into the workspace
    char* wb = states ? static_cast<char*>(states) : static_cast<char*>(ws);
    p.gam = pr.gate == DN_GATE_NONE ? nullptr : reinterpret_cast<float*>(wb + (states ? sl.gam : w.gam));
    p.Tm = wb + (states ? sl.Tm : w.Tm);
    p.Pm = wb + (states ? sl.Pm : w.Pm);
    p.Um = states ? wb + sl.Um : nullptr;   // written only with the saved states
    if (pr.kz) set_kaczmarz(&p, wb + (states ? sl.kz : w.kz), d, shape->eps);
    set_scan(&p, pr, static_cast<char*>(ws), w);
    const hipError_t e = dn::launch_forward(pr, p, states != nullptr, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(DN_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return DN_OK;
}

dn_status dn_chunk_fwd_noalloc(const dn_shape* shape, const void* q, const void* k, const void* v,
                               const float* beta, const float* g, const float* h0, void* o, float* hT,
                               void* stream) {
    g_err[0] = '\0';
    // a bad shape needs no scratch: dn_chunk_fwd reports it
    const size_t need = dn_workspace_bytes(shape, DN_PASS_FWD);
    if (need > DN_NOALLOC_SCRATCH_BYTES)
        return fail(DN_ERR_WORKSPACE,
                    "this shape needs %zu bytes of scratch; the allocation-free forward holds %zu (use "
                    "dn_chunk_fwd with a workspace)",
                    need, (size_t)DN_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (need > 0) {
        const hipError_t e = dn::noalloc_scratch(&ws, &ws_bytes);
        if (e != hipSuccess) return fail(DN_ERR_HIP, "scratch array not found: %s", hipGetErrorString(e));
    }
    return dn_chunk_fwd(shape, q, k, v, beta, g, h0, o, hT, nullptr, ws, ws_bytes, stream);
}

dn_status dn_chunk_bwd(const dn_shape* shape, const void* q, const void* k, const void* v,
                       const float* beta, const float* g, const float* h0, const void* dout,
                       const float* dhT, const void* states, void* dq, void* dk, void* dv,
                       float* dbeta, float* dg, float* dh0, void* ws, size_t ws_bytes,
                       void* stream) {
    g_err[0] = '\0';
    dn::Problem pr;
    Dims d;
    DN_TRY(check_shape(shape, &pr, &d));
    const size_t nk = d.BH * d.T * d.dk * d.E, nv = d.BH * d.T * d.dv * d.E;
    const size_t nb = d.BH * d.T * 4, ng = pr.gate == DN_GATE_NONE ? 0 : d.BH * d.T * d.gw * 4;
    const size_t ns = d.BH * d.dv * d.dk * 4;
    const dn::SavedLayout sl = dn::saved_layout(pr);
    const size_t nst = sl.total;
    if (pr.gate == DN_GATE_NONE && (g || dg)) return fail(DN_ERR_INVALID, "g and dg must be NULL without a gate");
    DN_TRY(need(q, nk, "q"));
    DN_TRY(need(k, nk, "k"));
    DN_TRY(need(v, nv, "v"));
    DN_TRY(need(beta, nb, "beta"));
    DN_TRY(need(g, ng, "g"));
    DN_TRY(need(dout, nv, "dout"));
    DN_TRY(need(dq, nk, "dq"));
    DN_TRY(need(dk, nk, "dk"));
    DN_TRY(need(dv, nv, "dv"));
    DN_TRY(need(dbeta, nb, "dbeta"));
    DN_TRY(need(dg, ng, "dg"));
    const bool have_states = states != nullptr;
    const dn::WsLayout w = dn::ws_layout(pr, have_states ? DN_PASS_BWD : DN_PASS_BWD_RECOMPUTE);
    if (ws_bytes < w.total) return fail(DN_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, w.total);
    DN_TRY(need(ws, w.total, "workspace"));
    DN_TRY(check_buffers({{"q", q, nk, false},
                          {"k", k, nk, false},
                          {"v", v, nv, false},
                          {"beta", beta, nb, false},
                          {"g", g, ng, false},
                          {"h0", h0, ns, false},
                          {"dout", dout, nv, false},
                          {"dhT", dhT, ns, false},
                          {"states", states, nst, false},
                          {"dq", dq, nk, true},
                          {"dk", dk, nk, true},
                          {"dv", dv, nv, true},
                          {"dbeta", dbeta, nb, true},
                          {"dg", dg, ng, true},
                          {"dh0", dh0, ns, true},
                          {"workspace", ws, w.total, true}}));
    dn::Params p{};
    p.BH = (int)d.BH;
    p.T = (int)d.T;
    p.NT = (int)d.NT;
    p.DKr = (int)d.dk;
    p.DVr = (int)d.dv;
    p.q = q;
    p.k = k;
    p.v = v;
    p.dout = dout;
    p.beta = beta;
    p.g = g;
    p.h0 = h0;
    p.dhT = dhT;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.dbeta = dbeta;
    p.dg = dg;
    p.dh0 = dh0;
    char* wb = static_cast<char*>(ws);
    char* sb = have_states ? static_cast<char*>(const_cast<void*>(states)) : nullptr;
    p.lam = wb + w.lam;
    p.dS1 = wb + w.dS1;
    if (have_states) {   // the forward's saved states, gam, T and P
        p.states = sb + sl.states;
        p.gam = pr.gate == DN_GATE_NONE ? nullptr : reinterpret_cast<float*>(sb + sl.gam);
        p.Tm = sb + sl.Tm;
        p.Pm = sb + sl.Pm;
        p.Um = sb + sl.Um;
        if (pr.kz) set_kaczmarz(&p, sb + sl.kz, d, shape->eps);
    } else {             // recomputed into the workspace
        p.states = wb + w.states;
        p.gam = pr.gate == DN_GATE_NONE ? nullptr : reinterpret_cast<float*>(wb + w.gam);
        p.Tm = wb + w.Tm;
        p.Pm = wb + w.Pm;
        if (pr.kz) set_kaczmarz(&p, wb + w.kz, d, shape->eps);
    }
    set_scan(&p, pr, wb, w);
    const hipError_t e = dn::launch_backward(pr, p, have_states, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(DN_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return DN_OK;
}

}  // extern "C"

namespace {

// Shape checks of the chunkwise phase-controlled gate (chunks of 16, d <= 128).
dn_status phase_shape(const dn_shape* s, dn::Problem* pr, Dims* d) {
    if (!s) return fail(DN_ERR_INVALID, "shape is NULL");
    if (s->B < 0 || s->H < 0 || s->T < 0) return fail(DN_ERR_SHAPE, "B, H, T must be >= 0");
    if (s->dtype != DN_F32 && s->dtype != DN_BF16) return fail(DN_ERR_DTYPE, "unknown dtype %d", s->dtype);
    if (s->gate < DN_GATE_NONE || s->gate > DN_GATE_VECTOR) return fail(DN_ERR_INVALID, "unknown gate %d", s->gate);
    DN_TRY(check_flags(s));
    if (s->flags & DN_FLAG_KACZMARZ) return fail(DN_ERR_UNSUPPORTED, "the chunkwise phase gate has no Kaczmarz step");
    if ((long long)s->B * s->H > 65535) return fail(DN_ERR_UNSUPPORTED, "B*H must be <= 65535");
    if (s->C != 16) return fail(DN_ERR_UNSUPPORTED, "the chunkwise phase gate runs chunks of 16 (C must be 16)");
    if (s->dk != s->dv) return fail(DN_ERR_UNSUPPORTED, "dk must equal dv");
    if (s->dk != 16 && s->dk != 32 && s->dk != 64 && s->dk != 128)
        return fail(DN_ERR_UNSUPPORTED, "dk must be 16, 32, 64 or 128");
    *pr = dn::Problem{};
    pr->B = s->B;
    pr->H = s->H;
    pr->T = s->T;
    pr->dk = s->dk;
    pr->dv = s->dv;
    pr->C = 16;
    pr->bf16 = s->dtype == DN_BF16;
    pr->gate = s->gate;
    d->BH = (size_t)s->B * s->H;
    d->T = (size_t)s->T;
    d->NT = s->T > 0 ? ((size_t)s->T + 15) / 16 : 0;
    d->dk = (size_t)s->dk;
    d->dv = (size_t)s->dv;
    d->E = pr->bf16 ? 2 : 4;
    d->gw = s->gate == DN_GATE_VECTOR ? (size_t)s->dk : 1;
    return DN_OK;
}

// Regions of the phase gate's buffers (fp32, each rounded up to 256 bytes):
// saved = chunk states, then the per-chunk T, P, G; backward workspace = lambda,
// then the state cotangent leaving each chunk (recomputing: then the saved
// buffer's regions).
struct PhaseSizes {
    size_t st, mats, lam, ds1;
};
PhaseSizes phase_sizes(const Dims& d) {
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    return {al(d.BH * d.NT * 2 * d.dv * d.dk * 4), al(d.BH * d.NT * 6 * 16 * 16 * 4), al(d.BH * d.NT * 2 * d.dv * 16 * 4),
            al(d.BH * d.NT * 2 * d.dv * d.dk * 4)};
}

}  // namespace

extern "C" {

size_t dn_phase_states_bytes(const dn_shape* shape) {
    dn::Problem pr;
    Dims d;
    if (phase_shape(shape, &pr, &d) != DN_OK) return 0;
    const PhaseSizes z = phase_sizes(d);
    return z.st + z.mats;
}

size_t dn_phase_workspace_bytes(const dn_shape* shape, int pass) {
    dn::Problem pr;
    Dims d;
    if (phase_shape(shape, &pr, &d) != DN_OK) return 0;
    const PhaseSizes z = phase_sizes(d);
    if (pass == DN_PASS_FWD) return z.mats;
    if (pass == DN_PASS_BWD) return z.lam + z.ds1;
    if (pass == DN_PASS_BWD_RECOMPUTE) return z.lam + z.ds1 + z.st + z.mats;
    return 0;
}

dn_status dn_chunk_phase_fwd(const dn_shape* shape, const void* q, const void* k, const void* v, const float* beta,
                             const float* g, const float* theta, const float* h0_re, const float* h0_im, void* o,
                             float* hT_re, float* hT_im, float* states, void* ws, size_t ws_bytes,
                             void* stream) {
    g_err[0] = '\0';
    dn::Problem pr;
    Dims d;
    DN_TRY(phase_shape(shape, &pr, &d));
    const size_t nk = d.BH * d.T * d.dk * d.E, nv = d.BH * d.T * d.dv * d.E, nb = d.BH * d.T * 4;
    const size_t ng = pr.gate == DN_GATE_NONE ? 0 : d.BH * d.T * d.gw * 4, nth = d.BH * d.T * d.dk * 4;
    const PhaseSizes z = phase_sizes(d);
    const size_t ns = d.BH * d.dv * d.dk * 4, nst = z.st + z.mats;
    const size_t nws = states ? 0 : z.mats;   // with saved states the matrices go there
    if (pr.gate == DN_GATE_NONE && g) return fail(DN_ERR_INVALID, "g must be NULL without a gate");
    if (ws_bytes < nws) return fail(DN_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, nws);
    DN_TRY(need(ws, nws, "workspace"));
    DN_TRY(need(q, nk, "q"));
    DN_TRY(need(k, nk, "k"));
    DN_TRY(need(v, nv, "v"));
    DN_TRY(need(beta, nb, "beta"));
    DN_TRY(need(g, ng, "g"));
    DN_TRY(need(theta, nth, "theta"));
    DN_TRY(need(o, nv, "o"));
    DN_TRY(check_buffers({{"q", q, nk, false},
                          {"k", k, nk, false},
                          {"v", v, nv, false},
                          {"beta", beta, nb, false},
                          {"g", g, ng, false},
                          {"theta", theta, nth, false},
                          {"h0_re", h0_re, ns, false},
                          {"h0_im", h0_im, ns, false},
                          {"o", o, nv, true},
                          {"hT_re", hT_re, ns, true},
                          {"hT_im", hT_im, ns, true},
                          {"states", states, nst, true},
                          {"workspace", ws, nws, true}}));
    dn::Params p{};
    p.BH = (int)d.BH;
    p.T = (int)d.T;
    p.NT = (int)d.NT;
    p.DKr = (int)d.dk;
    p.DVr = (int)d.dv;
    p.q = q;
    p.k = k;
    p.v = v;
    p.beta = beta;
    p.g = g;
    p.theta = theta;
    p.h0 = h0_re;
    p.h0_im = h0_im;
    p.o = o;
    p.hT = hT_re;
    p.hT_im = hT_im;
    dn::PhaseBufs f{};
    f.states = states;
    f.mats = states ? reinterpret_cast<float*>(reinterpret_cast<char*>(states) + z.st) : static_cast<float*>(ws);
    const hipError_t e = dn::launch_phase(pr, p, f, false, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(DN_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return DN_OK;
}

dn_status dn_chunk_phase_bwd(const dn_shape* shape, const void* q, const void* k, const void* v, const float* beta,
                             const float* g, const float* theta, const float* h0_re, const float* h0_im,
                             const void* dout, const float* dhT_re, const float* dhT_im, const float* states, void* dq,
                             void* dk, void* dv, float* dbeta, float* dg, float* dtheta, float* dh0_re, float* dh0_im,
                             void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = '\0';
    dn::Problem pr;
    Dims d;
    DN_TRY(phase_shape(shape, &pr, &d));
    const size_t nk = d.BH * d.T * d.dk * d.E, nv = d.BH * d.T * d.dv * d.E, nb = d.BH * d.T * 4;
    const size_t ng = pr.gate == DN_GATE_NONE ? 0 : d.BH * d.T * d.gw * 4, nth = d.BH * d.T * d.dk * 4;
    const PhaseSizes z = phase_sizes(d);
    const size_t ns = d.BH * d.dv * d.dk * 4, nst = z.st + z.mats;
    const bool recompute = states == nullptr;   // the states and matrices go to the workspace, after lambda, dS1
    const size_t nws = z.lam + z.ds1 + (recompute ? nst : 0);
    if (pr.gate == DN_GATE_NONE && (g || dg)) return fail(DN_ERR_INVALID, "g and dg must be NULL without a gate");
    if (ws_bytes < nws) return fail(DN_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, nws);
    DN_TRY(need(ws, nws, "workspace"));
    DN_TRY(need(q, nk, "q"));
    DN_TRY(need(k, nk, "k"));
    DN_TRY(need(v, nv, "v"));
    DN_TRY(need(beta, nb, "beta"));
    DN_TRY(need(g, ng, "g"));
    DN_TRY(need(theta, nth, "theta"));
    DN_TRY(need(dout, nv, "dout"));
    DN_TRY(need(dq, nk, "dq"));
    DN_TRY(need(dk, nk, "dk"));
    DN_TRY(need(dv, nv, "dv"));
    DN_TRY(need(dbeta, nb, "dbeta"));
    DN_TRY(need(dg, ng, "dg"));
    DN_TRY(need(dtheta, nth, "dtheta"));
    DN_TRY(check_buffers({{"q", q, nk, false},
                          {"k", k, nk, false},
                          {"v", v, nv, false},
                          {"beta", beta, nb, false},
                          {"g", g, ng, false},
                          {"theta", theta, nth, false},
                          {"h0_re", h0_re, recompute ? ns : 0, false},
                          {"h0_im", h0_im, recompute ? ns : 0, false},
                          {"dout", dout, nv, false},
                          {"dhT_re", dhT_re, ns, false},
                          {"dhT_im", dhT_im, ns, false},
                          {"states", states, nst, false},
                          {"dq", dq, nk, true},
                          {"dk", dk, nk, true},
                          {"dv", dv, nv, true},
                          {"dbeta", dbeta, nb, true},
                          {"dg", dg, ng, true},
                          {"dtheta", dtheta, nth, true},
                          {"dh0_re", dh0_re, ns, true},
                          {"dh0_im", dh0_im, ns, true},
                          {"workspace", ws, nws, true}}));
    dn::Params p{};
    p.BH = (int)d.BH;
    p.T = (int)d.T;
    p.NT = (int)d.NT;
    p.DKr = (int)d.dk;
    p.DVr = (int)d.dv;
    p.q = q;
    p.k = k;
    p.v = v;
    p.beta = beta;
    p.g = g;
    p.theta = theta;
    p.dout = dout;
    p.dhT = dhT_re;
    p.dhT_im = dhT_im;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.dbeta = dbeta;
    p.dg = dg;
    p.dtheta = dtheta;
    p.dh0 = dh0_re;
    p.dh0_im = dh0_im;
    dn::PhaseBufs f{};
    f.states = recompute ? reinterpret_cast<float*>(static_cast<char*>(ws) + z.lam + z.ds1) : const_cast<float*>(states);
    f.mats = reinterpret_cast<float*>(reinterpret_cast<char*>(f.states) + z.st);
    f.lam = static_cast<float*>(ws);
    f.dS1 = reinterpret_cast<float*>(static_cast<char*>(ws) + z.lam);
    if (recompute) {   // the forward's states and matrices again (no output)
        dn::Params pf = p;
        pf.h0 = h0_re;
        pf.h0_im = h0_im;
        const hipError_t e = dn::launch_phase(pr, pf, f, false, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return fail(DN_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    }
    const hipError_t e = dn::launch_phase(pr, p, f, true, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(DN_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return DN_OK;
}

}  // extern "C"

namespace {

// Both recurrent entry points: theta == nullptr is the plain recurrence (then
// state_im must be NULL too), else the phase-controlled gate with the complex
// state (state, state_im).
dn_status recurrent_call(const dn_shape* shape, const void* q, const void* k, const void* v, const float* beta,
                         const float* g, const float* theta, float* state, float* state_im, void* o, void* stream,
                         bool phase) {
    g_err[0] = '\0';
    if (!shape) return fail(DN_ERR_INVALID, "shape is NULL");
    const dn_shape* s = shape;
    if (s->B < 0 || s->H < 0 || s->T < 0) return fail(DN_ERR_SHAPE, "B, H, T must be >= 0");
    if (s->dtype != DN_F32 && s->dtype != DN_BF16) return fail(DN_ERR_DTYPE, "unknown dtype %d", s->dtype);
    if (s->gate < DN_GATE_NONE || s->gate > DN_GATE_VECTOR) return fail(DN_ERR_INVALID, "unknown gate %d", s->gate);
    DN_TRY(check_flags(s));
    if (s->dk != 16 && s->dk != 32 && s->dk != 64 && s->dk != 128)
        return fail(DN_ERR_UNSUPPORTED, "dk must be 16, 32, 64 or 128");
    if (s->dv <= 0 || s->dv % 16 != 0) return fail(DN_ERR_UNSUPPORTED, "dv must be a positive multiple of 16");
    if ((long long)s->B * s->H * (s->dv / 16) > 0x7fffffffLL) return fail(DN_ERR_UNSUPPORTED, "B*H*dv/16 too large");
    const size_t BH = (size_t)s->B * s->H, T = (size_t)s->T, E = s->dtype == DN_BF16 ? 2 : 4;
    const size_t gw = s->gate == DN_GATE_VECTOR ? (size_t)s->dk : 1;
    const size_t nk = BH * T * s->dk * E, nv = BH * T * s->dv * E, nb = BH * T * 4;
    const size_t ng = s->gate == DN_GATE_NONE ? 0 : BH * T * gw * 4, ns = BH * s->dv * s->dk * 4;
    const size_t nth = phase ? BH * T * s->dk * 4 : 0, nsi = phase ? ns : 0;
    if (s->gate == DN_GATE_NONE && g) return fail(DN_ERR_INVALID, "g must be NULL without a gate");
    DN_TRY(need(q, nk, "q"));
    DN_TRY(need(k, nk, "k"));
    DN_TRY(need(v, nv, "v"));
    DN_TRY(need(beta, nb, "beta"));
    DN_TRY(need(g, ng, "g"));
    DN_TRY(need(theta, nth, "theta"));
    DN_TRY(need(state, ns, "state"));
    DN_TRY(need(state_im, nsi, "state_im"));
    DN_TRY(need(o, nv, "o"));
    DN_TRY(check_buffers({{"q", q, nk, false},
                          {"k", k, nk, false},
                          {"v", v, nv, false},
                          {"beta", beta, nb, false},
                          {"g", g, ng, false},
                          {"theta", theta, nth, false},
                          {"state", state, ns, true},
                          {"state_im", state_im, nsi, true},
                          {"o", o, nv, true}}));
    dn::Problem pr{};
    pr.B = s->B;
    pr.H = s->H;
    pr.T = s->T;
    pr.dk = s->dk;
    pr.dv = s->dv;
    pr.C = s->C;
    pr.bf16 = s->dtype == DN_BF16;
    pr.gate = s->gate;
    pr.kz = (s->flags & DN_FLAG_KACZMARZ) ? 1 : 0;
    dn::Params p{};
    p.BH = (int)BH;
    p.T = s->T;
    p.DKr = s->dk;
    p.DVr = s->dv;
    p.q = q;
    p.k = k;
    p.v = v;
    p.beta = beta;
    p.g = g;
    p.hT = state;
    p.o = o;
    if (phase) {
        p.theta = theta;
        p.hT_im = state_im;
    }
    if (pr.kz) {   // the step size is formed per step in the kernel
        p.eta = beta;
        p.eps = s->eps;
        p.kz = 1;
    }
    const hipError_t e = dn::launch_recurrent(pr, p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(DN_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return DN_OK;
}

}  // namespace

extern "C" {

dn_status dn_recurrent_fwd(const dn_shape* shape, const void* q, const void* k, const void* v,
                           const float* beta, const float* g, float* state, void* o, void* stream) {
    return recurrent_call(shape, q, k, v, beta, g, nullptr, state, nullptr, o, stream, false);
}

dn_status dn_recurrent_phase_fwd(const dn_shape* shape, const void* q, const void* k, const void* v,
                                 const float* beta, const float* g, const float* theta, float* state_re,
                                 float* state_im, void* o, void* stream) {
    return recurrent_call(shape, q, k, v, beta, g, theta, state_re, state_im, o, stream, true);
}

const char* dn_status_string(dn_status status) {
    switch (status) {
        case DN_OK: return "ok";
        case DN_ERR_INVALID: return "invalid argument";
        case DN_ERR_SHAPE: return "invalid shape";
        case DN_ERR_DTYPE: return "invalid dtype";
        case DN_ERR_WORKSPACE: return "workspace too small";
        case DN_ERR_UNSUPPORTED: return "unsupported configuration";
        case DN_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char* dn_last_error(void) { return g_err; }

}  // extern "C"
