"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/dn.h declares, sizes its buffers, and rejects bad calls on the host
before any HIP call (so no test here launches anything)."""
import ctypes
import os
import re

import pytest

from delta_rule_linear_gated_amd import binding as B
from delta_rule_linear_gated_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    txt = open(os.path.join(ROOT, "include", "dn.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(dn_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    L = B.lib()
    names = declared_functions()
    assert set(names) == set(B.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for st in (B.DN_OK, B.DN_ERR_INVALID, B.DN_ERR_SHAPE, B.DN_ERR_DTYPE, B.DN_ERR_WORKSPACE,
               B.DN_ERR_UNSUPPORTED, B.DN_ERR_HIP):
        assert B.dn_status_string(st) not in ("", "unknown status")


@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_sizes_of_the_workloads(name):
    w = W.CONFIGS[name]
    sh = B.make_shape(w.B, w.H, w.T, w.dk, w.dv, w.C, w.dtype, w.gate, w.kaczmarz_eps)
    E = 2 if w.dtype == "bf16" else 4
    NT = -(-w.T // w.C)
    gw = 0 if w.gate == "none" else (w.dk if w.gate == "vector" else 1)
    al = lambda x: -(-x // 256) * 256
    sl = B.dn_states_layout(sh)
    # saved buffer: chunk-entry states, T, P, U (io type), cumulative log-decay (fp32)
    assert sl["states"] == 0
    assert sl["T"] == al(w.B * w.H * NT * w.dv * w.dk * E)
    assert sl["P"] - sl["T"] == sl["U"] - sl["P"] == al(w.B * w.H * NT * w.C * w.C * E)
    assert sl["gam"] - sl["U"] == al(w.B * w.H * NT * w.C * w.dv * E)
    assert sl["kz"] - sl["gam"] == al(w.B * w.H * w.T * gw * 4)
    # Kaczmarz step: beta and 1 / (||k||^2 + eps) per token (fp32)
    assert sl["total"] - sl["kz"] == (al(2 * w.B * w.H * w.T * 4) if w.kla else 0)
    assert B.dn_states_bytes(sh) == sl["total"]
    f = B.dn_workspace_bytes(sh, B.DN_PASS_FWD)
    b = B.dn_workspace_bytes(sh, B.DN_PASS_BWD)
    r = B.dn_workspace_bytes(sh, B.DN_PASS_BWD_RECOMPUTE)
    assert 0 < f and 0 < b < r
    lay = B.dn_workspace_layout(sh, B.DN_PASS_BWD_RECOMPUTE)
    assert lay["total"] == r
    offs = [lay[k] for k in ("gam", "T", "P", "lam", "dS1", "states", "kz", "seg_end", "seg_start", "total")]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    # the recomputing backward holds in its workspace what the saved buffer carries,
    # except U (the chunk backward forms it again there)
    assert r - b == B.dn_states_bytes(sh) - (sl["gam"] - sl["U"])
    # with a saved buffer the backward's workspace holds only lambda and dS1 (and the
    # scan buffers, when the scan is used)
    lb = B.dn_workspace_layout(sh, B.DN_PASS_BWD)
    scan = lb["total"] - lb["seg_end"]
    assert scan == scan_bytes(w.B, w.H, w.T, w.dk, w.dv, w.C)
    assert lb["gam"] == lb["T"] == lb["P"] == lb["lam"] == 0 and lb["states"] == lb["kz"] == lb["seg_end"]
    # the forward's workspace holds gam, T, P (used when it saves nothing; U is
    # written only beside saved states)
    assert f == sl["total"] - sl["T"] - (sl["gam"] - sl["U"]) + scan


def expected_segments(B_, H, T, dv, C):
    """The scan's segment count, restated: sequential unless (dv/16) * B * H < 128
    and at least 32 chunks; then min(512 // grid, 32, NT // 4) segments of equal
    length (the last shorter), at least 2."""
    NT = -(-T // C) if T > 0 else 0
    grid = (dv // 16) * B_ * H
    if NT < 32 or grid == 0 or 2 * grid >= 256:
        return 1
    g = min(512 // grid, 32, NT // 4)
    if g < 2:
        return 1
    ln = -(-NT // g)
    return -(-NT // ln)


def scan_bytes(B_, H, T, dk, dv, C):
    G = expected_segments(B_, H, T, dv, C)
    if G == 1:
        return 0
    al = lambda x: -(-x // 256) * 256
    return al(B_ * H * G * (dv + dk) * dk * 4) + al(B_ * H * G * dv * dk * 4)


@pytest.mark.parametrize("B_,H,T,d,C,nseg", [
    (1, 4, 32768, 128, 64, 16),     # few heads, long sequence: 16 segments of 32 chunks
    (2, 4, 1024, 64, 64, 1),        # 16 chunks: sequential
    (2, 4, 2048, 64, 64, 8),        # 8 heads at d = 64, 32 chunks: 8 segments of 4
    (1, 1, 64, 16, 16, 1),          # 4 chunks: sequential
    (8, 16, 4096, 128, 64, 1),      # 128 heads fill the device: sequential
    (1, 32, 32768, 128, 64, 1),     # 32 heads x 8 row blocks = 256: sequential
    (1, 8, 8192, 128, 64, 8),       # 64 blocks: 8 segments of 16 chunks
    (1, 1, 100 * 64 + 5, 128, 64, 21),   # 101 chunks, at most 101 // 4 = 25 -> segments of 5 -> 21
    (1, 1, 37 * 64, 64, 64, 8),     # 37 chunks: 9 asked, segments of 5 -> 8
])
def test_scan_plan_and_workspace(B_, H, T, d, C, nseg):
    assert expected_segments(B_, H, T, d, C) == nseg
    sh = B.make_shape(B_, H, T, d, d, C, "bf16", "scalar")
    for pass_ in (B.DN_PASS_FWD, B.DN_PASS_BWD, B.DN_PASS_BWD_RECOMPUTE):
        lay = B.dn_workspace_layout(sh, pass_)
        assert lay["total"] - lay["seg_end"] == scan_bytes(B_, H, T, d, d, C)
    off = B.make_shape(B_, H, T, d, d, C, "bf16", "scalar", no_scan=True)
    lay = B.dn_workspace_layout(off, B.DN_PASS_FWD)
    assert lay["total"] == lay["seg_end"]


FAKE = 1 << 20  # aligned, never dereferenced: every call below fails validation first


def fwd(sh, **over):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, beta=FAKE * 4, g=FAKE * 5, h0=None, o=FAKE * 6, hT=None,
             states=None, ws=FAKE * 7, ws_bytes=1 << 40)
    a.update(over)
    return B.dn_chunk_fwd(sh, a["q"], a["k"], a["v"], a["beta"], a["g"], a["h0"], a["o"], a["hT"],
                          a["states"], a["ws"], a["ws_bytes"], 0)


def bwd(sh, **over):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, beta=FAKE * 4, g=FAKE * 5, h0=None, dout=FAKE * 8,
             dhT=None, states=None, dq=FAKE * 9, dk=FAKE * 10, dv=FAKE * 11, dbeta=FAKE * 12,
             dg=FAKE * 13, dh0=None, ws=FAKE * 14, ws_bytes=1 << 40)
    a.update(over)
    return B.dn_chunk_bwd(sh, *(a[n] for n in ("q", "k", "v", "beta", "g", "h0", "dout", "dhT", "states",
                                               "dq", "dk", "dv", "dbeta", "dg", "dh0", "ws", "ws_bytes")), 0)


SMALL = dict(B=1, H=1, T=64, dk=16, dv=16, C=16, dtype="bf16", gate="scalar")


def sh_of(**over):
    d = dict(SMALL)
    d.update(over)
    return B.make_shape(**d)


def test_validation_errors_forward():
    assert fwd(sh_of(T=-1)) == B.DN_ERR_SHAPE
    assert fwd(sh_of(dk=0)) == B.DN_ERR_SHAPE
    assert fwd(sh_of(dtype=7)) == B.DN_ERR_DTYPE
    assert fwd(sh_of(gate=3)) == B.DN_ERR_INVALID
    assert fwd(sh_of(C=48)) == B.DN_ERR_UNSUPPORTED
    assert fwd(sh_of(dk=16, dv=32)) == B.DN_ERR_UNSUPPORTED
    assert fwd(sh_of(dk=96, dv=96)) == B.DN_ERR_UNSUPPORTED
    assert fwd(sh_of(dk=128, dv=128, C=64, dtype="fp32", gate="vector")) == B.DN_ERR_UNSUPPORTED
    assert fwd(sh_of(dk=64, dv=64, C=64, dtype="fp32", gate="vector")) == B.DN_ERR_UNSUPPORTED
    assert fwd(sh_of(B=300, H=300)) == B.DN_ERR_UNSUPPORTED
    assert fwd(sh_of(), q=None) == B.DN_ERR_INVALID
    assert fwd(sh_of(), g=None) == B.DN_ERR_INVALID
    assert fwd(sh_of(gate="none")) == B.DN_ERR_INVALID                 # g given without a gate
    assert fwd(sh_of(), q=FAKE + 8) == B.DN_ERR_INVALID                # misaligned
    assert fwd(sh_of(), ws_bytes=16) == B.DN_ERR_WORKSPACE
    assert fwd(sh_of(), o=FAKE * 3) == B.DN_ERR_INVALID                # output aliases v
    assert fwd(sh_of(), o=FAKE * 7) == B.DN_ERR_INVALID                # output aliases workspace
    assert "overlaps" in B.dn_last_error()
    assert fwd(sh_of(), v=None) == B.DN_ERR_INVALID
    L = B.lib()
    assert L.dn_chunk_fwd(None, None, None, None, None, None, None, None, None, None, None, 0, None) == B.DN_ERR_INVALID


def test_validation_errors_backward():
    assert bwd(sh_of(), dq=None) == B.DN_ERR_INVALID
    assert bwd(sh_of(), dg=None) == B.DN_ERR_INVALID
    assert bwd(sh_of(gate="none"), g=None) == B.DN_ERR_INVALID         # dg given without a gate
    assert bwd(sh_of(), ws_bytes=1024) == B.DN_ERR_WORKSPACE
    assert bwd(sh_of(), dk=FAKE * 9) == B.DN_ERR_INVALID               # dk aliases dq
    assert bwd(sh_of(), dq=FAKE) == B.DN_ERR_INVALID                   # dq aliases q
    assert bwd(sh_of(T=-5)) == B.DN_ERR_SHAPE


def test_validation_errors_kaczmarz():
    for eps in (-1.0, float("nan"), float("inf")):
        assert fwd(sh_of(kaczmarz_eps=eps)) == B.DN_ERR_INVALID and "eps" in B.dn_last_error()
        assert bwd(sh_of(kaczmarz_eps=eps)) == B.DN_ERR_INVALID
        assert rec(sh_of(kaczmarz_eps=eps)) == B.DN_ERR_INVALID
    sh = sh_of()
    sh.flags = 4   # no such flag
    assert fwd(sh) == B.DN_ERR_INVALID and "flags" in B.dn_last_error()
    assert B.dn_states_bytes(sh) == 0
    # eps is ignored without the flag; with it the saved buffer gains the step data
    sh = sh_of()
    sh.eps = float("nan")
    assert B.dn_states_bytes(sh) == B.dn_states_bytes(sh_of()) > 0
    kz = sh_of(kaczmarz_eps=0.0)
    assert B.dn_states_bytes(kz) - B.dn_states_bytes(sh_of()) == 512   # 2 x 64 fp32
    assert B.dn_workspace_bytes(kz, B.DN_PASS_BWD) == B.dn_workspace_bytes(sh_of(), B.DN_PASS_BWD)


def test_workspace_grows_with_recompute():
    sh = sh_of(T=4096, dk=128, dv=128, C=64)
    sl = B.dn_states_layout(sh)
    # everything the saved buffer carries except U, which the recomputing chunk backward forms itself
    assert B.dn_workspace_bytes(sh, B.DN_PASS_BWD_RECOMPUTE) - B.dn_workspace_bytes(sh, B.DN_PASS_BWD) \
        == B.dn_states_bytes(sh) - (sl["gam"] - sl["U"])
    assert B.dn_workspace_bytes(sh, 9) == 0


def rec(sh, **over):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, beta=FAKE * 4, g=FAKE * 5, state=FAKE * 6, o=FAKE * 7)
    a.update(over)
    return B.dn_recurrent_fwd(sh, a["q"], a["k"], a["v"], a["beta"], a["g"], a["state"], a["o"], 0)


def test_validation_errors_recurrent():
    assert rec(sh_of(T=-1)) == B.DN_ERR_SHAPE
    assert rec(sh_of(dtype=7)) == B.DN_ERR_DTYPE
    assert rec(sh_of(gate=3)) == B.DN_ERR_INVALID
    assert rec(sh_of(dk=48, dv=48)) == B.DN_ERR_UNSUPPORTED
    assert rec(sh_of(dv=24)) == B.DN_ERR_UNSUPPORTED                   # dv not a multiple of 16
    assert rec(sh_of(), q=None) == B.DN_ERR_INVALID
    assert rec(sh_of(), state=None) == B.DN_ERR_INVALID
    assert rec(sh_of(gate="none")) == B.DN_ERR_INVALID                 # g given without a gate
    assert rec(sh_of(), o=FAKE * 6) == B.DN_ERR_INVALID                # o aliases the state
    assert rec(sh_of(), state=FAKE + 8) == B.DN_ERR_INVALID            # misaligned
    assert "state" in B.dn_last_error() or "aligned" in B.dn_last_error()


def recp(sh, **over):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, beta=FAKE * 4, g=FAKE * 5, theta=FAKE * 6, state_re=FAKE * 7,
             state_im=FAKE * 8, o=FAKE * 9)
    a.update(over)
    return B.dn_recurrent_phase_fwd(sh, *(a[n] for n in ("q", "k", "v", "beta", "g", "theta", "state_re",
                                                         "state_im", "o")), 0)


def test_validation_errors_recurrent_phase():
    sh = sh_of(gate="vector", T=3, dk=32, dv=32)
    assert recp(sh, theta=None) == B.DN_ERR_INVALID and "theta" in B.dn_last_error()
    assert recp(sh, state_im=None) == B.DN_ERR_INVALID and "state_im" in B.dn_last_error()
    assert recp(sh, state_im=FAKE * 7) == B.DN_ERR_INVALID and "overlaps" in B.dn_last_error()
    assert recp(sh, o=FAKE * 8) == B.DN_ERR_INVALID
    assert recp(sh, theta=FAKE * 6 + 4) == B.DN_ERR_INVALID                     # misaligned
    assert recp(sh_of(gate="none", T=3), theta=FAKE * 6) == B.DN_ERR_INVALID    # g given without a gate
    assert recp(sh_of(gate="vector", T=3, dk=48, dv=48)) == B.DN_ERR_UNSUPPORTED
    assert recp(sh_of(gate="vector", T=3, dv=24)) == B.DN_ERR_UNSUPPORTED
    assert recp(sh_of(gate="vector", T=3, kaczmarz_eps=-1.0)) == B.DN_ERR_INVALID


def test_validation_errors_chunk_phase():
    """The chunkwise phase-controlled gate: chunks of 16, d in {16, 32, 64, 128}, no Kaczmarz step,
    theta required; the backward takes the forward's states or (states NULL) recomputes them in a
    larger workspace."""
    def sh(**over):
        d = dict(B=1, H=2, T=40, dk=32, dv=32, C=16, dtype="fp32", gate="vector")
        d.update(over)
        return B.make_shape(**d)

    def fwd(s, **over):
        a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, beta=FAKE * 4, g=FAKE * 5, theta=FAKE * 6, h0_re=None, h0_im=None,
                 o=FAKE * 7, hT_re=None, hT_im=None, states=None, ws=FAKE * 16, ws_bytes=1 << 30)
        a.update(over)
        return B.dn_chunk_phase_fwd(s, a["q"], a["k"], a["v"], a["beta"], a["g"], a["theta"], a["h0_re"],
                                    a["h0_im"], a["o"], a["hT_re"], a["hT_im"], a["states"], a["ws"], a["ws_bytes"], 0)

    def bwd(s, **over):
        a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, beta=FAKE * 4, g=FAKE * 5, theta=FAKE * 6, h0_re=None,
                 h0_im=None, dout=FAKE * 8, dhT_re=None, dhT_im=None, states=FAKE * 9, dq=FAKE * 10, dk=FAKE * 11,
                 dv=FAKE * 12, dbeta=FAKE * 13, dg=FAKE * 14, dtheta=FAKE * 15, dh0_re=None, dh0_im=None,
                 ws=FAKE * 16, ws_bytes=1 << 30)
        a.update(over)
        return B.dn_chunk_phase_bwd(s, *(a[n] for n in ("q", "k", "v", "beta", "g", "theta", "h0_re", "h0_im",
                                                        "dout", "dhT_re", "dhT_im", "states", "dq", "dk", "dv",
                                                        "dbeta", "dg", "dtheta", "dh0_re", "dh0_im", "ws",
                                                        "ws_bytes")), 0)

    al = lambda x: (x + 255) // 256 * 256
    # NT = ceil(40 / 16) = 3: chunk states, then T, P, G per chunk (complex, 16 x 16)
    assert B.dn_phase_states_bytes(sh()) == al(1 * 2 * 3 * 2 * 32 * 32 * 4) + al(1 * 2 * 3 * 6 * 16 * 16 * 4)
    assert B.dn_phase_workspace_bytes(sh(), B.DN_PASS_FWD) == al(1 * 2 * 3 * 6 * 16 * 16 * 4)
    assert B.dn_phase_workspace_bytes(sh(), B.DN_PASS_BWD) == al(2 * 3 * 2 * 32 * 16 * 4) + al(2 * 3 * 2 * 32 * 32 * 4)
    nbwd = al(2 * 3 * 2 * 32 * 16 * 4) + al(2 * 3 * 2 * 32 * 32 * 4)
    assert B.dn_phase_workspace_bytes(sh(), B.DN_PASS_BWD_RECOMPUTE) == nbwd + B.dn_phase_states_bytes(sh())
    assert B.dn_phase_states_bytes(sh(C=64)) == 0
    assert B.dn_phase_workspace_bytes(sh(C=64), B.DN_PASS_BWD) == 0
    assert fwd(sh(C=64)) == B.DN_ERR_UNSUPPORTED
    assert B.dn_phase_states_bytes(sh(dk=128, dv=128)) == al(2 * 3 * 2 * 128 * 128 * 4) + al(2 * 3 * 6 * 16 * 16 * 4)
    assert fwd(sh(dk=48, dv=48)) == B.DN_ERR_UNSUPPORTED
    assert fwd(sh(dk=256, dv=256)) == B.DN_ERR_UNSUPPORTED
    assert fwd(sh(dk=32, dv=16)) == B.DN_ERR_UNSUPPORTED
    assert fwd(B.make_shape(1, 2, 40, 32, 32, 16, "fp32", "vector", kaczmarz_eps=1e-6)) == B.DN_ERR_UNSUPPORTED
    assert fwd(sh(), theta=None) == B.DN_ERR_INVALID
    assert fwd(sh(gate="none")) == B.DN_ERR_INVALID                     # g given without a gate
    assert fwd(sh(), o=FAKE * 3) == B.DN_ERR_INVALID                    # output aliases v
    assert fwd(sh(), hT_re=FAKE * 20, hT_im=FAKE * 20) == B.DN_ERR_INVALID
    # states NULL: the workspace must also hold the recomputed states and matrices
    assert bwd(sh(), states=None, ws_bytes=nbwd) == B.DN_ERR_WORKSPACE
    assert bwd(sh(), states=None, h0_re=FAKE * 10) == B.DN_ERR_INVALID   # h0 (read to recompute) aliases dq
    assert fwd(sh(), ws=None) == B.DN_ERR_INVALID                       # no states: the matrices need a workspace
    assert fwd(sh(), ws_bytes=100) == B.DN_ERR_WORKSPACE
    assert fwd(sh(), o=FAKE * 16) == B.DN_ERR_INVALID                   # output aliases the workspace
    assert bwd(sh(), ws=None) == B.DN_ERR_INVALID
    assert bwd(sh(), ws_bytes=100) == B.DN_ERR_WORKSPACE
    assert bwd(sh(), dtheta=None) == B.DN_ERR_INVALID
    assert bwd(sh(), dg=None) == B.DN_ERR_INVALID
    assert bwd(sh(), dq=FAKE * 11) == B.DN_ERR_INVALID                  # dq aliases dk
    assert "overlaps" in B.dn_last_error()
