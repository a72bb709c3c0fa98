"""Guard bands around every buffer the library writes.  Each output, the saved
buffer and the workspace is the middle of a larger allocation whose bytes before
and after hold a fixed pattern; after the forward and the backward (both
policies, every gate, both I/O types, ragged lengths, the Kaczmarz step, the
chunk-parallel scan), the phase-controlled gate, the allocation-free forward and
decode, every pattern is intact and no input has changed."""
import pytest
import torch

from delta_rule_linear_gated_amd import binding as B
from delta_rule_linear_gated_amd import workloads as W
from helpers import say

pytestmark = pytest.mark.gpu

GUARD = 4096     # bytes on each side: a multiple of 256, so the middle keeps its alignment
PATTERN = 0xA5


class Guarded:
    """Outputs carved from the middle of pattern-filled byte allocations."""

    def __init__(self):
        self.bufs = []

    def buf(self, name, nbytes, dtype=torch.uint8, shape=None):
        raw = torch.full((nbytes + 2 * GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        mid = raw[GUARD:GUARD + nbytes]
        self.bufs.append((name, raw, nbytes))
        if dtype == torch.uint8:
            return mid
        t = mid.view(dtype)
        return t.view(shape) if shape is not None else t

    def like(self, name, t):
        return self.buf(name, t.numel() * t.element_size(), t.dtype, t.shape)

    def check(self, label):
        torch.cuda.synchronize()
        for name, raw, n in self.bufs:
            lo, hi = raw[:GUARD], raw[GUARD + n:]
            assert bool((lo == PATTERN).all()), f"{label}: bytes before {name} overwritten"
            assert bool((hi == PATTERN).all()), f"{label}: bytes after {name} overwritten"
        say(f"[guard] {label}: {len(self.bufs)} buffers intact")


def _inputs(w):
    inp = W.make_inputs(w)
    return {n: (None if t is None else t.cuda()) for n, t in inp.items()}


def _same_inputs(d, ref, label):
    for n, t in ref.items():
        if t is not None:
            assert torch.equal(d[n], t), f"{label}: input {n} changed"


def _ok(st):
    assert st == B.DN_OK, B.dn_last_error()


CHUNK_CASES = [
    # gate, dtype, B, H, T, d, C, kaczmarz
    ("scalar", "bf16", 2, 3, 64 * 2 + 17, 128, 64, False),
    ("vector", "bf16", 1, 2, 64 + 33, 128, 64, False),
    ("none", "fp32", 2, 2, 32 * 3 + 7, 64, 32, False),
    ("vector", "fp32", 1, 3, 16 * 5 + 9, 32, 16, False),
    ("scalar", "bf16", 1, 2, 64 * 3 + 1, 128, 64, True),
    ("scalar", "bf16", 1, 1, 16 * 37 + 3, 64, 16, False),   # few heads, 38 chunks: the scan
]


@pytest.mark.parametrize("policy", ["save", "recompute"])
@pytest.mark.parametrize("case", CHUNK_CASES, ids=lambda c: "-".join(map(str, c)))
def test_chunk_forward_backward_stay_in_bounds(case, policy):
    gate, dtype, Bn, H, T, d, C, kz = case
    w = W.custom(Bn, H, T, d, d, C, gate, dtype, h0_std=0.5, kla=kz, seed=90 + T)
    x = _inputs(w)
    ref = {n: (None if t is None else t.clone()) for n, t in x.items()}
    eps = w.kaczmarz_eps if kz else None
    sh = B.shape_of(x["q"], x["v"], x["g"], C, eps)
    g = Guarded()
    o, hT = g.like("o", x["v"]), g.like("hT", x["h0"])
    states = g.buf("states", B.dn_states_bytes(sh)) if policy == "save" else None
    nwf = B.dn_workspace_bytes(sh, B.DN_PASS_FWD)
    wsf = g.buf("ws_fwd", nwf)
    _ok(B.dn_chunk_fwd(sh, x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], o, hT, states, wsf, nwf))
    g.check(f"{case} {policy} forward")
    grads = {n: g.like(n, x[m]) for n, m in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dbeta", "beta"),
                                             ("dh0", "h0"))}
    grads["dg"] = None if x["g"] is None else g.like("dg", x["g"])
    nwb = B.dn_workspace_bytes(sh, B.DN_PASS_BWD if policy == "save" else B.DN_PASS_BWD_RECOMPUTE)
    wsb = g.buf("ws_bwd", nwb)
    _ok(B.dn_chunk_bwd(sh, x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], x["do"], x["dhT"], states,
                       grads["dq"], grads["dk"], grads["dv"], grads["dbeta"], grads["dg"], grads["dh0"], wsb, nwb))
    g.check(f"{case} {policy} backward")
    _same_inputs(x, ref, f"{case} {policy}")


def test_allocation_free_forward_stays_in_bounds():
    w = W.custom(2, 2, 64 * 2 + 5, 128, 128, 64, "scalar", "bf16", h0_std=0.5, seed=97)
    x = _inputs(w)
    sh = B.shape_of(x["q"], x["v"], x["g"], 64)
    g = Guarded()
    o, hT = g.like("o", x["v"]), g.like("hT", x["h0"])
    _ok(B.dn_chunk_fwd_noalloc(sh, x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], o, hT))
    g.check("allocation-free forward")


@pytest.mark.parametrize("gate,dtype,d", [("vector", "bf16", 64), ("scalar", "fp32", 32), ("none", "bf16", 16),
                                          ("vector", "fp32", 128)])
def test_chunk_phase_stays_in_bounds(gate, dtype, d):
    w = W.custom(2, 2, 16 * 3 + 7, d, d, 16, gate, dtype, h0_std=0.5, seed=98, phase=True)
    x = _inputs(w)
    ref = {n: (None if t is None else t.clone()) for n, t in x.items()}
    sh = B.make_shape(w.B, w.H, w.T, d, d, 16, dtype, gate)
    g = Guarded()
    o, hr, hi = g.like("o", x["v"]), g.like("hT_re", x["h0"]), g.like("hT_im", x["h0"])
    states = g.buf("states", B.dn_phase_states_bytes(sh))
    _ok(B.dn_chunk_phase_fwd(sh, x["q"], x["k"], x["v"], x["beta"], x["g"], x["theta"], x["h0"], x["h0_im"], o, hr,
                             hi, states))
    g.check(f"phase {gate} {dtype} d={d} forward")
    gr = {n: g.like(n, x[m]) for n, m in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dbeta", "beta"),
                                          ("dtheta", "theta"), ("dh0_re", "h0"), ("dh0_im", "h0"))}
    gr["dg"] = None if x["g"] is None else g.like("dg", x["g"])
    nws = B.dn_phase_workspace_bytes(sh, B.DN_PASS_BWD)
    ws = g.buf("ws", nws)
    _ok(B.dn_chunk_phase_bwd(sh, x["q"], x["k"], x["v"], x["beta"], x["g"], x["theta"], x["h0"], x["h0_im"],
                             x["do"], x["dhT"], x["dhT_im"], states, gr["dq"], gr["dk"], gr["dv"], gr["dbeta"],
                             gr["dg"], gr["dtheta"], gr["dh0_re"], gr["dh0_im"], ws, nws))
    g.check(f"phase {gate} {dtype} d={d} backward")
    nwr = B.dn_phase_workspace_bytes(sh, B.DN_PASS_BWD_RECOMPUTE)   # the backward recomputing the states
    wsr = g.buf("ws_recompute", nwr)
    _ok(B.dn_chunk_phase_bwd(sh, x["q"], x["k"], x["v"], x["beta"], x["g"], x["theta"], x["h0"], x["h0_im"],
                             x["do"], x["dhT"], x["dhT_im"], None, gr["dq"], gr["dk"], gr["dv"], gr["dbeta"],
                             gr["dg"], gr["dtheta"], gr["dh0_re"], gr["dh0_im"], wsr, nwr))
    g.check(f"phase {gate} {dtype} d={d} backward, recomputed states")
    _same_inputs(x, ref, f"phase {gate}")


@pytest.mark.parametrize("phase", [False, True])
def test_decode_stays_in_bounds(phase):
    w = W.custom(3, 2, 5, 64, 64, 16, "vector", "bf16", h0_std=0.5, seed=99, phase=phase)
    x = _inputs(w)
    sh = B.make_shape(w.B, w.H, w.T, 64, 64, 16, "bf16", "vector")
    g = Guarded()
    o = g.like("o", x["v"])
    sr = g.like("state", x["h0"])
    sr.copy_(x["h0"])
    if phase:
        si = g.like("state_im", x["h0"])
        si.copy_(x["h0_im"])
        _ok(B.dn_recurrent_phase_fwd(sh, x["q"], x["k"], x["v"], x["beta"], x["g"], x["theta"], sr, si, o))
    else:
        _ok(B.dn_recurrent_fwd(sh, x["q"], x["k"], x["v"], x["beta"], x["g"], sr, o))
    g.check(f"decode phase={phase}")
