"""Parity of the phase-controlled gate's recurrent entry point
(dn_recurrent_phase_fwd; SFDA summary, complex state, real inputs) with the
fp64 oracle (oracle/sfda.py): o for every step and the complex state after the
last one, for every gate type, both I/O types, dk in {16, ..., 128}, dv != dk,
with and without the Kaczmarz step; at zero phase it agrees with the plain
recurrent entry point; zero steps leave the state alone."""
import numpy as np
import pytest
import torch

from oracle import sfda
from delta_rule_linear_gated_amd import binding as B
from delta_rule_linear_gated_amd import workloads as W
from helpers import TOL, rel_err, say

pytestmark = pytest.mark.gpu

STATE_TOL = 1e-4   # the state is fp32 in the kernel whatever the I/O type

CASES = [
    # gate, dtype, B, H, T, dk, dv, kaczmarz eps
    ("vector", "bf16", 2, 4, 1, 128, 128, None),
    ("vector", "bf16", 1, 3, 9, 128, 128, None),
    ("scalar", "bf16", 2, 2, 5, 64, 64, None),
    ("none", "fp32", 1, 2, 7, 32, 32, None),
    ("vector", "fp32", 2, 2, 16, 16, 16, None),
    ("vector", "fp32", 1, 2, 3, 128, 64, None),
    ("vector", "bf16", 1, 2, 6, 64, 128, 1e-6),
]


def _inputs(gate, dtype, Bn, H, T, dk, dv, eps, seed):
    w = W.custom(Bn, H, T, dk, dv, 16, gate, dtype, h0_std=0.5, kla=eps is not None, seed=seed,
                 kz_eps=eps if eps is not None else 1e-6, phase=True)
    return w, W.make_inputs(w, cotangents=False)


def _run(inp, eps, gate):
    d = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    sr, si = d["h0"].clone(), d["h0_im"].clone()
    o = B.recurrent_phase_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["theta"], sr, si,
                              gate=gate, kaczmarz_eps=eps)
    torch.cuda.synchronize()
    return o.cpu(), sr.cpu(), si.cpu()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_phase_recurrent_matches_oracle(case):
    gate, dtype, Bn, H, T, dk, dv, eps = case
    say(f"[phase] gate={gate} dtype={dtype} B={Bn} H={H} T={T} dk={dk} dv={dv} eps={eps}")
    w, inp = _inputs(gate, dtype, Bn, H, T, dk, dv, eps, seed=37)
    o, sr, si = _run(inp, eps, gate)
    f = {n: W.to_f64(t) for n, t in inp.items()}
    o_ref, S_ref = sfda.forward(f["q"], f["k"], f["v"], f["beta"], f["g"], f["theta"], f["h0"], f["h0_im"],
                                eps=eps)
    S = W.to_f64(sr) + 1j * W.to_f64(si)
    eo, es = rel_err(W.to_f64(o), o_ref), float(np.max(np.abs(S - S_ref)) / np.max(np.abs(S_ref)))
    say(f"  o err {eo:.2e}  state err {es:.2e}")
    assert eo <= TOL[dtype]
    assert es <= STATE_TOL


def test_zero_phase_is_the_plain_recurrence():
    w, inp = _inputs("vector", "bf16", 2, 2, 7, 128, 128, None, seed=5)
    inp["theta"].zero_()
    inp["h0_im"].zero_()
    o, sr, si = _run(inp, None, "vector")
    d = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    state = d["h0"].clone()
    o2 = B.recurrent_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], state)
    torch.cuda.synchronize()
    assert rel_err(W.to_f64(o), W.to_f64(o2.cpu())) < 1e-5
    assert rel_err(W.to_f64(sr), W.to_f64(state.cpu())) < 1e-5
    assert torch.count_nonzero(si) == 0


def test_zero_steps_leave_the_state():
    w, inp = _inputs("vector", "bf16", 1, 2, 0, 64, 64, None, seed=3)
    o, sr, si = _run(inp, None, "vector")
    assert torch.equal(sr, inp["h0"]) and torch.equal(si, inp["h0_im"])
