"""Parity of the recurrent (decode) entry point dn_recurrent_fwd with the fp64
sequential oracle: o for every step and the state after the last one, for all
gates, both I/O types, dk in {16, ..., 128}, dv different from dk, one step and
several; a zero-step call leaves the state alone; and decoding after a chunkwise
prefill continues the same sequence."""
import numpy as np
import pytest
import torch

import oracle
from delta_rule_linear_gated_amd import binding as B
from delta_rule_linear_gated_amd import workloads as W
from helpers import TOL, nthreads, rel_err, say

pytestmark = pytest.mark.gpu

STATE_TOL = 1e-4   # the state is fp32 in the kernel whatever the I/O type

CASES = [
    # gate, dtype, B, H, T, dk, dv
    ("scalar", "bf16", 2, 4, 1, 128, 128),
    ("scalar", "bf16", 1, 3, 9, 128, 128),
    ("vector", "bf16", 2, 2, 5, 64, 64),
    ("none", "fp32", 1, 2, 7, 32, 32),
    ("scalar", "fp32", 2, 2, 16, 16, 16),
    ("vector", "fp32", 1, 2, 3, 128, 64),
    ("none", "bf16", 1, 1, 4, 64, 128),
]


def _inputs(gate, dtype, Bn, H, T, dk, dv, seed):
    w = W.custom(Bn, H, T, dk, dv, 16, gate, dtype, h0_std=0.5, seed=seed)
    inp = W.make_inputs(w)
    if inp["h0"] is None:
        inp["h0"] = torch.zeros(Bn, H, dv, dk)
    return inp


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_recurrent_matches_oracle(case):
    gate, dtype, Bn, H, T, dk, dv = case
    say(f"[recurrent] gate={gate} dtype={dtype} B={Bn} H={H} T={T} dk={dk} dv={dv}")
    inp = _inputs(gate, dtype, Bn, H, T, dk, dv, seed=31)
    d = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    state = d["h0"].clone()
    o = B.recurrent_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], state)
    torch.cuda.synchronize()
    f = {n: W.to_f64(t) for n, t in inp.items()}
    o_ref, s_ref = oracle.forward(f["q"], f["k"], f["v"], f["beta"], f["g"], f["h0"], nthreads=nthreads())
    eo, es = rel_err(W.to_f64(o.cpu()), o_ref), rel_err(W.to_f64(state.cpu()), s_ref)
    say(f"  o err {eo:.2e}  state err {es:.2e}")
    assert eo <= TOL[dtype]
    assert es <= STATE_TOL


def test_zero_steps_leave_the_state():
    inp = _inputs("scalar", "bf16", 1, 2, 0, 64, 64, seed=3)
    d = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    state = d["h0"].clone()
    B.recurrent_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], state)
    torch.cuda.synchronize()
    assert torch.equal(state, d["h0"])


@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_decode_after_chunked_prefill(gate):
    """Prefill T0 tokens with the chunkwise forward, then decode T1 more with the
    recurrent kernel from its hT: outputs and final state match the oracle run over
    all T0 + T1 tokens."""
    T0, T1 = 200, 6
    inp = _inputs(gate, "bf16", 1, 2, T0 + T1, 128, 128, seed=11)
    d = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    sl = lambda t, a, b: None if t is None else t[:, :, a:b].contiguous()
    o0, hT, _ = B.chunk_fwd(sl(d["q"], 0, T0), sl(d["k"], 0, T0), sl(d["v"], 0, T0), sl(d["beta"], 0, T0),
                            sl(d["g"], 0, T0), d["h0"], C=64, save_states=False)
    o1 = B.recurrent_fwd(sl(d["q"], T0, T0 + T1), sl(d["k"], T0, T0 + T1), sl(d["v"], T0, T0 + T1),
                         sl(d["beta"], T0, T0 + T1), sl(d["g"], T0, T0 + T1), hT)
    torch.cuda.synchronize()
    f = {n: W.to_f64(t) for n, t in inp.items()}
    o_ref, s_ref = oracle.forward(f["q"], f["k"], f["v"], f["beta"], f["g"], f["h0"], nthreads=nthreads())
    o = np.concatenate([W.to_f64(o0.cpu()), W.to_f64(o1.cpu())], axis=2)
    eo, es = rel_err(o, o_ref), rel_err(W.to_f64(hT.cpu()), s_ref)
    say(f"[prefill+decode] gate={gate}: o err {eo:.2e}  state err {es:.2e}")
    assert eo <= TOL["bf16"]
    assert es <= TOL["bf16"]   # the chunkwise prefill uses bf16 matrix-core operands
