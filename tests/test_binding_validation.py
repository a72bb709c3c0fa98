"""The convenience wrappers reject mismatched tensors before any C-ABI call
(CPU only: the checks run on the host and raise ValueError)."""
from __future__ import annotations

import pytest
import torch

from delta_rule_linear_gated_amd import binding as B


def _inputs(dtype=torch.bfloat16, gate="scalar", B_=2, H=3, T=40, dk=32, dv=32):
    q = torch.zeros(B_, H, T, dk, dtype=dtype)
    k = torch.zeros(B_, H, T, dk, dtype=dtype)
    v = torch.zeros(B_, H, T, dv, dtype=dtype)
    beta = torch.zeros(B_, H, T)
    g = None if gate == "none" else (torch.zeros(B_, H, T) if gate == "scalar" else torch.zeros(B_, H, T, dk))
    h0 = torch.zeros(B_, H, dv, dk)
    do = torch.zeros(B_, H, T, dv, dtype=dtype)
    dhT = torch.zeros(B_, H, dv, dk)
    return dict(q=q, k=k, v=v, beta=beta, g=g, h0=h0, do=do, dhT=dhT)


def _fwd(d):
    return B.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], C=16)


def _bwd(d):
    return B.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["do"], d["dhT"], None, C=16)


@pytest.mark.parametrize("call", [_fwd, _bwd])
@pytest.mark.parametrize("name,bad,msg", [
    ("k", lambda t: t.float(), "k must be"),
    ("v", lambda t: t.float(), "v must be"),
    ("beta", lambda t: t.bfloat16(), "beta must be"),
    ("g", lambda t: t.bfloat16(), "g must be"),
    ("h0", lambda t: t.double(), "h0 must be"),
    ("k", lambda t: t[:, :, :-1].contiguous(), "k must have shape"),
    ("v", lambda t: t[:, :2].contiguous(), "v must have shape"),
    ("beta", lambda t: t[..., :-1].contiguous(), "beta must have shape"),
    ("g", lambda t: torch.zeros(*t.shape, 5), "g must have shape"),
    ("h0", lambda t: t.transpose(-1, -2)[..., :16].contiguous(), "h0 must have shape"),
    ("q", lambda t: t.half(), "q must be float32 or bfloat16"),
    ("k", lambda t: t.transpose(-1, -2).contiguous().transpose(-1, -2), "contiguous"),
])
def test_wrappers_reject_mismatched_inputs(call, name, bad, msg):
    d = _inputs()
    d[name] = bad(d[name])
    with pytest.raises(ValueError, match=msg):
        call(d)


def test_backward_rejects_bad_cotangents():
    d = _inputs()
    d["do"] = d["do"].float()
    with pytest.raises(ValueError, match="do must be"):
        _bwd(d)
    d = _inputs()
    d["dhT"] = torch.zeros(2, 3, 32, 16)
    with pytest.raises(ValueError, match="dhT must have shape"):
        _bwd(d)


def test_vector_gate_shape_accepted_up_to_the_device_check():
    # every dtype and shape is right: the only complaint left is the CPU device
    for gate in ("none", "scalar", "vector"):
        d = _inputs(gate=gate)
        with pytest.raises(ValueError, match="CUDA device"):
            _fwd(d)
        with pytest.raises(ValueError, match="CUDA device"):
            _bwd(d)


def test_recurrent_wrappers_validate():
    d = _inputs(dtype=torch.float32)
    state = torch.zeros(2, 3, 32, 32)
    with pytest.raises(ValueError, match="beta must be"):
        B.recurrent_fwd(d["q"], d["k"], d["v"], d["beta"].double(), d["g"], state)
    with pytest.raises(ValueError, match="state must have shape"):
        B.recurrent_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], state[:, :, :16].contiguous())
    theta = torch.zeros(2, 3, 40, 32)
    with pytest.raises(ValueError, match="theta must have shape"):
        B.recurrent_phase_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], theta[:, :, :5].contiguous(), state,
                              state.clone())
    with pytest.raises(ValueError, match="CUDA device"):
        B.recurrent_phase_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], theta, state, state.clone())
