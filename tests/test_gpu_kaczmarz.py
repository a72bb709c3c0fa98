"""Parity of the fused Kaczmarz step (DN_FLAG_KACZMARZ: the caller passes eta and
the kernels use beta_t = eta_t / (||k_t||^2 + eps), KLA abstract) with the fp64
oracle's Kaczmarz wrappers: forward, backward (d eta and the step-size term of
dk) for every gate, both I/O types, both state policies and several eps; the step
data the forward saves; the fused call against the plain call fed the same beta;
and the recurrent (decode) entry point, alone and after a chunkwise prefill."""
import numpy as np
import pytest
import torch

import oracle
from delta_rule_linear_gated_amd import binding as B
from delta_rule_linear_gated_amd import workloads as W
from helpers import TOL, compare, gpu_run, nthreads, oracle_run, rel_err, say

pytestmark = pytest.mark.gpu

CASES = [
    # gate, dtype, B, H, T, d, C, eps
    ("scalar", "bf16", 1, 2, 200, 128, 64, 1e-6),
    ("vector", "bf16", 1, 2, 150, 128, 64, 1e-6),
    ("none", "bf16", 2, 1, 130, 64, 32, 1e-6),
    ("scalar", "fp32", 1, 2, 150, 64, 64, 0.5),
    ("vector", "fp32", 1, 2, 77, 32, 16, 1e-3),
    ("none", "fp32", 1, 1, 70, 16, 16, 0.0),
]


def _workload(case, seed):
    gate, dtype, Bn, H, T, d, C, eps = case
    return W.custom(Bn, H, T, d, d, C, gate, dtype, h0_std=0.5, kla=True, seed=seed, kz_eps=eps)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("policy", ["save", "recompute"])
def test_kaczmarz_matches_oracle(case, policy):
    w = _workload(case, 23 + case[4])
    say(f"[kaczmarz] {w.describe()} eps={w.kaczmarz_eps} policy={policy}")
    inp = W.make_inputs(w)
    gpu = gpu_run(w, inp, policy)
    ref = oracle_run(inp, kaczmarz_eps=w.kaczmarz_eps)
    compare(gpu, ref, TOL[w.dtype], label=f"{case} {policy}")
    if policy == "save":   # the step data the forward keeps for the backward
        k = W.to_f64(inp["k"])
        n = np.sum(k * k, axis=-1) + w.kaczmarz_eps
        eb = rel_err(gpu["saved_kz_beta"].double().numpy(), oracle.kaczmarz_beta(W.to_f64(inp["beta"]), k,
                                                                                  w.kaczmarz_eps))
        er = rel_err(gpu["saved_kz_rn"].double().numpy(), 1.0 / n)
        say(f"  saved beta err {eb:.2e}  1/n err {er:.2e}")
        assert eb < 1e-5 and er < 1e-5


@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_fused_equals_plain_call_with_the_same_beta(gate):
    """The fused call and the plain call given the beta it saved agree bitwise on
    everything but dk (which gains the step-size path) and dbeta (d eta = dbeta / n)."""
    w = W.custom(1, 3, 190, 128, 128, 64, gate, "bf16", h0_std=0.3, kla=True, seed=44)
    inp = W.make_inputs(w)
    d = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    eps = w.kaczmarz_eps
    o1, h1, s1 = B.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], C=64, kaczmarz_eps=eps)
    sv = B.saved_regions(s1, B.shape_of(d["q"], d["v"], d["g"], 64, eps))
    beta = sv["kz_beta"].clone()
    g1 = B.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["do"], d["dhT"], s1, C=64,
                     kaczmarz_eps=eps)
    o2, h2, s2 = B.chunk_fwd(d["q"], d["k"], d["v"], beta, d["g"], d["h0"], C=64)
    g2 = B.chunk_bwd(d["q"], d["k"], d["v"], beta, d["g"], d["h0"], d["do"], d["dhT"], s2, C=64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    for n in ("dq", "dv", "dg", "dh0"):
        assert torch.equal(g1[n], g2[n]), n
    assert torch.equal(g1["dbeta"], g2["dbeta"] * sv["kz_rn"])
    assert not torch.equal(g1["dk"], g2["dk"])


REC = [
    # gate, dtype, B, H, T, dk, dv, eps
    ("scalar", "bf16", 2, 4, 7, 128, 128, 1e-6),
    ("vector", "bf16", 1, 2, 5, 64, 64, 1e-6),
    ("none", "fp32", 1, 2, 9, 32, 48, 0.25),
]


@pytest.mark.parametrize("case", REC, ids=lambda c: "-".join(map(str, c)))
def test_recurrent_kaczmarz(case):
    gate, dtype, Bn, H, T, dk, dv, eps = case
    say(f"[kaczmarz recurrent] {case}")
    w = W.custom(Bn, H, T, dk, dv, 16, gate, dtype, h0_std=0.5, kla=True, seed=61, kz_eps=eps)
    inp = W.make_inputs(w)
    if inp["h0"] is None:
        inp["h0"] = torch.zeros(Bn, H, dv, dk)
    d = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    state = d["h0"].clone()
    o = B.recurrent_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], state, kaczmarz_eps=eps)
    torch.cuda.synchronize()
    f = {n: W.to_f64(t) for n, t in inp.items()}
    o_ref, s_ref = oracle.kaczmarz_forward(f["q"], f["k"], f["v"], f["beta"], f["g"], f["h0"], eps=eps,
                                           nthreads=nthreads())
    eo, es = rel_err(W.to_f64(o.cpu()), o_ref), rel_err(W.to_f64(state.cpu()), s_ref)
    say(f"  o err {eo:.2e}  state err {es:.2e}")
    assert eo <= TOL[dtype] and es <= 1e-4


def test_kaczmarz_prefill_then_decode():
    T0, T1, eps = 190, 5, 1e-6
    w = W.custom(1, 2, T0 + T1, 128, 128, 64, "scalar", "bf16", kla=True, seed=13, kz_eps=eps)
    inp = W.make_inputs(w)
    d = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    sl = lambda t, a, b: None if t is None else t[:, :, a:b].contiguous()
    part = lambda a, b: [sl(d[n], a, b) for n in ("q", "k", "v", "beta", "g")]
    o0, hT, _ = B.chunk_fwd(*part(0, T0), None, C=64, save_states=False, kaczmarz_eps=eps)
    o1 = B.recurrent_fwd(*part(T0, T0 + T1), hT, kaczmarz_eps=eps)
    torch.cuda.synchronize()
    f = {n: W.to_f64(t) for n, t in inp.items()}
    o_ref, s_ref = oracle.kaczmarz_forward(f["q"], f["k"], f["v"], f["beta"], f["g"], None, eps=eps,
                                           nthreads=nthreads())
    o = np.concatenate([W.to_f64(o0.cpu()), W.to_f64(o1.cpu())], axis=2)
    eo, es = rel_err(o, o_ref), rel_err(W.to_f64(hT.cpu()), s_ref)
    say(f"[kaczmarz prefill+decode] o err {eo:.2e}  state err {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
