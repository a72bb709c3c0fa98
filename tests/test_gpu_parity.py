"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

* the five workloads at their full sizes, every head compared element by
  element, in the state policy each one names (the same calls bench.py times);
* reduced shapes that span several chunks and end in a ragged chunk, for every
  gate, both I/O types and every chunk size;
* properties: recomputed states give bitwise the gradients of saved states,
  runs are bitwise deterministic, NULL h0 / dhT / hT / dh0 paths, empty inputs.
"""
import numpy as np
import pytest
import torch

from delta_rule_linear_gated_amd import binding as B
from delta_rule_linear_gated_amd import workloads as W
from helpers import TOL, compare, gpu_run, oracle_run, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_workload_full_size(name):
    w = W.CONFIGS[name]
    say(f"[parity] {w.describe()}")
    inp = W.make_inputs(w)
    gpu = gpu_run(w, inp)
    ref = oracle_run(inp, kaczmarz_eps=w.kaczmarz_eps)
    compare(gpu, ref, TOL[w.dtype], label=name)


REDUCED = [
    # gate, dtype, B, H, T, d, C
    ("scalar", "bf16", 1, 2, 200, 128, 64),
    ("vector", "bf16", 1, 2, 150, 128, 64),
    ("none", "bf16", 2, 1, 130, 128, 64),
    ("scalar", "bf16", 1, 2, 100, 64, 32),
    ("vector", "bf16", 2, 1, 90, 32, 16),
    ("none", "bf16", 1, 1, 33, 16, 16),
    ("scalar", "fp32", 1, 2, 150, 64, 64),
    ("vector", "fp32", 1, 2, 77, 32, 32),
    ("none", "fp32", 1, 2, 70, 16, 16),
    ("scalar", "bf16", 1, 1, 5, 128, 64),       # a single short chunk
]


@pytest.mark.parametrize("case", REDUCED, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("policy", ["save", "recompute"])
def test_reduced_shapes(case, policy):
    gate, dtype, Bb, H, T, d, C = case
    w = W.custom(Bb, H, T, d, d, C, gate, dtype, h0_std=0.5, seed=17 + T)
    say(f"[parity] {w.describe()} policy={policy}")
    inp = W.make_inputs(w)
    compare(gpu_run(w, inp, policy), oracle_run(inp), TOL[dtype], label=f"{case} {policy}")


def test_recompute_is_bitwise_save():
    w = W.custom(2, 3, 300, 128, 128, 64, "scalar", "bf16", h0_std=0.3, seed=5)
    inp = W.make_inputs(w)
    a = gpu_run(w, inp, "save")
    b = gpu_run(w, inp, "recompute")
    for n in ("dq", "dk", "dv", "dbeta", "dg", "dh0"):
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_bitwise_deterministic(gate):
    w = W.custom(1, 4, 256, 128, 128, 64, gate, "bf16", seed=9)
    inp = W.make_inputs(w)
    a = gpu_run(w, inp)
    b = gpu_run(w, inp)
    for n in ("o", "hT", "dq", "dk", "dv", "dbeta", "dg", "dh0", "states", "saved_T", "saved_P", "saved_gam"):
        assert torch.equal(a[n], b[n]), n


def test_null_paths():
    w = W.custom(1, 2, 96, 64, 64, 32, "scalar", "bf16", seed=3)
    inp = W.make_inputs(w)
    assert inp["h0"] is None
    d = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    zeros = torch.zeros(1, 2, 64, 64, device="cuda")
    o1, h1, s1 = B.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], None, C=32)
    o2, h2, s2 = B.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], zeros, C=32)
    o3, h3, s3 = B.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], None, C=32, want_hT=False)
    assert torch.equal(o1, o2) and torch.equal(h1, h2) and torch.equal(o1, o3) and h3 is None
    g1 = B.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], None, d["do"], None, s1, C=32)
    g2 = B.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], None, d["do"], zeros, s1, C=32)
    g3 = B.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], None, d["do"], None, s1, C=32,
                     want_dh0=False)
    for n in ("dq", "dk", "dv", "dbeta", "dg", "dh0"):
        assert torch.equal(g1[n], g2[n]), n
    assert g3["dh0"] is None and torch.equal(g3["dq"], g1["dq"])
    # and against the oracle without dhT
    ref = oracle_run(inp, dhT=False)
    compare({"o": o1.cpu(), "hT": h1.cpu(), **{n: t.cpu() for n, t in g1.items()}}, ref, TOL["bf16"],
            label="null dhT")


def test_empty_inputs():
    for T in (0,):
        w = W.custom(1, 2, T, 64, 64, 64, "scalar", "bf16", h0_std=1.0, seed=4)
        inp = W.make_inputs(w)
        d = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
        o, hT, st = B.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], C=64)
        gr = B.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["do"], d["dhT"], st, C=64)
        torch.cuda.synchronize()
        assert o.numel() == 0 and torch.equal(hT, d["h0"]) and torch.equal(gr["dh0"], d["dhT"])
    w = W.custom(0, 3, 64, 64, 64, 64, "vector", "bf16", seed=4)
    inp = W.make_inputs(w)
    d = {n: (None if t is None else t.cuda()) for n, t in inp.items()}
    o, hT, st = B.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], None, C=64)
    torch.cuda.synchronize()
    assert o.numel() == 0


def test_autograd_function():
    w = W.custom(1, 2, 130, 64, 64, 64, "vector", "bf16", h0_std=0.5, seed=12)
    inp = W.make_inputs(w)
    d = {n: (None if t is None else t.cuda().requires_grad_(n in ("q", "k", "v", "beta", "g", "h0")))
         for n, t in inp.items() if n not in ("do", "dhT")}
    o, hT = B.DeltaRule.apply(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], 64, False)
    (o.float() * inp["do"].cuda().float()).sum().backward(retain_graph=True)
    ref = oracle_run({**inp, "dhT": None}, dhT=False)
    got = {"o": o.detach().cpu(), "hT": hT.detach().cpu(), "dq": d["q"].grad.cpu(), "dk": d["k"].grad.cpu(),
           "dv": d["v"].grad.cpu(), "dbeta": d["beta"].grad.cpu(), "dg": d["g"].grad.cpu(),
           "dh0": d["h0"].grad.cpu()}
    compare(got, ref, TOL["bf16"], label="autograd")
